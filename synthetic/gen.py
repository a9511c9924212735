"""Seeded generators for the six W4A16 workloads (see the package docstring).

Workloads (shapes, dtypes and value ranges of the layer being exercised):

1. tiny      AWQ, fp16, g=128, zero points;  M in {1,4};  (K,N) = (512,256)
2. decode    AWQ, fp16, g=128, zero points;  M in {1,4,16};
             (K,N) in {(4096,12288), (4096,4096), (4096,22016), (11008,4096)}
3. mid       standard (GPTQ) symmetric (no zero points), bf16, g=128;
             M in {32,64,128,256};
             (K,N) in {(8192,10240), (8192,8192), (8192,57344), (28672,8192)}
4. prefill   AWQ, fp16, g=128, zero points;  M in {2048,8192};
             (K,N) in {(8192,28672), (28672,8192), (8192,8192)}
5. actorder  standard + g_idx, fp16, g=128, zero points; M in {1,16,64,512};
             (K,N) = (8192,8192); plus a per-channel variant (g=-1, no g_idx)
6. prefill_bf16  the prefill shapes and row counts as standard (GPTQ)
             symmetric bf16 layers, g=128 (the bf16 large-M path)

fp16 scales are U[0.002, 0.02]; bf16 scales are U[0.001, 0.01]; activations
are N(0, 1).  Seeds: weights from SeedSequence([cfg_id, K, N, variant]) so one
weight set serves every M; activations from SeedSequence([cfg_id, M, K, 1]).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def seeded(*key: int) -> np.random.Generator:
    """A numpy Generator seeded from a tuple of non-negative ints."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def random_words(rng: np.random.Generator, shape) -> np.ndarray:
    """int32 words of 32 uniformly random bits (eight uniform 4-bit codes each)."""
    return rng.integers(0, 2**32, size=shape, dtype=np.uint64).astype(np.uint32).view(np.int32)


def constant_words(shape, code: int) -> np.ndarray:
    """int32 words whose eight 4-bit fields all hold ``code`` (order-free)."""
    assert 0 <= code <= 15
    return np.full(shape, np.uint32(0x11111111 * code), dtype=np.uint32).view(np.int32)


def to_bf16_bits(a) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    NaN inputs map to a quiet NaN.  Used only to produce bf16 inputs.
    """
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        r = r.copy()
        r[nan] = np.uint16(0x7FC0)
    return r


def _round_to(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp16":
        return a.astype(np.float32).astype(np.float16)
    if dtype == "bf16":
        return to_bf16_bits(a)
    raise ValueError(dtype)


def uniform_scales(rng: np.random.Generator, shape, lo: float, hi: float, dtype: str) -> np.ndarray:
    """Scales ~ U[lo, hi] rounded to fp16 (np.float16) or bf16 (uint16 bits)."""
    return _round_to(rng.uniform(lo, hi, size=shape), dtype)


def normal_acts(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """Activations ~ N(0, 1) rounded to fp16 (np.float16) or bf16 (uint16 bits)."""
    return _round_to(rng.standard_normal(size=shape, dtype=np.float32), dtype)


def actorder_gidx(rng: np.random.Generator, K: int, group_size: int) -> np.ndarray:
    """GPTQ act-order group index: every group owns exactly ``group_size`` rows,
    scattered over the input dim by a seeded random permutation."""
    assert K % group_size == 0
    base = np.arange(K, dtype=np.int64) // group_size
    return base[rng.permutation(K)].astype(np.int32)


# ----------------------------------------------------------------------------
# Workload table
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class ConfigCase:
    cfg_id: int           # 1..6 in the order of the workload list above
    name: str
    fmt: str              # "awq" (input is AWQ-packed) or "std" (standard / GPTQ-packed)
    dtype: str            # "fp16" | "bf16"  (activations, scales, bias, output)
    group_size: int       # 32, 64, 128 or -1 (per-channel)
    has_zeros: bool
    has_gidx: bool
    K: int
    N: int
    Ms: tuple
    scale_lo: float
    scale_hi: float
    variant: int = 0      # distinguishes sub-variants that share (cfg_id, K, N)

    @property
    def G(self) -> int:
        return 1 if self.group_size == -1 else self.K // self.group_size

    @property
    def label(self) -> str:
        gs = "ch" if self.group_size == -1 else f"g{self.group_size}"
        return f"{self.name}-K{self.K}-N{self.N}-{gs}"


def _cases():
    out = []
    out.append(ConfigCase(1, "tiny", "awq", "fp16", 128, True, False, 512, 256, (1, 4), 0.002, 0.02))
    for K, N in ((4096, 12288), (4096, 4096), (4096, 22016), (11008, 4096)):
        out.append(ConfigCase(2, "decode", "awq", "fp16", 128, True, False, K, N, (1, 4, 16), 0.002, 0.02))
    for K, N in ((8192, 10240), (8192, 8192), (8192, 57344), (28672, 8192)):
        out.append(ConfigCase(3, "mid", "std", "bf16", 128, False, False, K, N, (32, 64, 128, 256), 0.001, 0.01))
    for K, N in ((8192, 28672), (28672, 8192), (8192, 8192)):
        out.append(ConfigCase(4, "prefill", "awq", "fp16", 128, True, False, K, N, (2048, 8192), 0.002, 0.02))
    out.append(ConfigCase(5, "actorder", "std", "fp16", 128, True, True, 8192, 8192, (1, 16, 64, 512), 0.002, 0.02))
    out.append(ConfigCase(5, "perchannel", "std", "fp16", -1, True, False, 8192, 8192, (1, 16, 64, 512), 0.002, 0.02,
                          variant=1))
    for K, N in ((8192, 28672), (28672, 8192), (8192, 8192)):
        out.append(ConfigCase(6, "prefill_bf16", "std", "bf16", 128, False, False, K, N, (2048, 8192), 0.001, 0.01))
    return tuple(out)


CONFIGS = _cases()


def config_cases(cfg_id: int):
    return [c for c in CONFIGS if c.cfg_id == cfg_id]


def workload_case(name: str) -> ConfigCase:
    """The first case of the workload called `name` ("tiny", "decode", ...)."""
    return next(c for c in CONFIGS if c.name == name)


def make_layer_inputs(c: ConfigCase) -> dict:
    """Weights of one layer, in the checkpoint format the workload names.

    Returns a dict with
      qweight  int32  [K, N/8] (fmt "awq") or [K/8, N] (fmt "std")
      qzeros   int32  [G, N/8] or None
      scales   [G, N] fp16 (np.float16) or bf16 (uint16 bits)
      g_idx    int32  [K] or None
    """
    rng = seeded(c.cfg_id, c.K, c.N, c.variant)
    if c.fmt == "awq":
        qweight = random_words(rng, (c.K, c.N // 8))
    else:
        qweight = random_words(rng, (c.K // 8, c.N))
    qzeros = random_words(rng, (c.G, c.N // 8)) if c.has_zeros else None
    scales = uniform_scales(rng, (c.G, c.N), c.scale_lo, c.scale_hi, c.dtype)
    g_idx = actorder_gidx(rng, c.K, c.group_size) if c.has_gidx else None
    return dict(qweight=qweight, qzeros=qzeros, scales=scales, g_idx=g_idx)


def make_acts(c: ConfigCase, M: int) -> np.ndarray:
    """Activations x [M, K] for one workload row count."""
    return normal_acts(seeded(c.cfg_id, M, c.K, 1), (M, c.K), c.dtype)
