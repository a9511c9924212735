"""GPU parity of the W4A8-fp8 path (INT4 weights x FP8-E4M3 activations)
against the oracle (oracle/w4a8_oracle.py).

* w4a8_quantize: the E4M3 codes in operand order must equal the oracle's
  bit for bit (an integer decision taken in fp32 on both sides: x / s_x in
  fp32, clamp, nearest even); the block row sums agree to fp32 rounding.
* w4a8_linear: y within max |y - ref| <= 1e-2 (1 + |ref|) elementwise and
  ||y - ref||_F / ||ref||_F <= 2e-3 of the float64 result for the same
  quantized activations, element by element.
"""
import numpy as np
import pytest

import oracle as O
from synthetic import actorder_gidx, normal_acts, random_words, seeded, uniform_scales
from tests._gpu import act_dtype, filled, say, to_dev, to_host

pytestmark = pytest.mark.gpu

ELEM_TOL, FRO_TOL = 1e-2, 2e-3
SX = 0.01171875        # 0.75 * 2^-6 (exact in fp32): N(0, 1) saturates past 5.25
SX_SMALL = 0.0021      # not a power of two: |x| > 0.94 saturates


@pytest.fixture(scope="module")
def W():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import weight_only_int4_gptq_amd as W
    W.lib()
    return W


def _spread_acts(rng, shape, dtype):
    """N(0, 1) activations times 10^U(-4, 1): values from the E4M3
    subnormals up to saturation."""
    import synthetic.gen as G
    v = rng.standard_normal(size=shape).astype(np.float32) * (10.0 ** rng.uniform(-4, 1, size=shape)).astype(np.float32)
    return G._round_to(v, dtype)


def _layer(W, fmt, K, N, gs, has_z, act, dtype, seed):
    G = 1 if gs == -1 else K // gs
    rng = seeded(1301, K, N, max(gs, 0), int(has_z), int(act), seed)
    lo, hi = (0.002, 0.02) if dtype == "fp16" else (0.001, 0.01)
    qw = random_words(rng, (K, N // 8) if fmt == "awq" else (K // 8, N))
    qz = random_words(rng, (G, N // 8)) if has_z else None
    sc = uniform_scales(rng, (G, N), lo, hi, dtype)
    gi = actorder_gidx(rng, K, gs) if act else None
    lyr = W.W4A16Linear(K, N, gs, has_z, act, dtype, fmt)
    lyr.process_weights_after_loading(to_dev(qw), to_dev(qz) if has_z else None, to_dev(sc),
                                      to_dev(gi) if act else None)
    return lyr, (qw, qz, sc, gi)


QUANT_CASES = [
    # (K, group_size, act_order, dtype, x_scale)
    (512, 128, False, "fp16", SX),
    (512, 128, True, "fp16", SX),
    (1152, 128, False, "bf16", SX_SMALL),
    (1152, 128, True, "bf16", SX),
    (224, -1, False, "fp16", SX_SMALL),     # K tail: padded columns
]


@pytest.mark.parametrize("case", QUANT_CASES, ids=[f"K{c[0]}-g{c[1]}-{'act' if c[2] else 'plain'}-{c[3]}"
                                                   for c in QUANT_CASES])
def test_w4a8_quantize_bit_exact(W, case):
    import torch
    K, gs, act, dtype, sx = case
    lyr, (qw, qz, sc, gi) = _layer(W, "std", K, 32, gs, True, act, dtype, 1)
    Kp = -(-K // 128) * 128
    for M in (1, 3, 17, 130):
        say(f"w4a8_quantize K={K} g={gs} act={act} {dtype} M={M}")
        x = _spread_acts(seeded(1302, M, K), (M, K), dtype)
        xs = torch.tensor([sx], dtype=torch.float32, device="cuda")
        Mr = -(-M // 4) * 4
        xq = filled((M, Kp), torch.uint8, 0xFF)
        rs = filled((Kp // 128, Mr), torch.float32, 0xFF)
        W.w4a8_quantize(lyr.layer, M, to_dev(x), xs, lyr.tiled["perm"], xq, rs)
        torch.cuda.synchronize()
        xsorted = x[:, O.actorder_perm(gi).astype(np.int64)] if act else x
        codes = O.quantize_acts_fp8(xsorted, dtype, sx)
        assert np.array_equal(to_host(xq), O.fp8_operand_order(codes, Kp))
        ref = O.fp8_block_sums(codes, Kp)
        got = to_host(rs).astype(np.float64)
        assert np.allclose(got, ref, rtol=1e-6, atol=1e-6), np.abs(got - ref).max()


LINEAR_CASES = [
    # (name, fmt, K, N, group_size, has_zeros, act_order, dtype, bias, x_scale)
    ("awq-fp16-g128", "awq", 384, 272, 128, True, False, "fp16", False, SX),
    ("awq-fp16-g128-bias", "awq", 384, 272, 128, True, False, "fp16", True, SX_SMALL),
    ("std-bf16-g128-sym", "std", 384, 272, 128, False, False, "bf16", False, SX),
    ("std-bf16-g128-sym-bias", "std", 1152, 264, 128, False, False, "bf16", True, SX),
    ("std-fp16-g128-z-act", "std", 512, 272, 128, True, True, "fp16", True, SX),
    ("std-fp16-ch-z", "std", 384, 272, -1, True, False, "fp16", False, SX),
    ("std-bf16-ch-sym-k224", "std", 224, 40, -1, False, False, "bf16", True, SX_SMALL),
    # 272 strips: the four-wave K-split kernel with LDS activation tiles at M <= 4
    ("awq-fp16-g128-n4352", "awq", 640, 4352, 128, True, False, "fp16", True, SX),
]
LINEAR_MS = (1, 4, 5, 16, 17, 64, 130, 300)


def _check(y_bits, ref, dtype, what):
    y = O.act_to_f64(y_bits, dtype)
    r = O.check(y, ref, ELEM_TOL, FRO_TOL)
    say(f"  {what}: max_ratio={r['max_ratio']:.3e} rel_fro={r['rel_fro']:.3e}")
    assert r["ok"], (what, r)


@pytest.mark.parametrize("v", LINEAR_CASES, ids=[v[0] for v in LINEAR_CASES])
def test_w4a8_linear_matches_the_oracle(W, v):
    import torch
    name, fmt, K, N, gs, has_z, act, dtype, with_bias, sx = v
    lyr, (qw, qz, sc, gi) = _layer(W, fmt, K, N, gs, has_z, act, dtype, len(name))
    bias = uniform_scales(seeded(1303, N), (N,), -1.0, 1.0, dtype) if with_bias else None
    xs = torch.tensor([sx], dtype=torch.float32, device="cuda")
    for M in LINEAR_MS:
        say(f"w4a8 {name} M={M} kernel={W.w4a8_kernel_name(lyr.layer, M)}")
        x = normal_acts(seeded(1304, M, K), (M, K), dtype)
        ref = O.reference_w4a8_linear(x, fmt, dtype, qw, qz, sc, gs, sx, g_idx=gi, bias=bias)
        buf = filled((M + 2, N), act_dtype(dtype), 0x7F)
        lyr.apply_fp8(to_dev(x), xs, to_dev(bias) if bias is not None else None, out=buf[:M])
        torch.cuda.synchronize()
        assert (to_host(buf[M:]).view(np.uint16) == 0x7F7F).all(), "write past row M"
        _check(to_host(buf[:M]), ref, dtype, f"{name} M={M}")


FULL_CASES = [
    # workload shapes with fp8 activations: (label, fmt, K, N, gs, has_z, act, dtype, Ms)
    ("decode-awq-fp16", "awq", 4096, 12288, 128, True, False, "fp16", (1, 4, 16)),
    ("decode-down-awq-fp16", "awq", 11008, 4096, 128, True, False, "fp16", (1, 4, 16)),
    ("mid-std-bf16-sym", "std", 8192, 8192, 128, False, False, "bf16", (64, 256)),
    ("prefill-awq-fp16", "awq", 8192, 8192, 128, True, False, "fp16", (2048,)),
    ("actorder-fp16", "std", 8192, 8192, 128, True, True, "fp16", (512,)),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("v", FULL_CASES, ids=[v[0] for v in FULL_CASES])
def test_w4a8_full_size_complete(W, v):
    import torch
    label, fmt, K, N, gs, has_z, act, dtype, Ms = v
    lyr, (qw, qz, sc, gi) = _layer(W, fmt, K, N, gs, has_z, act, dtype, 7)
    q, z = O.codes_from_inputs(fmt, qw, qz)
    Wd = O.dequant(q, z, O.act_to_f64(sc, dtype), O.group_index(K, gs, gi))
    del q, z
    xs = torch.tensor([SX], dtype=torch.float32, device="cuda")
    for M in Ms:
        say(f"w4a8 full {label} M={M} kernel={W.w4a8_kernel_name(lyr.layer, M)}")
        x = normal_acts(seeded(1305, M, K), (M, K), dtype)
        xq = O.e4m3_to_f64(O.quantize_acts_fp8(x, dtype, SX)) * float(np.float32(SX))
        ref = np.concatenate([O.linear_ref(xq[a:a + 512], Wd) for a in range(0, M, 512)])
        y = lyr.apply_fp8(to_dev(x), xs)
        torch.cuda.synchronize()
        _check(to_host(y), ref, dtype, f"{label} M={M} (all {M * N} outputs)")


@pytest.mark.timeout(600)
def test_w4a8_codes_beyond_4gib(W):
    # the fp8 codes span more than 4 GiB (M K bytes): rows at both ends and
    # across the 4 GiB mark, and a ragged last tile, against the oracle
    import torch
    K, N, gs = 65536, 256, 128
    edge = (1 << 32) // K                # first row starting at byte 2^32 of the codes
    M = edge + 512 + 37
    lyr, (qw, qz, sc, gi) = _layer(W, "awq", K, N, gs, True, False, "fp16", 11)
    q, z = O.codes_from_inputs("awq", qw, qz)
    Wd = O.dequant(q, z, O.act_to_f64(sc, "fp16"), O.group_index(K, gs, gi))
    del q, z
    say(f"w4a8 beyond 4 GiB M={M} K={K} kernel={W.w4a8_kernel_name(lyr.layer, M)}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1306)
    x = torch.empty((M, K), dtype=torch.float16, device="cuda")
    for r0 in range(0, M, 4096):
        r1 = min(M, r0 + 4096)
        x[r0:r1] = torch.randn((r1 - r0, K), generator=gen, device="cuda")
    xs = torch.tensor([SX], dtype=torch.float32, device="cuda")
    y = lyr.apply_fp8(x, xs)
    torch.cuda.synchronize()
    for r0, r1 in ((0, 32), (edge - 16, edge + 16), (M - 32, M)):
        xh = to_host(x[r0:r1])
        xq = O.e4m3_to_f64(O.quantize_acts_fp8(xh, "fp16", SX)) * float(np.float32(SX))
        _check(to_host(y[r0:r1]), O.linear_ref(xq, Wd), "fp16", f"rows {r0}..{r1}")
    del x, y
    torch.cuda.empty_cache()
