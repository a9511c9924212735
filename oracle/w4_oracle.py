"""Plain, slow, obviously-correct CPU oracle for weight-only INT4 linear layers.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check of the
entry module and by the benchmark's CPU-baseline leg; never by the product
path.  Integers are handled as int64, floating point as float64.

Sources (four web pages on vLLM / SGLang quantization):

* [P1] "Quantized layer loading: AWQ / GPTQ / Marlin / fp8" (vLLM architecture
  notes): section "Data flow" gives the AWQ parameter shapes; "Boundaries and
  failures" gives group_size = -1 => per-channel (group = input size);
  "Design motivation" says AWQ packs along the output dim in a non-standard
  nibble order and the kernels want the standard (GPTQ-like) input-dim
  packing, and that GPTQ act-order carries a g_idx.
* [P2] "vLLM AWQ 4-bit quantization practice" (AutoAWQ loading / kernel
  dispatch): section 5.1 gives the standard nibble order (bits 0,4,...,28
  <-> indices 0..7), the reverse-order constant [0,4,1,5,2,6,3,7],
  pack_factor = 32 // 4 = 8 and the repack of qweight to [K // 8, N];
  section 5.3 gives the dequantization (shift-and-mask each nibble, subtract
  the zero, multiply by the scale) and the supported group sizes.
* [P3] "01. Quantization" (vLLM learning book): section 5.2 (per-group scale
  per 128 elements).
* [P4] SGLang quantization design: section 1 (create_weights /
  process_weights_after_loading / apply split).

Readings where the pages leave a point open:

* AWQ order direction: logical column j of an AWQ word sits in nibble slot
  R[j], R = [0,4,1,5,2,6,3,7] (the constant is used to build the unpack
  shifts, [P2] 5.3).  Worked word: columns 0..7 holding 0..7 pack to
  0x75316420.
* Standard zeros keep the [G, N/8] shape of the AWQ zeros with the standard
  nibble order; [P2] 5.1 names a transposed [N/8, G] view, which
  ``std_zeros_transposed`` provides.
* Zero points are used as stored, for AWQ and standard alike (no +-1).
* Without zero points the zero is 8 (symmetric 4-bit).
* A g_idx group index replaces k // group_size.
* The gfx950 tile layout (``tile_layout``) is this library's own format,
  defined in that function's docstring.

Every function below is pinned by ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import numpy as np

PACK_FACTOR = 32 // 4                       # [P2] 5.1
AWQ_REVERSE_ORDER = (0, 4, 1, 5, 2, 6, 3, 7)  # [P2] 5.1 / 5.3: slot holding logical index j
SUPPORTED_GROUP_SIZES = (-1, 32, 64, 128)   # [P2] 5.3; -1 => per-channel ([P1] boundaries)

__all__ = [
    "PACK_FACTOR", "AWQ_REVERSE_ORDER", "SUPPORTED_GROUP_SIZES",
    "u32", "to_i32", "nib", "unpack_awq", "pack_awq",
    "pack_std", "unpack_std", "pack_std_zeros", "unpack_std_zeros", "std_zeros_transposed",
    "awq_to_std", "half_to_f64", "bf16_to_f64", "act_to_f64",
    "group_index", "dequant", "linear_ref", "codes_from_inputs", "reference_linear",
    "reference_entries", "reference_moe", "actorder_perm", "gidx_status", "GIDX_OUT_OF_RANGE", "GIDX_UNEQUAL_GROUPS",
    "tile_layout", "untile_codes",
    "TILE_N", "TILE_K", "TILE_SLOT_OF_OFFSET", "check",
]


# ----------------------------------------------------------------------------
# Integer words and nibbles
# ----------------------------------------------------------------------------

def u32(words) -> np.ndarray:
    """Unsigned 32-bit value of int32 words, as int64 (slot 7 >= 8 makes the
    int32 negative, so an unsigned view is needed before shifting)."""
    return np.asarray(words).astype(np.int64) & 0xFFFFFFFF


def to_i32(values) -> np.ndarray:
    """Reinterpret non-negative int64 values < 2**32 as int32 words."""
    v = np.asarray(values, dtype=np.int64)
    assert (v >= 0).all() and (v < 2**32).all()
    return v.astype(np.uint32).view(np.int32)


def nib(words, i: int) -> np.ndarray:
    """Nibble slot i (bits [4i, 4i+4)) of each word, as int64 in 0..15.
    Shift-then-mask as in the dequantization of [P2] 5.3."""
    return (u32(words) >> (4 * i)) & 0xF


def unpack_awq(words) -> np.ndarray:
    """AWQ words [R, C] (packed along the output dim) -> codes [R, 8C].

    Logical column 8c + j of row r is nibble slot AWQ_REVERSE_ORDER[j] of
    word [r, c]; [P1] "Data flow" (qweight [K, N/8], qzeros [G, N/8], both
    packed along dim 1) and [P2] 5.1 / 5.3 (reverse order)."""
    w = np.asarray(words)
    R, C = w.shape
    out = np.empty((R, C * 8), dtype=np.int64)
    for j in range(8):
        out[:, j::8] = nib(w, AWQ_REVERSE_ORDER[j])
    return out


def pack_awq(codes) -> np.ndarray:
    """Inverse of ``unpack_awq`` (codes [R, 8C] -> AWQ words [R, C])."""
    q = np.asarray(codes, dtype=np.int64)
    R, N = q.shape
    assert N % 8 == 0 and ((q >= 0) & (q <= 15)).all()
    acc = np.zeros((R, N // 8), dtype=np.int64)
    for j in range(8):
        acc |= q[:, j::8] << (4 * AWQ_REVERSE_ORDER[j])
    return to_i32(acc)


def pack_std(codes) -> np.ndarray:
    """Codes [K, N] -> standard words [K/8, N] packed along the input dim:
    slot i of word [r, n] holds row 8r + i ([P2] 5.1: standard order, shape
    [K // 8, N])."""
    q = np.asarray(codes, dtype=np.int64)
    K, N = q.shape
    assert K % 8 == 0 and ((q >= 0) & (q <= 15)).all()
    acc = np.zeros((K // 8, N), dtype=np.int64)
    for i in range(8):
        acc |= q[i::8, :] << (4 * i)
    return to_i32(acc)


def unpack_std(words) -> np.ndarray:
    """Standard words [K/8, N] -> codes [K, N] (inverse of ``pack_std``)."""
    w = np.asarray(words)
    R, N = w.shape
    out = np.empty((R * 8, N), dtype=np.int64)
    for i in range(8):
        out[i::8, :] = nib(w, i)
    return out


def pack_std_zeros(zeros) -> np.ndarray:
    """Zero codes [G, N] -> standard zero words [G, N/8]: slot i of word
    [g, c] holds column 8c + i (standard order, output-dim packing)."""
    z = np.asarray(zeros, dtype=np.int64)
    G, N = z.shape
    assert N % 8 == 0 and ((z >= 0) & (z <= 15)).all()
    acc = np.zeros((G, N // 8), dtype=np.int64)
    for i in range(8):
        acc |= z[:, i::8] << (4 * i)
    return to_i32(acc)


def unpack_std_zeros(words) -> np.ndarray:
    """Standard zero words [G, N/8] -> zero codes [G, N]."""
    w = np.asarray(words)
    G, C = w.shape
    out = np.empty((G, C * 8), dtype=np.int64)
    for i in range(8):
        out[:, i::8] = nib(w, i)
    return out


def std_zeros_transposed(words) -> np.ndarray:
    """The [N/8, G] view of standard zero words named in [P2] 5.1."""
    return np.ascontiguousarray(np.asarray(words).T)


def awq_to_std(awq_qweight, awq_qzeros=None):
    """AWQ -> standard conversion ([P2] 5.1; [P1] "Design motivation"):
    unpack each AWQ word with the reverse order, then repack qweight along
    the input dim to [K/8, N] and the zeros, bit order fixed, to [G, N/8]."""
    std_w = pack_std(unpack_awq(awq_qweight))
    std_z = None if awq_qzeros is None else pack_std_zeros(unpack_awq(awq_qzeros))
    return std_w, std_z


# ----------------------------------------------------------------------------
# Floating-point decoding (exact)
# ----------------------------------------------------------------------------

def half_to_f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float16).astype(np.float64)


def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64: bf16 is the top half of a
    float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def act_to_f64(a, dtype: str) -> np.ndarray:
    if dtype == "fp16":
        return half_to_f64(a)
    if dtype == "bf16":
        return bf16_to_f64(a)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# Dequantization and the linear layer
# ----------------------------------------------------------------------------

def group_index(K: int, group_size: int, g_idx=None) -> np.ndarray:
    """Group of each input row: g_idx[k] when act-order supplies one
    ([P1] "Design motivation"), else k // group_size, with group_size = -1
    meaning one group of K rows ([P1] "Boundaries and failures")."""
    if g_idx is not None:
        g = np.asarray(g_idx, dtype=np.int64)
        assert g.shape == (K,)
        return g
    gs = K if group_size == -1 else group_size
    assert K % gs == 0
    return np.arange(K, dtype=np.int64) // gs


def dequant(codes, zeros, scales_f64, grp) -> np.ndarray:
    """W[k, n] = (q[k, n] - z[grp[k], n]) * s[grp[k], n] in float64
    ([P2] 5.3).  ``zeros`` None means the symmetric zero 8."""
    q = np.asarray(codes, dtype=np.int64)
    s = np.asarray(scales_f64, dtype=np.float64)
    z = 8 if zeros is None else np.asarray(zeros, dtype=np.int64)[grp, :]
    return (q - z).astype(np.float64) * s[grp, :]


def linear_ref(x_f64, W_f64, bias_f64=None) -> np.ndarray:
    """y = x @ W (+ bias), accumulated in float64 (BLAS dgemm)."""
    y = np.asarray(x_f64, dtype=np.float64) @ np.asarray(W_f64, dtype=np.float64)
    if bias_f64 is not None:
        y = y + np.asarray(bias_f64, dtype=np.float64)[None, :]
    return y


def codes_from_inputs(fmt: str, qweight, qzeros=None):
    """Codes q [K, N] and zero codes z [G, N] (or None) of a checkpoint in
    AWQ ("awq") or standard ("std") format."""
    if fmt == "awq":
        q = unpack_awq(qweight)
        z = None if qzeros is None else unpack_awq(qzeros)
    elif fmt == "std":
        q = unpack_std(qweight)
        z = None if qzeros is None else unpack_std_zeros(qzeros)
    else:
        raise ValueError(fmt)
    return q, z


def reference_linear(x, fmt, dtype, qweight, qzeros, scales, group_size, g_idx=None, bias=None):
    """Float64 reference y [M, N] of the whole layer from checkpoint inputs:
    unpack, fix the order, dequantize per group, then matmul."""
    q, z = codes_from_inputs(fmt, qweight, qzeros)
    K, _ = q.shape
    grp = group_index(K, group_size, g_idx)
    W = dequant(q, z, act_to_f64(scales, dtype), grp)
    b = None if bias is None else act_to_f64(bias, dtype)
    return linear_ref(act_to_f64(x, dtype), W, b)


def reference_entries(x, fmt, dtype, qweight, qzeros, scales, group_size, rows, cols,
                      g_idx=None, bias=None) -> np.ndarray:
    """Float64 reference for selected outputs y[rows[i], cols[i]] only, each
    computed on its own from one dequantized weight column (for full-size
    shapes where the whole product is too slow on the CPU)."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    s = act_to_f64(scales, dtype)
    uniq, where = np.unique(rows, return_inverse=True)
    xs = act_to_f64(np.asarray(x)[uniq], dtype)          # only the sampled rows
    K = xs.shape[1]
    grp = group_index(K, group_size, g_idx)
    qw = np.asarray(qweight)
    out = np.empty(rows.shape[0], dtype=np.float64)
    for i, (mi, n) in enumerate(zip(where.tolist(), cols.tolist())):
        if fmt == "awq":
            qcol = (u32(qw[:, n // 8]) >> (4 * AWQ_REVERSE_ORDER[n % 8])) & 0xF
            zcol = None if qzeros is None else (u32(qzeros)[:, n // 8] >> (4 * AWQ_REVERSE_ORDER[n % 8])) & 0xF
        else:
            k = np.arange(K)
            qcol = (u32(qw[:, n])[k // 8] >> (4 * (k % 8))) & 0xF
            zcol = None if qzeros is None else (u32(qzeros)[:, n // 8] >> (4 * (n % 8))) & 0xF
        zk = 8 if zcol is None else zcol[grp]
        wcol = (qcol - zk).astype(np.float64) * s[grp, n]
        out[i] = float(np.dot(xs[mi], wcol))
        if bias is not None:
            out[i] += float(act_to_f64(bias, dtype)[n])
    return out


# ----------------------------------------------------------------------------
# Act-order row order and g_idx validation
# ----------------------------------------------------------------------------

def reference_moe(x, offsets, fmt, dtype, experts, group_size, bias=None) -> np.ndarray:
    """Grouped (mixture-of-experts) layer, float64 [total_rows, N]: rows
    [offsets[e], offsets[e + 1]) of x go through expert e's linear layer
    (experts: list of (qweight, qzeros, scales) checkpoint inputs; bias:
    [E, N] or None).  The experts share K, N, format and group size (the WNA16
    MoE path of [P2] 5.4); each expert is the plain layer of
    ``reference_linear``."""
    out = []
    for e, (qw, qz, sc) in enumerate(experts):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        b = None if bias is None else bias[e]
        out.append(reference_linear(np.asarray(x)[r0:r1], fmt, dtype, qw, qz, sc, group_size, bias=b))
    return np.concatenate(out, axis=0)


def actorder_perm(g_idx) -> np.ndarray:
    """Stable ascending sort of input rows by group (ties keep the original
    row order): sorted row k' is original row perm[k']."""
    return np.argsort(np.asarray(g_idx, dtype=np.int64), kind="stable").astype(np.int32)


GIDX_OUT_OF_RANGE = 1
GIDX_UNEQUAL_GROUPS = 2


def gidx_status(g_idx, G: int, group_size: int) -> int:
    """Status bits the repack reports for a g_idx: bit 0 if any entry lies
    outside [0, G); bit 1 if some group in [0, G) does not own exactly
    group_size rows."""
    g = np.asarray(g_idx, dtype=np.int64)
    st = 0
    if ((g < 0) | (g >= G)).any():
        st |= GIDX_OUT_OF_RANGE
    counts = np.bincount(g[(g >= 0) & (g < G)], minlength=G)
    if (counts != group_size).any():
        st |= GIDX_UNEQUAL_GROUPS
    return st


# ----------------------------------------------------------------------------
# gfx950 tile layout (this library's own format)
# ----------------------------------------------------------------------------

TILE_N = 16    # output columns per strip
TILE_K = 128   # input rows per block
# Nibble slot that holds K-offset e (0..7) inside a tiled word.
TILE_SLOT_OF_OFFSET = (0, 4, 1, 5, 2, 6, 3, 7)


def _one_bits(dtype: str) -> int:
    return 0x3C00 if dtype == "fp16" else 0x3F80


def tile_layout(std_qweight, std_qzeros, scales, group_size: int, dtype: str, g_idx=None) -> dict:
    """Repack standard weights into the tile layout consumed by the kernels.

    Definition (K % 32 == 0, N % 8 == 0, g = K when group_size == -1,
    G = K / g, every act-order group owning exactly g rows).  The column
    count is padded to Np = 16 ceil(N / 16) (the pages' tile padding, read
    as: a padded column has every code and its zero point equal to 8 and
    every scale equal to 1, so its weights are exactly 0).  The row count
    is padded the same way to Kp = 128 ceil(K / 128) (no act-order then):
    a padded row's code equals its zero point, which is the column's zero
    point when the layer has one group (per-channel, g = K) and 8 in the
    Gp - G padded groups (Gp = Kp / g) otherwise, whose scales are 1 and
    zero points 8.  Steps 3-5 then run over Kp rows, Gp groups and Np
    columns:

    1. Row order: perm = stable argsort of g_idx (identity without g_idx);
       sorted row k' holds original row perm[k'] and lies in group k' // g.
    2. Zero scales: where s[g, n] == 0 the stored scale is the stored scale
       of group g-1 in the same column (1.0 for g == 0), and every code of
       that group and column is stored equal to its zero point (8 when there
       are no zero points).  (q - z) * s = 0 either way.
    3. qweight: int32 words indexed [t, b, l, j] (t < N/16, b < K/128,
       l < 64, j < 4), flattened in that order.  The word holds the eight
       codes of column n = 16 t + l % 16 at sorted rows
       k' = 128 b + 32 j + 8 (l // 16) + e, e = 0..7, with K-offset e in
       nibble slot TILE_SLOT_OF_OFFSET[e].
    4. scales: [N/16, G, 16] entries (t, g, c) = stored scale (g, 16 t + c),
       as raw fp16 / bf16 bits (uint16).
    5. zeros (when present): int32 [N/16, G, 2]; nibble slot i of word
       (t, g, w) holds the zero code of column 16 t + 8 w + i.
    6. perm: int32 [K] (only with g_idx).
    """
    q = unpack_std(std_qweight)
    K, N = q.shape
    assert K % 32 == 0 and N % 8 == 0
    assert K % TILE_K == 0 or g_idx is None
    gs = K if group_size == -1 else group_size
    G = K // gs
    z = None if std_qzeros is None else unpack_std_zeros(std_qzeros)
    if dtype == "fp16":
        sbits = np.asarray(scales, dtype=np.float16).view(np.uint16).astype(np.int64)
    else:
        sbits = np.asarray(scales, dtype=np.uint16).astype(np.int64)
    assert sbits.shape == (G, N)

    perm = None
    if g_idx is not None:
        assert gidx_status(g_idx, G, gs) == 0
        perm = actorder_perm(g_idx)
        q = q[perm.astype(np.int64), :]

    # Step 2: zero-scale substitution, group by group.
    is_zero = (sbits & 0x7FFF) == 0
    stored = sbits.copy()
    for g in range(G):
        prev = np.full(N, _one_bits(dtype), dtype=np.int64) if g == 0 else stored[g - 1]
        stored[g] = np.where(is_zero[g], prev, sbits[g])
    zfull = np.full((G, N), 8, dtype=np.int64) if z is None else z
    rows_group = np.arange(K) // gs
    q = np.where(is_zero[rows_group, :], zfull[rows_group, :], q)

    # Padding to Np columns: codes and zero points 8, scales 1.
    Np = -(-N // TILE_N) * TILE_N
    if Np != N:
        q = np.concatenate([q, np.full((K, Np - N), 8, dtype=np.int64)], axis=1)
        stored = np.concatenate([stored, np.full((G, Np - N), _one_bits(dtype), dtype=np.int64)], axis=1)
        if z is not None:
            z = np.concatenate([z, np.full((G, Np - N), 8, dtype=np.int64)], axis=1)
    N = Np

    # Padding to Kp rows: per-channel rows take the column's zero point,
    # grouped rows fill new groups with zero points 8 and scales 1.
    Kp = -(-K // TILE_K) * TILE_K
    if Kp != K:
        if G == 1 and gs == K:
            zrow = np.full(N, 8, dtype=np.int64) if z is None else z[0]
            pad_codes = np.broadcast_to(zrow, (Kp - K, N))
        else:
            pad_codes = np.full((Kp - K, N), 8, dtype=np.int64)
            Gp = Kp // gs
            stored = np.concatenate([stored, np.full((Gp - G, N), _one_bits(dtype), dtype=np.int64)], axis=0)
            if z is not None:
                z = np.concatenate([z, np.full((Gp - G, N), 8, dtype=np.int64)], axis=0)
            G = Gp
        q = np.concatenate([q, np.asarray(pad_codes, dtype=np.int64)], axis=0)
    K = Kp

    # Step 3: words [t, b, l, j] built from explicit index arithmetic.
    T, B = N // TILE_N, K // TILE_K
    t = np.arange(T)[:, None, None, None]
    b = np.arange(B)[None, :, None, None]
    lane = np.arange(64)[None, None, :, None]
    j = np.arange(4)[None, None, None, :]
    n = TILE_N * t + lane % 16
    word = np.zeros((T, B, 64, 4), dtype=np.int64)
    for e in range(8):
        k = TILE_K * b + 32 * j + 8 * (lane // 16) + e
        word |= q[k, n] << (4 * TILE_SLOT_OF_OFFSET[e])
    out = {"qweight": to_i32(word.reshape(-1))}

    # Step 4: scales [N/16, G, 16].
    out["scales"] = stored.reshape(G, T, TILE_N).transpose(1, 0, 2).astype(np.uint16).copy()

    # Step 5: zeros [N/16, G, 2].
    if z is not None:
        zw = np.zeros((T, G, 2), dtype=np.int64)
        for w in range(2):
            for i in range(8):
                col = TILE_N * np.arange(T) + 8 * w + i       # one column per strip
                zw[:, :, w] |= z[:, col].T << (4 * i)          # [G, T] -> [T, G]
        out["zeros"] = to_i32(zw)
    else:
        out["zeros"] = None
    out["perm"] = perm
    return out


def untile_codes(tiled_qweight, K: int, N: int) -> np.ndarray:
    """Inverse of step 3 of ``tile_layout``: walk every (k', n) and read its
    nibble back.  Written from the definition independently of the packer."""
    w = u32(np.asarray(tiled_qweight).reshape(-1))
    B = K // TILE_K
    out = np.empty((K, N), dtype=np.int64)
    kk = np.arange(K)[:, None]
    nn = np.arange(N)[None, :]
    t, c = nn // TILE_N, nn % TILE_N
    b, r = kk // TILE_K, kk % TILE_K
    j, rr = r // 32, r % 32
    lane = 16 * (rr // 8) + c
    e = rr % 8
    idx = ((t * B + b) * 64 + lane) * 4 + j
    slot = np.asarray(TILE_SLOT_OF_OFFSET)[e]
    out[:, :] = (w[idx] >> (4 * slot)) & 0xF
    return out


# ----------------------------------------------------------------------------
# Acceptance
# ----------------------------------------------------------------------------

def check(y_f64, ref_f64, elem_tol: float = 1e-2, fro_tol: float = 2e-3) -> dict:
    """Acceptance test of a GEMM result against the float64 reference:
    max |y - ref| <= elem_tol * (1 + |ref|) elementwise and
    ||y - ref||_F / ||ref||_F <= fro_tol."""
    y = np.asarray(y_f64, dtype=np.float64)
    r = np.asarray(ref_f64, dtype=np.float64)
    assert y.shape == r.shape
    d = np.abs(y - r)
    finite = bool(np.isfinite(y).all())
    ratio = d / (1.0 + np.abs(r))
    nr = float(np.linalg.norm(r))
    nd = float(np.linalg.norm(y - r)) if finite else float("inf")
    if nr == 0.0:
        rel_fro = 0.0 if nd == 0.0 else float("inf")
    else:
        rel_fro = nd / nr
    max_ratio = float(ratio.max()) if ratio.size else 0.0
    ok = finite and max_ratio <= elem_tol and rel_fro <= fro_tol
    return {"ok": bool(ok), "max_abs": float(d.max()) if d.size else 0.0, "max_ratio": max_ratio,
            "rel_fro": rel_fro, "finite": finite}
