"""CPU oracle for INT4 weights x FP8 activations (W4A8-fp8).

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by the tests
and the benchmark's CPU-baseline leg, never by the product path.

Sources:

* [P1] vLLM "Quantized layer loading: AWQ / GPTQ / Marlin / fp8", section
  "Boundaries and failures": when the kernel's activation type is fp8
  (float8_e4m3fn) the int4 weights are preprocessed for fp8 activations and
  the scales are multiplied by 512.
* [P4] SGLang quantization design, section 5 (W4AFp8): int4 weights with one
  scale per group of 128 elements, fp8 activations quantized with a static
  input scale (per-expert input scales reduced to one scalar by their max).

Readings:

* FP8 format: E4M3 with no infinities ("fn"), the float8_e4m3fn the
  loading page names: sign bit, four exponent bits (bias 7), three mantissa
  bits; exponent 0 holds subnormals m/8 * 2^-6; 0x7F and 0xFF are NaN; the
  largest finite magnitude is 448.
* Activation quantization: x_q = e4m3(clamp(x / s_x, -448, 448)) with one
  per-tensor scale s_x (the static input scale), x / s_x computed in
  float32 (x is exact in float32) and rounded to the nearest e4m3 value,
  ties to the even mantissa.  The layer computes y = s_x * x_q W + bias with
  W = (q - z) s as in the W4A16 layer.
* The factor 512 = 2^9: the e4m3 byte whose value is v * 2^-9 is the integer
  v itself for v = 0..15 (subnormals 0..7, then exponent 1), so a 4-bit code
  written into a byte is an fp8 operand worth code / 512; the scales carry
  the 512 back.  (A property of the format, pinned in the tests; the oracle
  itself computes with exact values.)
"""
from __future__ import annotations

import numpy as np

from .w4_oracle import act_to_f64, codes_from_inputs, dequant, group_index, linear_ref

E4M3_MAX = 448.0

__all__ = ["E4M3_MAX", "e4m3_to_f64", "e4m3_rne", "quantize_acts_fp8", "reference_w4a8_linear",
           "FP8_BYTE_OFFSETS", "fp8_operand_order", "fp8_block_sums"]


def e4m3_to_f64(codes) -> np.ndarray:
    """Value of each E4M3 (fn) byte, from the format's definition."""
    b = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    sub = m / 8.0 * 2.0 ** -6
    nor = (1.0 + m / 8.0) * np.power(2.0, e - 7)
    v = sign * np.where(e == 0, sub, nor)
    return np.where((b & 0x7F) == 0x7F, np.nan, v)


def _finite_positive_table():
    """(values, codes) of the non-negative finite E4M3 bytes, ascending."""
    codes = np.arange(0x7F, dtype=np.int64)  # 0x00 .. 0x7E
    return e4m3_to_f64(codes), codes


def e4m3_rne(v) -> np.ndarray:
    """Nearest E4M3 byte of each value (float32 or float64 input, taken
    exactly), ties to the byte with the even mantissa; magnitudes above 448
    saturate to 448; -0 and negative values keep the sign bit."""
    v = np.asarray(v, dtype=np.float64)
    assert not np.isnan(v).any()
    vals, codes = _finite_positive_table()
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(vals, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0) & (hi != lo))
    exact = vals[hi] == a
    c = np.where(exact | pick_hi, codes[hi], codes[lo])
    neg = np.signbit(v)
    return (np.where(neg, c | 0x80, c)).astype(np.uint8)


def quantize_acts_fp8(x, dtype: str, x_scale) -> np.ndarray:
    """E4M3 codes of x / s_x (float32 division, clamped to +-448, nearest
    even): the activation quantization with a static per-tensor scale
    ([P4] section 5.2)."""
    xf = act_to_f64(x, dtype).astype(np.float32)        # exact
    q = xf / np.float32(x_scale)                        # IEEE float32 division
    q = np.clip(q, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_rne(q)


def reference_w4a8_linear(x, fmt, dtype, qweight, qzeros, scales, group_size, x_scale, g_idx=None, bias=None):
    """Float64 reference y [M, N] of the W4A8 layer: activations quantized to
    E4M3 with the static scale, then y = s_x x_q W + bias with the
    dequantized int4 weight W = (q - z) s of the W4A16 layer."""
    xq = e4m3_to_f64(quantize_acts_fp8(x, dtype, x_scale)) * float(np.float32(x_scale))
    q, z = codes_from_inputs(fmt, qweight, qzeros)
    K, _ = q.shape
    W = dequant(q, z, act_to_f64(scales, dtype), group_index(K, group_size, g_idx))
    b = None if bias is None else act_to_f64(bias, dtype)
    return linear_ref(xq, W, b)


# ----------------------------------------------------------------------------
# The library's layout of quantized activations (its own format, like the
# tile layout of the weights): within each 128-column block of a row, byte
# 32 q + 8 j + i holds column 32 j + 8 q + FP8_BYTE_OFFSETS[i].
# ----------------------------------------------------------------------------

FP8_BYTE_OFFSETS = (0, 4, 1, 5, 2, 6, 3, 7)


def fp8_operand_order(codes, Kp: int) -> np.ndarray:
    """Codes [M][K] (sorted column order) -> bytes [M][Kp] in operand order,
    columns K .. Kp - 1 zero."""
    c = np.asarray(codes, dtype=np.uint8)
    M, K = c.shape
    assert Kp % 128 == 0 and Kp >= K
    src = np.zeros((M, Kp), dtype=np.uint8)
    src[:, :K] = c
    out = np.zeros((M, Kp), dtype=np.uint8)
    for b in range(Kp // 128):
        for q in range(4):
            for j in range(4):
                for i in range(8):
                    out[:, 128 * b + 32 * q + 8 * j + i] = src[:, 128 * b + 32 * j + 8 * q + FP8_BYTE_OFFSETS[i]]
    return out


def fp8_block_sums(codes, Kp: int) -> np.ndarray:
    """Sums of the E4M3 values of each 128-column block of each row (sorted
    order), [Kp / 128][Mr] with Mr = M rounded up to 4 (extra rows zero)."""
    v = e4m3_to_f64(np.asarray(codes, dtype=np.uint8))
    M, K = v.shape
    Mr = (M + 3) // 4 * 4
    out = np.zeros((Kp // 128, Mr), dtype=np.float64)
    for b in range(Kp // 128):
        out[b, :M] = v[:, 128 * b:min(128 * (b + 1), K)].sum(axis=1)
    return out
