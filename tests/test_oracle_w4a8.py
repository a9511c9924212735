"""Pins of the W4A8-fp8 oracle (INT4 weights x FP8-E4M3 activations).

Each pin is fixed by the FP8 format's definition (hand-derived values in
tests/golden/e4m3_values.txt), by rounding rules worked out by hand, by
closed forms, by reduction to the W4A16 oracle where the quantization is
exact, or by brute force; mutation tests plant mistakes in the oracle.
"""
import os

import numpy as np
import pytest

import oracle as O
from synthetic import constant_words, normal_acts, random_words, seeded, uniform_scales

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_values.txt")


def _golden():
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            b, v, *_ = line.split()
            yield int(b, 16), float(v)


def test_e4m3_golden_values():
    n = 0
    for b, v in _golden():
        got = float(O.e4m3_to_f64(np.array([b]))[0])
        assert got == v and np.signbit(got) == np.signbit(v), (hex(b), got, v)
        n += 1
    assert n >= 15
    assert np.isnan(O.e4m3_to_f64(np.array([0x7F, 0xFF]))).all()


def test_e4m3_every_finite_byte_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    vals = O.e4m3_to_f64(codes)
    assert np.array_equal(O.e4m3_rne(vals), codes.astype(np.uint8))
    pos = np.sort(vals[vals > 0])
    assert len(np.unique(pos)) == len(pos) == 126        # 7 subnormals + 119 normals


def test_e4m3_rounding_ties_to_even_and_saturation():
    cases = [
        (1.0625, 0x38),     # midway 1.0 (m=0) / 1.125 (m=1): even m=0
        (1.1875, 0x3A),     # midway 1.125 (m=1) / 1.25 (m=2): even m=2
        (1.1, 0x39),        # nearest 1.125
        (0.5 * 2 ** -9, 0x00),   # midway 0 / 2^-9: even code 0
        (1.5 * 2 ** -9, 0x02),   # midway 1*2^-9 / 2*2^-9: even code 2
        (2 ** -6 + 2 ** -10, 0x08),  # midway 2^-6 (m=0) / 2^-6 * 1.125 (m=1): even
        (464.0, 0x7E),      # midway 448 / (480, not finite): saturates to 448
        (1e6, 0x7E), (-1e6, 0xFE), (-1.0625, 0xB8),
    ]
    for v, b in cases:
        assert int(O.e4m3_rne(np.array([v]))[0]) == b, (v, hex(b))


def test_code_written_as_a_byte_is_code_over_512():
    # why the pages multiply the scales by 512 for fp8 activations: the
    # byte holding v (0..15) is the E4M3 value v * 2^-9
    v = np.arange(16)
    assert np.array_equal(O.e4m3_to_f64(v), v * 2.0 ** -9)


def test_quantize_divides_in_float32_then_rounds():
    # s = 0.75: 3 / 0.75 = 4 exactly (0x48); 100 / 0.75 = 133.3 lies between
    # 128 (e=14, m=0) and 144 (m=1), nearest 128 = 0x70; 400 / 0.75 = 533.3
    # is above 448 and saturates (0x7E, 0xFE)
    x = np.array([[3.0, -3.0, 0.0, 100.0, 400.0, -400.0]], dtype=np.float16)
    q = O.quantize_acts_fp8(x, "fp16", 0.75)
    assert q.tolist() == [[0x48, 0xC8, 0x00, 0x70, 0x7E, 0xFE]]


def _w4a16_inputs(K, N, gs, seed):
    G = K // gs
    rng = seeded(1201, K, N, seed)
    return (random_words(rng, (K // 8, N)), random_words(rng, (G, N // 8)),
            uniform_scales(rng, (G, N), 0.002, 0.02, "fp16"))


def test_exactly_representable_activations_reduce_to_w4a16():
    # activations already on the E4M3 grid with s_x = 1: quantization is the
    # identity and the W4A8 layer is the W4A16 layer
    K, N, gs = 256, 32, 128
    qw, qz, sc = _w4a16_inputs(K, N, gs, 1)
    rng = seeded(1202)
    grid = np.array([0.0, 0.5, 1.0, -1.5, 2.0, -3.0, 0.25, 7.0], dtype=np.float16)
    x = grid[rng.integers(0, len(grid), size=(3, K))]
    ref16 = O.reference_linear(x, "std", "fp16", qw, qz, sc, gs)
    ref8 = O.reference_w4a8_linear(x, "std", "fp16", qw, qz, sc, gs, 1.0)
    assert np.array_equal(ref8, ref16)
    # a power-of-two scale only moves the exponent: s_x = 2^-3, x on the grid * 2^-3
    x3 = (x.astype(np.float32) * 0.125).astype(np.float16)
    assert np.array_equal(O.reference_w4a8_linear(x3, "std", "fp16", qw, qz, sc, gs, 0.125), ref16 * 0.125)


def test_closed_form_constant_codes():
    # q = c, z = z0, s = s0: y[m, n] = (c - z0) s0 s_x sum_k x_q[m, k]
    K, N, gs = 256, 16, 128
    G = K // gs
    c, z0, s0, sx = 11, 3, 0.0078125, 0.02
    qw, qz = constant_words((K // 8, N), c), constant_words((G, N // 8), z0)
    sc = np.full((G, N), s0, dtype=np.float16)
    x = normal_acts(seeded(1203), (4, K), "fp16")
    xq = O.e4m3_to_f64(O.quantize_acts_fp8(x, "fp16", sx)) * float(np.float32(sx))
    expect = np.repeat(((c - z0) * s0 * xq.sum(axis=1))[:, None], N, axis=1)
    got = O.reference_w4a8_linear(x, "std", "fp16", qw, qz, sc, gs, sx)
    assert np.allclose(got, expect, rtol=1e-12, atol=1e-12)


def test_brute_force_triple_loop():
    K, N, M, gs = 128, 8, 2, 128
    qw, qz, sc = _w4a16_inputs(K, N, gs, 2)
    x = normal_acts(seeded(1204), (M, K), "bf16")
    sx = 0.015
    # plain loops over the definitions: bits of x, float32 division, nearest
    # E4M3 by exhaustive search over the 254 finite bytes, nibble unpack
    xs = O.act_to_f64(x, "bf16")
    finite = [b for b in range(256) if (b & 0x7F) != 0x7F]
    fvals = {b: float(O.e4m3_to_f64(np.array([b]))[0]) for b in finite}
    sc16 = uniform_scales(seeded(1205), (1, N), 0.001, 0.01, "bf16")
    scf = O.bf16_to_f64(sc16)
    qwu = qw.view(np.uint32)
    qzu = qz.view(np.uint32)
    y = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                t = float(np.float32(np.float32(xs[m, k]) / np.float32(sx)))
                t = max(-448.0, min(448.0, t))
                best = min(finite, key=lambda b: (abs(fvals[b] - t), (b & 1), -int(np.signbit(fvals[b]) == np.signbit(t))))
                xq = fvals[best] * float(np.float32(sx))
                q = (int(qwu[k // 8, n]) >> (4 * (k % 8))) & 0xF
                z = (int(qzu[0, n // 8]) >> (4 * (n % 8))) & 0xF
                acc += xq * (q - z) * scf[0, n]
            y[m, n] = acc
    got = O.reference_w4a8_linear(x, "std", "bf16", qw, qz, sc16, gs, sx)
    assert np.allclose(got, y, rtol=1e-12, atol=1e-12)


def test_mutation_truncating_instead_of_rounding_is_caught(monkeypatch):
    real = O.e4m3_rne

    def trunc(v):
        v = np.asarray(v, dtype=np.float64)
        vals = O.e4m3_to_f64(np.arange(0x7F))
        a = np.minimum(np.abs(v), 448.0)
        idx = np.searchsorted(vals, a, side="right") - 1
        c = np.arange(0x7F)[idx]
        return np.where(np.signbit(v), c | 0x80, c).astype(np.uint8)

    monkeypatch.setattr(O, "e4m3_rne", trunc)
    with pytest.raises(AssertionError):
        test_e4m3_rounding_ties_to_even_and_saturation()
    monkeypatch.setattr(O, "e4m3_rne", real)


def test_mutation_wrong_exponent_bias_is_caught(monkeypatch):
    real = O.e4m3_to_f64

    def bias8(codes):
        return real(codes) / 2.0

    monkeypatch.setattr(O, "e4m3_to_f64", bias8)
    with pytest.raises(AssertionError):
        test_e4m3_golden_values()


def test_operand_order_worked_bytes_and_bijection():
    # column -> byte, derived by hand from "byte 32 q + 8 j + i holds column
    # 32 j + 8 q + [0,4,1,5,2,6,3,7][i]": column 1 is offset 1 = entry 2 of
    # the list with j = q = 0, so byte 2; column 4 -> byte 1; column 8 (q = 1)
    # -> byte 32; column 32 (j = 1) -> byte 8; column 127 (j = 3, q = 3,
    # offset 7 = entry 7) -> byte 127; column 130 -> block 1, byte 128 + 4
    K = 256
    expect = {1: 2, 4: 1, 8: 32, 32: 8, 127: 127, 130: 132, 0: 0}
    for col, byte in expect.items():
        codes = np.zeros((1, K), dtype=np.uint8)
        codes[0, col] = 0x38
        out = O.fp8_operand_order(codes, K)
        assert out[0, byte] == 0x38 and out.sum() == 0x38, (col, byte)
    # a permutation of each block (every byte used once)
    codes = (np.arange(256) % 251).astype(np.uint8)[None, :]
    out = O.fp8_operand_order(codes, 256)
    assert sorted(out[0].tolist()) == sorted(codes[0].tolist())
    # K tail: the padded columns are zero
    out = O.fp8_operand_order(np.full((2, 96), 0x38, dtype=np.uint8), 128)
    assert int((out != 0).sum()) == 2 * 96


def test_block_sums_closed_form():
    codes = np.full((3, 256), 0x38, dtype=np.uint8)       # every value 1.0
    codes[1, 128:] = 0xB8                                  # -1.0
    s = O.fp8_block_sums(codes, 256)
    assert s.shape == (2, 4)
    assert s[:, :3].tolist() == [[128.0, 128.0, 128.0], [128.0, -128.0, 128.0]]
    assert (s[:, 3] == 0).all()
