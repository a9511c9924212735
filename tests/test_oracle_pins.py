"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

No test here re-derives a result with the oracle's own formula: each checks
worked values derived by hand (tests/golden/), closed forms, invariants,
special cases, or brute force on tiny inputs.  The mutation tests at the end
plant plausible mistakes in the oracle and show that a pin catches each.
"""
import os

import numpy as np
import pytest

import oracle as O
from synthetic import (
    constant_words, make_acts, make_layer_inputs, config_cases, random_words, seeded,
    to_bf16_bits, uniform_scales, normal_acts, actorder_gidx,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


# ----------------------------------------------------------------------------
# Nibbles, packing, AWQ order
# ----------------------------------------------------------------------------

def test_nibble_exhaustive_every_value_every_slot():
    for slot in range(8):
        for v in range(16):
            word = np.array([v << (4 * slot)], dtype=np.uint32).view(np.int32)
            for i in range(8):
                assert int(O.nib(word, i)[0]) == (v if i == slot else 0)


def test_nibble_negative_words():
    # 0x80000000 is negative as int32: slot 7 must read 8, the rest 0.
    w = np.array([0x80000000, 0xFFFFFFFF], dtype=np.uint32).view(np.int32)
    assert w[0] < 0
    assert [int(O.nib(w, i)[0]) for i in range(8)] == [0] * 7 + [8]
    assert [int(O.nib(w, i)[1]) for i in range(8)] == [15] * 8


def test_golden_awq_and_std_words():
    n = 0
    for kind, hexword, *vals in _golden_lines("awq_words.txt"):
        word = np.array([[int(hexword, 16)]], dtype=np.uint32).view(np.int32)
        vals = [int(v) for v in vals]
        if kind == "awq":
            assert O.unpack_awq(word)[0].tolist() == vals
            assert O.pack_awq(np.array([vals]))[0, 0] == word[0, 0]
        else:
            assert O.unpack_std(word)[:, 0].tolist() == vals
            assert O.pack_std(np.array(vals)[:, None])[0, 0] == word[0, 0]
        n += 1
    assert n >= 10


def test_awq_order_is_a_permutation_with_known_inverse():
    R = O.AWQ_REVERSE_ORDER
    P = (0, 2, 4, 6, 1, 3, 5, 7)  # packer order: slot i holds column P[i]
    assert sorted(R) == list(range(8))
    assert all(P[R[j]] == j for j in range(8))


def test_std_pack_roundtrip_random_words():
    rng = seeded(11)
    w = random_words(rng, (64, 48))
    assert (w < 0).any()
    assert np.array_equal(O.pack_std(O.unpack_std(w)), w)
    assert np.array_equal(O.pack_std_zeros(O.unpack_std_zeros(w)), w)
    assert np.array_equal(O.pack_awq(O.unpack_awq(w)), w)


def test_unpack_layouts_index_rows_and_columns():
    # Standard: word [r, n] carries rows 8r..8r+7 of column n.  Put a distinct
    # code in one row and check it lands at (8r + i, n) only.
    Sw = np.zeros((3, 5), dtype=np.int32)
    Sw[2, 4] = np.int32(0x00500000)  # slot 5 = 5
    q = O.unpack_std(Sw)
    assert q.shape == (24, 5)
    nz = np.argwhere(q)
    assert nz.tolist() == [[8 * 2 + 5, 4]] and q[21, 4] == 5
    # AWQ: word [k, c] carries columns 8c..8c+7 of row k.
    Aw = np.zeros((4, 3), dtype=np.int32)
    Aw[1, 2] = np.int32(0x00000F00)  # slot 2 -> logical column 4
    q = O.unpack_awq(Aw)
    assert q.shape == (4, 24)
    assert np.argwhere(q).tolist() == [[1, 8 * 2 + 4]]


def test_awq_to_std_identity_and_shapes():
    rng = seeded(12)
    K, N, G = 256, 64, 2
    aw = random_words(rng, (K, N // 8))
    az = random_words(rng, (G, N // 8))
    sw, sz = O.awq_to_std(aw, az)
    assert sw.shape == (K // 8, N) and sz.shape == (G, N // 8)
    assert np.array_equal(O.unpack_std(sw), O.unpack_awq(aw))
    assert np.array_equal(O.unpack_std_zeros(sz), O.unpack_awq(az))
    assert O.std_zeros_transposed(sz).shape == (N // 8, G)


def test_awq_to_std_worked_word():
    # One AWQ word per row, rows 0..7 all equal to the golden 0x75316420
    # (columns 0..7 hold 0..7).  Then column n of the standard word holds
    # the value n in all eight rows: 0x11111111 * n.
    aw = np.full((8, 1), 0x75316420, dtype=np.uint32).view(np.int32)
    sw, _ = O.awq_to_std(aw)
    assert [int(v) for v in O.u32(sw[0])] == [0x11111111 * n for n in range(8)]


# ----------------------------------------------------------------------------
# Floating point decoding
# ----------------------------------------------------------------------------

def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0x4300, 0xC000, 0x0000, 0x8000, 0x3C24, 0x7F80], dtype=np.uint16)
    v = O.bf16_to_f64(bits)
    assert v[0] == 1.0 and v[1] == 128.0 and v[2] == -2.0 and v[3] == 0.0
    assert np.signbit(v[4]) and v[4] == 0.0
    assert v[5] == 0.010009765625  # 0x3C24 = 2^-7 * (1 + 36/128)
    assert np.isinf(v[6])


def test_bf16_generator_round_to_nearest_even():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins (1.0).
    # 1 + 3*2^-8 is a tie between 1+2^-7 and 1+2^-6: even wins (1+2^-6).
    b = to_bf16_bits(np.array([1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-20], dtype=np.float32))
    assert O.bf16_to_f64(b).tolist() == [1.0, 1 + 2**-6, 1 + 2**-7]


# ----------------------------------------------------------------------------
# Dequantization and the linear layer: closed forms and special cases
# ----------------------------------------------------------------------------

def _tiny_layer(code=None, zero=None, K=256, N=32, gs=128, dtype="fp16", seed=21):
    rng = seeded(seed)
    G = K // gs if gs != -1 else 1
    qw = random_words(rng, (K, N // 8)) if code is None else constant_words((K, N // 8), code)
    qz = random_words(rng, (G, N // 8)) if zero is None else constant_words((G, N // 8), zero)
    s = uniform_scales(rng, (G, N), 0.002, 0.02, dtype)
    return qw, qz, s


def test_closed_form_constant_codes():
    # q = c, z = z0, s = s0 everywhere => y[m, n] = (c - z0) * s0 * sum_k x[m, k]
    K, N, gs = 256, 32, 128
    G = K // gs
    for c, z0 in ((13, 2), (1, 9), (7, 7)):
        qw = constant_words((K, N // 8), c)
        qz = constant_words((G, N // 8), z0)
        s = np.full((G, N), 0.0078125, dtype=np.float16)
        x = normal_acts(seeded(3), (3, K), "fp16")
        y = O.reference_linear(x, "awq", "fp16", qw, qz, s, gs)
        expect = (c - z0) * 0.0078125 * x.astype(np.float64).sum(axis=1)
        np.testing.assert_allclose(y, np.repeat(expect[:, None], N, axis=1), rtol=1e-13, atol=1e-13)


def test_one_hot_row_selects_dequantized_row_with_its_group_scale():
    # x = e_k selects W[k, :] = (c - z[g(k), :]) * s[g(k), :].  Zeros and
    # scales differ per group and per column, so a wrong group map, a wrong
    # zero index or a transposed operand all change the value.
    K, N, gs = 256, 16, 64
    G = K // gs
    zc = np.arange(G * N).reshape(G, N) % 16
    qz = O.pack_awq(zc)
    sv = (1 + np.arange(G * N).reshape(G, N)).astype(np.float16) / 1024
    qw = constant_words((K, N // 8), 11)
    for k in (0, 63, 64, 130, 255):
        x = np.zeros((1, K), dtype=np.float16)
        x[0, k] = 1.0
        y = O.reference_linear(x, "awq", "fp16", qw, qz, sv, gs)[0]
        g = k // gs
        expect = [(11 - zc[g, n]) * float(sv[g, n]) for n in range(N)]
        assert y.tolist() == expect


def test_zero_scales_or_codes_equal_zero_point_give_bias():
    K, N, gs = 256, 32, 128
    rng = seeded(4)
    x = normal_acts(rng, (2, K), "fp16")
    bias = uniform_scales(rng, (N,), -1, 1, "fp16")
    qw, qz, s = _tiny_layer()
    y = O.reference_linear(x, "awq", "fp16", qw, qz, np.zeros_like(s), gs, bias=bias)
    assert np.array_equal(y, np.repeat(bias.astype(np.float64)[None, :], 2, axis=0))
    qw9 = constant_words((K, N // 8), 9)
    qz9 = constant_words((K // gs, N // 8), 9)
    y = O.reference_linear(x, "awq", "fp16", qw9, qz9, s, gs, bias=bias)
    assert np.array_equal(y, np.repeat(bias.astype(np.float64)[None, :], 2, axis=0))


def test_symmetric_equals_explicit_zero_eight():
    K, N, gs = 256, 32, 128
    rng = seeded(5)
    qw = random_words(rng, (K // 8, N))
    s = uniform_scales(rng, (K // gs, N), 0.001, 0.01, "bf16")
    x = normal_acts(rng, (3, K), "bf16")
    a = O.reference_linear(x, "std", "bf16", qw, None, s, gs)
    b = O.reference_linear(x, "std", "bf16", qw, constant_words((K // gs, N // 8), 8), s, gs)
    assert np.array_equal(a, b)


def test_per_channel_equals_group_of_K():
    K, N = 256, 32
    rng = seeded(6)
    qw = random_words(rng, (K // 8, N))
    qz = random_words(rng, (1, N // 8))
    s = uniform_scales(rng, (1, N), 0.002, 0.02, "fp16")
    x = normal_acts(rng, (2, K), "fp16")
    a = O.reference_linear(x, "std", "fp16", qw, qz, s, -1)
    b = O.reference_linear(x, "std", "fp16", qw, qz, s, K)
    assert np.array_equal(a, b)


def test_gidx_identity_equals_grouped():
    K, N, gs = 512, 32, 128
    rng = seeded(7)
    qw = random_words(rng, (K // 8, N))
    qz = random_words(rng, (K // gs, N // 8))
    s = uniform_scales(rng, (K // gs, N), 0.002, 0.02, "fp16")
    x = normal_acts(rng, (2, K), "fp16")
    a = O.reference_linear(x, "std", "fp16", qw, qz, s, gs)
    b = O.reference_linear(x, "std", "fp16", qw, qz, s, gs, g_idx=np.arange(K) // gs)
    assert np.array_equal(a, b)


def test_joint_row_permutation_invariance():
    # Permuting x columns, weight rows and g_idx together leaves y unchanged.
    K, N, gs = 512, 32, 128
    rng = seeded(8)
    q = rng.integers(0, 16, size=(K, N))
    qz = random_words(rng, (K // gs, N // 8))
    s = uniform_scales(rng, (K // gs, N), 0.002, 0.02, "fp16")
    x = normal_acts(rng, (3, K), "fp16")
    g_idx = actorder_gidx(rng, K, gs)
    p = rng.permutation(K)
    a = O.reference_linear(x, "std", "fp16", O.pack_std(q), qz, s, gs, g_idx=g_idx)
    b = O.reference_linear(x[:, p], "std", "fp16", O.pack_std(q[p]), qz, s, gs, g_idx=g_idx[p])
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_linearity_in_x():
    qw, qz, s = _tiny_layer()
    rng = seeded(9)
    x1 = normal_acts(rng, (2, 256), "fp16").astype(np.float64)
    x2 = normal_acts(rng, (2, 256), "fp16").astype(np.float64)
    q, z = O.codes_from_inputs("awq", qw, qz)
    W = O.dequant(q, z, O.half_to_f64(s), O.group_index(256, 128))
    np.testing.assert_allclose(O.linear_ref(x1 + 3 * x2, W), O.linear_ref(x1, W) + 3 * O.linear_ref(x2, W),
                               rtol=1e-12, atol=1e-10)


def test_brute_force_triple_loop_on_tiny_config():
    # Pure-Python integer/float loops straight from the definitions, against
    # the vectorized oracle on the tiny workload (AWQ, K=512, N=256, M=1,4).
    c = config_cases(1)[0]
    L = make_layer_inputs(c)
    aw = [[int(v) & 0xFFFFFFFF for v in row] for row in L["qweight"].tolist()]
    az = [[int(v) & 0xFFFFFFFF for v in row] for row in L["qzeros"].tolist()]
    s = L["scales"].astype(np.float64).tolist()
    R = (0, 4, 1, 5, 2, 6, 3, 7)
    for M in c.Ms:
        x = make_acts(c, M)
        ref = O.reference_linear(x, "awq", "fp16", L["qweight"], L["qzeros"], L["scales"], c.group_size)
        xs = x.astype(np.float64).tolist()
        for m in range(M):
            for n in range(0, c.N, 7):   # every 7th column keeps the loop short
                acc = 0.0
                for k in range(c.K):
                    g = k // 128
                    qv = (aw[k][n // 8] >> (4 * R[n % 8])) & 15
                    zv = (az[g][n // 8] >> (4 * R[n % 8])) & 15
                    acc += xs[m][k] * ((qv - zv) * s[g][n])
                assert abs(acc - ref[m, n]) <= 1e-12 * (1 + abs(ref[m, n]))


def test_reference_entries_match_full_reference():
    for fmt, cfg in (("awq", 1),):
        c = config_cases(cfg)[0]
        L = make_layer_inputs(c)
        x = make_acts(c, 4)
        full = O.reference_linear(x, fmt, c.dtype, L["qweight"], L["qzeros"], L["scales"], c.group_size)
        rows, cols = np.array([0, 3, 2, 1]), np.array([0, 255, 17, 128])
        e = O.reference_entries(x, fmt, c.dtype, L["qweight"], L["qzeros"], L["scales"], c.group_size, rows, cols)
        np.testing.assert_allclose(e, full[rows, cols], rtol=1e-12, atol=1e-12)
    # standard format with g_idx and bf16, against the full reference
    K, N, gs = 512, 64, 128
    rng = seeded(10)
    qw = random_words(rng, (K // 8, N))
    qz = random_words(rng, (K // gs, N // 8))
    s = uniform_scales(rng, (K // gs, N), 0.001, 0.01, "bf16")
    x = normal_acts(rng, (3, K), "bf16")
    gi = actorder_gidx(rng, K, gs)
    bias = uniform_scales(rng, (N,), -1, 1, "bf16")
    full = O.reference_linear(x, "std", "bf16", qw, qz, s, gs, g_idx=gi, bias=bias)
    rows, cols = np.array([0, 2, 1]), np.array([63, 0, 40])
    e = O.reference_entries(x, "std", "bf16", qw, qz, s, gs, rows, cols, g_idx=gi, bias=bias)
    np.testing.assert_allclose(e, full[rows, cols], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# Act-order, g_idx validation, tile layout
# ----------------------------------------------------------------------------

def test_actorder_perm_is_stable():
    g = np.array([2, 0, 1, 0, 2, 1, 0, 1])
    assert O.actorder_perm(g).tolist() == [1, 3, 6, 2, 5, 7, 0, 4]


def test_gidx_status_bits():
    assert O.gidx_status([0, 1, 1, 0], 2, 2) == 0
    assert O.gidx_status([0, 1, 2, 0], 2, 2) == O.GIDX_OUT_OF_RANGE | O.GIDX_UNEQUAL_GROUPS
    assert O.gidx_status([0, 0, 0, 1], 2, 2) == O.GIDX_UNEQUAL_GROUPS
    assert O.gidx_status([-1, 1, 1, 0], 2, 2) == O.GIDX_OUT_OF_RANGE | O.GIDX_UNEQUAL_GROUPS


def test_tile_golden_words():
    K, N, gs = 256, 32, 128
    q = (np.arange(K)[:, None] + np.arange(N)[None, :]) % 16
    s = np.full((K // gs, N), 0.5, dtype=np.float16)
    t = O.tile_layout(O.pack_std(q), None, s, gs, "fp16")
    assert t["qweight"].shape == (K * N // 8,)
    for idx, hexword in _golden_lines("tile_words.txt"):
        assert int(O.u32(t["qweight"][int(idx)])) == int(hexword, 16)


def test_tile_is_a_bijection_and_untile_inverts_it():
    K, N, gs = 384, 48, 128
    rng = seeded(13)
    q = rng.integers(0, 16, size=(K, N))
    s = uniform_scales(rng, (K // gs, N), 0.002, 0.02, "fp16")
    t = O.tile_layout(O.pack_std(q), None, s, gs, "fp16")
    assert np.array_equal(O.untile_codes(t["qweight"], K, N), q)
    # bijection: tile a matrix of distinct (k, n) ids, 4 bits at a time
    ids = np.arange(K * N).reshape(K, N)
    seen = np.zeros((K, N), dtype=np.int64)
    for shift in range(0, 16, 4):
        part = (ids >> shift) & 0xF
        back = O.untile_codes(O.tile_layout(O.pack_std(part), None, s, gs, "fp16")["qweight"], K, N)
        seen |= back << shift
    assert np.array_equal(seen, ids)


def test_tile_scales_zeros_layout_and_actorder_rows():
    K, N, gs = 256, 32, 64
    G = K // gs
    rng = seeded(14)
    q = rng.integers(0, 16, size=(K, N))
    z = rng.integers(0, 16, size=(G, N))
    s = uniform_scales(rng, (G, N), 0.002, 0.02, "fp16")
    gi = actorder_gidx(rng, K, gs)
    t = O.tile_layout(O.pack_std(q), O.pack_std_zeros(z), s, gs, "fp16", g_idx=gi)
    perm = t["perm"]
    assert sorted(perm.tolist()) == list(range(K))
    assert (gi[perm] == np.arange(K) // gs).all()            # sorted rows grouped in order
    assert np.array_equal(O.untile_codes(t["qweight"], K, N), q[perm])
    sb = s.view(np.uint16)
    for tt in range(N // 16):
        for g in range(G):
            assert t["scales"][tt, g].tolist() == sb[g, 16 * tt:16 * tt + 16].tolist()
            for w in range(2):
                word = int(O.u32(t["zeros"][tt, g, w]))
                assert [(word >> (4 * i)) & 15 for i in range(8)] == z[g, 16 * tt + 8 * w:16 * tt + 8 * w + 8].tolist()


def test_tile_zero_scale_substitution_keeps_the_product():
    K, N, gs = 256, 16, 64
    G = K // gs
    rng = seeded(15)
    q = rng.integers(0, 16, size=(K, N))
    z = rng.integers(0, 16, size=(G, N))
    s = uniform_scales(rng, (G, N), 0.002, 0.02, "fp16")
    s[0, 3] = 0
    s[2, 3] = -0.0
    s[2, 5] = 0
    t = O.tile_layout(O.pack_std(q), O.pack_std_zeros(z), s, gs, "fp16")
    st = t["scales"][0].view(np.float16)
    assert st[0, 3] == 1.0 and st[1, 3] == s[1, 3] and st[2, 3] == s[1, 3] and st[2, 5] == s[1, 5]
    qt = O.untile_codes(t["qweight"], K, N)
    assert (qt[0:64, 3] == z[0, 3]).all() and (qt[128:192, 3] == z[2, 3]).all()
    assert (qt[128:192, 5] == z[2, 5]).all()
    # The product from the tiled operands equals the product from the inputs.
    x = normal_acts(rng, (2, K), "fp16")
    W_in = O.dequant(q, z, O.half_to_f64(s), O.group_index(K, gs))
    W_t = O.dequant(qt, z, st.astype(np.float64), O.group_index(K, gs))
    assert np.array_equal(O.linear_ref(x.astype(np.float64), W_in), O.linear_ref(x.astype(np.float64), W_t))


# ----------------------------------------------------------------------------
# Acceptance function
# ----------------------------------------------------------------------------

def test_check_thresholds():
    ref = np.array([[0.0, 10.0], [-3.0, 1.0]])
    assert O.check(ref, ref)["ok"]
    y = ref.copy()
    y[0, 0] = 0.011                       # 1.1e-2 > 1e-2 * (1 + 0)
    assert not O.check(y, ref)["ok"]
    y = ref.copy()
    y[0, 1] = 10.1                        # 0.1 <= 1e-2 * 11 but Frobenius 0.1/10.5 > 2e-3
    r = O.check(y, ref)
    assert r["max_ratio"] <= 1e-2 and not r["ok"]
    y = ref * (1 + 1e-3)
    assert O.check(y, ref)["ok"]
    y = ref.copy()
    y[1, 1] = np.nan
    assert not O.check(y, ref)["ok"]


def test_tile_layout_pads_columns_to_whole_strips():
    # N = 24: one full strip and one half strip; the padded columns hold
    # codes and zero points 8 and scale 1 (weights exactly 0), the real
    # columns are untouched
    K, N, gs = 256, 24, 128
    G = K // gs
    rng = seeded(920)
    sw = random_words(rng, (K // 8, N))
    sz = random_words(rng, (G, N // 8))
    sc = uniform_scales(rng, (G, N), 0.002, 0.02, "fp16")
    t = O.tile_layout(sw, sz, sc, gs, "fp16")
    assert t["qweight"].size == K * 32 // 8 and t["scales"].shape == (2, G, 16) and t["zeros"].shape == (2, G, 2)
    full = O.untile_codes(t["qweight"], K, 32)
    np.testing.assert_array_equal(full[:, :N], O.unpack_std(sw))
    assert (full[:, N:] == 8).all()
    assert (t["scales"][1, :, 8:] == 0x3C00).all()
    np.testing.assert_array_equal(t["scales"][:, :, :].transpose(1, 0, 2).reshape(G, 32)[:, :N],
                                  sc.view(np.uint16))
    zw = O.u32(t["zeros"])
    assert (zw[1, :, 1] == 0x88888888).all()
    np.testing.assert_array_equal(zw[:, :, :].transpose(1, 0, 2).reshape(G, 4)[:, :3], O.u32(sz))
    # the padded layer computes the same outputs as the unpadded definition
    q, z = O.codes_from_inputs("std", sw, sz)
    W = O.dequant(q, z, O.half_to_f64(sc), O.group_index(K, gs))
    qp = full
    zp = np.concatenate([z, np.full((G, 8), 8)], axis=1)
    sp = np.concatenate([O.half_to_f64(sc), np.ones((G, 8))], axis=1)
    Wp = O.dequant(qp, zp, sp, O.group_index(K, gs))
    np.testing.assert_array_equal(Wp[:, :N], W)
    assert (Wp[:, N:] == 0).all()


@pytest.mark.parametrize("K,gs,has_z", [(96, 32, True), (192, 64, False), (320, 64, True), (224, -1, True), (32, -1, False)])
def test_tile_layout_pads_rows_to_whole_blocks(K, gs, has_z):
    # K % 128 != 0: rows K .. Kp-1 are padded.  A padded row's code equals
    # its zero point, so every padded weight is exactly 0; grouped layers
    # get new groups (scale 1, zero point 8), a per-channel layer keeps its
    # one group and its zero point
    N = 16
    Kp = -(-K // 128) * 128
    g = K if gs == -1 else gs
    G, Gp = K // g, (1 if gs == -1 else Kp // g)
    rng = seeded(921)
    sw = random_words(rng, (K // 8, N))
    sz = random_words(rng, (G, N // 8)) if has_z else None
    sc = uniform_scales(rng, (G, N), 0.002, 0.02, "fp16")
    t = O.tile_layout(sw, sz, sc, gs, "fp16")
    assert t["qweight"].size == Kp * N // 8 and t["scales"].shape == (1, Gp, 16)
    full = O.untile_codes(t["qweight"], Kp, N)
    np.testing.assert_array_equal(full[:K], O.unpack_std(sw))
    q, z = O.codes_from_inputs("std", sw, sz)
    if gs == -1:
        want = np.broadcast_to(z[0] if has_z else np.full(N, 8), (Kp - K, N))
        np.testing.assert_array_equal(full[K:], want)
    else:
        assert (full[K:] == 8).all()
        assert (t["scales"][0, G:] == 0x3C00).all()
        if has_z:
            assert (O.u32(t["zeros"])[0, G:] == 0x88888888).all()
    np.testing.assert_array_equal(t["scales"][0, :G], sc.view(np.uint16))
    # dequantizing the padded layout gives the layer's weights and zero rows
    sp = O.half_to_f64(t["scales"][0].view(np.float16))
    zp = None
    if has_z:
        zw = O.u32(t["zeros"])[0]
        zp = np.array([[(int(zw[gg, c // 8]) >> (4 * (c % 8))) & 0xF for c in range(N)] for gg in range(Gp)])
    Wp = O.dequant(full, zp, sp, O.group_index(Kp, Kp if gs == -1 else gs))
    W = O.dequant(q, z, O.half_to_f64(sc), O.group_index(K, gs))
    np.testing.assert_array_equal(Wp[:K], W)
    assert (Wp[K:] == 0).all()


# ----------------------------------------------------------------------------
# Grouped (mixture-of-experts) reference
# ----------------------------------------------------------------------------

def _moe_experts(E, K, N, gs, seed):
    out = []
    for e in range(E):
        rng = seeded(909, seed, e)
        G = K // gs
        out.append((random_words(rng, (K, N // 8)), random_words(rng, (G, N // 8)),
                    uniform_scales(rng, (G, N), 0.002, 0.02, "fp16")))
    return out


def test_moe_closed_form_constant_experts():
    # expert e with constant code c_e, zero z_e and scale s_e maps row r of its
    # range to (c_e - z_e) s_e sum_k x[r, k] (+ its bias), whatever the others hold
    K, N, gs = 256, 16, 128
    G = K // gs
    consts = [(13, 2, 0.0078125), (0, 15, 0.015625), (9, 9, 0.5)]
    experts = [(constant_words((K, N // 8), c), constant_words((G, N // 8), z), np.full((G, N), s, np.float16))
               for c, z, s in consts]
    offsets = np.array([0, 2, 2, 5])          # the second expert owns no row
    x = normal_acts(seeded(910), (5, K), "fp16")
    bias = uniform_scales(seeded(911), (3, N), -1, 1, "fp16")
    y = O.reference_moe(x, offsets, "awq", "fp16", experts, gs, bias=bias)
    xs = x.astype(np.float64).sum(axis=1)
    expect = np.empty((5, N))
    for e, (c, z, s) in enumerate(consts):
        for r in range(offsets[e], offsets[e + 1]):
            expect[r] = (c - z) * s * xs[r] + bias[e].astype(np.float64)
    np.testing.assert_allclose(y, expect, rtol=1e-13, atol=1e-13)


def test_moe_one_expert_is_the_dense_layer_and_experts_are_independent():
    K, N, gs = 256, 32, 128
    experts = _moe_experts(3, K, N, gs, 1)
    x = normal_acts(seeded(912), (7, K), "fp16")
    # one expert owning every row == the plain layer
    y1 = O.reference_moe(x, np.array([0, 7]), "awq", "fp16", experts[:1], gs)
    qw, qz, sc = experts[0]
    np.testing.assert_array_equal(y1, O.reference_linear(x, "awq", "fp16", qw, qz, sc, gs))
    # reordering the experts together with their row ranges reorders the output rows
    offs = np.array([0, 3, 4, 7])
    y = O.reference_moe(x, offs, "awq", "fp16", experts, gs)
    order = [2, 0, 1]
    xr = np.concatenate([x[offs[e]:offs[e + 1]] for e in order])
    offr = np.concatenate([[0], np.cumsum([offs[e + 1] - offs[e] for e in order])])
    yr = O.reference_moe(xr, offr, "awq", "fp16", [experts[e] for e in order], gs)
    np.testing.assert_array_equal(yr, np.concatenate([y[offs[e]:offs[e + 1]] for e in order]))
    # an expert's rows do not depend on another expert's weights
    other = _moe_experts(3, K, N, gs, 2)
    y2 = O.reference_moe(x, offs, "awq", "fp16", [experts[0], other[1], experts[2]], gs)
    np.testing.assert_array_equal(y2[:3], y[:3])
    np.testing.assert_array_equal(y2[4:], y[4:])
    assert not np.array_equal(y2[3:4], y[3:4])


# ----------------------------------------------------------------------------
# Mutation tests: plant a mistake in the oracle and show a pin catches it
# ----------------------------------------------------------------------------

def test_mutation_wrong_awq_direction_is_caught(monkeypatch):
    # Reading the constant the other way round (column j in slot P[j]).
    import oracle.w4_oracle as W
    monkeypatch.setattr(W, "AWQ_REVERSE_ORDER", (0, 2, 4, 6, 1, 3, 5, 7))
    with pytest.raises(AssertionError):
        test_golden_awq_and_std_words()


def test_mutation_sign_flip_in_dequant_is_caught(monkeypatch):
    import oracle.w4_oracle as W
    orig = W.dequant

    def flipped(codes, zeros, s, grp):
        return -orig(codes, zeros, s, grp)
    monkeypatch.setattr(W, "dequant", flipped)
    with pytest.raises(AssertionError):
        test_closed_form_constant_codes()


def test_mutation_group_index_modulo_is_caught(monkeypatch):
    import oracle.w4_oracle as W

    def modulo(K, group_size, g_idx=None):
        gs = K if group_size == -1 else group_size
        return np.arange(K) % (K // gs)
    monkeypatch.setattr(W, "group_index", modulo)
    with pytest.raises(AssertionError):
        test_one_hot_row_selects_dequantized_row_with_its_group_scale()


def test_mutation_tile_slot_order_is_caught(monkeypatch):
    import oracle.w4_oracle as W
    monkeypatch.setattr(W, "TILE_SLOT_OF_OFFSET", tuple(range(8)))
    with pytest.raises(AssertionError):
        test_tile_golden_words()
