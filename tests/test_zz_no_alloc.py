"""The no-allocation entry point (w4a16_linear_noalloc) against w4a16_linear
with a caller workspace, through the C ABI: bit-identical outputs (both run
the same kernels) on two calls in a row, the second with a smaller input, for
each path that uses a workspace (act-order gather, K-tail padding, split-K
partials, bf16 row sums and fp16 copy of x) and one that uses none; and a
bf16 call whose fp16 copy would not fit the static array, which runs the
wide kernel instead, against the oracle."""
import numpy as np
import pytest

import oracle as O
from synthetic import actorder_gidx, normal_acts, random_words, seeded, uniform_scales
from tests._gpu import act_dtype, filled, say, to_dev, to_host

pytestmark = pytest.mark.gpu

CASES = [
    # (name, K, N, group_size, has_zeros, act_order, dtype, Ms: first, then smaller)
    ("act-order gather + split-K", 1152, 4096, 128, True, True, "fp16", (40, 17)),
    ("act-order gather, large M", 1152, 4096, 128, True, True, "fp16", (300, 3)),
    ("K-tail padding", 1120, 272, 32, True, False, "fp16", (33, 1)),
    ("split-K partials, bf16", 8192, 8192, 128, False, False, "bf16", (64, 32)),
    ("fp16 copy of x, then row sums, bf16", 1152, 8200, 128, True, False, "bf16", (1100, 300)),
    ("no workspace", 1152, 4096, 128, True, False, "fp16", (8, 1)),
]


@pytest.fixture(scope="module")
def W():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import weight_only_int4_gptq_amd as W
    W.lib()
    return W


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_the_workspace_entry_point(W, case):
    import torch
    name, K, N, gs, has_z, act, dtype, Ms = case
    G = K // gs
    rng = seeded(909, K, N, gs, int(act))
    lo, hi = (0.002, 0.02) if dtype == "fp16" else (0.001, 0.01)
    lyr = W.W4A16Linear(K, N, gs, has_z, act, dtype, "std")
    lyr.process_weights_after_loading(to_dev(random_words(rng, (K // 8, N))),
                                      to_dev(random_words(rng, (G, N // 8))) if has_z else None,
                                      to_dev(uniform_scales(rng, (G, N), lo, hi, dtype)),
                                      to_dev(actorder_gidx(rng, K, gs)) if act else None)
    t = lyr.tiled
    bias = to_dev(uniform_scales(seeded(910, N), (N,), -1.0, 1.0, dtype))
    for M in Ms:
        say(f"noalloc {name} M={M} kernel={lyr.kernel_name(M)} workspace={W.w4_workspace_size(lyr.layer, M)}")
        x = to_dev(normal_acts(seeded(911, M, K), (M, K), dtype))
        ws_b = W.w4_workspace_size(lyr.layer, M)
        ws = torch.empty((max(ws_b, 1),), dtype=torch.uint8, device="cuda")
        y_ref = filled((M, N), act_dtype(dtype), 0x00)
        W.w4a16_linear(lyr.layer, M, x, t["qweight"], t["scales"], t["qzeros"], t["perm"], bias, y_ref,
                       ws if ws_b else None, ws_b)
        y = filled((M + 1, N), act_dtype(dtype), 0xFF)
        W.w4a16_linear_noalloc(lyr.layer, M, x, t["qweight"], t["scales"], t["qzeros"], t["perm"], bias, y[:M])
        torch.cuda.synchronize()
        assert np.array_equal(to_host(y[:M]).view(np.uint16), to_host(y_ref).view(np.uint16)), (name, M)
        assert (to_host(y[M:]).view(np.uint16) == 0xFFFF).all(), "write past row M"


def test_noalloc_bf16_copy_too_large_runs_the_wide_kernel(W):
    # at M = 2048, K = 16384 the fp16 copy of x (64 MiB + the row factors)
    # exceeds the static array: the no-allocation call runs the wide kernel
    # with row sums, within the layer's accuracy bound; a smaller second call
    # runs the same kernel as w4a16_linear again
    import torch
    K, N, gs = 16384, 4104, 128
    G = K // gs
    rng = seeded(912, K, N)
    qweight = random_words(rng, (K // 8, N))
    scales = uniform_scales(rng, (G, N), 0.001, 0.01, "bf16")
    lyr = W.W4A16Linear(K, N, gs, False, False, "bf16", "std")
    lyr.process_weights_after_loading(to_dev(qweight), None, to_dev(scales))
    t = lyr.tiled
    assert W.w4_workspace_size(lyr.layer, 2048) > W.w4_noalloc_scratch_bytes()
    for M in (2048, 1100):
        say(f"noalloc bf16 M={M} K={K} kernel={lyr.kernel_name(M)} workspace={W.w4_workspace_size(lyr.layer, M)}")
        xh = normal_acts(seeded(913, M, K), (M, K), "bf16")
        x = to_dev(xh)
        ws_b = W.w4_workspace_size(lyr.layer, M)
        ws = torch.empty((max(ws_b, 1),), dtype=torch.uint8, device="cuda")
        y_ref = filled((M, N), act_dtype("bf16"), 0x00)
        W.w4a16_linear(lyr.layer, M, x, t["qweight"], t["scales"], t["qzeros"], t["perm"], None, y_ref,
                       ws if ws_b else None, ws_b)
        y = filled((M + 1, N), act_dtype("bf16"), 0xFF)
        W.w4a16_linear_noalloc(lyr.layer, M, x, t["qweight"], t["scales"], t["qzeros"], t["perm"], None, y[:M])
        torch.cuda.synchronize()
        assert (to_host(y[M:]).view(np.uint16) == 0xFFFF).all(), "write past row M"
        yb, rb = to_host(y[:M]).view(np.uint16), to_host(y_ref).view(np.uint16)
        if M == 1100:
            assert np.array_equal(yb, rb), M
            continue
        rows = np.r_[0:32, M - 32:M]
        ref = O.reference_linear(xh[rows], "std", "bf16", qweight, None, scales, gs)
        for what, out in (("noalloc", yb), ("workspace", rb)):
            r = O.check(O.bf16_to_f64(out[rows]), ref, 1e-2, 2e-3)
            say(f"  {what}: max_ratio={r['max_ratio']:.3e} rel_fro={r['rel_fro']:.3e}")
            assert r["ok"], (what, r)
