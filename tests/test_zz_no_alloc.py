"""The no-allocation entry point (w4a16_linear_noalloc) against w4a16_linear
with a caller workspace, through the C ABI: bit-identical outputs (both run
the same kernels) on two calls in a row, the second with a smaller input, for
each path that uses a workspace (act-order gather, K-tail padding, split-K
partials) and one that uses none."""
import numpy as np
import pytest

from synthetic import actorder_gidx, normal_acts, random_words, seeded, uniform_scales
from tests._gpu import act_dtype, filled, say, to_dev, to_host

pytestmark = pytest.mark.gpu

CASES = [
    # (name, K, N, group_size, has_zeros, act_order, dtype, Ms: first, then smaller)
    ("act-order gather + split-K", 1152, 4096, 128, True, True, "fp16", (40, 17)),
    ("act-order gather, large M", 1152, 4096, 128, True, True, "fp16", (300, 3)),
    ("K-tail padding", 1120, 272, 32, True, False, "fp16", (33, 1)),
    ("split-K partials, bf16", 8192, 8192, 128, False, False, "bf16", (64, 32)),
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
