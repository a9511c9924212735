"""Host-side checks of libw4hip that need no GPU: the library loads, exports
every call include/w4hip.h declares, and rejects bad arguments before any
device work."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4hip.h")


@pytest.fixture(scope="module")
def W():
    import weight_only_int4_gptq_amd as W
    from weight_only_int4_gptq_amd import _abi
    if not os.path.exists(_abi._LIB_PATH):
        # CPU-only convenience: cross-compile in-tree when nothing is built yet.
        from weight_only_int4_gptq_amd import build
        build.build()
    W.lib()
    return W


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:w4_status|const\s+char\s*\*|size_t)\s*(w4\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_lifecycle_calls():
    names = declared_functions()
    for n in ("w4_check_layer", "w4_sizes", "w4_workspace_size", "w4_kernel_name", "w4_status_str",
              "w4_repack_awq", "w4_repack_gptq", "w4a16_linear"):
        assert n in names


def test_library_exports_every_declared_symbol(W):
    L = W.lib()
    for n in declared_functions():
        assert hasattr(L, n), n


def test_check_layer_status_codes(W):
    ok = W.make_layer(512, 256, 128, True, False, "fp16")
    assert W.w4_check_layer(ok) == W.W4_OK
    assert W.lib().w4_check_layer(None) == W.W4_ERR_INVALID_ARGUMENT
    bad = [
        (dict(K=0), W.W4_ERR_INVALID_ARGUMENT), (dict(N=-16), W.W4_ERR_INVALID_ARGUMENT),
        (dict(group_size=16), W.W4_ERR_UNSUPPORTED), (dict(group_size=256), W.W4_ERR_UNSUPPORTED),
        (dict(group_size=0), W.W4_ERR_UNSUPPORTED), (dict(K=200), W.W4_ERR_UNSUPPORTED),
        (dict(N=20), W.W4_ERR_UNSUPPORTED), (dict(K=2 ** 21), W.W4_ERR_UNSUPPORTED),
        (dict(group_size=-1, has_g_idx=True), W.W4_ERR_UNSUPPORTED), (dict(dtype=2), W.W4_ERR_UNSUPPORTED),
    ]
    for over, expect in bad:
        kw = dict(K=512, N=256, group_size=128, has_zero_points=True, has_g_idx=False, dtype="fp16")
        kw.update(over)
        assert W.w4_check_layer(W.make_layer(**kw)) == expect, over
    for gs in (-1, 32, 64, 128):
        assert W.w4_check_layer(W.make_layer(384, 48, gs, False, False, "bf16")) == W.W4_OK
    # N % 16 == 8 is accepted: the tile layout pads the last strip to 16 columns
    assert W.w4_check_layer(W.make_layer(512, 24)) == W.W4_OK
    s = W.w4_sizes(W.make_layer(512, 24, 128, True, False, "fp16"))
    assert s["tiled_qweight"] == 512 * 32 // 2 and s["tiled_scales"] == 4 * 32 * 2
    assert s["tiled_qzeros"] == 2 * 4 * 2 * 4 and s["std_qweight"] == 64 * 24 * 4
    # K % 128 != 0 (K % 32 == 0) is accepted for group sizes 32, 64 and
    # per-channel without act-order: the tile layout pads rows to Kp
    for K, gs in ((96, 32), (320, 64), (320, -1), (32, -1), (1120, 32)):
        assert W.w4_check_layer(W.make_layer(K, 256, gs, True, False, "fp16")) == W.W4_OK, (K, gs)
    for K, gs, gi in ((320, 64, True), (672, 128, False), (336, 32, False), (96, 32, True)):
        assert W.w4_check_layer(W.make_layer(K, 256, gs, True, gi, "fp16")) == W.W4_ERR_UNSUPPORTED, (K, gs, gi)
    s = W.w4_sizes(W.make_layer(320, 24, 64, True, False, "fp16"))
    assert s["tiled_qweight"] == 384 * 32 // 2 and s["tiled_scales"] == 6 * 32 * 2
    assert s["tiled_qzeros"] == 2 * 6 * 2 * 4 and s["std_qweight"] == 40 * 24 * 4 and s["scales"] == 5 * 24 * 2
    s = W.w4_sizes(W.make_layer(320, 256, -1, True, False, "bf16"))
    assert s["tiled_qweight"] == 384 * 256 // 2 and s["tiled_scales"] == 256 * 2 and s["tiled_qzeros"] == 16 * 2 * 4


def test_sizes_of_the_tiny_layer(W):
    s = W.w4_sizes(W.make_layer(512, 256, 128, True, False, "fp16"))
    assert s == dict(awq_qweight=512 * 32 * 4, qzeros=4 * 32 * 4, scales=4 * 256 * 2, std_qweight=64 * 256 * 4,
                     tiled_qweight=512 * 256 // 2, tiled_scales=4 * 256 * 2, tiled_qzeros=16 * 4 * 2 * 4, perm=0)
    s = W.w4_sizes(W.make_layer(8192, 8192, 128, True, True, "fp16"))
    assert s["perm"] == 8192 * 4
    s = W.w4_sizes(W.make_layer(8192, 8192, -1, False, False, "bf16"))
    assert s["scales"] == 8192 * 2 and s["qzeros"] == 0 and s["tiled_qzeros"] == 0
    with pytest.raises(W.W4Error):
        W.w4_sizes(W.make_layer(100, 256))


def test_workspace_and_kernel_name(W):
    L = W.make_layer(4096, 4096)
    assert W.w4_workspace_size(L, 0) == 0
    assert W.w4_workspace_size(L, 16) >= 0
    with pytest.raises(W.W4Error):
        W.w4_workspace_size(L, -1)
    assert W.w4_kernel_name(L, 0) == "none"
    assert W.w4_kernel_name(L, -3) == "invalid"
    assert W.w4_kernel_name(W.make_layer(100, 16), 1) == "invalid"
    assert W.w4_kernel_name(L, 1).startswith("w4_")
    # a K tail needs the zero-padded activations in the workspace
    Lt = W.make_layer(320, 256, 64, True, False, "fp16")
    assert W.w4_workspace_size(Lt, 4) >= 4 * 384 * 2 and W.w4_kernel_name(Lt, 4).startswith("w4_")
    assert W.w4_workspace_size(W.make_layer(384, 256, 64, True, False, "fp16"), 4) == 0
    for s in range(5):
        assert W.w4_status_str(s)
    assert W.w4_status_str(99) == "unknown status"


def test_launch_dims_follow_the_kernel_choice(W):
    # skinny, activations in LDS: one workgroup of 8 waves per 16-column strip
    L = W.make_layer(4096, 12288)
    assert W.w4_kernel_name(L, 1) == "w4_skinny_lds_k8"
    assert W.w4_launch_dims(L, 1) == ((768, 1, 1), 512)
    # narrow layer, M <= 4: 16 waves, the activation rows copied per block
    L = W.make_layer(4096, 4096)
    assert W.w4_kernel_name(L, 1) == "w4_skinny_dma4_k16"
    assert W.w4_launch_dims(L, 4) == ((256, 1, 1), 1024)
    # skinny, 16 waves, one strip per workgroup (M < 8 on a narrow layer)
    assert W.w4_kernel_name(L, 5) == "w4_skinny_k16"
    assert W.w4_launch_dims(L, 5) == ((256, 1, 1), 1024)
    # activation tiles through LDS: eight waves, one strip (narrow) or two
    assert W.w4_kernel_name(L, 16) == "w4_skinny_dma_k8"
    assert W.w4_launch_dims(L, 16) == ((256, 1, 1), 512)
    L8 = W.make_layer(8192, 8192)
    assert W.w4_kernel_name(L8, 9) == "w4_skinny_dma_n2_k8"
    assert W.w4_launch_dims(L8, 9) == ((256, 1, 1), 512)
    # three strips per workgroup on 513..768 strips divisible by three (one
    # round of at most 256 workgroups), else the shared-tile 16-row kernel
    L = W.make_layer(4096, 12288)
    assert W.w4_kernel_name(L, 16) == "w4_skinny_dma_n3_k8"
    assert W.w4_launch_dims(L, 16) == ((256, 1, 1), 512)
    assert W.w4_kernel_name(W.make_layer(4096, 9216), 9) == "w4_skinny_dma_n3_k8"
    assert W.w4_launch_dims(W.make_layer(4096, 9216), 9) == ((192, 1, 1), 512)
    L = W.make_layer(4096, 10240)
    assert W.w4_kernel_name(L, 16) == "w4_wide_16x64_w4"
    assert W.w4_launch_dims(L, 16) == ((160, 1, 1), 256)
    assert W.w4_kernel_name(W.make_layer(4096, 22016), 8) == "w4_wide_16x32_w2"
    # large M: one 1-D grid of 128 x 256 tiles of four waves
    L = W.make_layer(8192, 8192)
    assert W.w4_kernel_name(L, 2048) == "w4_big_128x256"
    assert W.w4_launch_dims(L, 2048) == ((16 * 32, 1, 1), 256)
    # split-K wide tiles: the K ranges along z
    name = W.w4_kernel_name(L, 64)
    (gx, gy, gz), t = W.w4_launch_dims(L, 64)
    assert name.endswith("_splitk") and gz > 1 and t % 64 == 0
    with pytest.raises(W.W4Error):
        W.w4_launch_dims(L, 0)


def test_w4a8_kernel_choice(W):
    # decode rows: K split over the waves of a workgroup on narrow layers
    assert W.w4a8_kernel_name(W.make_layer(4096, 4096), 1) == "w4a8_f8_skinny_k16"
    assert W.w4a8_kernel_name(W.make_layer(11008, 4096), 16) == "w4a8_f8_skinny_dma_k8"
    assert W.w4a8_kernel_name(W.make_layer(4096, 4096), 16) == "w4a8_f8_skinny_dma_k16"
    assert W.w4a8_kernel_name(W.make_layer(4096, 12288), 4) == "w4a8_f8_skinny_dma_k4"
    assert W.w4a8_kernel_name(W.make_layer(11008, 4096), 1) == "w4a8_f8_skinny_k16_r2"
    assert W.w4a8_kernel_name(W.make_layer(4096, 12288), 16) == "w4a8_f8_skinny_dma_k8"
    assert W.w4a8_kernel_name(W.make_layer(4096, 22016), 1) == "w4a8_f8_16x16"
    assert W.w4a8_kernel_name(W.make_layer(8192, 8192), 64) == "w4a8_f8_64x128"
    assert W.w4a8_kernel_name(W.make_layer(8192, 8192), 2048) == "w4a8_f8_64x256"


def test_floor_library_exports_its_kernels():
    from weight_only_int4_gptq_amd import build
    if not os.path.exists(build.FLOOR_LIB):
        build.build()
    F = ctypes.CDLL(build.FLOOR_LIB)
    assert hasattr(F, "w4floor_stream") and hasattr(F, "w4floor_empty")
    # bad sizes and grids are refused on the host (no GPU call is made)
    F.w4floor_stream.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint32),
                                 ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    F.w4floor_empty.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p]
    g = (ctypes.c_uint32 * 3)(4, 1, 1)
    assert F.w4floor_stream(16, 24, g, 256, 16, 0, None) != 0        # bytes not a multiple of 16
    assert F.w4floor_stream(16, 32, g, 100, 16, 0, None) != 0        # workgroup not whole waves
    assert F.w4floor_empty((ctypes.c_uint32 * 3)(0, 1, 1), 256, 0, None) != 0


def _lin(W, L, M, x=16, qw=16, sc=16, qz=16, perm=None, bias=None, y=16, ws=None, ws_bytes=0):
    return W.lib().w4a16_linear(ctypes.byref(L), M, x, qw, sc, qz, perm, bias, y, ws, ws_bytes, None)


def test_linear_rejects_bad_arguments_before_any_launch(W):
    L = W.make_layer(512, 256, 128, True, False, "fp16")
    assert _lin(W, L, -1) == W.W4_ERR_INVALID_ARGUMENT
    assert _lin(W, L, 1, x=None) == W.W4_ERR_INVALID_ARGUMENT
    assert _lin(W, L, 1, y=None) == W.W4_ERR_INVALID_ARGUMENT
    assert _lin(W, L, 1, y=18) == W.W4_ERR_INVALID_ARGUMENT              # y must be 4-byte aligned
    assert _lin(W, L, 1, qz=None) == W.W4_ERR_INVALID_ARGUMENT          # zero points declared, none given
    assert _lin(W, L, 1, x=24) == W.W4_ERR_INVALID_ARGUMENT             # x not 16-byte aligned
    assert _lin(W, L, 1, qw=8) == W.W4_ERR_INVALID_ARGUMENT
    assert _lin(W, L, 1, perm=16) == W.W4_ERR_INVALID_ARGUMENT          # perm without act-order
    assert _lin(W, L, 2 ** 25) == W.W4_ERR_UNSUPPORTED
    assert _lin(W, L, 0) == W.W4_OK                                     # M == 0: nothing to do
    La = W.make_layer(512, 256, 128, True, True, "fp16")
    assert _lin(W, La, 1) == W.W4_ERR_INVALID_ARGUMENT                  # act-order needs perm
    Ls = W.make_layer(512, 256, 128, False, False, "bf16")
    assert _lin(W, Ls, 1) == W.W4_ERR_INVALID_ARGUMENT                  # zeros given for a symmetric layer
    bad = W.make_layer(100, 256)
    assert _lin(W, bad, 1) == W.W4_ERR_UNSUPPORTED


def test_repacks_reject_bad_arguments(W):
    lib = W.lib()
    L = W.make_layer(512, 256, 128, True, False, "fp16")
    sym = W.make_layer(512, 256, 128, False, False, "fp16")
    assert lib.w4_repack_awq(ctypes.byref(sym), 16, 16, 16, 16, None) == W.W4_ERR_UNSUPPORTED
    assert lib.w4_repack_awq(ctypes.byref(L), None, 16, 16, 16, None) == W.W4_ERR_INVALID_ARGUMENT
    assert lib.w4_repack_awq(ctypes.byref(L), 16, 16, 20, 16, None) == W.W4_ERR_INVALID_ARGUMENT
    g = lib.w4_repack_gptq
    assert g(ctypes.byref(L), 16, None, 16, None, 16, 16, 16, None, None, None) == W.W4_ERR_INVALID_ARGUMENT
    assert g(ctypes.byref(sym), 16, 16, 16, None, 16, 16, None, None, None, None) == W.W4_ERR_INVALID_ARGUMENT
    act = W.make_layer(512, 256, 128, True, True, "fp16")
    assert g(ctypes.byref(act), 16, 16, 16, None, 16, 16, 16, 16, None, None) == W.W4_ERR_INVALID_ARGUMENT
    assert g(ctypes.byref(act), 16, 16, 16, 16, 16, 16, 16, 20, None, None) == W.W4_ERR_INVALID_ARGUMENT


def test_split_k_workspace_is_sized_and_checked(W):
    # mid-size M on a layer with N <= 16384 splits K over four workgroups:
    # fp32 partials [4][M][N] live in the workspace
    L = W.make_layer(8192, 8192, 128, False, False, "bf16")
    assert W.w4_kernel_name(L, 32).endswith("splitk")
    assert W.w4_workspace_size(L, 32) == 4 * 32 * 8192 * 4
    assert W.w4_workspace_size(L, 64) == 4 * 64 * 8192 * 4
    assert W.w4_workspace_size(L, 128) == 4 * 128 * 8192 * 4
    assert W.w4_workspace_size(L, 1) == 0
    # bf16 from M = 256 (and M = 64 on long or wide layers): the row sums of x
    # per 128-row block follow, [K / 128][M] fp32; above 128 rows a K of
    # 8192 splits two ways
    assert W.w4_workspace_size(L, 256) == 2 * 256 * 8192 * 4 + 64 * 256 * 4
    # with >= 256 tiles of 128 x 256 the 32x32x16 kernel runs on an fp16
    # copy of x [M][K] and its row factors, fp32 for whole 128-row tiles
    assert W.w4_kernel_name(L, 2048) == "w4_big_128x256"
    assert W.w4_workspace_size(L, 2048) == 2048 * 8192 * 2 + 2048 * 4
    assert W.w4_workspace_size(L, 1000) == 1000 * 8192 * 2 + 1024 * 4
    assert W.w4_workspace_size(L, 1030) == 1030 * 8192 * 2 + 1152 * 4
    # fewer tiles: the 128 x 128 wide tile with row sums
    L4 = W.make_layer(8192, 4096, 128, False, False, "bf16")
    assert W.w4_kernel_name(L4, 1024) == "w4_wide_128x128"
    assert W.w4_workspace_size(L4, 1024) == 64 * 1024 * 4
    # a longer K splits eight ways (four at M = 256)
    L2 = W.make_layer(28672, 8192, 128, False, False, "bf16")
    assert W.w4_workspace_size(L2, 32) == 8 * 32 * 8192 * 4
    assert W.w4_workspace_size(L2, 64) == 8 * 64 * 8192 * 4 + 224 * 64 * 4
    assert W.w4_workspace_size(L2, 256) == 4 * 256 * 8192 * 4 + 224 * 256 * 4
    # N = 57344 has workgroups enough: no split, only the row sums
    assert W.w4_workspace_size(W.make_layer(8192, 57344, 128, False, False, "bf16"), 128) == 64 * 128 * 4
    # g = 32: four sums per block; fp16 layers need none
    assert W.w4_workspace_size(W.make_layer(8192, 57344, 32, False, False, "bf16"), 128) == 256 * 128 * 4
    assert W.w4_workspace_size(W.make_layer(8192, 57344, 128, False, False, "fp16"), 128) == 0
    # act-order: the gathered activations (256-byte aligned) come first
    La = W.make_layer(8192, 8192, 128, True, True, "fp16")
    assert W.w4_workspace_size(La, 64) == 64 * 8192 * 2 + 4 * 64 * 8192 * 4
    # too small a workspace is refused before any launch
    need = W.w4_workspace_size(L, 32)
    assert _lin(W, L, 32, qz=None, ws=16, ws_bytes=need - 1) == W.W4_ERR_WORKSPACE
    assert _lin(W, L, 32, qz=None, ws=None, ws_bytes=0) == W.W4_ERR_WORKSPACE


def test_moe_rejects_k_tails_and_act_order(W):
    # the grouped launch runs whole 128-row blocks only, without act-order
    for L in (W.make_layer(320, 256, 64, True, False, "fp16"), W.make_layer(512, 256, 128, True, True, "fp16")):
        st = W.lib().w4a16_moe_linear(ctypes.byref(L), 2, 8, 4, 16, 16, 16, 16, 16, None, 16, None)
        assert st == W.W4_ERR_UNSUPPORTED


def test_noalloc_linear_rejects_before_any_launch(W):
    # the static workspace bounds what a no-allocation call can run; every
    # refusal happens on the host
    lib = W.lib()
    assert W.w4_noalloc_scratch_bytes() == 64 << 20

    def na(L, M, x=16, qw=16, sc=16, qz=16, perm=None, bias=None, y=16):
        return lib.w4a16_linear_noalloc(ctypes.byref(L), M, x, qw, sc, qz, perm, bias, y, None)

    L = W.make_layer(512, 256, 128, True, False, "fp16")
    assert na(L, -1) == W.W4_ERR_INVALID_ARGUMENT
    assert na(L, 1, x=None) == W.W4_ERR_INVALID_ARGUMENT
    assert na(L, 1, y=18) == W.W4_ERR_INVALID_ARGUMENT
    assert na(L, 0) == W.W4_OK
    # act-order at M = 8192, K = 8192 needs a 128 MiB gather: over the limit
    La = W.make_layer(8192, 8192, 128, True, True, "fp16")
    assert W.w4_workspace_size(La, 8192) > W.w4_noalloc_scratch_bytes()
    assert na(La, 8192, perm=16) == W.W4_ERR_WORKSPACE
    # every mid-batch split-K workspace fits
    for K, N in ((8192, 10240), (8192, 8192), (28672, 8192)):
        for M in (32, 64, 128, 256):
            assert W.w4_workspace_size(W.make_layer(K, N, 128, False, False, "bf16"), M) <= W.w4_noalloc_scratch_bytes()


def test_w4a8_rejects_before_any_launch(W):
    lib = W.lib()
    # group sizes other than 128 and per-channel are not W4A8 layers
    for gs in (32, 64):
        L = W.make_layer(512, 256, gs, True, False, "fp16")
        assert W.w4a8_kernel_name(L, 4) == "invalid"
        assert lib.w4a8_linear(ctypes.byref(L), 4, 16, 16, 16, 16, 16, None, None, 16, 16, 1 << 20, None) == \
            W.W4_ERR_UNSUPPORTED
    L = W.make_layer(512, 256, 128, True, False, "fp16")
    # workspace: quantized activations [M][Kp] (256-byte aligned), then the
    # block sums [Kp/128][M rounded up to 4] fp32
    assert W.w4a8_workspace_size(L, 5) == 5 * 512 + (512 // 128) * 8 * 4          # 2560 is 256-aligned
    assert W.w4a8_workspace_size(L, 3) == 1536 + 4 * 4 * 4
    assert W.w4a8_workspace_size(L, 1) == 512 + 4 * 4 * 4
    assert W.w4a8_workspace_size(W.make_layer(256, 40, 128, True, False, "fp16"), 1) == 256 + 2 * 4 * 4
    assert W.w4a8_workspace_size(W.make_layer(224, 40, -1, False, False, "bf16"), 3) == 3 * 256 + 2 * 4 * 4
    assert W.w4a8_workspace_size(W.make_layer(128, 40, -1, False, False, "bf16"), 1) == 256 + 1 * 4 * 4

    def lin(M, x=16, xs=16, ws=16, wsb=1 << 20):
        return lib.w4a8_linear(ctypes.byref(L), M, x, xs, 16, 16, 16, None, None, 16, ws, wsb, None)

    assert lin(0) == W.W4_OK
    assert lin(4, x=None) == W.W4_ERR_INVALID_ARGUMENT
    assert lin(4, xs=None) == W.W4_ERR_INVALID_ARGUMENT
    assert lin(4, xs=18) == W.W4_ERR_INVALID_ARGUMENT      # fp32 scale, 4-byte aligned
    assert lin(4, wsb=W.w4a8_workspace_size(L, 4) - 1) == W.W4_ERR_WORKSPACE
    q = lib.w4a8_quantize
    assert q(ctypes.byref(L), 4, 16, 16, 16, 16, 16, None) == W.W4_ERR_INVALID_ARGUMENT   # perm without act-order
    assert q(ctypes.byref(L), 4, 16, 16, None, 12, 16, None) == W.W4_ERR_INVALID_ARGUMENT  # xq 8-byte aligned
    assert q(ctypes.byref(L), 0, 16, 16, None, 16, 16, None) == W.W4_OK
