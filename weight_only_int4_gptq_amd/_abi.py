"""ctypes binding of libw4hip (include/w4hip.h): same names, argument
marshalling only.  Device buffers may be passed as torch tensors (their
data_ptr() is used) or as integer addresses; ``stream`` is a torch stream, an
integer hipStream_t or None for torch's current stream.  A nonzero status
raises ``W4Error``.

The library must have been built (``python -m weight_only_int4_gptq_amd.build``);
loading fails loudly otherwise -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw4hip.so")

W4_OK, W4_ERR_INVALID_ARGUMENT, W4_ERR_UNSUPPORTED, W4_ERR_WORKSPACE, W4_ERR_HIP = range(5)
W4_FP16, W4_BF16 = 0, 1
DTYPES = {"fp16": W4_FP16, "bf16": W4_BF16}


class W4Error(RuntimeError):
    def __init__(self, call: str, status: int, msg: str):
        super().__init__(f"{call}: {msg} (status {status})")
        self.status = status


class w4_layer(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int64), ("N", ctypes.c_int64), ("group_size", ctypes.c_int32),
                ("has_zero_points", ctypes.c_int32), ("has_g_idx", ctypes.c_int32), ("act_dtype", ctypes.c_int32)]


class w4_sizes_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("awq_qweight", "qzeros", "scales", "std_qweight", "tiled_qweight",
                                                "tiled_scales", "tiled_qzeros", "perm")]

    def as_dict(self) -> dict:
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


def make_layer(K: int, N: int, group_size: int = 128, has_zero_points: bool = True, has_g_idx: bool = False,
               dtype: str = "fp16") -> w4_layer:
    return w4_layer(int(K), int(N), int(group_size), int(bool(has_zero_points)), int(bool(has_g_idx)),
                    DTYPES[dtype] if isinstance(dtype, str) else int(dtype))


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libw4hip; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"libw4hip.so not found at {_LIB_PATH}; build it with "
                              f"`python -m weight_only_int4_gptq_amd.build` (no fallback path exists)")
        L = ctypes.CDLL(_LIB_PATH)
        P, I64, SZ, VP = ctypes.POINTER, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
        sig = {
            "w4_check_layer": ([P(w4_layer)], ctypes.c_int),
            "w4_sizes": ([P(w4_layer), P(w4_sizes_t)], ctypes.c_int),
            "w4_workspace_size": ([P(w4_layer), I64, P(SZ)], ctypes.c_int),
            "w4_kernel_name": ([P(w4_layer), I64], ctypes.c_char_p),
            "w4_launch_dims": ([P(w4_layer), I64, P(ctypes.c_uint32), P(ctypes.c_uint32)], ctypes.c_int),
            "w4_status_str": ([ctypes.c_int], ctypes.c_char_p),
            "w4_repack_awq": ([P(w4_layer), VP, VP, VP, VP, VP], ctypes.c_int),
            "w4_repack_gptq": ([P(w4_layer), VP, VP, VP, VP, VP, VP, VP, VP, VP, VP], ctypes.c_int),
            "w4a16_linear": ([P(w4_layer), I64, VP, VP, VP, VP, VP, VP, VP, VP, SZ, VP], ctypes.c_int),
            "w4_dequant_dense": ([P(w4_layer), VP, VP, VP, VP, VP, VP], ctypes.c_int),
            "w4a16_moe_linear": ([P(w4_layer), ctypes.c_int32, I64, I64, VP, VP, VP, VP, VP, VP, VP, VP],
                                 ctypes.c_int),
            "w4a16_linear_noalloc": ([P(w4_layer), I64, VP, VP, VP, VP, VP, VP, VP, VP], ctypes.c_int),
            "w4a8_quantize": ([P(w4_layer), I64, VP, VP, VP, VP, VP, VP], ctypes.c_int),
            "w4a8_workspace_size": ([P(w4_layer), I64, P(SZ)], ctypes.c_int),
            "w4a8_linear": ([P(w4_layer), I64, VP, VP, VP, VP, VP, VP, VP, VP, VP, SZ, VP], ctypes.c_int),
            "w4a8_kernel_name": ([P(w4_layer), I64], ctypes.c_char_p),
            "w4_noalloc_scratch_bytes": ([], SZ),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _raise(call: str, st: int):
    if st != W4_OK:
        raise W4Error(call, st, w4_status_str(st))


def w4_status_str(status: int) -> str:
    return lib().w4_status_str(int(status)).decode()


def w4_check_layer(layer: w4_layer) -> int:
    """Status code of the descriptor check (does not raise)."""
    return lib().w4_check_layer(ctypes.byref(layer))


def w4_sizes(layer: w4_layer) -> dict:
    out = w4_sizes_t()
    _raise("w4_sizes", lib().w4_sizes(ctypes.byref(layer), ctypes.byref(out)))
    return out.as_dict()


def w4_workspace_size(layer: w4_layer, M: int) -> int:
    b = ctypes.c_size_t(0)
    _raise("w4_workspace_size", lib().w4_workspace_size(ctypes.byref(layer), int(M), ctypes.byref(b)))
    return int(b.value)


def w4_kernel_name(layer: w4_layer, M: int) -> str:
    return lib().w4_kernel_name(ctypes.byref(layer), int(M)).decode()


def w4_launch_dims(layer: w4_layer, M: int):
    """((gx, gy, gz), threads) of the GEMM kernel w4a16_linear runs for M rows."""
    g = (ctypes.c_uint32 * 3)()
    t = ctypes.c_uint32(0)
    _raise("w4_launch_dims", lib().w4_launch_dims(ctypes.byref(layer), int(M), g, ctypes.byref(t)))
    return (int(g[0]), int(g[1]), int(g[2])), int(t.value)


def w4_repack_awq(layer, awq_qweight, awq_qzeros, std_qweight, std_qzeros, stream=None) -> None:
    _raise("w4_repack_awq", lib().w4_repack_awq(ctypes.byref(layer), _ptr(awq_qweight), _ptr(awq_qzeros),
                                                _ptr(std_qweight), _ptr(std_qzeros), _stream(stream)))


def w4_repack_gptq(layer, std_qweight, std_qzeros, scales, g_idx, tiled_qweight, tiled_scales, tiled_qzeros,
                   perm, status_dev=None, stream=None) -> None:
    _raise("w4_repack_gptq", lib().w4_repack_gptq(
        ctypes.byref(layer), _ptr(std_qweight), _ptr(std_qzeros), _ptr(scales), _ptr(g_idx), _ptr(tiled_qweight),
        _ptr(tiled_scales), _ptr(tiled_qzeros), _ptr(perm), _ptr(status_dev), _stream(stream)))


def w4a16_linear(layer, M, x, tiled_qweight, tiled_scales, tiled_qzeros, perm, bias, y, workspace=None,
                 workspace_bytes: int = 0, stream=None) -> None:
    _raise("w4a16_linear", lib().w4a16_linear(
        ctypes.byref(layer), int(M), _ptr(x), _ptr(tiled_qweight), _ptr(tiled_scales), _ptr(tiled_qzeros),
        _ptr(perm), _ptr(bias), _ptr(y), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def w4_dequant_dense(layer, tiled_qweight, tiled_scales, tiled_qzeros, perm, w, stream=None) -> None:
    """Dense W [K][N] in the activation dtype (the unfused comparison path)."""
    _raise("w4_dequant_dense", lib().w4_dequant_dense(
        ctypes.byref(layer), _ptr(tiled_qweight), _ptr(tiled_scales), _ptr(tiled_qzeros), _ptr(perm), _ptr(w),
        _stream(stream)))


def w4a16_moe_linear(layer, num_experts, total_rows, max_rows, x, expert_offsets, tiled_qweight, tiled_scales,
                     tiled_qzeros, bias, y, stream=None) -> None:
    """Grouped W4A16 linear of a mixture-of-experts layer (rows grouped by expert)."""
    _raise("w4a16_moe_linear", lib().w4a16_moe_linear(
        ctypes.byref(layer), int(num_experts), int(total_rows), int(max_rows), _ptr(x), _ptr(expert_offsets),
        _ptr(tiled_qweight), _ptr(tiled_scales), _ptr(tiled_qzeros), _ptr(bias), _ptr(y), _stream(stream)))


def w4a16_linear_noalloc(layer, M, x, tiled_qweight, tiled_scales, tiled_qzeros, perm, bias, y, stream=None) -> None:
    """w4a16_linear with the library's static device workspace (allocates nothing)."""
    _raise("w4a16_linear_noalloc", lib().w4a16_linear_noalloc(
        ctypes.byref(layer), int(M), _ptr(x), _ptr(tiled_qweight), _ptr(tiled_scales), _ptr(tiled_qzeros),
        _ptr(perm), _ptr(bias), _ptr(y), _stream(stream)))


def w4_noalloc_scratch_bytes() -> int:
    return int(lib().w4_noalloc_scratch_bytes())


def w4a8_quantize(layer, M, x, x_scale, perm, xq, rowsum, stream=None) -> None:
    """E4M3 activations in operand order and their 128-column block sums."""
    _raise("w4a8_quantize", lib().w4a8_quantize(ctypes.byref(layer), int(M), _ptr(x), _ptr(x_scale), _ptr(perm),
                                                _ptr(xq), _ptr(rowsum), _stream(stream)))


def w4a8_workspace_size(layer, M) -> int:
    b = ctypes.c_size_t(0)
    _raise("w4a8_workspace_size", lib().w4a8_workspace_size(ctypes.byref(layer), int(M), ctypes.byref(b)))
    return int(b.value)


def w4a8_linear(layer, M, x, x_scale, tiled_qweight, tiled_scales, tiled_qzeros, perm, bias, y, workspace,
                workspace_bytes, stream=None) -> None:
    """INT4 weights x FP8 activations (static per-tensor scale x_scale[0])."""
    _raise("w4a8_linear", lib().w4a8_linear(
        ctypes.byref(layer), int(M), _ptr(x), _ptr(x_scale), _ptr(tiled_qweight), _ptr(tiled_scales),
        _ptr(tiled_qzeros), _ptr(perm), _ptr(bias), _ptr(y), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def w4a8_kernel_name(layer, M) -> str:
    return lib().w4a8_kernel_name(ctypes.byref(layer), int(M)).decode()
