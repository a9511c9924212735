"""create_weights / process_weights_after_loading / apply for one W4A16
linear layer (the three-phase split of the SGLang quantization design page,
section 1, and of the vLLM loading page, "Responsibilities").

torch is used only to allocate device memory and to name the current stream;
every step of the computation runs in libw4hip's HIP kernels.
"""
from __future__ import annotations

import torch

from . import _abi as A

_TORCH_DTYPE = {"fp16": torch.float16, "bf16": torch.bfloat16}


class W4A16Linear:
    """One weight-only INT4 linear layer on the current CUDA (HIP) device.

    fmt "awq": checkpoint qweight int32 [K, N/8] packed along N in the AWQ
    order (the vLLM loading page, "Data flow"); fmt "std": standard/GPTQ
    qweight int32 [K/8, N].  qzeros int32 [G, N/8] (absent when symmetric),
    scales [G, N] in the activation dtype, g_idx int32 [K] with act-order.
    """

    def __init__(self, K: int, N: int, group_size: int = 128, has_zero_points: bool = True,
                 has_g_idx: bool = False, dtype: str = "fp16", fmt: str = "awq", device="cuda"):
        if fmt not in ("awq", "std"):
            raise ValueError(fmt)
        self.layer = A.make_layer(K, N, group_size, has_zero_points, has_g_idx, dtype)
        st = A.w4_check_layer(self.layer)
        if st != A.W4_OK:
            raise A.W4Error("w4_check_layer", st, A.w4_status_str(st))
        self.K, self.N, self.group_size, self.dtype, self.fmt = K, N, group_size, dtype, fmt
        self.has_zero_points, self.has_g_idx = has_zero_points, has_g_idx
        self.G = 1 if group_size == -1 else K // group_size
        self.device = torch.device(device)
        self.sizes = A.w4_sizes(self.layer)
        self.tiled = None

    # -- create_weights ----------------------------------------------------
    def create_weights(self) -> dict:
        """Empty checkpoint parameters with the shapes of the chosen format."""
        d, i32 = self.device, torch.int32
        K, N, G = self.K, self.N, self.G
        qweight = torch.empty((K, N // 8) if self.fmt == "awq" else (K // 8, N), dtype=i32, device=d)
        return {
            "qweight": qweight,
            "qzeros": torch.empty((G, N // 8), dtype=i32, device=d) if self.has_zero_points else None,
            "scales": torch.empty((G, N), dtype=_TORCH_DTYPE[self.dtype], device=d),
            "g_idx": torch.empty((K,), dtype=i32, device=d) if self.has_g_idx else None,
        }

    # -- process_weights_after_loading -------------------------------------
    def process_weights_after_loading(self, qweight, qzeros, scales, g_idx=None, stream=None,
                                      keep_standard: bool = False) -> dict:
        """AWQ -> standard (fmt "awq") then standard -> tile layout.  Re-runnable.
        With act-order the g_idx status word is read back once and a bad
        g_idx raises ValueError."""
        d, i32 = self.device, torch.int32
        K, N, G = self.K, self.N, self.G
        std_w, std_z = qweight, qzeros
        if self.fmt == "awq":
            std_w = torch.empty((K // 8, N), dtype=i32, device=d)
            std_z = torch.empty((G, N // 8), dtype=i32, device=d)
            A.w4_repack_awq(self.layer, qweight, qzeros, std_w, std_z, stream)
        # the tile layout's byte sizes come from the library (w4_sizes), the
        # one place that knows its padding
        sz = self.sizes
        tiled = {
            "qweight": torch.empty((sz["tiled_qweight"] // 4,), dtype=i32, device=d),
            "scales": torch.empty((sz["tiled_scales"] // 2,), dtype=_TORCH_DTYPE[self.dtype], device=d),
            "qzeros": torch.empty((sz["tiled_qzeros"] // 4,), dtype=i32, device=d) if self.has_zero_points else None,
            "perm": torch.empty((sz["perm"] // 4,), dtype=i32, device=d) if self.has_g_idx else None,
        }
        status = torch.empty((1,), dtype=i32, device=d) if self.has_g_idx else None
        A.w4_repack_gptq(self.layer, std_w, std_z, scales, g_idx, tiled["qweight"], tiled["scales"],
                         tiled["qzeros"], tiled["perm"], status, stream)
        if status is not None:
            st = int(status.cpu().item())
            if st != 0:
                raise ValueError(f"invalid g_idx (status bits {st:#x}: 1 = out of range, 2 = group size != "
                                 f"{self.group_size})")
        if keep_standard:
            tiled["std_qweight"], tiled["std_qzeros"] = std_w, std_z
        self.tiled = tiled
        return tiled

    # -- apply -------------------------------------------------------------
    def apply(self, x: torch.Tensor, bias=None, out=None, stream=None) -> torch.Tensor:
        """y = x W + bias; x [..., K] in the activation dtype, leading dims flattened.
        ``out`` (optional) must be a contiguous [M, N] tensor of that dtype on
        the layer's device."""
        if self.tiled is None:
            raise RuntimeError("process_weights_after_loading has not run")
        dt = _TORCH_DTYPE[self.dtype]
        dev = self.tiled["qweight"].device
        if x.dtype != dt or x.device != dev or x.shape[-1] != self.K:
            raise ValueError(f"x must be [..., {self.K}] {dt} on {dev}; got {tuple(x.shape)} {x.dtype} on {x.device}")
        if bias is not None and (bias.dtype != dt or bias.device != dev or tuple(bias.shape) != (self.N,)
                                 or not bias.is_contiguous()):
            raise ValueError(f"bias must be a contiguous [{self.N}] {dt} tensor on {dev}")
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.K)
        if not x2.is_contiguous():
            x2 = x2.contiguous()
        M = x2.shape[0]
        if out is not None and (out.dtype != dt or out.device != dev or tuple(out.shape) != (M, self.N)
                                or not out.is_contiguous()):
            raise ValueError(f"out must be a contiguous [{M}, {self.N}] {dt} tensor on {dev}; got "
                             f"{tuple(out.shape)} {out.dtype} contiguous={out.is_contiguous()}")
        y = out if out is not None else torch.empty((M, self.N), dtype=dt, device=dev)
        ws_bytes = A.w4_workspace_size(self.layer, M)
        st = stream if stream is not None else torch.cuda.current_stream(dev)
        ws = self._workspace(ws_bytes, st) if ws_bytes else None
        t = self.tiled
        A.w4a16_linear(self.layer, M, x2, t["qweight"], t["scales"], t["qzeros"], t["perm"], bias, y, ws, ws_bytes,
                       st)
        return y.reshape(*lead, self.N)

    def _workspace(self, nbytes: int, stream) -> "torch.Tensor":
        """A scratch buffer of at least nbytes for calls on ``stream``: one per
        stream (calls on different streams may overlap; calls on one stream
        are ordered), allocated by torch's caching allocator on that stream,
        so a buffer that is replaced is not reused while the stream still has
        work on it."""
        cache = self.__dict__.setdefault("_ws", {})
        key = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        ws = cache.get(key)
        if ws is None or ws.numel() < nbytes:
            if isinstance(stream, torch.cuda.Stream):
                with torch.cuda.stream(stream):
                    ws = torch.empty((nbytes,), dtype=torch.uint8, device=stream.device)
            else:
                ws = torch.empty((nbytes,), dtype=torch.uint8, device=self.tiled["qweight"].device)
                ws.record_stream(torch.cuda.ExternalStream(key))
            cache[key] = ws
        return ws

    def apply_fp8(self, x: torch.Tensor, x_scale: torch.Tensor, bias=None, out=None, stream=None) -> torch.Tensor:
        """y = s_x x_q W + bias with fp8 (E4M3) activations x_q = e4m3(x / s_x):
        the W4A8 path (w4a8_linear).  x [..., K] in the activation dtype,
        x_scale a one-element float32 tensor on the device (the static
        per-tensor input scale).  Group size 128 or per-channel."""
        if self.tiled is None:
            raise RuntimeError("process_weights_after_loading has not run")
        dt = _TORCH_DTYPE[self.dtype]
        dev = self.tiled["qweight"].device
        if x.dtype != dt or x.device != dev or x.shape[-1] != self.K:
            raise ValueError(f"x must be [..., {self.K}] {dt} on {dev}; got {tuple(x.shape)} {x.dtype} on {x.device}")
        if x_scale.dtype != torch.float32 or x_scale.device != dev or x_scale.numel() != 1:
            raise ValueError("x_scale must be a one-element float32 tensor on the layer's device")
        if bias is not None and (bias.dtype != dt or bias.device != dev or tuple(bias.shape) != (self.N,)
                                 or not bias.is_contiguous()):
            raise ValueError(f"bias must be a contiguous [{self.N}] {dt} tensor on {dev}")
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.K)
        if not x2.is_contiguous():
            x2 = x2.contiguous()
        M = x2.shape[0]
        if out is not None and (out.dtype != dt or out.device != dev or tuple(out.shape) != (M, self.N)
                                or not out.is_contiguous()):
            raise ValueError(f"out must be a contiguous [{M}, {self.N}] {dt} tensor on {dev}")
        y = out if out is not None else torch.empty((M, self.N), dtype=dt, device=dev)
        ws_bytes = A.w4a8_workspace_size(self.layer, M)
        st = stream if stream is not None else torch.cuda.current_stream(dev)
        ws = self._workspace(ws_bytes, st) if ws_bytes else None
        t = self.tiled
        A.w4a8_linear(self.layer, M, x2, x_scale, t["qweight"], t["scales"], t["qzeros"], t["perm"], bias, y, ws,
                      ws_bytes, st)
        return y.reshape(*lead, self.N)

    def dequantize_dense(self, out=None, stream=None) -> torch.Tensor:
        """The dense weight W [K, N] in the activation dtype (for the unfused
        dequantize-then-matmul comparison; the fused apply() never builds it)."""
        if self.tiled is None:
            raise RuntimeError("process_weights_after_loading has not run")
        t = self.tiled
        w = out if out is not None else torch.empty((self.K, self.N), dtype=t["scales"].dtype,
                                                    device=t["qweight"].device)
        A.w4_dequant_dense(self.layer, t["qweight"], t["scales"], t["qzeros"], t["perm"], w, stream)
        return w

    def kernel_name(self, M: int) -> str:
        return A.w4_kernel_name(self.layer, M)


class W4A16MoELinear:
    """The grouped (mixture-of-experts) layer: E experts of one shape, each
    repacked into its slice of stacked tile buffers, applied in one launch to
    rows grouped by expert (w4a16_moe_linear).  Act-order and K % 128 != 0
    are not supported."""

    def __init__(self, num_experts: int, K: int, N: int, group_size: int = 128, has_zero_points: bool = True,
                 dtype: str = "fp16", fmt: str = "awq", device="cuda"):
        if K % 128 != 0:
            raise A.W4Error("W4A16MoELinear", A.W4_ERR_UNSUPPORTED, "the grouped launch needs K % 128 == 0")
        self.E = int(num_experts)
        self.experts = [W4A16Linear(K, N, group_size, has_zero_points, False, dtype, fmt, device=device)
                        for _ in range(self.E)]
        self.K, self.N, self.dtype = K, N, dtype
        self.layer = self.experts[0].layer
        self.tiled = None

    def process_weights_after_loading(self, weights, stream=None) -> dict:
        """weights: per expert (qweight, qzeros, scales) as loaded."""
        tiled = [ex.process_weights_after_loading(qw, qz, sc, None, stream) for ex, (qw, qz, sc) in
                 zip(self.experts, weights)]
        self.tiled = {k: (torch.stack([t[k] for t in tiled]).contiguous() if tiled[0][k] is not None else None)
                      for k in ("qweight", "scales", "qzeros")}
        for ex in self.experts:
            ex.tiled = None  # the stacked copy is the one kept
        return self.tiled

    def apply(self, x: torch.Tensor, expert_offsets: torch.Tensor, max_rows: int = 0, bias=None, out=None,
              stream=None) -> torch.Tensor:
        """y [R, N] for rows x [R, K] grouped by expert (expert_offsets int32 [E + 1] on the device)."""
        if self.tiled is None:
            raise RuntimeError("process_weights_after_loading has not run")
        x2 = x.contiguous()
        R = x2.shape[0]
        y = out if out is not None else torch.empty((R, self.N), dtype=x.dtype, device=x.device)
        t = self.tiled
        A.w4a16_moe_linear(self.layer, self.E, R, max_rows, x2, expert_offsets, t["qweight"], t["scales"],
                           t["qzeros"], bias, y, stream)
        return y
