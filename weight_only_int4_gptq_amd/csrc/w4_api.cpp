// extern "C" entry points of libw4hip: host-side validation, sizes and the
// launches of the repack and GEMM kernels.  See include/w4hip.h for the
// contract of every call.
#include <atomic>
#include <cstring>

#include "w4_internal.h"

namespace {

using w4::Shape;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Device check (gfx950 only), cached per device ordinal.
std::atomic<int> g_dev_state[64];  // 0 unknown, 1 gfx950, 2 other

constexpr int64_t kMaxDim = int64_t(1) << 20;
constexpr int64_t kMaxM = int64_t(1) << 24;

}  // namespace

namespace w4 {

w4_status device_status() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return W4_ERR_HIP;
  if (dev < 64) {
    const int st = g_dev_state[dev].load(std::memory_order_relaxed);
    if (st == 1) return W4_OK;
    if (st == 2) return W4_ERR_UNSUPPORTED;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return W4_ERR_HIP;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_dev_state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? W4_OK : W4_ERR_UNSUPPORTED;
}

w4_status linear_checks(const w4_layer* L, int64_t M, const void* x, const int32_t* tiled_qweight,
                        const void* tiled_scales, const int32_t* tiled_qzeros, const int32_t* perm, const void* bias,
                        const void* y) {
  const w4_status st = w4_check_layer(L);
  if (st != W4_OK) return st;
  if (M < 0) return W4_ERR_INVALID_ARGUMENT;
  if (M > kMaxM) return W4_ERR_UNSUPPORTED;
  const Shape s = shape_of(L);
  if (!x || !tiled_qweight || !tiled_scales || !y) return W4_ERR_INVALID_ARGUMENT;
  if (s.has_z != (tiled_qzeros != nullptr) || s.has_perm != (perm != nullptr)) return W4_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(tiled_qweight, 16) || !aligned(tiled_scales, 2) || !aligned(y, 4) ||
      (bias && !aligned(bias, 2)) || (tiled_qzeros && !aligned(tiled_qzeros, 4)) || (perm && !aligned(perm, 16)))
    return W4_ERR_INVALID_ARGUMENT;
  return W4_OK;
}

}  // namespace w4

using w4::device_status;

extern "C" {

w4_status w4_check_layer(const w4_layer* L) {
  if (L == nullptr) return W4_ERR_INVALID_ARGUMENT;
  if (L->K <= 0 || L->N <= 0) return W4_ERR_INVALID_ARGUMENT;
  if (L->act_dtype != W4_FP16 && L->act_dtype != W4_BF16) return W4_ERR_UNSUPPORTED;
  const int gs = L->group_size;
  if (gs != -1 && gs != 32 && gs != 64 && gs != 128) return W4_ERR_UNSUPPORTED;
  if (L->K > kMaxDim || L->N > kMaxDim) return W4_ERR_UNSUPPORTED;
  // N tail: a padded last strip.  K tail (K % 128 != 0): padded rows, for
  // K % 32 == 0 with group sizes 32, 64 or per-channel and no act-order
  if (L->N % 8 != 0 || L->K % 32 != 0) return W4_ERR_UNSUPPORTED;
  if (L->K % w4::kTileK != 0 && (gs == 128 || L->has_g_idx)) return W4_ERR_UNSUPPORTED;
  if (gs != -1 && L->K % gs != 0) return W4_ERR_UNSUPPORTED;
  if (L->has_g_idx && gs == -1) return W4_ERR_UNSUPPORTED;
  return W4_OK;
}

w4_status w4_sizes(const w4_layer* L, w4_sizes_t* out) {
  const w4_status st = w4_check_layer(L);
  if (st != W4_OK) return st;
  if (out == nullptr) return W4_ERR_INVALID_ARGUMENT;
  const Shape s = w4::shape_of(L);
  const size_t K = (size_t)s.K, N = (size_t)s.N, G = (size_t)s.G;
  out->awq_qweight = K * (N / 8) * 4;
  out->qzeros = s.has_z ? G * (N / 8) * 4 : 0;
  out->scales = G * N * 2;
  out->std_qweight = (K / 8) * N * 4;
  const size_t Np = (size_t)s.Np, Kp = (size_t)s.Kp, Gp = (size_t)s.Gp;
  out->tiled_qweight = Kp * Np / 2;
  out->tiled_scales = Gp * Np * 2;
  out->tiled_qzeros = s.has_z ? (Np / w4::kTileN) * Gp * 2 * 4 : 0;
  out->perm = s.has_perm ? K * 4 : 0;
  return W4_OK;
}

w4_status w4_workspace_size(const w4_layer* L, int64_t M, size_t* bytes) {
  const w4_status st = w4_check_layer(L);
  if (st != W4_OK) return st;
  if (bytes == nullptr || M < 0) return W4_ERR_INVALID_ARGUMENT;
  if (M > kMaxM) return W4_ERR_UNSUPPORTED;
  *bytes = M == 0 ? 0 : w4::gemm_workspace_bytes(w4::shape_of(L), M);
  return W4_OK;
}

const char* w4_kernel_name(const w4_layer* L, int64_t M) {
  if (w4_check_layer(L) != W4_OK || M < 0 || M > kMaxM) return "invalid";
  if (M == 0) return "none";
  return w4::plan_gemm(w4::padded_k(w4::shape_of(L)), M).name;
}

w4_status w4_launch_dims(const w4_layer* L, int64_t M, uint32_t grid[3], uint32_t* threads) {
  const w4_status st = w4_check_layer(L);
  if (st != W4_OK) return st;
  if (grid == nullptr || threads == nullptr || M < 1) return W4_ERR_INVALID_ARGUMENT;
  if (M > kMaxM) return W4_ERR_UNSUPPORTED;
  unsigned g[3], t = 0;
  w4::gemm_launch_dims(w4::shape_of(L), M, g, &t);
  for (int i = 0; i < 3; ++i) grid[i] = g[i];
  *threads = t;
  return W4_OK;
}

const char* w4_status_str(w4_status s) {
  switch (s) {
    case W4_OK: return "ok";
    case W4_ERR_INVALID_ARGUMENT: return "invalid argument";
    case W4_ERR_UNSUPPORTED: return "unsupported layer, shape or device";
    case W4_ERR_WORKSPACE: return "workspace too small";
    case W4_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

w4_status w4_repack_awq(const w4_layer* L, const int32_t* awq_qweight, const int32_t* awq_qzeros,
                        int32_t* std_qweight, int32_t* std_qzeros, void* stream) {
  w4_status st = w4_check_layer(L);
  if (st != W4_OK) return st;
  if (!L->has_zero_points || L->has_g_idx) return W4_ERR_UNSUPPORTED;
  if (!awq_qweight || !awq_qzeros || !std_qweight || !std_qzeros) return W4_ERR_INVALID_ARGUMENT;
  if (!aligned(awq_qweight, 4) || !aligned(awq_qzeros, 4) || !aligned(std_qweight, 16) || !aligned(std_qzeros, 4))
    return W4_ERR_INVALID_ARGUMENT;
  st = device_status();
  if (st != W4_OK) return st;
  const Shape s = w4::shape_of(L);
  if (w4::launch_awq_to_std(s, awq_qweight, awq_qzeros, std_qweight, std_qzeros, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return W4_ERR_HIP;
  return W4_OK;
}

w4_status w4_repack_gptq(const w4_layer* L, const int32_t* std_qweight, const int32_t* std_qzeros,
                         const void* scales, const int32_t* g_idx, int32_t* tiled_qweight, void* tiled_scales,
                         int32_t* tiled_qzeros, int32_t* perm, int32_t* status_dev, void* stream) {
  w4_status st = w4_check_layer(L);
  if (st != W4_OK) return st;
  const Shape s = w4::shape_of(L);
  if (!std_qweight || !scales || !tiled_qweight || !tiled_scales) return W4_ERR_INVALID_ARGUMENT;
  if (s.has_z != (std_qzeros != nullptr) || s.has_z != (tiled_qzeros != nullptr)) return W4_ERR_INVALID_ARGUMENT;
  if (s.has_perm != (g_idx != nullptr) || s.has_perm != (perm != nullptr)) return W4_ERR_INVALID_ARGUMENT;
  if (!aligned(std_qweight, 4) || !aligned(scales, 2) || !aligned(tiled_qweight, 16) || !aligned(tiled_scales, 2) ||
      (std_qzeros && !aligned(std_qzeros, 4)) || (tiled_qzeros && !aligned(tiled_qzeros, 4)) ||
      (g_idx && !aligned(g_idx, 4)) || (perm && !aligned(perm, 16)) || (status_dev && !aligned(status_dev, 4)))
    return W4_ERR_INVALID_ARGUMENT;
  st = device_status();
  if (st != W4_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (s.has_perm) {
    if (w4::launch_actorder_perm(s, g_idx, perm, status_dev, hs) != hipSuccess) return W4_ERR_HIP;
  } else if (status_dev != nullptr) {
    if (w4::launch_status_zero(status_dev, hs) != hipSuccess) return W4_ERR_HIP;
  }
  if (w4::launch_tile(s, std_qweight, std_qzeros, static_cast<const uint16_t*>(scales), perm, tiled_qweight,
                      static_cast<uint16_t*>(tiled_scales), tiled_qzeros, hs) != hipSuccess)
    return W4_ERR_HIP;
  return W4_OK;
}

w4_status w4a16_linear(const w4_layer* L, int64_t M, const void* x, const int32_t* tiled_qweight,
                       const void* tiled_scales, const int32_t* tiled_qzeros, const int32_t* perm, const void* bias,
                       void* y, void* workspace, size_t workspace_bytes, void* stream) {
  w4_status st = w4::linear_checks(L, M, x, tiled_qweight, tiled_scales, tiled_qzeros, perm, bias, y);
  if (st != W4_OK || M == 0) return st;
  const Shape s = w4::shape_of(L);
  const size_t need = w4::gemm_workspace_bytes(s, M);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return W4_ERR_WORKSPACE;
  if (workspace != nullptr && !aligned(workspace, 16)) return W4_ERR_INVALID_ARGUMENT;
  st = w4::device_status();
  if (st != W4_OK) return st;
  if (w4::launch_gemm(s, M, x, tiled_qweight, tiled_scales, tiled_qzeros, perm, bias, y, workspace,
                      static_cast<hipStream_t>(stream)) != hipSuccess)
    return W4_ERR_HIP;
  return W4_OK;
}

w4_status w4a16_moe_linear(const w4_layer* L, int32_t num_experts, int64_t total_rows, int64_t max_rows,
                           const void* x, const int32_t* expert_offsets, const int32_t* tiled_qweight,
                           const void* tiled_scales, const int32_t* tiled_qzeros, const void* bias, void* y,
                           void* stream) {
  w4_status st = w4_check_layer(L);
  if (st != W4_OK) return st;
  const Shape s = w4::shape_of(L);
  if (s.has_perm || s.K != s.Kp) return W4_ERR_UNSUPPORTED;  // act-order experts, K tails
  if (num_experts < 0 || total_rows < 0 || max_rows < 0) return W4_ERR_INVALID_ARGUMENT;
  if (num_experts > 65535 || total_rows > kMaxM) return W4_ERR_UNSUPPORTED;
  if (num_experts == 0 || total_rows == 0) return W4_OK;
  if (max_rows == 0 || max_rows > total_rows) max_rows = total_rows;
  if (!x || !expert_offsets || !tiled_qweight || !tiled_scales || !y) return W4_ERR_INVALID_ARGUMENT;
  if (s.has_z != (tiled_qzeros != nullptr)) return W4_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(tiled_qweight, 16) || !aligned(tiled_scales, 2) || !aligned(y, 2) ||
      !aligned(expert_offsets, 4) || (bias && !aligned(bias, 2)) || (tiled_qzeros && !aligned(tiled_qzeros, 4)))
    return W4_ERR_INVALID_ARGUMENT;
  st = device_status();
  if (st != W4_OK) return st;
  if (w4::launch_moe(s, num_experts, total_rows, max_rows, x, expert_offsets, tiled_qweight, tiled_scales,
                     tiled_qzeros, bias, y, static_cast<hipStream_t>(stream)) != hipSuccess)
    return W4_ERR_HIP;
  return W4_OK;
}

w4_status w4_dequant_dense(const w4_layer* L, const int32_t* tiled_qweight, const void* tiled_scales,
                           const int32_t* tiled_qzeros, const int32_t* perm, void* w, void* stream) {
  w4_status st = w4_check_layer(L);
  if (st != W4_OK) return st;
  const Shape s = w4::shape_of(L);
  if (!tiled_qweight || !tiled_scales || !w) return W4_ERR_INVALID_ARGUMENT;
  if (s.has_z != (tiled_qzeros != nullptr) || s.has_perm != (perm != nullptr)) return W4_ERR_INVALID_ARGUMENT;
  if (!aligned(tiled_qweight, 16) || !aligned(tiled_scales, 2) || !aligned(w, 2) ||
      (tiled_qzeros && !aligned(tiled_qzeros, 4)) || (perm && !aligned(perm, 4)))
    return W4_ERR_INVALID_ARGUMENT;
  st = device_status();
  if (st != W4_OK) return st;
  if (w4::launch_dequant_dense(s, tiled_qweight, tiled_scales, tiled_qzeros, perm, w,
                               static_cast<hipStream_t>(stream)) != hipSuccess)
    return W4_ERR_HIP;
  return W4_OK;
}

// ---- INT4 weights x FP8 activations ----

namespace {
w4_status w4a8_layer_ok(const w4_layer* L) {
  const w4_status st = w4_check_layer(L);
  if (st != W4_OK) return st;
  // one MFMA step covers 128 rows: one group of 128, or any number of
  // blocks of a per-channel layer
  if (L->group_size != 128 && L->group_size != -1) return W4_ERR_UNSUPPORTED;
  return W4_OK;
}
}  // namespace

w4_status w4a8_workspace_size(const w4_layer* L, int64_t M, size_t* bytes) {
  const w4_status st = w4a8_layer_ok(L);
  if (st != W4_OK) return st;
  if (bytes == nullptr || M < 0) return W4_ERR_INVALID_ARGUMENT;
  if (M > kMaxM) return W4_ERR_UNSUPPORTED;
  *bytes = M == 0 ? 0 : w4::f8_workspace_bytes(w4::padded_k(w4::shape_of(L)), M);
  return W4_OK;
}

w4_status w4a8_quantize(const w4_layer* L, int64_t M, const void* x, const float* x_scale, const int32_t* perm,
                        uint8_t* xq, float* rowsum, void* stream) {
  w4_status st = w4a8_layer_ok(L);
  if (st != W4_OK) return st;
  if (M < 0) return W4_ERR_INVALID_ARGUMENT;
  if (M > kMaxM) return W4_ERR_UNSUPPORTED;
  const Shape s = w4::shape_of(L);
  if (!x || !x_scale || !xq || !rowsum) return W4_ERR_INVALID_ARGUMENT;
  if (s.has_perm != (perm != nullptr)) return W4_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 2) || !aligned(x_scale, 4) || !aligned(xq, 8) || !aligned(rowsum, 4) || (perm && !aligned(perm, 4)))
    return W4_ERR_INVALID_ARGUMENT;
  if (M == 0) return W4_OK;
  st = device_status();
  if (st != W4_OK) return st;
  if (w4::launch_f8_quantize(s, M, x, x_scale, perm, xq, rowsum, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return W4_ERR_HIP;
  return W4_OK;
}

w4_status w4a8_linear(const w4_layer* L, int64_t M, const void* x, const float* x_scale,
                      const int32_t* tiled_qweight, const void* tiled_scales, const int32_t* tiled_qzeros,
                      const int32_t* perm, const void* bias, void* y, void* workspace, size_t workspace_bytes,
                      void* stream) {
  w4_status st = w4a8_layer_ok(L);
  if (st != W4_OK) return st;
  st = w4::linear_checks(L, M, x, tiled_qweight, tiled_scales, tiled_qzeros, perm, bias, y);
  if (st != W4_OK || M == 0) return st;
  if (x_scale == nullptr || !aligned(x_scale, 4)) return W4_ERR_INVALID_ARGUMENT;
  const Shape s0 = w4::shape_of(L);
  const Shape s = w4::padded_k(s0);
  const size_t need = w4::f8_workspace_bytes(s, M);
  if (workspace == nullptr || workspace_bytes < need) return W4_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return W4_ERR_INVALID_ARGUMENT;
  st = device_status();
  if (st != W4_OK) return st;
  uint8_t* xq = static_cast<uint8_t*>(workspace);
  float* rs = reinterpret_cast<float*>(xq + w4::f8_xq_bytes(s, M));
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (w4::launch_f8_quantize(s0, M, x, x_scale, perm, xq, rs, hs) != hipSuccess) return W4_ERR_HIP;
  if (w4::launch_f8_gemm(s, M, xq, rs, x_scale, tiled_qweight, tiled_scales, tiled_qzeros, bias, y, hs) !=
      hipSuccess)
    return W4_ERR_HIP;
  return W4_OK;
}

const char* w4a8_kernel_name(const w4_layer* L, int64_t M) {
  if (w4a8_layer_ok(L) != W4_OK || M < 0 || M > kMaxM) return "invalid";
  if (M == 0) return "none";
  return w4::f8_kernel_name(w4::padded_k(w4::shape_of(L)), M);
}

}  // extern "C"
