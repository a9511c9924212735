// w4a16_linear_noalloc: w4a16_linear for callers that cannot allocate device
// memory (code under HIP graph capture, serving loops, harnesses that forbid
// allocation).  The workspace of w4a16_linear (act-order gather, K-tail
// padding, split-K partials, bf16 row sums or fp16 copy of x) lives in a
// file-scope device array instead of a caller buffer.  The kernels are those
// of w4a16_linear, except that a bf16 call at large M whose fp16 copy of x
// would not fit the array runs the wide kernel instead of the large-M one.
#include <mutex>

#include "w4_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // per device, held until the process ends

// The workspace of every w4a16_linear_noalloc call on a device.  Its name is
// a host-side stand-in: host code uses only the device address returned by
// hipGetSymbolAddress for the current device.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch`, per device

// Device address of the array on the current device, resolved once per
// device (with that device current) and kept.
w4_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return W4_ERR_HIP;
  if (dev >= kMaxDevices) return W4_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return W4_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return W4_OK;
}

}  // namespace

extern "C" {

size_t w4_noalloc_scratch_bytes(void) { return kScratchBytes; }

w4_status w4a16_linear_noalloc(const w4_layer* L, int64_t M, const void* x, const int32_t* tiled_qweight,
                               const void* tiled_scales, const int32_t* tiled_qzeros, const int32_t* perm,
                               const void* bias, void* y, void* stream) {
  w4_status st = w4::linear_checks(L, M, x, tiled_qweight, tiled_scales, tiled_qzeros, perm, bias, y);
  if (st != W4_OK || M == 0) return st;
  const w4::Shape s = w4::shape_of(L);
  if (w4::gemm_workspace_bytes(s, M, kScratchBytes) > kScratchBytes) return W4_ERR_WORKSPACE;
  st = w4::device_status();
  if (st != W4_OK) return st;
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != W4_OK) return st;
  if (w4::launch_gemm(s, M, x, tiled_qweight, tiled_scales, tiled_qzeros, perm, bias, y, ws,
                      static_cast<hipStream_t>(stream), kScratchBytes) != hipSuccess)
    return W4_ERR_HIP;
  return W4_OK;
}

}  // extern "C"
