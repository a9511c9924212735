// Large-M launches of bf16 layers (w4_big.h): an exact fp16 copy of x and
// the fp16 kernel with bf16 scales, bias and output.  A file of its own so
// that its kernels compile in parallel with the fp16 ones.
#include "w4_big.h"

namespace w4 {

hipError_t launch_big_h16(const Shape& s, int64_t M, const uint16_t* x, const int32_t* tiled_w, const void* tiled_s,
                          const int32_t* tiled_z, const void* bias, void* y, uint16_t* xh, float* rowf,
                          hipStream_t st) {
  if (!s.bf16) return hipErrorInvalidValue;
  return big_gm<true>(big_args(s, M, tiled_w, tiled_s, tiled_z, bias, y), x, xh, rowf, s.has_z, st);
}

}  // namespace w4
