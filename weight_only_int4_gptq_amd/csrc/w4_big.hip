// Large-M launches on the 32x32x16 MFMA kernel (w4_big.h): fp16 and bf16
// layers (bf16 through an exact fp16 copy of x), every group mode, with or
// without zero points.
#include "w4_big.h"

namespace w4 {
namespace {

template <int GM>
hipError_t big_grouped_z(const Args& a, bool has_z, hipStream_t st) {
  return has_z ? run_big_grouped<kBigWM, kBigWN, kBigMT, kBigNT, kBigS, GM, true>(a, st)
               : run_big_grouped<kBigWM, kBigWN, kBigMT, kBigNT, kBigS, GM, false>(a, st);
}

}  // namespace

int64_t big_tile_rows() { return BigCfg<kBigWM, kBigWN, kBigMT, kBigNT, kBigS>::BM; }
int64_t big_tile_cols() { return BigCfg<kBigWM, kBigWN, kBigMT, kBigNT, kBigS>::BN; }
int big_threads() { return 64 * kBigWM * kBigWN; }

hipError_t launch_big(const Shape& s, int64_t M, const uint16_t* x, const int32_t* tiled_w, const void* tiled_s,
                      const int32_t* tiled_z, const void* bias, void* y, uint16_t* xh, float* rowf,
                      hipStream_t st) {
  if (s.bf16) return launch_big_h16(s, M, x, tiled_w, tiled_s, tiled_z, bias, y, xh, rowf, st);
  return big_gm<false>(big_args(s, M, tiled_w, tiled_s, tiled_z, bias, y), x, nullptr, nullptr, s.has_z, st);
}

hipError_t launch_big_moe(const Shape& s, int experts, int64_t total_rows, int64_t max_rows, const void* x,
                          const int32_t* offsets, const int32_t* tiled_w, const void* tiled_s,
                          const int32_t* tiled_z, const void* bias, void* y, hipStream_t st) {
  if (s.bf16) return hipErrorInvalidValue;
  Args a{};
  a.x = static_cast<const uint16_t*>(x);
  a.qw = reinterpret_cast<const u4*>(tiled_w);
  a.sc = static_cast<const uint16_t*>(tiled_s);
  a.zs = reinterpret_cast<const uint32_t*>(tiled_z);
  a.bias = static_cast<const uint16_t*>(bias);
  a.y = static_cast<uint16_t*>(y);
  a.offs = offsets;
  a.groups = experts;
  a.max_rows = max_rows;
  a.M = total_rows;
  a.K = s.K;
  a.N = s.N;
  a.G = s.G;
  a.gs = s.gs;
  switch (group_mode(a.gs, a.K)) {
    case GM_32: return big_grouped_z<GM_32>(a, s.has_z, st);
    case GM_64: return big_grouped_z<GM_64>(a, s.has_z, st);
    case GM_128: return big_grouped_z<GM_128>(a, s.has_z, st);
    default: return big_grouped_z<GM_CH>(a, s.has_z, st);
  }
}

}  // namespace w4
