// Large-M launches on the 32x32x16 MFMA kernel (w4_big.h): fp16 activations,
// every group mode, with or without zero points.
#include "w4_big.h"

namespace w4 {
namespace {

// The shipped configuration: four waves side by side, each 128 rows x 64
// columns (workgroup tile 128 x 256), double-buffered (64 KiB of LDS, two
// workgroups per CU); tile order in bands of four row tiles.  Chosen from
// sweeps of the prefill shapes on MI355X against 2 x 2 and 2 x 4 wave
// arrangements, 64 x 64 and 64 x 128 wave tiles and three- and four-deep
// pipelines.
constexpr int kBigWM = 1, kBigWN = 4, kBigMT = 4, kBigNT = 2, kBigS = 2;
constexpr int64_t kBigGroupM = 4;

template <int GM>
hipError_t big_z(const Args& a, const uint16_t* x, bool has_z, hipStream_t st) {
  return has_z ? run_big<kBigWM, kBigWN, kBigMT, kBigNT, kBigS, GM, true>(a, x, kBigGroupM, st)
               : run_big<kBigWM, kBigWN, kBigMT, kBigNT, kBigS, GM, false>(a, x, kBigGroupM, st);
}

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
                      const int32_t* tiled_z, const void* bias, void* y, hipStream_t st) {
  if (s.bf16) return hipErrorInvalidValue;  // the bf16 operand needs the zero-term correction of the wide kernel
  Args a{};
  a.qw = reinterpret_cast<const u4*>(tiled_w);
  a.sc = static_cast<const uint16_t*>(tiled_s);
  a.zs = reinterpret_cast<const uint32_t*>(tiled_z);
  a.bias = static_cast<const uint16_t*>(bias);
  a.y = static_cast<uint16_t*>(y);
  a.part = nullptr;
  a.splits = 1;
  a.M = M;
  a.K = s.K;
  a.N = s.N;
  a.G = s.G;
  a.gs = s.gs;
  switch (group_mode(a.gs, a.K)) {
    case GM_32: return big_z<GM_32>(a, x, s.has_z, st);
    case GM_64: return big_z<GM_64>(a, x, s.has_z, st);
    case GM_128: return big_z<GM_128>(a, x, s.has_z, st);
    default: return big_z<GM_CH>(a, x, s.has_z, st);
  }
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
