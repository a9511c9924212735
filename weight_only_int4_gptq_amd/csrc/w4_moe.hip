// Grouped (mixture-of-experts) launches of the wide kernel: one launch over
// all experts, the expert in the third grid dimension.
#include "w4_kern.h"

namespace w4 {

constexpr int64_t kMoeBigRows = 128;

GemmPlan plan_moe(const Shape& s, int64_t max_rows, int experts) {
  // grouped launch of the wide kernel (no split-K): 16-row tiles for up to
  // 16 rows per expert (two waves of one strip each once there are >= 1024
  // strips over all experts, else one wave of one strip), else the largest
  // tile not taller than the rows that still gives >= 256 workgroups over
  // all experts
  const int64_t T = s.Np / kTileN;
  if (!s.bf16 && max_rows >= kMoeBigRows) {
    // fp16 experts of at least kMoeBigRows rows: 128 x 256 tiles of 32x32x16
    // MFMAs, as for large-M fp16 layers
    return GemmPlan{GemmKind::kBig, 0, 0, 0, false, "w4_big_128x256_grouped"};
  }
  int idx = kNumWide - 1;
  if (max_rows <= 16) {
    idx = T * experts >= 1024 ? kWide16x32w2 : kWide16x16;
  } else {
    for (int i = 0; i < kNumWide; ++i) {
      const WideChoice& w = kWide[i];
      const int64_t bm = 16 * w.mt, bn = 16 * w.ns * w.wn;
      const int64_t wgs = ((s.N + bn - 1) / bn) * ((max_rows + bm - 1) / bm) * experts;
      if (max_rows >= w.min_m && (bm <= max_rows || bm == 32) && wgs >= 256) {
        idx = i;
        break;
      }
    }
  }
  const WideChoice& w = kWide[idx];
  GemmPlan p{GemmKind::kWide, w.mt, w.ns, w.wn, false, w.name};
  p.wide = idx;
  return p;
}

hipError_t launch_moe(const Shape& s, int experts, int64_t total_rows, int64_t max_rows, const void* x,
                      const int32_t* offsets, const int32_t* tiled_w, const void* tiled_s, const int32_t* tiled_z,
                      const void* bias, void* y, hipStream_t st) {
  Args a{};
  a.x = static_cast<const uint16_t*>(x);
  a.qw = reinterpret_cast<const u4*>(tiled_w);
  a.sc = static_cast<const uint16_t*>(tiled_s);
  a.zs = reinterpret_cast<const uint32_t*>(tiled_z);
  a.perm = nullptr;
  a.bias = static_cast<const uint16_t*>(bias);
  a.y = static_cast<uint16_t*>(y);
  a.part = nullptr;
  a.splits = 1;
  a.offs = offsets;
  a.groups = experts;
  a.max_rows = max_rows;
  a.M = total_rows;
  a.K = s.K;
  a.N = s.N;
  a.G = s.G;
  a.gs = s.gs;
  const GemmPlan p = plan_moe(s, max_rows, experts);
  if (p.kind == GemmKind::kBig)
    return launch_big_moe(s, experts, total_rows, max_rows, x, offsets, tiled_w, tiled_s, tiled_z, bias, y, st);
  return wide_dispatch<true>(p.wide, s, a, a.x, st);
}

}  // namespace w4
