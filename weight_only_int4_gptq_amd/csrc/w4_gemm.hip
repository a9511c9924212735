// Plain (one layer) launches of the fused dequantize + GEMM: kernel choice
// by shape, workspace layout, act-order gather, K-tail padding.
#include "w4_kern.h"

namespace w4 {
namespace {

// Workspace of a call: first the activations the kernels read instead of x
// (gathered through perm with act-order, on every path; or padded to whole
// 128-row blocks when K % 128 != 0; the two never coincide), then the
// split-K partials.
inline size_t front_bytes(const Shape& s, const GemmPlan& p, int64_t M) {
  size_t b = 0;
  if (s.has_perm) b = (size_t)M * (size_t)s.K * sizeof(uint16_t);
  else if (s.K != s.Kp) b = (size_t)M * (size_t)s.Kp * sizeof(uint16_t);
  return (b + 255) / 256 * 256;
}

// Workspace layout: front bytes (gathered or padded activations), split-K
// partials [splits][M][N] fp32, row sums [Kp / L][M] fp32 (bf16 pre-pass),
// the fp16 copy of x and its row factors (bf16 on the large-M kernel), each
// part 256-byte aligned.
size_t partial_bytes(const Shape& s, const GemmPlan& p, int64_t M) {
  const size_t b = p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)s.N * sizeof(float) : 0;
  return (b + 255) / 256 * 256;
}

size_t rowsum_bytes(const Shape& sp, const GemmPlan& p, int64_t M) {
  if (!p.rsin) return 0;
  const size_t periods = (size_t)(sp.Kp / kTileK) * (size_t)(sp.gs == 32 ? 4 : (sp.gs == 64 ? 2 : 1));
  return (periods * (size_t)M * sizeof(float) + 255) / 256 * 256;
}

// bf16 on the large-M kernel: the fp16 copy of x [M][Kp], then the row
// factors, fp32 for whole 128-row tiles (the epilogue reads a tile's
// factors in 16-byte pieces; rows >= M are read, never used)
size_t h16_x_bytes(const Shape& sp, const GemmPlan& p, int64_t M) {
  return p.h16 ? ((size_t)M * (size_t)sp.Kp * sizeof(uint16_t) + 255) / 256 * 256 : 0;
}
size_t h16_bytes(const Shape& sp, const GemmPlan& p, int64_t M) {
  return p.h16 ? h16_x_bytes(sp, p, M) + (size_t)((M + 127) / 128 * 128) * sizeof(float) : 0;
}

// Act-order first gathers the columns of x into the workspace (front bytes
// of the workspace in use by the caller: `front`).
hipError_t launch_wide(const Shape& s, const GemmPlan& p, const Args& a0, void* ws, size_t front, hipStream_t st) {
  Args a = a0;
  const uint16_t* x = a.x;
  if (s.has_perm) {
    uint16_t* xp = static_cast<uint16_t*>(ws);
    const hipError_t e = launch_gather(a.x, a.perm, xp, a.M, a.K, st);
    if (e != hipSuccess) return e;
    x = xp;
  }
  a.splits = p.splits;
  a.part = p.splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + front) : nullptr;
  a.rsum = p.rsin ? reinterpret_cast<float*>(static_cast<char*>(ws) + front + partial_bytes(s, p, a.M)) : nullptr;
  return wide_dispatch<false>(p.wide, s, a, x, st);
}

template <int MT, int NB, int KW, bool XL, bool BF16, bool HZ, int D, int AR>
hipError_t pick_gm(const Args& a, hipStream_t st) {
  switch (group_mode(a.gs, a.K)) {
    case GM_32: return run_skinny<MT, NB, KW, GM_32, BF16, HZ, XL, D, AR>(a, st);
    case GM_64: return run_skinny<MT, NB, KW, GM_64, BF16, HZ, XL, D, AR>(a, st);
    case GM_128: return run_skinny<MT, NB, KW, GM_128, BF16, HZ, XL, D, AR>(a, st);
    default: return run_skinny<MT, NB, KW, GM_CH, BF16, HZ, XL, D, AR>(a, st);
  }
}

// (act-order activations arrive gathered: the skinny kernels never see perm)
// D: ring depth (the measured default for the configuration unless given)
template <int MT, int NB, int KW, bool XL, int AR = 0, int D = skinny_depth<MT, NB, KW, XL>()>
hipError_t pick_flags(const Shape& s, const Args& a, hipStream_t st) {
  if (s.bf16)
    return s.has_z ? pick_gm<MT, NB, KW, XL, true, true, D, AR>(a, st)
                   : pick_gm<MT, NB, KW, XL, true, false, D, AR>(a, st);
  return s.has_z ? pick_gm<MT, NB, KW, XL, false, true, D, AR>(a, st)
                 : pick_gm<MT, NB, KW, XL, false, false, D, AR>(a, st);
}

}  // namespace

namespace {
GemmPlan plan_tiles(const Shape& s, int64_t M, bool bf16_big);
}  // namespace

GemmPlan plan_gemm(const Shape& s, int64_t M, bool bf16_big) {
  GemmPlan p = plan_tiles(s, M, bf16_big);
  // bf16 wide kernels take the zero-point row sums from a pre-pass
  // (row_sums_bf16) instead of a ones-operand MFMA per row tile and step
  // where that measured faster: M >= 256, or M >= 64 on long (K >= 16384)
  // or wide (> 1024 strips) layers (5-13% there; the extra launch cost more
  // than it saved below that, e.g. 45.6 -> 46.9 us at 8192 x 10240, M = 128)
  const int64_t T = s.Np / kTileN;
  if (s.bf16 && p.kind == GemmKind::kWide && (M >= 256 || (M >= 64 && (s.K >= 16384 || T > 1024))))
    p.rsin = true;
  p.h16 = s.bf16 && p.kind == GemmKind::kBig;
  return p;
}

namespace {
GemmPlan plan_tiles(const Shape& s, int64_t M, bool bf16_big) {
  // (mt, nb, kw, xl): 16-row tiles per wave, strips per workgroup, waves per
  // workgroup (splitting K), activations staged in LDS; the ring depth
  // follows from them (skinny_depth).  Chosen from timing sweeps of the
  // decode shapes on MI355X.  K is never split across
  // workgroups: the agent-scope release fence that a cross-workgroup fix-up
  // needs writes back the XCD's whole L2 on gfx950 and cost far more than it
  // saved at these sizes (measured).
  GemmPlan p;
  const int64_t T = s.Np / kTileN;
  if (M <= 4 && T <= 256) {
    // few strips (N <= 4096): sixteen waves per strip, each copying the (at
    // most four) activation rows of every block into its LDS ring as it
    // goes; measured 3-11% faster than staging the rows once up front
    p = GemmPlan{GemmKind::kSkinny, 1, 1, 16, false, "w4_skinny_dma4_k16"};
    p.ar = 4;
  } else if (M <= 4 && skinny_lds_bytes(1, 1, 8, true, M, s.K) <= kMaxSkinnyLds) {
    // activations staged in LDS once per workgroup
    p = GemmPlan{GemmKind::kSkinny, 1, 1, 8, true, "w4_skinny_lds_k8"};
  } else if (M <= 16 && T > 512 && !(T <= 768 && T % 3 == 0)) {
    // many strips (N > 8192): every wave walks all of K for one strip with
    // the activation tile in LDS shared by the workgroup's waves (four for
    // up to 1024 strips, else two with a six-deep pipeline), which measured
    // faster than splitting K, and than the per-wave kernels below once
    // those would need a second round of workgroups (10240 x 4096 at
    // M = 16: 14.0 -> 10.7 us)
    const int idx = T <= 1024 ? kWide16x64w4 : kWide16x32w2;
    const WideChoice& w = kWide[idx];
    p = GemmPlan{GemmKind::kWide, w.mt, w.ns, w.wn, false, w.name};
    p.wide = idx;
  } else if (M <= 16 && ((T <= 256 && M >= 8) || (T > 256 && T <= 512 && T % 2 == 0) || T > 512)) {
    // each wave copies every block's activation tile into its own LDS ring
    // slot with direct-to-LDS loads (whole rows) and reads its operands from
    // there: loading them into registers touches 16 half-used cache lines per
    // load, which measured 12-19% slower at M = 16 on the narrow layers
    // (11008 x 4096: 13.6 -> 11.0 us; 4096 x 4096: 6.6 -> 5.8 us) and 15% at
    // 8192 x 8192.  Eight waves with a 3-deep ring (11008 x 4096: 11.3 ->
    // 10.9 us against 2-deep); the ring and the reduction take one CU's LDS,
    // so the strips per workgroup keep the grid to one round of at most 256
    // workgroups: one strip up to 256 strips, two up to 512, three up to 768
    // (12288: 10.9 -> 10.3 us against the shared-tile kernel above; 9216:
    // 13.7 -> 9.5 us against two strips)
    if (T <= 256)
      p = GemmPlan{GemmKind::kSkinny, 1, 1, 8, false, "w4_skinny_dma_k8"};
    else if (T <= 512)
      p = GemmPlan{GemmKind::kSkinny, 1, 2, 8, false, "w4_skinny_dma_n2_k8"};
    else
      p = GemmPlan{GemmKind::kSkinny, 1, 3, 8, false, "w4_skinny_dma_n3_k8"};
    p.ar = 16;
  } else if (M <= 16) {
    // activations from registers; two strips per workgroup share them
    // (halving the activation traffic) unless N is small: then one strip
    // per workgroup, sixteen waves for short K, eight for long K
    if (T <= 256 && s.K <= 4096) {
      p = GemmPlan{GemmKind::kSkinny, 1, 1, 16, false, "w4_skinny_k16"};
    } else if (T % 2 == 0 && (T >= 512 || s.K <= 4096)) {
      p = s.K >= 8192 ? GemmPlan{GemmKind::kSkinny, 1, 2, 8, false, "w4_skinny_n2_k8"}
                      : GemmPlan{GemmKind::kSkinny, 1, 2, 16, false, "w4_skinny_n2_k16"};
    } else {
      p = GemmPlan{GemmKind::kSkinny, 1, 1, 8, false, "w4_skinny_k8"};
    }
  } else if ((!s.bf16 || bf16_big) && ((M + big_tile_rows() - 1) / big_tile_rows()) *
                                ((s.Np + big_tile_cols() - 1) / big_tile_cols()) >= 256) {
    // large M (fp16, or bf16 on its exact fp16 copy of x), at least one
    // 128 x 256 tile of 32x32x16 MFMAs per CU (with fewer tiles, splitting K
    // measured slower than the wide kernel's smaller tiles: act-order
    // M = 512 at 8192 x 8192, 94 vs 86 us; bf16 M = 128 at 8192 x 8192,
    // 47 vs 32 us)
    p = GemmPlan{GemmKind::kBig, 0, 0, 0, false, "w4_big_128x256"};
  } else {
    // wide kernel: the largest tile that is not taller than M (32 rows at
    // least) and still gives >= 256 workgroups (one per CU), else the
    // smallest.  Mid-size M
    // (<= 256) on layers with N <= 16384 instead splits K over 4 or 8
    // workgroups per tile (fp32 partials in the workspace, summed by
    // split_reduce): enough workgroups and weight streams in flight; measured
    // 1.35-2x faster at M <= 64 and 1.1-1.45x at M = 128/256 than any
    // unsplit tile there.  Above 128 rows two splits suffice for K < 16384
    // (bf16 8192 x 8192, M = 256: 59.8 -> 52.4 us against four).
    const int64_t nblk = s.K / kTileK;
    if (M <= 256 && T <= 1024 && nblk >= 4) {
      // 32x128 (M <= 32), 64x128, or 64x256 for long K at M > 64
      const int idx = M <= 32 ? 3 : (M > 64 && s.K >= 16384 ? 1 : 2);
      int splits = M > 64 ? (s.K >= 16384 ? (M <= 128 ? 8 : 4) : (M <= 128 ? 4 : 2)) : (s.K >= 16384 ? 8 : 4);
      while (splits > 1 && splits * 2 > nblk) splits /= 2;  // >= 2 blocks per split
      static const char* split_names[] = {"", "w4_wide_64x256_splitk", "w4_wide_64x128_splitk",
                                          "w4_wide_32x128_splitk"};
      const WideChoice& w = kWide[idx];
      p = GemmPlan{GemmKind::kWide, w.mt, w.ns, w.wn, false, splits > 1 ? split_names[idx] : w.name};
      p.wide = idx;
      p.splits = splits;
      return p;
    }
    int pick = kNumWide - 1;
    for (int i = 0; i < kNumWide; ++i) {
      if (i == 1 && T <= 1024) continue;  // 64x256 only on wide layers (64x128 measured faster below)
      const WideChoice& w = kWide[i];
      const int64_t bm = 16 * w.mt, bn = 16 * w.ns * w.wn;
      const int64_t wgs = ((s.N + bn - 1) / bn) * ((M + bm - 1) / bm);
      if (M >= w.min_m && (bm <= M || bm == 32) && wgs >= 256) {
        pick = i;
        break;
      }
    }
    const WideChoice& w = kWide[pick];
    p = GemmPlan{GemmKind::kWide, w.mt, w.ns, w.wn, false, w.name};
    p.wide = pick;
  }
  return p;
}

}  // namespace

// Grid and workgroup size of the GEMM kernel launch_gemm runs for M rows
// (the dimensions the run_* launchers compute; s is the unpadded shape).
void gemm_launch_dims(const Shape& s0, int64_t M, unsigned grid[3], unsigned* threads) {
  const Shape s = padded_k(s0);
  const GemmPlan p = plan_gemm(s, M);
  const int64_t T = s.Np / kTileN;
  grid[0] = grid[1] = grid[2] = 1;
  if (p.kind == GemmKind::kSkinny) {
    grid[0] = (unsigned)(T / p.nb);
    grid[1] = (unsigned)((M + 16 * p.mt - 1) / (16 * p.mt));
    *threads = 64u * (unsigned)p.kw;
  } else if (p.kind == GemmKind::kBig) {
    grid[0] = (unsigned)(((M + big_tile_rows() - 1) / big_tile_rows()) *
                         ((s.Np + big_tile_cols() - 1) / big_tile_cols()));
    *threads = (unsigned)big_threads();
  } else {
    const WideChoice& w = kWide[p.wide];
    grid[0] = (unsigned)((T + w.ns * w.wn - 1) / (w.ns * w.wn));
    grid[1] = (unsigned)((M + 16 * w.mt - 1) / (16 * w.mt));
    grid[2] = (unsigned)p.splits;
    *threads = 64u * (unsigned)w.wn;
  }
}

namespace {
size_t plan_bytes(const Shape& s, const Shape& sp, const GemmPlan& p, int64_t M) {
  return front_bytes(s, p, M) + partial_bytes(s, p, M) + rowsum_bytes(sp, p, M) + h16_bytes(sp, p, M);
}

// The plan of a call with at most ws_cap bytes of workspace (s unpadded).
GemmPlan plan_capped(const Shape& s, int64_t M, size_t ws_cap) {
  const Shape sp = padded_k(s);
  const GemmPlan p = plan_gemm(sp, M);
  if (p.h16 && plan_bytes(s, sp, p, M) > ws_cap) return plan_gemm(sp, M, false);
  return p;
}
}  // namespace

size_t gemm_workspace_bytes(const Shape& s, int64_t M, size_t ws_cap) {
  return plan_bytes(s, padded_k(s), plan_capped(s, M, ws_cap), M);
}

hipError_t launch_gemm(const Shape& s0, int64_t M, const void* x, const int32_t* tiled_w, const void* tiled_s,
                       const int32_t* tiled_z, const int32_t* perm, const void* bias, void* y, void* ws,
                       hipStream_t st, size_t ws_cap) {
  // the kernels run the padded shape (K a whole number of blocks)
  const Shape s = padded_k(s0);
  Args a;
  a.x = static_cast<const uint16_t*>(x);
  a.qw = reinterpret_cast<const u4*>(tiled_w);
  a.sc = static_cast<const uint16_t*>(tiled_s);
  a.zs = reinterpret_cast<const uint32_t*>(tiled_z);
  a.perm = perm;
  a.bias = static_cast<const uint16_t*>(bias);
  a.y = static_cast<uint16_t*>(y);
  a.part = nullptr;
  a.splits = 1;
  a.offs = nullptr;
  a.groups = 0;
  a.max_rows = M;
  a.rsum = nullptr;
  a.M = M;
  a.K = s.K;
  a.N = s.N;
  a.G = s.G;
  a.gs = s.gs;
  const GemmPlan p = plan_capped(s0, M, ws_cap);
  const size_t front = front_bytes(s0, p, M);
  if (s0.K != s0.Kp) {
    // zero-padded copy of x in the workspace (act-order is excluded here)
    uint16_t* xp = static_cast<uint16_t*>(ws);
    const int64_t total = M * (s.K / 8);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    pad_columns<<<(unsigned)blocks, 256, 0, st>>>(reinterpret_cast<const uint4*>(a.x), reinterpret_cast<uint4*>(xp),
                                                  M, s0.K / 8, s.K / 8);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.x = xp;
  }
  if (p.kind == GemmKind::kWide) return launch_wide(s, p, a, ws, front, st);
  if (p.kind == GemmKind::kBig) {
    const uint16_t* xb = a.x;
    if (s.has_perm) {
      uint16_t* xp = static_cast<uint16_t*>(ws);
      const hipError_t e = launch_gather(a.x, a.perm, xp, a.M, a.K, st);
      if (e != hipSuccess) return e;
      xb = xp;
    }
    uint16_t* xh = nullptr;
    float* rowf = nullptr;
    if (p.h16) {
      char* h = static_cast<char*>(ws) + front + partial_bytes(s, p, M) + rowsum_bytes(s, p, M);
      xh = reinterpret_cast<uint16_t*>(h);
      rowf = reinterpret_cast<float*>(h + h16_x_bytes(s, p, M));
    }
    return launch_big(s, M, xb, tiled_w, tiled_s, tiled_z, bias, y, xh, rowf, st);
  }
  Shape sk = s;
  if (s.has_perm) {
    // gather x[:, perm] into the workspace, then run without act-order
    uint16_t* xp = static_cast<uint16_t*>(ws);
    const hipError_t e = launch_gather(a.x, a.perm, xp, a.M, a.K, st);
    if (e != hipSuccess) return e;
    a.x = xp;
    a.perm = nullptr;
    sk.has_perm = false;
  }
  if (p.ar == 4) return pick_flags<1, 1, 16, false, 4, 3>(sk, a, st);
  if (p.ar == 16) {
    if (p.nb == 3) return pick_flags<1, 3, 8, false, 16, 3>(sk, a, st);
    return p.nb == 2 ? pick_flags<1, 2, 8, false, 16, 3>(sk, a, st) : pick_flags<1, 1, 8, false, 16, 3>(sk, a, st);
  }
  if (p.xl) return pick_flags<1, 1, 8, true>(sk, a, st);
  if (p.nb == 2) return p.kw == 16 ? pick_flags<1, 2, 16, false>(sk, a, st) : pick_flags<1, 2, 8, false>(sk, a, st);
  return p.kw == 16 ? pick_flags<1, 1, 16, false>(sk, a, st) : pick_flags<1, 1, 8, false>(sk, a, st);
}

}  // namespace w4
