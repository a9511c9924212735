// Large-M fused dequantize + GEMM on v_mfma_f32_32x32x16_f16 (gfx950).
//
// y[m, n] = sum_k x[m, k] * (q[k, n] - z[g(k), n]) * s[g(k), n] + bias[n]
// (dequantization of the vLLM AWQ practice page, section 5.3, fused into the
// matrix multiply as the learning-book page, section 5.3, describes; that
// page's section 1 names large batches compute-bound).
//
// Why 32x32x16.  A 32x32x16 MFMA does twice the work of a 16x16x32 one per
// operand register, so per flop it needs half the activation bytes from LDS
// and half the weight dequantization.  With 16x16x32 tiles and the
// activations read from LDS, a wave reads 0.5 KiB of LDS per 16-cycle MFMA
// even with two strips per wave, which alone fills the CU's LDS read
// bandwidth at the MFMA peak; a 128 x 64 wave tile of 32x32x16 MFMAs reads
// 4 KiB per eight 32-cycle MFMAs, a quarter of it.
//
// Operand layout of v_mfma_f32_32x32x16_f16: lane l supplies row (A) or
// column (B) l % 32 and the eight K values 8 (l / 32) .. 8 (l / 32) + 7 of
// the 16-deep step; output element r of lane l is row
// 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
//
// The weights stay in the library's tile layout (16-column strips, words
// [t][b][l'][j] holding column 16 t + l' % 16 at rows
// 128 b + 32 j + 8 (l' / 16) + e).  Lane l of a 32-column tile (strips 2 T
// and 2 T + 1) needs column c = l % 32 at rows 16 s + 8 h + e (h = l / 32)
// for the eight 16-deep steps s of a block: for even s that is word j = s / 2
// of lane l' = 16 h + c % 16 of strip 2 T + c / 16, for odd s word j = s / 2
// of lane l' + 32.  So each lane loads two 16-byte chunks per tile and block,
// and a step's B operand is one word, dequantized to eight exact (q - z)
// halves exactly as in the 16x16x32 kernels.
//
// Numerics: exact integer operands, fp32 accumulation, one fp32 scale per
// period applied with the ratio rescale of the wide kernel (the accumulator
// holding sum_{h<g} P_h s_h / s_{g-1} is multiplied by s_{g-1} / s_g at the
// start of period g and by the last scale at the end; the tile layout never
// stores a zero scale), y rounded once.
//
// Workgroup: WM x WN waves, each owning MT 32-row tiles and NT 32-column
// tiles (workgroup tile 32 MT WM x 32 NT WN).  K is walked in 128-row blocks
// through an S-deep pipeline: the activation tile of block b sits in LDS slot
// b % S (direct global->LDS loads, 16-byte chunk j of row r stored at chunk
// position j ^ (r % 16), so the rows one A read touches fall on distinct
// banks), the packed words, scales and zeros of block b in register slot
// b % S.  Iteration b waits until its own block has landed (vmcnt counted as
// in the wide kernel), passes one barrier, issues block b + S - 1 and
// computes block b.
//
// bf16 layers run the same fp16 kernel: a pre-pass (bf16_rows_to_f16)
// converts x to fp16.  A bf16 value has 8 significant bits and an fp16
// normal 11, so every bf16 value in fp16's normal range converts without
// rounding.  Each row is first multiplied by the power of two 2^-e (exact)
// that brings its largest finite magnitude into [2^14, 2^15), and the
// epilogue multiplies that row's result by 2^e.  So every value of the row
// down to 2^-29 of its largest is exact; smaller ones are rounded to fp16's
// subnormal grid, an error of at most 2^-39 of the row's largest magnitude
// per element.  Scales, bias and output stay bf16.
//
// Workgroup -> tile: the dispatcher hands consecutive workgroups to the
// eight XCDs in turn; the grid is remapped so that each XCD walks a
// contiguous range of tiles, in bands of group_m row tiles, so tiles that
// share activation rows or weight columns run on the same L2.
#pragma once

#include "w4_kern.h"

namespace w4 {
namespace {

typedef float f16v __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f16v mfma32(u4 a, u4 b, f16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(bit_as<h8>(a), bit_as<h8>(b), c, 0, 0, 0);
}

template <int WM, int WN, int MT, int NT, int S>
struct BigCfg {
  static constexpr int NW = WM * WN;
  static constexpr int BM = 32 * MT * WM;                    // rows per workgroup tile
  static constexpr int BN = 32 * NT * WN;                    // columns per workgroup tile
  static constexpr int NA = BM * kTileK * 2 / (1024 * NW);   // 1 KiB direct-to-LDS loads per wave per block
  static constexpr int kAfter = (S - 2) * (2 * NT + NA);     // loads of the S - 2 later blocks
  static_assert(NA >= 1 && NA * 1024 * NW == BM * kTileK * 2, "the activation tile splits evenly over the waves");
  static_assert(S >= 2 && S <= 4 && kAfter < 64, "pipeline depth");
};

// Workgroup id -> (row tile, column tile), see the header comment.
__device__ __forceinline__ void big_tile_of(int64_t L, int64_t tiles_m, int64_t tiles_n, int64_t group_m,
                                            int64_t& tm, int64_t& tn) {
  const int64_t ntiles = tiles_m * tiles_n;
  if (ntiles % 8 == 0) L = (L % 8) * (ntiles / 8) + L / 8;
  const int64_t per_band = group_m * tiles_n;
  const int64_t band = L / per_band, first = band * group_m;
  const int64_t rows = tiles_m - first < group_m ? tiles_m - first : group_m;
  const int64_t in = L - band * per_band;
  tm = first + in % rows;
  tn = in / rows;
}

// GROUPED: a mixture-of-experts launch, grid (column tiles, row tiles,
// experts); expert e owns rows [offs[e], offs[e + 1]) of x and y (clamped
// into the M rows given) and the e-th copy of the tiled weights, scales,
// zeros and bias, each following the previous expert's.
//
// OB16: a bf16 layer (bf16 scales, bias and output) on fp16 activations from
// bf16_rows_to_f16, with rowf[m] = 2^e the factor of row m.  Plain launches.
// With one scale period per block it is held to two waves per SIMD, as the
// fp16 kernel runs: left free, the compiler takes two registers more than
// that allows (with zero points) and one wave per SIMD runs.
template <int WM, int WN, int MT, int NT, int S, int GM, bool HAS_Z, bool GROUPED = false, bool OB16 = false>
__global__ __launch_bounds__(64 * WM * WN, OB16 && Groups<GM>::kPeriods == 1 ? 2 : 1) void gemm_big(const uint16_t* __restrict__ x_in,
                                                             const u4* __restrict__ qw_in,
                                                             const uint16_t* __restrict__ sc_in,
                                                             const uint32_t* __restrict__ zs_in,
                                                             const uint16_t* __restrict__ bias_in,
                                                             uint16_t* __restrict__ y_in, int64_t M_in, int64_t K,
                                                             int64_t N, int G,
                                                             int64_t tiles_m, int64_t tiles_n, int64_t group_m,
                                                             const int32_t* __restrict__ offs,
                                                             const float* __restrict__ rowf) {
  using C = BigCfg<WM, WN, MT, NT, S>;
  static_assert(!(OB16 && GROUPED), "bf16 layers: plain launches");
  constexpr int NP = Groups<GM>::kPeriods;  // scale periods per 128-row block
  constexpr int SPP = 8 / NP;               // 16-deep steps per period
  constexpr int NA = C::NA;
  constexpr int kSlot = C::BM * kTileK, kNone = 8;
  // one LDS array per pipeline slot (see the wide kernel)
  __shared__ __attribute__((aligned(1024))) uint16_t lds0[kSlot];
  __shared__ __attribute__((aligned(1024))) uint16_t lds1[kSlot];
  __shared__ __attribute__((aligned(1024))) uint16_t lds2[S > 2 ? kSlot : kNone];
  __shared__ __attribute__((aligned(1024))) uint16_t lds3[S > 3 ? kSlot : kNone];
  auto slot_lds = [&](int u) __attribute__((always_inline)) -> uint16_t* {
    switch (u) {
      case 0: return lds0;
      case 1: return lds1;
      case 2: return lds2;
      default: return lds3;
    }
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int c = lane & 31, h = lane >> 5;
  const int64_t T = (N + kTileN - 1) / kTileN;  // strips; the last may be half padding
  const int64_t nblk = K / kTileK;
  constexpr int64_t kb0 = 0;  // the whole of K (the issue and pipeline code count blocks from kb0)
  const int64_t nb = nblk;
  const uint32_t zshift = 4u * (uint32_t)(c & 7);
  const NibbleMasks nm = NibbleMasks::make();

  // one 32 MT WM x 32 NT WN output tile at (m0, n0) of an M-row problem
  auto tile = [&](const int64_t m0, const int64_t n0, const uint16_t* __restrict__ x, const u4* __restrict__ qw,
                  const uint16_t* __restrict__ sc, const uint32_t* __restrict__ zs,
                  const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, const int64_t M)
                  __attribute__((always_inline)) {

  // Operand addresses: a uniform base per 32-column tile (and per row tile
  // for the activations) plus a 32-bit per-lane byte offset, so the loads
  // take the scalar-base + vector-offset form and the lanes hold one
  // register per address instead of two.  Weights, scales and zeros of the
  // lane's column: a strip past the end reads the tile's first strip, a
  // tile past the end strip 0 (neither is stored).
  const char* wb[NT];
  const char* sb[NT];
  const char* zb[NT];
  uint32_t wo[NT], so[NT], zo[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int64_t t0 = (n0 + (int64_t)(wn * NT + nt) * 32) / kTileN;  // uniform
    const int64_t tb = t0 < T ? t0 : 0;
    const uint32_t ls = t0 + (c >> 4) < T ? (uint32_t)(c >> 4) : 0u;  // lane's strip within the tile
    wb[nt] = reinterpret_cast<const char*>(qw + tb * nblk * 64);
    sb[nt] = reinterpret_cast<const char*>(sc + tb * G * kTileN);
    zb[nt] = reinterpret_cast<const char*>(HAS_Z ? zs + tb * G * 2 : zs);
    wo[nt] = (uint32_t)((ls * nblk * 64 + (c & 15) + 16 * h) * sizeof(u4));
    so[nt] = (uint32_t)((ls * G * kTileN + (c & 15)) * sizeof(uint16_t));
    zo[nt] = (uint32_t)((ls * G * 2 + ((c & 15) >> 3)) * sizeof(uint32_t));
  }
  // staging: load i of this wave fills rows 4 (NA wave + i) .. + 3 of the
  // tile; lane l lands at chunk position l % 16 of row base + l / 16 and so
  // loads logical chunk (l % 16) ^ (row % 16)
  const char* ab = reinterpret_cast<const char*>(x + m0 * K);
  uint32_t ao[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int row = 4 * (NA * wave + i) + (lane >> 4);
    const int64_t r = m0 + row < M ? row : M - 1 - m0;
    ao[i] = (uint32_t)((r * K + 8 * ((lane & 15) ^ (row & 15))) * sizeof(uint16_t));
  }

  struct Slot {
    u4 w[NT][2];
    uint16_t s[NT][NP];
    uint32_t z[NT][NP];
  };
  Slot rg[S];

  auto issue = [&](int64_t b, Slot& r, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint32_t g = (uint32_t)Groups<GM>::group((int)b, p);
        r.s[nt][p] = *reinterpret_cast<const uint16_t*>(sb[nt] + (so[nt] + g * (uint32_t)(kTileN * sizeof(uint16_t))));
        r.z[nt][p] = HAS_Z ? *reinterpret_cast<const uint32_t*>(zb[nt] + (zo[nt] + g * 8u)) : 0u;
      }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint32_t bo = wo[nt] + (uint32_t)b * 1024u;
      r.w[nt][0] = *reinterpret_cast<const u4*>(wb[nt] + bo);
      r.w[nt][1] = *reinterpret_cast<const u4*>(wb[nt] + (bo + 512u));
    }
#pragma unroll
    for (int i = 0; i < NA; ++i)
      load_lds16(reinterpret_cast<const uint16_t*>(ab + (ao[i] + (uint32_t)b * (uint32_t)(kTileK * sizeof(uint16_t)))),
                 slot_lds(slot) + 4 * (NA * wave + i) * kTileK);
  };

  f16v acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][nt][r] = 0.f;
  float s_prev[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) s_prev[nt] = 1.f;

  // Each row tile's rescale is applied just before its first MFMA of the
  // period, and the scheduler is asked to issue the 16 multiplies of one
  // tile after the MFMA of the tile before it: the matrix core works through
  // that MFMA while the vector ALU rescales the next tile, instead of all
  // 16 MT NT multiplies running ahead of the period's first MFMA.
  constexpr bool RESCALE = GM != GM_CH;
  auto compute = [&](const Slot& r, int slot) __attribute__((always_inline)) {
    // row of this lane in row tile i: 32 (MT wm + i) + c, so row % 16 == c % 16
    const uint16_t* xa = slot_lds(slot) + (wm * MT * 32 + c) * kTileK;
    // A operands double-buffered: step s + 1's LDS reads are issued at the
    // start of step s (the scheduling barrier keeps the compiler from
    // sinking them back to just before their first use), so their latency
    // is covered by a whole step of MFMAs
    u4 abuf[2][MT];
    auto read_a = [&](int step, u4 (&dst)[MT]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
        dst[i] = *reinterpret_cast<const u4*>(xa + i * 32 * kTileK + 8 * ((2 * step + h) ^ (c & 15)));
    };
    read_a(0, abuf[0]);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      uint32_t n1[NT], n2[NT];
      float ratio[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint32_t z = HAS_Z ? (r.z[nt][p] >> zshift) & 0xFu : 8u;
        n1[nt] = nz1024_bits(z);
        n2[nt] = nz64_bits(z);
        const float s_cur = act_to_f32<OB16>(r.s[nt][p]);
        ratio[nt] = s_prev[nt] * __builtin_amdgcn_rcpf(s_cur);
        s_prev[nt] = s_cur;
      }
#pragma unroll
      for (int st = 0; st < SPP; ++st) {
        const int step = p * SPP + st;  // 16-deep step of the block, 0..7
        if (step + 1 < 8) read_a(step + 1, abuf[(step + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        const u4(&a)[MT] = abuf[step & 1];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint32_t w = r.w[nt][step & 1][step >> 1];
          const u4 bq = dq_f16(w, n1[nt], n2[nt], nm);
#pragma unroll
          for (int i = 0; i < MT; ++i) {
            if (RESCALE && st == 0) {
#pragma unroll
              for (int q = 0; q < 16; ++q) acc[i][nt][q] *= ratio[nt];
            }
            acc[i][nt] = mfma32(a[i], bq, acc[i][nt]);
          }
        }
        if (RESCALE && st == 0) {
#pragma unroll
          for (int t = 0; t < MT * NT; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x0002, 16, 0);  // 16 VALU: one tile's rescale
            __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);   // then its MFMA
          }
        }
      }
    }
  };

  auto iterate = [&](int64_t b, int u) __attribute__((always_inline)) {
    const int un = (u + S - 1) % S;
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<C::kAfter>();
    lds_barrier();
    const int64_t bn = b + S - 1 < nb ? b + S - 1 : nb - 1;  // clamped: a redundant in-bounds load
    issue(kb0 + bn, rg[un], un);
    compute(rg[u], u);
  };

#pragma unroll
  for (int u = 0; u < S - 1; ++u) issue(kb0 + (u < nb ? u : nb - 1), rg[u], u);
  int64_t b = 0;
  for (; b + S <= nb; b += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) iterate(b + u, u);
  }
#pragma unroll
  for (int u = 0; u < S - 1; ++u)
    if (b + u < nb) iterate(b + u, u);

  // epilogue: element r of lane l is row 8 (r / 4) + 4 h + r % 4 of each row
  // tile, column c of each column tile
  if constexpr (OB16) {
    // row tile by row tile, so that only one tile's row factors are live:
    // rowf[m .. m + 3] for m = 8 j + 4 h of the tile (rowf holds whole
    // 128-row tiles; rows >= M are never stored)
    float bv[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int64_t n = n0 + (int64_t)(wn * NT + nt) * 32 + c;
      bv[nt] = bias != nullptr && n < N ? act_to_f32<true>(bias[n]) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int64_t mb = m0 + (int64_t)(wm * MT + i) * 32 + 4 * h;
      f4 rf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) rf[j] = *reinterpret_cast<const f4*>(rowf + mb + 8 * j);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int64_t n = n0 + (int64_t)(wn * NT + nt) * 32 + c;
        if (n >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = mb + 8 * (r >> 2) + (r & 3);
          if (m >= M) continue;
          y[m * N + n] = f32_to_act<true>(acc[i][nt][r] * s_prev[nt] * rf[r >> 2][r & 3] + bv[nt]);
        }
      }
    }
  } else {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int64_t n = n0 + (int64_t)(wn * NT + nt) * 32 + c;
      if (n >= N) continue;  // padded columns, or tiles past the last strip
      const float bv = bias != nullptr ? act_to_f32<false>(bias[n]) : 0.f;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = m0 + (int64_t)(wm * MT + i) * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (m >= M) continue;
          y[m * N + n] = f32_to_act<false>(acc[i][nt][r] * s_prev[nt] + bv);
        }
    }
  }
  };

  if constexpr (GROUPED) {
    const int64_t e = blockIdx.z;
    int64_t r0 = offs[e], r1 = offs[e + 1];
    r0 = r0 < 0 ? 0 : (r0 > M_in ? M_in : r0);
    r1 = r1 < r0 ? r0 : (r1 > M_in ? M_in : r1);
    const int64_t Me = r1 - r0;
    const u4* qwe = qw_in + e * (K * T * kTileN / 32);
    const uint16_t* sce = sc_in + e * T * kTileN * G;
    const uint32_t* zse = HAS_Z ? zs_in + e * T * 2 * G : zs_in;
    const uint16_t* biase = bias_in != nullptr ? bias_in + e * N : nullptr;
    // every row tile of the expert, in steps of gridDim.y (an expert with
    // more rows than the launch height is still computed whole); the weight
    // bases pass through an opaque zero made inside the loop so that the
    // compiler cannot hoist the prologue's weight loads out of it (the
    // counted vmcnt waits assume the issue order)
    for (int64_t m0 = (int64_t)blockIdx.y * C::BM; m0 < Me; m0 += (int64_t)gridDim.y * C::BM) {
      int64_t z0;
      asm volatile("s_mov_b64 %0, 0" : "=s"(z0));
      tile(m0, (int64_t)blockIdx.x * C::BN, x_in + r0 * K, qwe + z0, sce + z0, zse + z0, biase, y_in + r0 * N, Me);
      // the clamped prefetches of the last blocks may still be landing in
      // the LDS slots: drain them, and let every wave finish with the slots,
      // before the next row tile's prologue refills them
      wait_vmcnt<0>();
      lds_barrier();
    }
  } else {
    int64_t tm, tn;
    big_tile_of(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    tile(tm * C::BM, tn * C::BN, x_in, qw_in, sc_in, zs_in, bias_in, y_in, M_in);
  }
}

// xh[m][k] = fp16(x[m][k] 2^-e_m) and rowf[m] = 2^e_m for bf16 x [M][K]
// (K a multiple of 8): e_m brings the row's largest finite magnitude into
// [2^14, 2^15) (e_m >= -126; 0 for a row without a finite nonzero value).
// One workgroup per row: the row's maximum first, then the conversion
// (round to nearest even, exact in fp16's normal range).  CH > 0: rows of
// at most 256 CH 16-byte chunks, kept in registers between the two passes
// (one read of x); CH = 0: any K, read twice.
template <int CH>
__global__ __launch_bounds__(256) void bf16_rows_to_f16(const uint16_t* __restrict__ x, uint16_t* __restrict__ xh,
                                                        float* __restrict__ rowf, int64_t M, int64_t K) {
  __shared__ float red[4];
  const int64_t K8 = K / 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  auto upd = [](float& mx, const u4& v) __attribute__((always_inline)) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = __builtin_fabsf(bit_as<float>(w[j] << 16));
      const float hi = __builtin_fabsf(bit_as<float>(w[j] & 0xFFFF0000u));
      // infinities and NaNs do not count (scaled, they stay what they are)
      if (lo < __builtin_inff() && lo > mx) mx = lo;
      if (hi < __builtin_inff() && hi > mx) mx = hi;
    }
  };
  auto cvt = [](const u4& v, float down) __attribute__((always_inline)) -> u4 {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = (uint32_t)f32_to_act<false>(bit_as<float>(w[j] << 16) * down) |
             ((uint32_t)f32_to_act<false>(bit_as<float>(w[j] & 0xFFFF0000u) * down) << 16);
    return u4{o[0], o[1], o[2], o[3]};
  };
  for (int64_t m = blockIdx.x; m < M; m += gridDim.x) {
    const u4* src = reinterpret_cast<const u4*>(x + m * K);
    u4* dst = reinterpret_cast<u4*>(xh + m * K);
    float mx = 0.f;
    u4 keep[CH > 0 ? CH : 1];
    if constexpr (CH > 0) {
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int64_t c = threadIdx.x + 256 * j;
        keep[j] = c < K8 ? src[c] : u4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < CH; ++j) upd(mx, keep[j]);
    } else {
      for (int64_t c = threadIdx.x; c < K8; c += 256) upd(mx, src[c]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, off));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
    __syncthreads();  // red is rewritten for the next row
    // exponent of mx (-127 for a subnormal mx, which the clamp covers: every
    // bf16 value is at least 2^-133 and so stays exact after 2^126)
    const int ex = (int)((bit_as<uint32_t>(mx) >> 23) & 0xFFu) - 127;
    const int e = mx > 0.f ? (ex - 14 < -126 ? -126 : ex - 14) : 0;
    const float down = bit_as<float>((uint32_t)(127 - e) << 23);
    if (threadIdx.x == 0) rowf[m] = bit_as<float>((uint32_t)(127 + e) << 23);
    if constexpr (CH > 0) {
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int64_t c = threadIdx.x + 256 * j;
        if (c < K8) dst[c] = cvt(keep[j], down);
      }
    } else {
      for (int64_t c = threadIdx.x; c < K8; c += 256) dst[c] = cvt(src[c], down);
    }
  }
}

// Launch of one configuration (the whole of K per workgroup); `group_m` row
// tiles per band of the tile order.  OB16: x is bf16, converted into xh
// ([M][K] fp16) and rowf ([M] fp32) first.
template <int WM, int WN, int MT, int NT, int S, int GM, bool HZ, bool OB16 = false>
hipError_t run_big(const Args& a, const uint16_t* x, uint16_t* xh, float* rowf, int64_t group_m, hipStream_t st) {
  using C = BigCfg<WM, WN, MT, NT, S>;
  const int64_t Np = (a.N + kTileN - 1) / kTileN * kTileN;
  const int64_t tiles_m = (a.M + C::BM - 1) / C::BM, tiles_n = (Np + C::BN - 1) / C::BN;
  if (tiles_m * tiles_n > 0x7FFFFFFF || group_m < 1) return hipErrorInvalidValue;
  if constexpr (OB16) {
    if (xh == nullptr || rowf == nullptr || a.K % 8 != 0) return hipErrorInvalidValue;
    const unsigned blocks = (unsigned)(a.M < 65535 ? a.M : 65535);
    if (a.K <= 8 * 256 * 16)
      bf16_rows_to_f16<16><<<blocks, 256, 0, st>>>(x, xh, rowf, a.M, a.K);
    else
      bf16_rows_to_f16<0><<<blocks, 256, 0, st>>>(x, xh, rowf, a.M, a.K);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    x = xh;
  }
  gemm_big<WM, WN, MT, NT, S, GM, HZ, false, OB16><<<(unsigned)(tiles_m * tiles_n), 64 * WM * WN, 0, st>>>(
      x, a.qw, a.sc, a.zs, a.bias, a.y, a.M, a.K, a.N, a.G, tiles_m, tiles_n, group_m, nullptr,
      OB16 ? rowf : nullptr);
  return hipGetLastError();
}

// Grouped launch: a.offs [a.groups + 1] expert row offsets, a.max_rows the
// most rows any expert has (the launch height; a larger expert is still
// computed whole).
template <int WM, int WN, int MT, int NT, int S, int GM, bool HZ>
hipError_t run_big_grouped(const Args& a, hipStream_t st) {
  using C = BigCfg<WM, WN, MT, NT, S>;
  const int64_t Np = (a.N + kTileN - 1) / kTileN * kTileN;
  const int64_t tiles_n = (Np + C::BN - 1) / C::BN, tiles_m = (a.max_rows + C::BM - 1) / C::BM;
  if (a.offs == nullptr || a.groups < 1 || a.groups > 65535 || tiles_m < 1 || tiles_m > 65535 ||
      tiles_n > 0x7FFFFFFF)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)tiles_n, (unsigned)tiles_m, (unsigned)a.groups);
  gemm_big<WM, WN, MT, NT, S, GM, HZ, true><<<grid, 64 * WM * WN, 0, st>>>(
      a.x, a.qw, a.sc, a.zs, a.bias, a.y, a.M, a.K, a.N, a.G, tiles_m, tiles_n, 1, a.offs, nullptr);
  return hipGetLastError();
}

// The shipped configuration: four waves side by side, each 128 rows x 64
// columns (workgroup tile 128 x 256), double-buffered (64 KiB of LDS, two
// workgroups per CU); tile order in bands of four row tiles.  Chosen from
// sweeps of the prefill shapes on MI355X against 2 x 2 and 2 x 4 wave
// arrangements, 64 x 64 and 64 x 128 wave tiles and three- and four-deep
// pipelines.
constexpr int kBigWM = 1, kBigWN = 4, kBigMT = 4, kBigNT = 2, kBigS = 2;
constexpr int64_t kBigGroupM = 4;

template <int GM, bool OB16>
hipError_t big_z(const Args& a, const uint16_t* x, uint16_t* xh, float* rowf, bool has_z, hipStream_t st) {
  return has_z ? run_big<kBigWM, kBigWN, kBigMT, kBigNT, kBigS, GM, true, OB16>(a, x, xh, rowf, kBigGroupM, st)
               : run_big<kBigWM, kBigWN, kBigMT, kBigNT, kBigS, GM, false, OB16>(a, x, xh, rowf, kBigGroupM, st);
}

template <bool OB16>
hipError_t big_gm(const Args& a, const uint16_t* x, uint16_t* xh, float* rowf, bool has_z, hipStream_t st) {
  switch (group_mode(a.gs, a.K)) {
    case GM_32: return big_z<GM_32, OB16>(a, x, xh, rowf, has_z, st);
    case GM_64: return big_z<GM_64, OB16>(a, x, xh, rowf, has_z, st);
    case GM_128: return big_z<GM_128, OB16>(a, x, xh, rowf, has_z, st);
    default: return big_z<GM_CH, OB16>(a, x, xh, rowf, has_z, st);
  }
}

// Arguments of a plain large-M launch.
inline Args big_args(const Shape& s, int64_t M, const int32_t* tiled_w, const void* tiled_s, const int32_t* tiled_z,
                     const void* bias, void* y) {
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
  return a;
}

}  // namespace
}  // namespace w4
