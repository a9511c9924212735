// Fused dequantize + GEMM kernels of libw4hip for gfx950 (MI355X).
//
// y[m, n] = sum_k x[m, k] * (q[k, n] - z[g(k), n]) * s[g(k), n] + bias[n]
// (dequantization of the vLLM AWQ practice page, section 5.3, fused into the
// matrix multiply as the learning-book page, section 5.3, describes).
//
// Numerics.  The MFMA operands are exact small integers: for fp16 the
// operand is (q - z) itself, for bf16 it is (128 + q) and the zero term
// (128 + z) * sum_k x[m, k] is removed with per-row sums computed by an MFMA
// against a ones operand.  Products are accumulated in fp32 over one
// group-period, the period sum is multiplied by the fp32 scale and added to an
// fp32 total; y is rounded once.  Folding the scale into a 16-bit weight
// would round every weight and, at K = 28672, exceed the elementwise error
// bound; exact operands avoid that.
//
// Operand construction ("magic number" dequantization).  A tiled word holds
// K-offsets (0,1) in nibble slots (0,4), (2,3) in (1,5), (4,5) in (2,6) and
// (6,7) in (3,7), i.e. the two halves of a 32-bit register receive two
// consecutive K values with one mask:
//   fp16: (w & 0x000F000F) | 0x64006400 = (1024 + q0, 1024 + q1); adding
//         -(1024 + z) with v_pk_add_f16 gives (q - z) exactly.  The high
//         nibble pair (w & 0x00F000F0) | 0x64006400 = 1024 + 16 q; one
//         v_pk_fma_f16 by 1/16 and -(64 + z) gives (q - z) exactly.
//   bf16: 0x4300 is 128.0 with unit spacing; (w >> 4j) masked and ored gives
//         (128 + q) exactly (gfx950 has no packed bf16 add, hence the row-sum
//         correction above).
//
// MFMA v_mfma_f32_16x16x32_{f16,bf16}: lane l supplies row/column l % 16 and
// eight K values 8 (l / 16) .. 8 (l / 16) + 7 of the 32-deep step in each
// operand; A and B use the same (lane, slot) -> k map, so the sum pairs
// x[m, k] with w[k, n].  Output: lane l holds column l % 16, rows
// 4 (l / 16) + i, i = 0..3.
//
// Skinny kernel (the small-M, bandwidth-bound path): a workgroup owns NB
// strips of 16 output columns and MT 16-row tiles of M; its KW waves split the
// 128-row blocks of K between them (wave w takes blocks w, w + KW, ...), each
// wave streaming 16 bytes per lane per block with one coalesced 1 KiB load,
// and the KW partial results are summed in LDS at the end.
#include "w4_internal.h"

namespace w4 {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

template <typename T, typename F>
__device__ __forceinline__ T bit_as(F f) {
  return __builtin_bit_cast(T, f);
}

__device__ __forceinline__ uint32_t h2_bits(float a) {
  const h2 v = {(_Float16)a, (_Float16)a};
  return bit_as<uint32_t>(v);
}

// fp16 operand: exact (q - z) for the eight K-offsets of a tiled word.
__device__ __forceinline__ u4 dq_f16(uint32_t w, uint32_t nz1024_bits, uint32_t nz64_bits) {
  const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const h2 nz1024 = bit_as<h2>(nz1024_bits);
  const h2 nz64 = bit_as<h2>(nz64_bits);
  const uint32_t w8 = w >> 8;
  const h2 a = bit_as<h2>((w & 0x000F000Fu) | 0x64006400u) + nz1024;
  const h2 b = __builtin_elementwise_fma(bit_as<h2>((w & 0x00F000F0u) | 0x64006400u), sixteenth, nz64);
  const h2 c = bit_as<h2>((w8 & 0x000F000Fu) | 0x64006400u) + nz1024;
  const h2 d = __builtin_elementwise_fma(bit_as<h2>((w8 & 0x00F000F0u) | 0x64006400u), sixteenth, nz64);
  return u4{bit_as<uint32_t>(a), bit_as<uint32_t>(b), bit_as<uint32_t>(c), bit_as<uint32_t>(d)};
}

// bf16 operand: exact (128 + q) for the eight K-offsets of a tiled word.
__device__ __forceinline__ u4 dq_bf16(uint32_t w) {
  return u4{(w & 0x000F000Fu) | 0x43004300u, ((w >> 4) & 0x000F000Fu) | 0x43004300u,
            ((w >> 8) & 0x000F000Fu) | 0x43004300u, ((w >> 12) & 0x000F000Fu) | 0x43004300u};
}

template <bool BF16>
__device__ __forceinline__ f4 mfma(u4 a, u4 b, f4 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bit_as<b8>(a), bit_as<b8>(b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(bit_as<h8>(a), bit_as<h8>(b), c, 0, 0, 0);
}

template <bool BF16>
__device__ __forceinline__ float act_to_f32(uint16_t bits) {
  if constexpr (BF16)
    return bit_as<float>((uint32_t)bits << 16);
  else
    return (float)bit_as<_Float16>(bits);
}

template <bool BF16>
__device__ __forceinline__ uint16_t f32_to_act(float v) {
  if constexpr (BF16)
    return bit_as<uint16_t>((__bf16)v);
  else
    return bit_as<uint16_t>((_Float16)v);
}

// Group mode of a layer (compile time, so no division in the kernels):
//   GM_CH  per-channel, one group of K rows (g(k) = 0)
//   GM_128 g = 128: one group per 128-row block (g = block)
//   GM_64  g = 64: two groups per block, one per pair of 32-deep steps
//   GM_32  g = 32: four groups per block, one per step
enum GroupMode { GM_CH = 0, GM_128 = 1, GM_64 = 2, GM_32 = 3 };

template <int GM>
struct Groups {
  static constexpr int kPeriods = GM == GM_64 ? 2 : (GM == GM_32 ? 4 : 1);  // scale periods per block
  static constexpr int kSteps = 4 / kPeriods;                               // 32-deep steps per period
  __device__ static __forceinline__ int group(int kb, int p) {
    if constexpr (GM == GM_CH) return 0;
    else return kb * kPeriods + p;
  }
};

// fp16 -(1024 + z) and -(64 + z), packed twice (z = 0..15): 1024 has unit
// spacing, so its mantissa is z; 64 has spacing 1/16, so its mantissa is 16 z.
__device__ __forceinline__ uint32_t nz1024_bits(uint32_t z) { return (0xE400u + z) * 0x10001u; }
__device__ __forceinline__ uint32_t nz64_bits(uint32_t z) { return (0xD400u + 16u * z) * 0x10001u; }

// Accumulate one 128-row block of NB strips for MT row tiles.
//   a[i][j]  A operand of row tile i, step j
//   wv[s]    tiled words of strip s (one per step)
//   sraw/zraw[s][p]  scale bits / zero word of strip s, period p
template <int MT, int NB, int GM, bool BF16, bool HAS_Z>
__device__ __forceinline__ void block_mac(f4 (&tot)[MT][NB], const u4 (&a)[MT][4], const u4 (&wv)[NB],
                                          const uint16_t (&sraw)[NB][Groups<GM>::kPeriods],
                                          const uint32_t (&zraw)[NB][Groups<GM>::kPeriods], uint32_t zshift) {
  constexpr int NP = Groups<GM>::kPeriods, SP = Groups<GM>::kSteps;
  const u4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  f4 rs[MT][NP];
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        f4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = p * SP; j < (p + 1) * SP; ++j) r = mfma<true>(a[i][j], ones, r);
        rs[i][p] = r;
      }
  }
#pragma unroll
  for (int s = 0; s < NB; ++s) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const float sf = act_to_f32<BF16>(sraw[s][p]);
      const uint32_t z = HAS_Z ? (zraw[s][p] >> zshift) & 0xFu : 8u;
      f4 acc[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) acc[i] = f4{0.f, 0.f, 0.f, 0.f};
      const uint32_t n1 = nz1024_bits(z), n2 = nz64_bits(z);
#pragma unroll
      for (int j = p * SP; j < (p + 1) * SP; ++j) {
        u4 b;
        if constexpr (BF16)
          b = dq_bf16(wv[s][j]);
        else
          b = dq_f16(wv[s][j], n1, n2);
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[i] = mfma<BF16>(a[i][j], b, acc[i]);
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        if constexpr (BF16) {
          const float nzz = -(128.0f + (float)z);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][r] = __builtin_fmaf(nzz, rs[i][p][r], acc[i][r]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[i][s][r] = __builtin_fmaf(sf, acc[i][r], tot[i][s][r]);
      }
    }
  }
}

// Per-lane view of the operands of one workgroup, with every pointer
// computed once.  Rows >= M are clamped to row M-1: their MFMA outputs are
// valid numbers that are never stored, so no lane needs a mask.
template <int MT, int NB, int GM, bool HAS_Z, bool HAS_PERM>
struct LaneView {
  const u4* w[NB];            // tiled words of strip s at block 0 (lane's 16 bytes)
  const uint16_t* sc[NB];     // scale of column c of strip s, group 0
  const uint32_t* zs[NB];     // zero word holding column c of strip s, group 0
  const uint16_t* xr[MT];     // x row of tile i, offset 8 * quad
  const int32_t* pm;          // perm + 8 * quad
  int64_t nblk;

  __device__ __forceinline__ void init(const uint16_t* x, const u4* qw, const uint16_t* scl, const uint32_t* zsp,
                                       const int32_t* perm, int64_t t0, int64_t m0, int64_t M, int64_t K, int G,
                                       int lane) {
    const int c = lane & 15, quad = lane >> 4;
    nblk = K / kTileK;
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      w[s] = qw + (t0 + s) * nblk * 64 + lane;
      sc[s] = scl + (t0 + s) * G * kTileN + c;
      zs[s] = HAS_Z ? zsp + (t0 + s) * G * 2 + (c >> 3) : nullptr;
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      int64_t m = m0 + 16 * i + c;
      m = m < M ? m : M - 1;
      xr[i] = x + m * K + (HAS_PERM ? 0 : 8 * quad);
    }
    pm = perm + 8 * quad;
  }

  __device__ __forceinline__ void load(int kb, u4 (&a)[MT][4], u4 (&wv)[NB], uint16_t (&sraw)[NB][Groups<GM>::kPeriods],
                                       uint32_t (&zraw)[NB][Groups<GM>::kPeriods]) const {
    constexpr int NP = Groups<GM>::kPeriods;
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      wv[s] = w[s][(int64_t)kb * 64];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int g = Groups<GM>::group(kb, p);
        sraw[s][p] = sc[s][(int64_t)g * kTileN];
        zraw[s][p] = HAS_Z ? zs[s][(int64_t)g * 2] : 0u;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = kb * kTileK + 32 * j;
      if constexpr (!HAS_PERM) {
#pragma unroll
        for (int i = 0; i < MT; ++i) a[i][j] = *reinterpret_cast<const u4*>(xr[i] + k);
      } else {
        const int4 p0 = *reinterpret_cast<const int4*>(pm + k);
        const int4 p1 = *reinterpret_cast<const int4*>(pm + k + 4);
        const uint32_t idx[8] = {(uint32_t)p0.x, (uint32_t)p0.y, (uint32_t)p0.z, (uint32_t)p0.w,
                                 (uint32_t)p1.x, (uint32_t)p1.y, (uint32_t)p1.z, (uint32_t)p1.w};
        const uint32_t Ku = (uint32_t)(nblk * kTileK);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) h[e] = xr[i][idx[e] < Ku ? idx[e] : 0u];
          a[i][j] = u4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        }
      }
    }
  }
};

template <int MT, int NB, int KW, int U, int GM, bool BF16, bool HAS_Z, bool HAS_PERM>
__global__ __launch_bounds__(64 * KW) void gemm_skinny(const uint16_t* __restrict__ x, const u4* __restrict__ qw,
                                                        const uint16_t* __restrict__ sc,
                                                        const uint32_t* __restrict__ zs,
                                                        const int32_t* __restrict__ perm,
                                                        const uint16_t* __restrict__ bias,
                                                        uint16_t* __restrict__ y, int64_t M, int64_t K, int64_t N,
                                                        int G, uint32_t* __restrict__ counters,
                                                        float* __restrict__ partials) {
  constexpr int NP = Groups<GM>::kPeriods;
  constexpr int R = MT * NB * 4;
  extern __shared__ float red[];  // [KW][R][64]
  __shared__ int last_arrival;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t0 = (int64_t)blockIdx.x * NB;
  const int64_t m0 = (int64_t)blockIdx.y * 16 * MT;
  const int KS = (int)gridDim.z, split = (int)blockIdx.z;

  LaneView<MT, NB, GM, HAS_Z, HAS_PERM> v;
  v.init(x, qw, sc, zs, perm, t0, m0, M, K, G, lane);
  const int nblk = (int)v.nblk;
  // split z of the workgroup grid owns blocks [z nblk / KS, (z + 1) nblk / KS);
  // wave w owns the contiguous part [lo, hi) of it
  const int64_t slo = ((int64_t)nblk * split) / KS, shi = ((int64_t)nblk * (split + 1)) / KS;
  const int lo = (int)(slo + ((shi - slo) * wave) / KW);
  const int hi = (int)(slo + ((shi - slo) * (wave + 1)) / KW);
  const uint32_t zshift = 4u * (uint32_t)(lane & 7);

  f4 tot[MT][NB];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int s = 0; s < NB; ++s) tot[i][s] = f4{0.f, 0.f, 0.f, 0.f};

  int kb = lo;
  // Runs of U blocks: all loads of a run are issued before any is used.
  for (; kb + U <= hi; kb += U) {
    u4 a[U][MT][4];
    u4 wv[U][NB];
    uint16_t sraw[U][NB][NP];
    uint32_t zraw[U][NB][NP];
#pragma unroll
    for (int u = 0; u < U; ++u) v.load(kb + u, a[u], wv[u], sraw[u], zraw[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) block_mac<MT, NB, GM, BF16, HAS_Z>(tot, a[u], wv[u], sraw[u], zraw[u], zshift);
  }
  for (; kb < hi; ++kb) {
    u4 a[MT][4];
    u4 wv[NB];
    uint16_t sraw[NB][NP];
    uint32_t zraw[NB][NP];
    v.load(kb, a, wv, sraw, zraw);
    block_mac<MT, NB, GM, BF16, HAS_Z>(tot, a, wv, sraw, zraw, zshift);
  }

  // Sum the KW waves' partial results in LDS, then bias, round and store.
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int s = 0; s < NB; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[((wave * R) + (i * NB + s) * 4 + r) * 64 + lane] = tot[i][s][r];
  __syncthreads();
  constexpr int kPer = (R * 64 + 64 * KW - 1) / (64 * KW);  // outputs per thread
  float acc[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int e = threadIdx.x + q * 64 * KW;
    acc[q] = 0.f;
    if (e < R * 64) {
#pragma unroll
      for (int w = 0; w < KW; ++w) acc[q] += red[w * R * 64 + e];
    }
  }
  if (KS > 1) {
    // Split-K fix-up.  Each workgroup stores its partial tile; the last of the
    // KS workgroups of a tile to arrive sums the KS partials in split order
    // (deterministic), finishes the tile and clears its counter for the next
    // call.  No workgroup waits for another.
    const int64_t tile = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    float* part = partials + tile * KS * (R * 64);
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int e = threadIdx.x + q * 64 * KW;
      if (e < R * 64) part[(int64_t)split * (R * 64) + e] = acc[q];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t old = __hip_atomic_fetch_add(counters + tile, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      last_arrival = old == (uint32_t)(KS - 1);
    }
    __syncthreads();
    if (!last_arrival) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int e = threadIdx.x + q * 64 * KW;
      if (e < R * 64) {
        float v = 0.f;
        for (int z = 0; z < KS; ++z) v += part[(int64_t)z * (R * 64) + e];
        acc[q] = v;
      }
    }
    if (threadIdx.x == 0) __hip_atomic_store(counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int e = threadIdx.x + q * 64 * KW;
    if (e >= R * 64) continue;
    const int rr = e >> 6, l = e & 63;
    const int i = rr / (NB * 4), s = (rr >> 2) % NB, r = rr & 3;
    const int64_t m = m0 + 16 * i + 4 * (l >> 4) + r;
    const int64_t n = (t0 + s) * kTileN + (l & 15);
    if (m < M) {
      float o = acc[q];
      if (bias != nullptr) o += act_to_f32<BF16>(bias[n]);
      y[m * N + n] = f32_to_act<BF16>(o);
    }
  }
}

struct Args {
  const uint16_t* x;
  const u4* qw;
  const uint16_t* sc;
  const uint32_t* zs;
  const int32_t* perm;
  const uint16_t* bias;
  uint16_t* y;
  int64_t M, K, N;
  int G, gs;
  int ks;               // workgroups splitting K (gridDim.z)
  uint32_t* counters;   // split-K arrival counters (zero between calls)
  float* partials;      // split-K partial tiles
};

template <int MT, int NB, int KW, int U, int GM, bool BF16, bool HZ, bool HP>
hipError_t run_skinny(const Args& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.N / (kTileN * NB)), (unsigned)((a.M + 16 * MT - 1) / (16 * MT)), (unsigned)a.ks);
  const size_t lds = (size_t)KW * MT * NB * 4 * 64 * sizeof(float);
  gemm_skinny<MT, NB, KW, U, GM, BF16, HZ, HP><<<grid, 64 * KW, lds, st>>>(
      a.x, a.qw, a.sc, a.zs, a.perm, a.bias, a.y, a.M, a.K, a.N, a.G, a.counters, a.partials);
  return hipGetLastError();
}

inline int group_mode(int gs, int64_t K) {
  if (gs == 32) return GM_32;
  if (gs == 64) return GM_64;
  if (gs == 128) return GM_128;
  return GM_CH;  // per-channel: one group of K rows
}

template <int MT, int NB, int KW, int U, bool BF16, bool HZ, bool HP>
hipError_t pick_gm(const Args& a, hipStream_t st) {
  switch (group_mode(a.gs, a.K)) {
    case GM_32: return run_skinny<MT, NB, KW, U, GM_32, BF16, HZ, HP>(a, st);
    case GM_64: return run_skinny<MT, NB, KW, U, GM_64, BF16, HZ, HP>(a, st);
    case GM_128: return run_skinny<MT, NB, KW, U, GM_128, BF16, HZ, HP>(a, st);
    default: return run_skinny<MT, NB, KW, U, GM_CH, BF16, HZ, HP>(a, st);
  }
}

template <int MT, int NB, int KW, int U>
hipError_t pick_flags(const Shape& s, const Args& a, hipStream_t st) {
  if (s.bf16) {
    if (s.has_z)
      return s.has_perm ? pick_gm<MT, NB, KW, U, true, true, true>(a, st) : pick_gm<MT, NB, KW, U, true, true, false>(a, st);
    return s.has_perm ? pick_gm<MT, NB, KW, U, true, false, true>(a, st) : pick_gm<MT, NB, KW, U, true, false, false>(a, st);
  }
  if (s.has_z)
    return s.has_perm ? pick_gm<MT, NB, KW, U, false, true, true>(a, st) : pick_gm<MT, NB, KW, U, false, true, false>(a, st);
  return s.has_perm ? pick_gm<MT, NB, KW, U, false, false, true>(a, st) : pick_gm<MT, NB, KW, U, false, false, false>(a, st);
}

}  // namespace

GemmPlan plan_gemm(const Shape& s, int64_t M) {
  // (mt, nb, kw, u, ks): 16-row tiles per wave, strips per workgroup, waves
  // per workgroup (splitting K), blocks per load run, workgroups splitting K.
  GemmPlan p{GemmKind::kSkinny, 1, 1, 8, 1, 1, "w4_skinny_m16_n16"};
  if (M <= 16) {
    if (s.N >= 16384) p = GemmPlan{GemmKind::kSkinny, 1, 2, 8, 1, 1, "w4_skinny_m16_n32"};
    else if (s.K >= 8192 || s.N <= 4096) p = GemmPlan{GemmKind::kSkinny, 1, 1, 16, 2, 1, "w4_skinny_m16_n16_k16"};
  } else if (M <= 32) {
    p = GemmPlan{GemmKind::kSkinny, 2, 1, 8, 1, 1, "w4_skinny_m32"};
  } else {
    p = GemmPlan{GemmKind::kSkinny, 4, 1, 4, 1, 1, "w4_skinny_m64"};
  }
  // No split of K across workgroups: the agent-scope release fence that the
  // split-K fix-up needs writes back the XCD's whole L2 on gfx950 and costs
  // far more than it saves at these sizes (measured).
  p.ks = 1;
  return p;
}

namespace {
int64_t tiles_of(const Shape& s, int64_t M, const GemmPlan& p) {
  return (s.N / (kTileN * p.nb)) * ((M + 16 * p.mt - 1) / (16 * p.mt));
}
constexpr size_t kCounterAlign = 256;
}  // namespace

size_t gemm_workspace_bytes(const Shape& s, int64_t M) {
  const GemmPlan p = plan_gemm(s, M);
  if (p.ks <= 1) return 0;
  const size_t tiles = (size_t)tiles_of(s, M, p);
  const size_t counters = (tiles * sizeof(uint32_t) + kCounterAlign - 1) / kCounterAlign * kCounterAlign;
  return counters + tiles * p.ks * (size_t)(p.mt * p.nb * 4 * 64) * sizeof(float);
}

hipError_t launch_gemm(const Shape& s, int64_t M, const void* x, const int32_t* tiled_w, const void* tiled_s,
                       const int32_t* tiled_z, const int32_t* perm, const void* bias, void* y, void* ws,
                       hipStream_t st) {
  Args a;
  a.x = static_cast<const uint16_t*>(x);
  a.qw = reinterpret_cast<const u4*>(tiled_w);
  a.sc = static_cast<const uint16_t*>(tiled_s);
  a.zs = reinterpret_cast<const uint32_t*>(tiled_z);
  a.perm = perm;
  a.bias = static_cast<const uint16_t*>(bias);
  a.y = static_cast<uint16_t*>(y);
  a.M = M;
  a.K = s.K;
  a.N = s.N;
  a.G = s.G;
  a.gs = s.gs;
  const GemmPlan p = plan_gemm(s, M);
  a.ks = p.ks;
  a.counters = nullptr;
  a.partials = nullptr;
  if (p.ks > 1) {
    const size_t tiles = (size_t)tiles_of(s, M, p);
    const size_t counters = (tiles * sizeof(uint32_t) + kCounterAlign - 1) / kCounterAlign * kCounterAlign;
    a.counters = static_cast<uint32_t*>(ws);
    a.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + counters);
  }
  if (p.mt == 1 && p.nb == 2) return pick_flags<1, 2, 8, 1>(s, a, st);
  if (p.mt == 1 && p.kw == 16) return pick_flags<1, 1, 16, 2>(s, a, st);
  if (p.mt == 1) return pick_flags<1, 1, 8, 1>(s, a, st);
  if (p.mt == 2) return pick_flags<2, 1, 8, 1>(s, a, st);
  return pick_flags<4, 1, 4, 1>(s, a, st);
}

}  // namespace w4
