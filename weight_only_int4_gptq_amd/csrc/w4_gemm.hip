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

// Nibble masks held in VGPRs.  (w & mask) | bits is one v_and_or_b32, but a
// gfx9 VOP3 encoding takes no literal, so with literal masks the compiler
// emits a separate AND and OR.  Producing the masks once through an opaque
// move makes them register values and lets the compiler select
// v_and_or_b32 itself (keeping its hazard tracking around the MFMAs, which
// inline asm on the operand path would bypass).
struct NibbleMasks {
  uint32_t lo, hi;  // 0x000F000F, 0x00F000F0
  __device__ __forceinline__ static NibbleMasks make() {
    NibbleMasks m;
    asm volatile("v_mov_b32 %0, 0x000F000F" : "=v"(m.lo));
    asm volatile("v_mov_b32 %0, 0x00F000F0" : "=v"(m.hi));
    return m;
  }
};

// fp16 operand: exact (q - z) for the eight K-offsets of a tiled word.
__device__ __forceinline__ u4 dq_f16(uint32_t w, uint32_t nz1024_bits, uint32_t nz64_bits, NibbleMasks m) {
  const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const h2 nz1024 = bit_as<h2>(nz1024_bits);
  const h2 nz64 = bit_as<h2>(nz64_bits);
  const uint32_t w8 = w >> 8;
  const h2 a = bit_as<h2>((w & m.lo) | 0x64006400u) + nz1024;
  const h2 b = __builtin_elementwise_fma(bit_as<h2>((w & m.hi) | 0x64006400u), sixteenth, nz64);
  const h2 c = bit_as<h2>((w8 & m.lo) | 0x64006400u) + nz1024;
  const h2 d = __builtin_elementwise_fma(bit_as<h2>((w8 & m.hi) | 0x64006400u), sixteenth, nz64);
  return u4{bit_as<uint32_t>(a), bit_as<uint32_t>(b), bit_as<uint32_t>(c), bit_as<uint32_t>(d)};
}

// bf16 operand: exact (128 + q) for the eight K-offsets of a tiled word.
__device__ __forceinline__ u4 dq_bf16(uint32_t w, NibbleMasks m) {
  return u4{(w & m.lo) | 0x43004300u, ((w >> 4) & m.lo) | 0x43004300u, ((w >> 8) & m.lo) | 0x43004300u,
            ((w >> 12) & m.lo) | 0x43004300u};
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
                                          const uint32_t (&zraw)[NB][Groups<GM>::kPeriods], uint32_t zshift,
                                          NibbleMasks nm) {
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
          b = dq_bf16(wv[s][j], nm);
        else
          b = dq_f16(wv[s][j], n1, n2, nm);
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

// Activation rows staged in LDS (XL kernels): row r of the workgroup's
// 16-row tile at xs + r * (K + kXPad); the pad of 8 halves moves consecutive
// rows to different banks.
constexpr int kXPad = 8;

// Registers of one run of U blocks: weights, scales and zeros of NB strips,
// and (unless the activations come from LDS) the A operands of MT row tiles.
template <int U, int MT, int NB, int NP, bool XL>
struct RunRegs {
  u4 wv[U][NB];
  uint16_t sraw[U][NB][NP];
  uint32_t zraw[U][NB][NP];
  u4 a[XL ? 1 : U][MT][4];
};

// Per-lane view of the operands of one workgroup, with every pointer
// computed once.  Lanes whose row is >= M read row M - 1 and select zero.
// The selection is branch-free on purpose: an exec-masked load region here
// let the compiler fold the row mask into the loop's active-lane mask, so
// the next block's B operands were built for the masked lanes only.
template <int MT, int NB, int GM, bool HAS_Z, bool HAS_PERM, bool XL>
struct LaneView {
  static constexpr int NP = Groups<GM>::kPeriods;
  const u4* w[NB];            // tiled words of strip s at block 0 (lane's 16 bytes)
  const uint16_t* sc[NB];     // scale of column c of strip s, group 0
  const uint32_t* zs[NB];     // zero word holding column c of strip s, group 0
  const uint16_t* xr[MT];     // x row of tile i (+ 8 * quad without act-order)
  const int32_t* pm;          // perm + 8 * quad
  const uint16_t* xl;         // XL: LDS row of this lane + 8 * quad
  bool row_ok[MT];            // row of tile i is < M
  int64_t nblk;

  __device__ __forceinline__ void init(const uint16_t* x, const u4* qw, const uint16_t* scl, const uint32_t* zsp,
                                       const int32_t* perm, const uint16_t* xlds, int64_t t0, int64_t m0, int64_t M,
                                       int64_t K, int G, int lane) {
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
      row_ok[i] = m < M;
      m = m < M ? m : M - 1;
      xr[i] = x + m * K + (HAS_PERM ? 0 : 8 * quad);
    }
    pm = perm + 8 * quad;
    // LDS rows >= M are never staged; read row 0 instead (its value is discarded)
    xl = xlds + (row_ok[0] ? c : 0) * (K + kXPad) + 8 * quad;
  }

  __device__ static __forceinline__ u4 masked(bool ok, u4 v) {
    const u4 z = {0u, 0u, 0u, 0u};
    return ok ? v : z;
  }

  // A operands of block kb straight from global memory.
  __device__ __forceinline__ void load_a_global(int kb, u4 (&a)[MT][4]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = kb * kTileK + 32 * j;
      if constexpr (!HAS_PERM) {
#pragma unroll
        for (int i = 0; i < MT; ++i) a[i][j] = masked(row_ok[i], *reinterpret_cast<const u4*>(xr[i] + k));
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
          a[i][j] = masked(row_ok[i], u4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                         h[6] | (h[7] << 16)});
        }
      }
    }
  }

  // A operands of block kb from the LDS copy (one row tile).
  __device__ __forceinline__ void load_a_lds(int kb, u4 (&a)[MT][4]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) a[0][j] = masked(row_ok[0], *reinterpret_cast<const u4*>(xl + kb * kTileK + 32 * j));
  }

  // Weights, scales, zeros (and global A operands) of blocks kb .. kb+U-1 < hi.
  template <int U>
  __device__ __forceinline__ void load_run(int kb, int hi, RunRegs<U, MT, NB, NP, XL>& r) const {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = kb + u;
      if (b < hi) {  // wave-uniform
#pragma unroll
      for (int s = 0; s < NB; ++s) {
        r.wv[u][s] = w[s][(int64_t)b * 64];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int g = Groups<GM>::group(b, p);
          r.sraw[u][s][p] = sc[s][(int64_t)g * kTileN];
          r.zraw[u][s][p] = HAS_Z ? zs[s][(int64_t)g * 2] : 0u;
        }
      }
      if constexpr (!XL) load_a_global(b, r.a[u]);
      }
    }
  }
};

// Skinny kernel: see the header comment.  XL: activations staged in LDS.
template <int MT, int NB, int KW, int U, int GM, bool BF16, bool HAS_Z, bool HAS_PERM, bool XL>
__global__ __launch_bounds__(64 * KW) void gemm_skinny(const uint16_t* __restrict__ x, const u4* __restrict__ qw,
                                                        const uint16_t* __restrict__ sc,
                                                        const uint32_t* __restrict__ zs,
                                                        const int32_t* __restrict__ perm,
                                                        const uint16_t* __restrict__ bias,
                                                        uint16_t* __restrict__ y, int64_t M, int64_t K, int64_t N,
                                                        int G, uint32_t* __restrict__ counters,
                                                        float* __restrict__ partials) {
  static_assert(!XL || MT == 1, "LDS activations hold one 16-row tile");
  constexpr int NP = Groups<GM>::kPeriods;
  constexpr int R = MT * NB * 4;
  extern __shared__ float smem[];  // [KW][R][64] reduction buffer, then (XL) the activation rows
  float* red = smem;
  uint16_t* xlds = reinterpret_cast<uint16_t*>(smem + KW * R * 64);
  __shared__ int last_arrival;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t0 = (int64_t)blockIdx.x * NB;
  const int64_t m0 = (int64_t)blockIdx.y * 16 * MT;
  const int KS = (int)gridDim.z, split = (int)blockIdx.z;

  LaneView<MT, NB, GM, HAS_Z, HAS_PERM, XL> v;
  v.init(x, qw, sc, zs, perm, xlds, t0, m0, M, K, G, lane);
  const int nblk = (int)v.nblk;
  // split z of the workgroup grid owns blocks [z nblk / KS, (z + 1) nblk / KS);
  // wave w owns the contiguous part [lo, hi) of it
  const int64_t slo = ((int64_t)nblk * split) / KS, shi = ((int64_t)nblk * (split + 1)) / KS;
  const int lo = __builtin_amdgcn_readfirstlane((int)(slo + ((shi - slo) * wave) / KW));
  const int hi = __builtin_amdgcn_readfirstlane((int)(slo + ((shi - slo) * (wave + 1)) / KW));
  const uint32_t zshift = 4u * (uint32_t)(lane & 7);
  const NibbleMasks nm = NibbleMasks::make();

  f4 tot[MT][NB];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int s = 0; s < NB; ++s) tot[i][s] = f4{0.f, 0.f, 0.f, 0.f};

  // Runs of U blocks.  With LDS activations the runs are double buffered
  // (the loads of run r + 1 are in flight while run r is computed) and the
  // first run is issued before the staging so that its latency overlaps it;
  // with register activations a single buffer keeps the register count, and
  // so the occupancy, up (measured faster at M = 4..16).
  RunRegs<U, MT, NB, NP, XL> ra, rb;
  int kb = lo;
  v.template load_run<U>(kb, hi, ra);
  if constexpr (XL) {
    const int64_t rows = (M - m0) < 16 ? (M - m0) : 16;
    const int64_t K8 = K / 8;
    for (int64_t r = 0; r < rows; ++r) {
      const uint16_t* src = x + (m0 + r) * K;
      uint16_t* dst = xlds + r * (K + kXPad);
      for (int64_t k8 = threadIdx.x; k8 < K8; k8 += 64 * KW) {
        u4 val;
        if constexpr (!HAS_PERM) {
          val = *reinterpret_cast<const u4*>(src + 8 * k8);
        } else {
          const int4 p0 = *reinterpret_cast<const int4*>(perm + 8 * k8);
          const int4 p1 = *reinterpret_cast<const int4*>(perm + 8 * k8 + 4);
          const uint32_t idx[8] = {(uint32_t)p0.x, (uint32_t)p0.y, (uint32_t)p0.z, (uint32_t)p0.w,
                                   (uint32_t)p1.x, (uint32_t)p1.y, (uint32_t)p1.z, (uint32_t)p1.w};
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) h[e] = src[idx[e] < (uint32_t)K ? idx[e] : 0u];
          val = u4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        }
        *reinterpret_cast<u4*>(dst + 8 * k8) = val;
      }
    }
    __syncthreads();
  }

  auto compute = [&](int k0, RunRegs<U, MT, NB, NP, XL>& r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k0 + u < hi) {  // wave-uniform
        if constexpr (XL) {
          u4 a[MT][4];
          v.load_a_lds(k0 + u, a);
          block_mac<MT, NB, GM, BF16, HAS_Z>(tot, a, r.wv[u], r.sraw[u], r.zraw[u], zshift, nm);
        } else {
          block_mac<MT, NB, GM, BF16, HAS_Z>(tot, r.a[u], r.wv[u], r.sraw[u], r.zraw[u], zshift, nm);
        }
      }
    }
  };
  if constexpr (XL) {
    for (; kb < hi; kb += 2 * U) {
      v.template load_run<U>(kb + U, hi, rb);
      compute(kb, ra);
      v.template load_run<U>(kb + 2 * U, hi, ra);
      compute(kb + U, rb);
    }
  } else {
    for (; kb < hi; kb += U) {
      compute(kb, ra);
      v.template load_run<U>(kb + U, hi, ra);
    }
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

// ---------------------------------------------------------------------------
// Wide kernel (the large-M, MFMA-bound path)
//
// Workgroup: 256 threads = 4 waves in a 2 x 2 grid over a 128 x 128 output
// tile; wave (wm, wn) owns rows 64 wm .. 64 wm + 63 and strips 4 wn .. 4 wn + 3
// of the tile (4 x 4 MFMA tiles of 16 x 16).  Per 128-row group of K:
//   * the 128 x 128 activation tile is staged in LDS, double buffered, one
//     barrier per group, by direct global->LDS loads (no registers): 16-byte
//     chunk j of row r is stored at chunk position j ^ (r % 16) of the row,
//     so the 16 rows that one A-operand read touches fall on distinct banks;
//   * each wave streams the packed words of its 4 strips straight from HBM
//     into registers (one 16-byte load per strip per lane), prefetched one
//     group ahead together with scales and zeros;
//   * for each K step the four strips are dequantized in registers and fed
//     to 16 MFMAs.
// Scaling uses one accumulator set per tile: at the start of scale period g
// the fp32 accumulator (which holds sum_{h<g} P_h s_h / s_{g-1}) is
// multiplied by s_{g-1} / s_g, the MFMAs then add the exact integer-weighted
// sums P_g of period g, and the result is multiplied by the last scale at
// the end.  The tile layout never stores a zero scale (the repack replaces
// it and zeroes the codes' contribution), so every ratio is finite; each
// multiply adds one fp32 rounding (relative 2^-24 per period).
// Rows >= M are staged as zeros and never stored; strips >= N/16 are skipped.
// ---------------------------------------------------------------------------
constexpr int kWideBM = 128, kWideBN = 128, kWideThreads = 256;
constexpr int kWideLdsStride = kTileK;  // halves per staged activation row (swizzled, unpadded)

typedef __attribute__((address_space(3))) void lds_void;

template <int GM, bool BF16, bool HAS_Z>
__global__ __launch_bounds__(kWideThreads, 2) void gemm_wide(const uint16_t* __restrict__ x,
                                                               const u4* __restrict__ qw,
                                                               const uint16_t* __restrict__ sc,
                                                               const uint32_t* __restrict__ zs,
                                                               const uint16_t* __restrict__ bias,
                                                               uint16_t* __restrict__ y, int64_t M, int64_t K,
                                                               int64_t N, int G) {
  constexpr int NP = Groups<GM>::kPeriods, SP = Groups<GM>::kSteps;
  __shared__ __attribute__((aligned(1024))) uint16_t xs[2][kWideBM * kWideLdsStride];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int c = lane & 15, quad = lane >> 4;
  const int64_t T = N / kTileN;
  const int64_t nblk = K / kTileK;
  const int64_t m0 = (int64_t)blockIdx.y * kWideBM;
  const int64_t tw0 = (int64_t)blockIdx.x * (kWideBN / kTileN) + 4 * wn;  // first strip of this wave
  const uint32_t zshift = 4u * (uint32_t)(c & 7);
  const NibbleMasks nm = NibbleMasks::make();

  // staging: instruction i of wave w fills rows 32 w + 4 i .. + 3 of the
  // tile; lane l lands at chunk position l % 16 of row 32 w + 4 i + l / 16
  // and so loads logical chunk (l % 16) ^ (row % 16).  Rows >= M load row
  // M - 1: their outputs are never stored.
  auto stage = [&](int64_t kb, int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 32 * wave + 4 * i + (lane >> 4);
      int64_t m = m0 + row;
      m = m < M ? m : M - 1;
      const int j = (lane & 15) ^ (row & 15);
      const uint16_t* src = x + m * K + kb * kTileK + 8 * j;
      __builtin_amdgcn_global_load_lds(src, (lds_void*)&xs[buf][(32 * wave + 4 * i) * kWideLdsStride], 16, 0, 0);
    }
  };
  struct Meta {
    u4 w[4];
    uint16_t s[4][NP];
    uint32_t z[4][NP];
  };
  auto load_meta = [&](int64_t kb, Meta& mt) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t t = tw0 + nt;
      const bool ok = t < T;
      const int64_t tt = ok ? t : 0;
      mt.w[nt] = u4{0u, 0u, 0u, 0u};
      if (ok) mt.w[nt] = qw[(tt * nblk + kb) * 64 + lane];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int64_t g = Groups<GM>::group((int)kb, p);
        mt.s[nt][p] = ok ? sc[(tt * G + g) * kTileN + c] : (uint16_t)0;
        mt.z[nt][p] = (HAS_Z && ok) ? zs[(tt * G + g) * 2 + (c >> 3)] : 0u;
      }
    }
  };

  f4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
  const u4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  float s_prev[4] = {1.f, 1.f, 1.f, 1.f};

  Meta cur, nxt;
  stage(0, 0);
  load_meta(0, cur);
  __builtin_amdgcn_s_waitcnt(0);  // the direct-to-LDS loads of tile 0 have landed
  for (int64_t kb = 0; kb < nblk; ++kb) {
    const int buf = (int)(kb & 1);
    __syncthreads();  // tile kb visible; buffer buf ^ 1 free
    const bool more = kb + 1 < nblk;
    if (more) {
      stage(kb + 1, buf ^ 1);
      load_meta(kb + 1, nxt);
    }
    // row of this lane in tile i: 64 wm + 16 i + c, so row % 16 == c
    const uint16_t* xa = &xs[buf][(64 * wm + c) * kWideLdsStride];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      uint32_t n1[4], n2[4];
      float nzz[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const uint32_t z = HAS_Z ? (cur.z[nt][p] >> zshift) & 0xFu : 8u;
        n1[nt] = nz1024_bits(z);
        n2[nt] = nz64_bits(z);
        nzz[nt] = -(128.0f + (float)z);
        const float s_cur = act_to_f32<BF16>(cur.s[nt][p]);
        if constexpr (GM != GM_CH) {
          const float r = s_prev[nt] * __builtin_amdgcn_rcpf(s_cur);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][nt][q] *= r;
        }
        s_prev[nt] = s_cur;
      }
      f4 rs[4];
      if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) rs[i] = f4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = p * SP; j < (p + 1) * SP; ++j) {
        u4 a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a[i] = *reinterpret_cast<const u4*>(xa + 16 * i * kWideLdsStride + 8 * ((4 * j + quad) ^ c));
        if constexpr (BF16) {
#pragma unroll
          for (int i = 0; i < 4; ++i) rs[i] = mfma<true>(a[i], ones, rs[i]);
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          u4 b;
          if constexpr (BF16)
            b = dq_bf16(cur.w[nt][j], nm);
          else
            b = dq_f16(cur.w[nt][j], n1[nt], n2[nt], nm);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i][nt] = mfma<BF16>(a[i], b, acc[i][nt]);
        }
      }
      if constexpr (BF16) {
        // remove (128 + z) * sum_k x[m, k] of this period
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][nt][q] = __builtin_fmaf(nzz[nt], rs[i][q], acc[i][nt][q]);
      }
    }
    if (more) cur = nxt;
    __builtin_amdgcn_s_waitcnt(0);  // tile kb + 1 has landed before the barrier publishes it
  }
  f4 tot[4][4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) tot[i][nt][q] = acc[i][nt][q] * s_prev[nt];

  // epilogue: lane holds column c of each strip, rows 4 quad + r of each tile
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int64_t t = tw0 + nt;
    if (t >= T) continue;
    const int64_t n = t * kTileN + c;
    const float b = bias != nullptr ? act_to_f32<BF16>(bias[n]) : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + 64 * wm + 16 * i + 4 * quad + r;
        if (m < M) y[m * N + n] = f32_to_act<BF16>(tot[i][nt][r] + b);
      }
  }
}

// x_perm[m][k'] = x[m][perm[k']] for the act-order wide path (perm entries
// outside [0, K) read column 0).
__global__ void gather_columns(const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
                               uint16_t* __restrict__ xp, int64_t M, int64_t K) {
  const int64_t total = M * K;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = idx / K, k = idx - m * K;
    const uint32_t p = (uint32_t)perm[k];
    xp[idx] = x[m * K + (p < (uint32_t)K ? p : 0u)];
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

// LDS bytes of a skinny launch: the reduction buffer, plus the staged
// activation rows (at most 16, row stride K + kXPad halves) when XL.
constexpr size_t kMaxSkinnyLds = 64 * 1024;

inline size_t skinny_lds_bytes(int mt, int nb, int kw, bool xl, int64_t M, int64_t K) {
  size_t b = (size_t)kw * mt * nb * 4 * 64 * sizeof(float);
  if (xl) b += (size_t)(M < 16 ? M : 16) * (size_t)(K + kXPad) * sizeof(uint16_t);
  return b;
}

template <int MT, int NB, int KW, int U, int GM, bool BF16, bool HZ, bool HP, bool XL>
hipError_t run_skinny(const Args& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.N / (kTileN * NB)), (unsigned)((a.M + 16 * MT - 1) / (16 * MT)), (unsigned)a.ks);
  const size_t lds = skinny_lds_bytes(MT, NB, KW, XL, a.M, a.K);
  gemm_skinny<MT, NB, KW, U, GM, BF16, HZ, HP, XL><<<grid, 64 * KW, lds, st>>>(
      a.x, a.qw, a.sc, a.zs, a.perm, a.bias, a.y, a.M, a.K, a.N, a.G, a.counters, a.partials);
  return hipGetLastError();
}

inline int group_mode(int gs, int64_t K) {
  if (gs == 32) return GM_32;
  if (gs == 64) return GM_64;
  if (gs == 128) return GM_128;
  return GM_CH;  // per-channel: one group of K rows
}

template <int GM, bool BF16, bool HZ>
hipError_t run_wide(const Args& a, const uint16_t* x, hipStream_t st) {
  const dim3 grid((unsigned)((a.N / kTileN + (kWideBN / kTileN) - 1) / (kWideBN / kTileN)),
                  (unsigned)((a.M + kWideBM - 1) / kWideBM));
  gemm_wide<GM, BF16, HZ><<<grid, kWideThreads, 0, st>>>(x, a.qw, a.sc, a.zs, a.bias, a.y, a.M, a.K, a.N, a.G);
  return hipGetLastError();
}

template <bool BF16, bool HZ>
hipError_t wide_gm(const Args& a, const uint16_t* x, hipStream_t st) {
  switch (group_mode(a.gs, a.K)) {
    case GM_32: return run_wide<GM_32, BF16, HZ>(a, x, st);
    case GM_64: return run_wide<GM_64, BF16, HZ>(a, x, st);
    case GM_128: return run_wide<GM_128, BF16, HZ>(a, x, st);
    default: return run_wide<GM_CH, BF16, HZ>(a, x, st);
  }
}

// Act-order first gathers the columns of x into the workspace.
hipError_t launch_wide(const Shape& s, const Args& a, void* ws, hipStream_t st) {
  const uint16_t* x = a.x;
  if (s.has_perm) {
    uint16_t* xp = static_cast<uint16_t*>(ws);
    const int64_t total = a.M * a.K;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    gather_columns<<<(unsigned)blocks, 256, 0, st>>>(a.x, a.perm, xp, a.M, a.K);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    x = xp;
  }
  if (s.bf16) return s.has_z ? wide_gm<true, true>(a, x, st) : wide_gm<true, false>(a, x, st);
  return s.has_z ? wide_gm<false, true>(a, x, st) : wide_gm<false, false>(a, x, st);
}

template <int MT, int NB, int KW, int U, bool XL, bool BF16, bool HZ, bool HP>
hipError_t pick_gm(const Args& a, hipStream_t st) {
  switch (group_mode(a.gs, a.K)) {
    case GM_32: return run_skinny<MT, NB, KW, U, GM_32, BF16, HZ, HP, XL>(a, st);
    case GM_64: return run_skinny<MT, NB, KW, U, GM_64, BF16, HZ, HP, XL>(a, st);
    case GM_128: return run_skinny<MT, NB, KW, U, GM_128, BF16, HZ, HP, XL>(a, st);
    default: return run_skinny<MT, NB, KW, U, GM_CH, BF16, HZ, HP, XL>(a, st);
  }
}

template <int MT, int NB, int KW, int U, bool XL>
hipError_t pick_flags(const Shape& s, const Args& a, hipStream_t st) {
  if (s.bf16) {
    if (s.has_z)
      return s.has_perm ? pick_gm<MT, NB, KW, U, XL, true, true, true>(a, st)
                        : pick_gm<MT, NB, KW, U, XL, true, true, false>(a, st);
    return s.has_perm ? pick_gm<MT, NB, KW, U, XL, true, false, true>(a, st)
                      : pick_gm<MT, NB, KW, U, XL, true, false, false>(a, st);
  }
  if (s.has_z)
    return s.has_perm ? pick_gm<MT, NB, KW, U, XL, false, true, true>(a, st)
                      : pick_gm<MT, NB, KW, U, XL, false, true, false>(a, st);
  return s.has_perm ? pick_gm<MT, NB, KW, U, XL, false, false, true>(a, st)
                    : pick_gm<MT, NB, KW, U, XL, false, false, false>(a, st);
}

}  // namespace

GemmPlan plan_gemm(const Shape& s, int64_t M) {
  // (mt, nb, kw, u, ks, xl): 16-row tiles per wave, strips per workgroup,
  // waves per workgroup (splitting K), blocks per load run, workgroups
  // splitting K, activations staged in LDS.  Chosen from timing sweeps of
  // the decode shapes on MI355X.
  GemmPlan p;
  const bool deep_k = s.K >= 8192 || s.N <= 4096;  // few strips: more waves per strip
  if (M == 1 && skinny_lds_bytes(1, 1, 16, true, M, s.K) <= kMaxSkinnyLds) {
    p = deep_k ? GemmPlan{GemmKind::kSkinny, 1, 1, 16, 1, 1, true, "w4_skinny_m1_lds_k16"}
               : GemmPlan{GemmKind::kSkinny, 1, 1, 8, 1, 1, true, "w4_skinny_m1_lds_k8"};
  } else if (M <= 16) {
    if (s.N >= 12288) p = GemmPlan{GemmKind::kSkinny, 1, 2, 16, 1, 1, false, "w4_skinny_m16_n2_k16"};
    else if (M <= 4) p = GemmPlan{GemmKind::kSkinny, 1, 1, 16, 1, 1, false, "w4_skinny_m16_k16"};
    else p = GemmPlan{GemmKind::kSkinny, 1, 1, 8, 1, 1, false, "w4_skinny_m16_k8"};
  } else if (M <= 32) {
    p = GemmPlan{GemmKind::kSkinny, 2, 1, 8, 1, 1, false, "w4_skinny_m32"};
  } else if (M <= 64) {
    p = GemmPlan{GemmKind::kSkinny, 4, 1, 4, 1, 1, false, "w4_skinny_m64"};
  } else {
    p = GemmPlan{GemmKind::kWide, 0, 0, 0, 0, 1, false, s.has_perm ? "w4_wide_128x128_gather" : "w4_wide_128x128"};
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
  if (p.kind == GemmKind::kWide) return s.has_perm ? (size_t)M * (size_t)s.K * sizeof(uint16_t) : 0;
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
  if (p.kind == GemmKind::kWide) return launch_wide(s, a, ws, st);
  if (p.xl) return p.kw == 16 ? pick_flags<1, 1, 16, 1, true>(s, a, st) : pick_flags<1, 1, 8, 1, true>(s, a, st);
  if (p.mt == 1 && p.nb == 2) return pick_flags<1, 2, 16, 1, false>(s, a, st);
  if (p.mt == 1) return p.kw == 16 ? pick_flags<1, 1, 16, 1, false>(s, a, st) : pick_flags<1, 1, 8, 1, false>(s, a, st);
  if (p.mt == 2) return pick_flags<2, 1, 8, 1, false>(s, a, st);
  return pick_flags<4, 1, 4, 1, false>(s, a, st);
}

}  // namespace w4
