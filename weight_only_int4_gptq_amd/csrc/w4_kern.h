// Fused dequantize + GEMM kernels of libw4hip for gfx950 (MI355X): kernel
// templates and launch helpers shared by the plain (w4_gemm.hip) and grouped
// (w4_moe.hip) launch paths; everything sits in an anonymous namespace, so
// each translation unit instantiates the kernels it launches.
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
// 128-row blocks of K into KW contiguous ranges, each wave streaming 16 bytes
// per lane per block with one coalesced 1 KiB load, and the KW partial
// results are summed in LDS at the end.  Each scale period (one group, at
// most 128 rows) is accumulated exactly in fp32 from integer operands and
// then added, times its fp32 scale, to the fp32 total.
#pragma once

#include <atomic>

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
// 16-row tile at xs + r * (K + kXPad).  An A-operand read puts the four
// 16-byte quads of a row on four consecutive 4-bank groups (16 banks); with
// K a multiple of 128 the pad of 32 halves starts each row 16 banks after
// the previous one, so the (at most four) staged rows and their quads fall
// on 64 distinct banks.  (A pad of 8 halves, one 4-bank group per row,
// overlapped row r + 1 with quad 1 of row r: 0.6-0.75 bank-conflict cycles
// per LDS-active cycle at M = 4 in the SQ counters.)
constexpr int kXPad = 32;
constexpr int kXlRows = 4;  // at most this many rows are staged (M <= 4)

// Memory helpers shared by the kernels below.
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
// vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] in bits 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes
// land at dst + 16 l (dst is wave-uniform).
__device__ __forceinline__ void load_lds16(const uint16_t* src, uint16_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}

// 4 bytes per lane: lane l's word lands at dst + l (dst is wave-uniform).
__device__ __forceinline__ void load_lds4(const float* src, float* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 4, 0, 0);
}

// Workgroup barrier for the pipeline.  __syncthreads() would add a release
// fence, which waits for every outstanding direct-to-LDS load (they count as
// LDS writes) and so drains the whole pipeline at every block.  Here each
// wave has already waited for its own loads of the block about to be read
// (wait_vmcnt), so the bare barrier suffices; the empty asm statements keep
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Registers of one 128-row block: weights, scales and zeros of NB strips,
// and (unless the activations come from LDS) the A operands of MT row tiles.
template <int MT, int NB, int NP, bool XL>
struct BlockRegs {
  u4 wv[NB];
  uint16_t sraw[NB][NP];
  uint32_t zraw[NB][NP];
  u4 a[XL ? 1 : MT][4];
};

// Per-lane view of the operands of one workgroup, with every pointer
// computed once.  Lanes whose row is >= M read a valid row (M - 1, or row 0
// of the LDS copy) unmasked: an output row of the MFMA depends only on its
// own A row, and rows >= M are never stored.  The loads are unconditional on
// purpose: an exec-masked load region here let the compiler fold the row
// mask into the loop's active-lane mask, so the next block's B operands were
// built for the masked lanes only.
template <int MT, int NB, int GM, bool HAS_Z, bool XL>
struct LaneView {
  static constexpr int NP = Groups<GM>::kPeriods;
  // Addresses as a uniform base (per strip, per row tile) plus a 32-bit
  // per-lane byte offset, so the loads take the scalar-base form.
  const char* wb[NB];         // tiled words of strip s at block 0
  const char* sb[NB];         // scales of strip s, group 0
  const char* zb[NB];         // zero words of strip s, group 0
  const char* xb;             // x row m0
  uint32_t wo, so, zo;        // lane's 16 bytes of a block, its column's scale and zero word
  uint32_t xo[MT];            // x row of tile i + 8 * quad, relative to xb
  uint32_t xdo[4];            // AD: source of this lane's 16 bytes in direct-to-LDS load i of a block
  const uint16_t* xl;         // XL: LDS row of this lane + 8 * quad
  bool row_ok[MT];            // row of tile i is < M
  int64_t nblk;

  __device__ __forceinline__ void init(const uint16_t* x, const u4* qw, const uint16_t* scl, const uint32_t* zsp,
                                       const uint16_t* xlds, int64_t t0, int64_t m0, int64_t M, int64_t K, int G,
                                       int lane) {
    const int c = lane & 15, quad = lane >> 4;
    nblk = K / kTileK;
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      wb[s] = reinterpret_cast<const char*>(qw + (t0 + s) * nblk * 64);
      sb[s] = reinterpret_cast<const char*>(scl + (t0 + s) * G * kTileN);
      zb[s] = reinterpret_cast<const char*>(HAS_Z ? zsp + (t0 + s) * G * 2 : zsp);
    }
    wo = (uint32_t)lane * (uint32_t)sizeof(u4);
    so = (uint32_t)c * (uint32_t)sizeof(uint16_t);
    zo = (uint32_t)(c >> 3) * (uint32_t)sizeof(uint32_t);
    xb = reinterpret_cast<const char*>(x + m0 * K);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      int64_t m = m0 + 16 * i + c;
      row_ok[i] = m < M;
      m = m < M ? m : M - 1;
      xo[i] = (uint32_t)(((m - m0) * K + 8 * quad) * (int64_t)sizeof(uint16_t));
    }
    // LDS rows >= M are never staged; read row 0 instead
    xl = xlds + (row_ok[0] ? c : 0) * (K + kXPad) + 8 * quad;
    // AD (one 16-row tile): load i of a block fills rows 4 i .. 4 i + 3 of
    // the wave's 16 x 128 copy, lane l landing at chunk position l % 16 of
    // row 4 i + l / 16, which holds logical chunk (l % 16) ^ row (rows >= M
    // read row M - 1, never stored)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * i + quad;
      int64_t m = m0 + row;
      m = m < M ? m : M - 1;
      xdo[i] = (uint32_t)(((m - m0) * K + 8 * (c ^ row)) * (int64_t)sizeof(uint16_t));
    }
  }

  // AD: the first AR rows (4 or 16) of the block's activation tile into the
  // wave's LDS copy dst (AR / 4 direct-to-LDS loads of 1 KiB, each of four
  // whole 256-byte rows).
  template <int AR>
  __device__ __forceinline__ void load_a_dma(int kb, uint16_t* dst) const {
#pragma unroll
    for (int i = 0; i < AR / 4; ++i)
      load_lds16(reinterpret_cast<const uint16_t*>(xb + (xdo[i] + (uint32_t)kb * (uint32_t)(kTileK * sizeof(uint16_t)))),
                 dst + 4 * i * kTileK);
  }

  // A operands of block kb straight from global memory.
  __device__ __forceinline__ void load_a_global(int kb, u4 (&a)[MT][4]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t k = ((uint32_t)kb * kTileK + 32u * j) * (uint32_t)sizeof(uint16_t);
#pragma unroll
      for (int i = 0; i < MT; ++i) a[i][j] = *reinterpret_cast<const u4*>(xb + (xo[i] + k));
    }
  }

  // A operands of block kb from the LDS copy (one row tile).
  __device__ __forceinline__ void load_a_lds(int kb, u4 (&a)[MT][4]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) a[0][j] = *reinterpret_cast<const u4*>(xl + kb * kTileK + 32 * j);
  }

  // Weights, scales, zeros (and global A operands) of block b.
  template <bool NOA>
  __device__ __forceinline__ void load_block(int b, BlockRegs<MT, NB, NP, NOA>& r) const {
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      r.wv[s] = *reinterpret_cast<const u4*>(wb[s] + (wo + (uint32_t)b * 1024u));
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint32_t g = (uint32_t)Groups<GM>::group(b, p);
        r.sraw[s][p] = *reinterpret_cast<const uint16_t*>(sb[s] + (so + g * (uint32_t)(kTileN * sizeof(uint16_t))));
        r.zraw[s][p] = HAS_Z ? *reinterpret_cast<const uint32_t*>(zb[s] + (zo + g * 8u)) : 0u;
      }
    }
    if constexpr (!NOA) load_a_global(b, r.a);
  }
};

// Skinny kernel: see the header comment.  XL: activations staged in LDS.
// AD: each wave copies every block's 16 x 128 activation tile into its own
// LDS ring slot with direct-to-LDS loads (whole 256-byte rows, 8 cache lines
// per load) and reads its MFMA operands from there; loading them straight
// into registers instead touches 16 half-used lines per load.
template <int MT, int NB, int KW, int GM, bool BF16, bool HAS_Z, bool XL, int D, int AR = 0>
__global__ __launch_bounds__(64 * KW) void gemm_skinny(const uint16_t* __restrict__ x, const u4* __restrict__ qw,
                                                        const uint16_t* __restrict__ sc,
                                                        const uint32_t* __restrict__ zs,
                                                        const uint16_t* __restrict__ bias,
                                                        uint16_t* __restrict__ y, int64_t M, int64_t K, int64_t N,
                                                        int G) {
  static_assert(!XL || MT == 1, "LDS activations hold one 16-row tile");
  static_assert(AR == 0 || ((AR == 4 || AR == 16) && MT == 1 && !XL && D <= 6),
                "per-block LDS activations: 4 or 16 rows of one tile, ring <= 6");
  static_assert((D - 1) * (NB + AR / 4) < 64, "vmcnt is six bits");
  // AD ring: one array per slot (so a read of slot u waits only for the
  // loads into slot u), KW copies of 16 x 128 halves each
  constexpr int kAdSlot = AR ? KW * AR * kTileK : 8;
  __shared__ __attribute__((aligned(1024))) uint16_t ad0[kAdSlot];
  __shared__ __attribute__((aligned(1024))) uint16_t ad1[AR && D > 1 ? kAdSlot : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t ad2[AR && D > 2 ? kAdSlot : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t ad3[AR && D > 3 ? kAdSlot : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t ad4[AR && D > 4 ? kAdSlot : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t ad5[AR && D > 5 ? kAdSlot : 8];
  auto slot_ad = [&](int u) __attribute__((always_inline)) -> uint16_t* {
    switch (u) {
      case 0: return ad0;
      case 1: return ad1;
      case 2: return ad2;
      case 3: return ad3;
      case 4: return ad4;
      default: return ad5;
    }
  };
  constexpr int NP = Groups<GM>::kPeriods;
  constexpr int R = MT * NB * 4;
  // [KW][R][64] reduction buffer; with XL the staged activation rows occupy
  // the same bytes first (the reduction starts after a barrier), so the
  // launch needs the larger of the two, not their sum
  extern __shared__ float smem[];
  float* red = smem;
  uint16_t* xlds = reinterpret_cast<uint16_t*>(smem);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t0 = (int64_t)blockIdx.x * NB;
  const int64_t m0 = (int64_t)blockIdx.y * 16 * MT;

  LaneView<MT, NB, GM, HAS_Z, XL> v;
  v.init(x, qw, sc, zs, xlds, t0, m0, M, K, G, lane);
  const int nblk = (int)v.nblk;
  // wave w owns the contiguous blocks [lo, hi) of K (wave-uniform bounds)
  const int lo = __builtin_amdgcn_readfirstlane((int)(((int64_t)nblk * wave) / KW));
  const int hi = __builtin_amdgcn_readfirstlane((int)(((int64_t)nblk * (wave + 1)) / KW));
  const uint32_t zshift = 4u * (uint32_t)(lane & 7);
  const NibbleMasks nm = NibbleMasks::make();

  f4 tot[MT][NB];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int s = 0; s < NB; ++s) tot[i][s] = f4{0.f, 0.f, 0.f, 0.f};

  // Blocks go through a D-deep register ring: the loads of blocks b + 1 ..
  // b + D - 1 (weights, scales, zeros and, without LDS staging, the
  // activations) are in flight while block b is computed, so a wave with at
  // most D blocks pays one memory latency, not one per block.  With LDS
  // activations the first blocks are issued before the staging so that
  // their latency overlaps it.  The ring loops are fully unrolled (constant
  // slot indices keep the ring in registers) and branch-free in steady
  // state: the prefetch index is clamped to the wave's last block (redundant
  // in-bounds loads at the end), so no branch join makes the compiler wait
  // for every outstanding load.
  static_assert(D >= 2, "ring depth");
  const bool has_blocks = lo < hi;  // wave-uniform
  const int last = hi - 1;
  BlockRegs<MT, NB, NP, XL || AR != 0> ring[D];
  // the loads of block b into ring slot u (with AD also the activation tile
  // into the wave's copy in LDS slot u, issued last).  kPerBlock is a lower
  // bound on the loads one fill issues: the NB weight loads and the four
  // direct-to-LDS loads; the scale and zero loads are left out because the
  // compiler may merge them or hoist them out of the loop (per-channel
  // scales), and leaving them out only makes the wait below longer.
  constexpr int kPerBlock = NB + AR / 4;
  auto fill = [&](int b, int u) __attribute__((always_inline)) {
    v.load_block(b, ring[u]);
    if constexpr (AR != 0) v.template load_a_dma<AR>(b, slot_ad(u) + wave * AR * kTileK);
  };
  if (has_blocks) {
#pragma unroll
    for (int u = 0; u < D - 1; ++u) {
      fill(lo + u < last ? lo + u : last, u);
      if constexpr (AR != 0) __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (XL) {
    // Stage the (at most kXlRows) activation rows: the loads of every row of
    // a chunk column are issued before any is written, so one memory latency
    // covers the whole chunk column (rows >= M are neither loaded nor
    // written).
    const int rows = (int)((M - m0) < kXlRows ? (M - m0) : kXlRows);
    const int64_t K8 = K / 8;
    for (int64_t k8 = threadIdx.x; k8 < K8; k8 += 64 * KW) {
      u4 val[kXlRows];
#pragma unroll
      for (int r = 0; r < kXlRows; ++r)
        if (r < rows) val[r] = *reinterpret_cast<const u4*>(x + (m0 + r) * K + 8 * k8);
#pragma unroll
      for (int r = 0; r < kXlRows; ++r)
        if (r < rows) *reinterpret_cast<u4*>(xlds + r * (K + kXPad) + 8 * k8) = val[r];
    }
    __syncthreads();
  }

  auto compute = [&](int b, int u) __attribute__((always_inline)) {
    auto& r = ring[u];
    if constexpr (XL) {
      u4 a[MT][4];
      v.load_a_lds(b, a);
      block_mac<MT, NB, GM, BF16, HAS_Z>(tot, a, r.wv, r.sraw, r.zraw, zshift, nm);
    } else if constexpr (AR != 0) {
      // row c % AR of the wave's copy, chunk position (4 j + quad) ^ c: for
      // c < AR that is logical chunk 4 j + quad of row c; with 4 rows the
      // lanes past them (rows >= M, never stored) read some other chunk, at
      // a position of their own, so the 16 lanes of a quad hit 16 distinct
      // 16-byte bank groups
      const int c = lane & 15, quad = lane >> 4;
      const uint16_t* base = slot_ad(u) + wave * AR * kTileK + (c & (AR - 1)) * kTileK;
      u4 a[MT][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) a[0][j] = *reinterpret_cast<const u4*>(base + 8 * ((4 * j + quad) ^ c));
      block_mac<MT, NB, GM, BF16, HAS_Z>(tot, a, r.wv, r.sraw, r.zraw, zshift, nm);
    } else {
      block_mac<MT, NB, GM, BF16, HAS_Z>(tot, r.a, r.wv, r.sraw, r.zraw, zshift, nm);
    }
  };
  if (has_blocks) {
    int kb = lo;
    for (; kb + D <= hi; kb += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const int nb = kb + u + D - 1;
        fill(nb < last ? nb : last, (u + D - 1) % D);
        if constexpr (AR != 0) {
          // block kb + u's activation tile has landed once at most the loads
          // of the D - 1 later fills are outstanding (loads complete in issue
          // order; the scheduling barriers keep the fills in block order and
          // each fill's direct-to-LDS loads come after its register loads)
          __builtin_amdgcn_sched_barrier(0);
          wait_vmcnt<(D - 1) * kPerBlock>();
        }
        compute(kb + u, u);
        if constexpr (AR != 0) __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int u = 0; u < D - 1; ++u)
      if (kb + u < hi) {
        if constexpr (AR != 0) wait_vmcnt<0>();
        compute(kb + u, u);
      }
  }

  // Sum the KW waves' partial results in LDS, then bias, round and store.
  if constexpr (XL) __syncthreads();  // every wave is done with the activation rows
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
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int e = threadIdx.x + q * 64 * KW;
    if (e >= R * 64) continue;
    const int rr = e >> 6, l = e & 63;
    const int i = rr / (NB * 4), s = (rr >> 2) % NB, r = rr & 3;
    const int64_t m = m0 + 16 * i + 4 * (l >> 4) + r;
    const int64_t n = (t0 + s) * kTileN + (l & 15);
    if (m < M && n < N) {  // n >= N: the padded half of the last strip
      float o = acc[q];
      if (bias != nullptr) o += act_to_f32<BF16>(bias[n]);
      y[m * N + n] = f32_to_act<BF16>(o);
    }
  }
}

// ---------------------------------------------------------------------------
// Wide kernel (M > 16: LDS-staged activations, pipelined over K)
//
// Workgroup: WN waves side by side.  Every wave owns the same BM = 16 MT rows
// and NS strips of its own, so the workgroup tile is 16 MT x 16 NS WN.  The
// dequantization of a strip is shared by the MT row tiles of the wave, so a
// tall wave tile keeps the vector ALU work per MFMA low.
//
// K is walked in 128-row blocks through an S-deep pipeline:
//   * the BM x 128 activation tile of block b sits in LDS slot b % S, written
//     by direct global->LDS loads (no registers): 16-byte chunk j of row r is
//     stored at chunk position j ^ (r % 16), so the 16 rows that one
//     A-operand read touches fall on distinct banks;
//   * the packed words, scales and zeros of block b sit in register slot
//     b % S of each wave.
// Iteration b waits until its own block has landed (the loads of the S - 2
// later blocks stay in flight), passes one barrier (every wave's part of the
// tile is visible, and every wave is done with slot (b - 1) % S), issues the
// loads of block b + S - 1 into that slot and computes block b.
//
// The wait is a vector-memory counter wait: at most kAfter = (S - 2) (NS + NA)
// loads may remain outstanding, where NS word loads and NA direct-to-LDS
// loads are issued per block by each wave.  The scale and zero loads of the
// later blocks are not counted, which only makes the count smaller than the
// number of loads truly issued after block b (the wait is never too short).
//
// Scaling uses one accumulator set per tile: at the start of scale period g
// the fp32 accumulator (which holds sum_{h<g} P_h s_h / s_{g-1}) is
// multiplied by s_{g-1} / s_g, the MFMAs then add the exact integer-weighted
// sums P_g of period g, and the result is multiplied by the last scale at
// the end.  The tile layout never stores a zero scale (the repack replaces
// it and zeroes the codes' contribution), so every ratio is finite; each
// multiply adds one fp32 rounding (relative 2^-24 per period).
// Rows >= M are staged from row M - 1 and never stored; strips >= N/16 read
// strip 0 and are never stored.
// ---------------------------------------------------------------------------

template <int MT, int NS, int WN, int S>
struct WideCfg {
  static constexpr int BM = 16 * MT;          // rows per workgroup tile
  static constexpr int BN = 16 * NS * WN;     // columns per workgroup tile
  static constexpr int NA = BM / (4 * WN);    // direct-to-LDS loads per wave per block
  static constexpr int kAfter = (S - 2) * (NS + NA);
  static_assert(NA >= 1 && NA * 4 * WN == BM, "the activation tile splits evenly over the waves");
  static_assert(S >= 2 && kAfter < 64, "pipeline depth");
};

// RSIN (bf16 only): the zero-point term's row sums come from rsum[pd][m]
// (fp32 sums of x over scale period pd, row_sums_bf16) instead of a ones-operand
// MFMA per row tile and step: each wave copies the tile's sums of block b into
// its own LDS area with direct-to-LDS loads in the same pipeline slot.
template <int MT, int NS, int WN, int S, int GM, bool BF16, bool HAS_Z, bool GROUPED, bool RSIN = false>
__global__ __launch_bounds__(64 * WN, 1) void gemm_wide(const uint16_t* __restrict__ x,
                                                          const u4* __restrict__ qw,
                                                          const uint16_t* __restrict__ sc,
                                                          const uint32_t* __restrict__ zs,
                                                          const uint16_t* __restrict__ bias,
                                                          uint16_t* __restrict__ y, float* __restrict__ part,
                                                          const int32_t* __restrict__ offs,
                                                          const float* __restrict__ rsum, int64_t M,
                                                          int64_t K, int64_t N, int G) {
  using C = WideCfg<MT, NS, WN, S>;
  constexpr int NP = Groups<GM>::kPeriods, SP = Groups<GM>::kSteps;
  constexpr int NA = C::NA;
  static_assert(!RSIN || (BF16 && !GROUPED), "row sums from memory: plain bf16 launches");
  // row-sum copies: per wave and period RW floats (the tile's BM rows, at
  // least one 64-lane load), NR direct-to-LDS loads of 4 bytes per block
  constexpr int RW = C::BM < 64 ? 64 : C::BM;
  constexpr int NR = RSIN ? NP * (RW / 64) : 0;
  constexpr int kAfter = (S - 2) * (NS + NA + NR);
  static_assert(kAfter < 64, "vmcnt is six bits");
  // One LDS array per pipeline slot (BM x 128 halves each).  Separate
  // objects let the compiler tell the slots apart: a read of slot u then
  // waits only for the direct-to-LDS loads into slot u, not for every such
  // load in flight.
  constexpr int kSlot = C::BM * kTileK, kNone = 8;
  __shared__ __attribute__((aligned(1024))) uint16_t lds0[kSlot];
  __shared__ __attribute__((aligned(1024))) uint16_t lds1[kSlot];
  __shared__ __attribute__((aligned(1024))) uint16_t lds2[S > 2 ? kSlot : kNone];
  __shared__ __attribute__((aligned(1024))) uint16_t lds3[S > 3 ? kSlot : kNone];
  __shared__ __attribute__((aligned(1024))) uint16_t lds4[S > 4 ? kSlot : kNone];
  __shared__ __attribute__((aligned(1024))) uint16_t lds5[S > 5 ? kSlot : kNone];
  __shared__ __attribute__((aligned(1024))) uint16_t lds6[S > 6 ? kSlot : kNone];
  __shared__ __attribute__((aligned(1024))) uint16_t lds7[S > 7 ? kSlot : kNone];
  static_assert(S <= 8, "at most eight LDS slots");
  constexpr int kRsSlot = RSIN ? WN * NP * RW : 1;
  __shared__ __attribute__((aligned(256))) float rsl0[kRsSlot];
  __shared__ __attribute__((aligned(256))) float rsl1[kRsSlot];
  __shared__ __attribute__((aligned(256))) float rsl2[S > 2 ? kRsSlot : 1];
  __shared__ __attribute__((aligned(256))) float rsl3[S > 3 ? kRsSlot : 1];
  __shared__ __attribute__((aligned(256))) float rsl4[S > 4 ? kRsSlot : 1];
  __shared__ __attribute__((aligned(256))) float rsl5[S > 5 ? kRsSlot : 1];
  __shared__ __attribute__((aligned(256))) float rsl6[S > 6 ? kRsSlot : 1];
  __shared__ __attribute__((aligned(256))) float rsl7[S > 7 ? kRsSlot : 1];
  auto slot_rs = [&](int u) __attribute__((always_inline)) -> float* {
    switch (u) {
      case 0: return rsl0;
      case 1: return rsl1;
      case 2: return rsl2;
      case 3: return rsl3;
      case 4: return rsl4;
      case 5: return rsl5;
      case 6: return rsl6;
      default: return rsl7;
    }
  };
  auto slot_lds = [&](int u) __attribute__((always_inline)) -> uint16_t* {
    switch (u) {
      case 0: return lds0;
      case 1: return lds1;
      case 2: return lds2;
      case 3: return lds3;
      case 4: return lds4;
      case 5: return lds5;
      case 6: return lds6;
      default: return lds7;
    }
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, quad = lane >> 4;
  const int64_t T = (N + kTileN - 1) / kTileN;  // strips; the last may be half padding
  const int64_t nblk = K / kTileK;
  // split-K: workgroup z of gridDim.z walks blocks [kb0, kb0 + nb) (nb >= 1:
  // the host never splits finer than one block)
  int64_t split = blockIdx.z, nsplit = gridDim.z;
  if constexpr (GROUPED) {
    // grouped (mixture-of-experts) launch: workgroup z serves expert z, whose
    // rows [offs[z], offs[z + 1]) of x and y are contiguous (clamped into the
    // M rows given) and whose tiled weights, scales, zeros and bias follow
    // those of the previous expert
    const int64_t e = blockIdx.z;
    int64_t r0 = offs[e], r1 = offs[e + 1];
    r0 = r0 < 0 ? 0 : (r0 > M ? M : r0);
    r1 = r1 < r0 ? r0 : (r1 > M ? M : r1);
    M = r1 - r0;
    x += r0 * K;
    y += r0 * N;
    qw += e * (K * T * kTileN / 32);
    sc += e * T * kTileN * G;
    if (HAS_Z) zs += e * T * 2 * G;
    if (bias != nullptr) bias += e * N;
    split = 0;
    nsplit = 1;
  }
  const int64_t kb0 = nblk * split / nsplit;
  const int64_t nb = nblk * (split + 1) / nsplit - kb0;
  const int64_t tw0 = ((int64_t)blockIdx.x * WN + wave) * NS;  // first strip of this wave
  const uint32_t zshift = 4u * (uint32_t)(c & 7);
  const NibbleMasks nm = NibbleMasks::make();

  // One row tile m0 .. m0 + BM - 1 (qwb, scb, zsb: the weight, scale and
  // zero bases)
  auto tile = [&](const int64_t m0, const u4* qwb, const uint16_t* scb, const uint32_t* zsb)
                  __attribute__((always_inline)) {
  // Operand addresses: a uniform base per strip (and per row tile for the
  // activations) plus a 32-bit per-lane byte offset, so the loads take the
  // scalar-base + vector-offset form.  Strips past the end read strip 0.
  const char* wb[NS];
  const char* sb[NS];
  const char* zb[NS];
#pragma unroll
  for (int nt = 0; nt < NS; ++nt) {
    const int64_t t = tw0 + nt;
    const int64_t tt = t < T ? t : 0;
    wb[nt] = reinterpret_cast<const char*>(qwb + tt * nblk * 64);
    sb[nt] = reinterpret_cast<const char*>(scb + tt * G * kTileN);
    zb[nt] = reinterpret_cast<const char*>(HAS_Z ? zsb + tt * G * 2 : zsb);
  }
  const uint32_t wo = (uint32_t)lane * (uint32_t)sizeof(u4);
  const uint32_t so = (uint32_t)c * (uint32_t)sizeof(uint16_t);
  const uint32_t zo = (uint32_t)(c >> 3) * (uint32_t)sizeof(uint32_t);
  // staging: load i of this wave fills rows 4 (NA wave + i) .. + 3 of the
  // tile; lane l lands at chunk position l % 16 of row base + l / 16 and so
  // loads logical chunk (l % 16) ^ (row % 16)
  const char* ab = reinterpret_cast<const char*>(x + m0 * K);
  uint32_t ao[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int row = 4 * (NA * wave + i) + quad;
    const int64_t r = m0 + row < M ? row : M - 1 - m0;
    ao[i] = (uint32_t)((r * K + 8 * (c ^ (row & 15))) * sizeof(uint16_t));
  }

  struct Slot {
    u4 w[NS];
    uint16_t s[NS][NP];
    uint32_t z[NS][NP];
  };
  Slot rg[S];

  auto issue = [&](int64_t b, Slot& r, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < NS; ++nt)
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint32_t g = (uint32_t)Groups<GM>::group((int)b, p);
        r.s[nt][p] = *reinterpret_cast<const uint16_t*>(sb[nt] + (so + g * (uint32_t)(kTileN * sizeof(uint16_t))));
        r.z[nt][p] = HAS_Z ? *reinterpret_cast<const uint32_t*>(zb[nt] + (zo + g * 8u)) : 0u;
      }
#pragma unroll
    for (int nt = 0; nt < NS; ++nt) r.w[nt] = *reinterpret_cast<const u4*>(wb[nt] + (wo + (uint32_t)b * 1024u));
#pragma unroll
    for (int i = 0; i < NA; ++i)
      load_lds16(reinterpret_cast<const uint16_t*>(ab + (ao[i] + (uint32_t)b * (uint32_t)(kTileK * sizeof(uint16_t)))),
                 slot_lds(slot) + 4 * (NA * wave + i) * kTileK);
    if constexpr (RSIN) {
      // lane l of load (p, h): the sum of row m0 + 64 h + l over period
      // b NP + p (rows past M read row M - 1; never used)
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int h = 0; h < RW / 64; ++h) {
          const int64_t row = m0 + 64 * h + lane;
          load_lds4(rsum + (b * NP + p) * M + (row < M ? row : M - 1),
                    slot_rs(slot) + (wave * NP + p) * RW + 64 * h);
        }
    }
  };

  f4 acc[MT][NS];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NS; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
  const u4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  // Both dtypes keep the exact integer operand: rounding (q - z) s to a
  // 16-bit weight would add an error per weight that, summed over a long K
  // (28672), exceeds the elementwise bound near outputs close to zero.
  float s_prev[NS];
#pragma unroll
  for (int nt = 0; nt < NS; ++nt) s_prev[nt] = 1.f;

  auto compute = [&](const Slot& r, int slot) __attribute__((always_inline)) {
    // row of this lane in tile i: 16 i + c, so row % 16 == c
    const uint16_t* xa = slot_lds(slot) + c * kTileK;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      uint32_t n1[NS], n2[NS];
      float nzz[NS];
#pragma unroll
      for (int nt = 0; nt < NS; ++nt) {
        const uint32_t z = HAS_Z ? (r.z[nt][p] >> zshift) & 0xFu : 8u;
        n1[nt] = nz1024_bits(z);
        n2[nt] = nz64_bits(z);
        nzz[nt] = -(128.0f + (float)z);
        const float s_cur = act_to_f32<BF16>(r.s[nt][p]);
        if constexpr (GM != GM_CH) {
          const float ratio = s_prev[nt] * __builtin_amdgcn_rcpf(s_cur);
#pragma unroll
          for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][nt][q] *= ratio;
        }
        s_prev[nt] = s_cur;
      }
      f4 rs[MT];
      if constexpr (RSIN) {
        // rows 16 i + 4 quad .. + 3 of the tile (this wave's copy)
        const float* rsp = slot_rs(slot) + (wave * NP + p) * RW + 4 * quad;
#pragma unroll
        for (int i = 0; i < MT; ++i) rs[i] = *reinterpret_cast<const f4*>(rsp + 16 * i);
      } else if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < MT; ++i) rs[i] = f4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = p * SP; j < (p + 1) * SP; ++j) {
        u4 a[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i)
          a[i] = *reinterpret_cast<const u4*>(xa + 16 * i * kTileK + 8 * ((4 * j + quad) ^ c));
        if constexpr (BF16 && !RSIN) {
#pragma unroll
          for (int i = 0; i < MT; ++i) rs[i] = mfma<true>(a[i], ones, rs[i]);
        }
#pragma unroll
        for (int nt = 0; nt < NS; ++nt) {
          u4 bq;
          if constexpr (BF16)
            bq = dq_bf16(r.w[nt][j], nm);
          else
            bq = dq_f16(r.w[nt][j], n1[nt], n2[nt], nm);
#pragma unroll
          for (int i = 0; i < MT; ++i) acc[i][nt] = mfma<BF16>(a[i], bq, acc[i][nt]);
        }
      }
      if constexpr (BF16) {
        // remove (128 + z) * sum_k x[m, k] of this period
#pragma unroll
        for (int nt = 0; nt < NS; ++nt)
#pragma unroll
          for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][nt][q] = __builtin_fmaf(nzz[nt], rs[i][q], acc[i][nt][q]);
      }
    }
  };

  // one pipeline iteration on block b, register/LDS slot U (compile time)
  // (called with compile-time slots only: every loop around it is fully
  // unrolled, so the slot arrays stay in registers)
  auto iterate = [&](int64_t b, int u) __attribute__((always_inline)) {
    const int un = (u + S - 1) % S;
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<kAfter>();
    lds_barrier();
    const int64_t bn = b + S - 1 < nb ? b + S - 1 : nb - 1;  // clamped: a redundant in-bounds load
    issue(kb0 + bn, rg[un], un);
    compute(rg[u], u);
  };

  // prologue: blocks 0 .. S - 2 of the range (clamped to its last block)
#pragma unroll
  for (int u = 0; u < S - 1; ++u) issue(kb0 + (u < nb ? u : nb - 1), rg[u], u);
  int64_t b = 0;
  for (; b + S <= nb; b += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) iterate(b + u, u);
  }
  // the last nb % S blocks
#pragma unroll
  for (int u = 0; u < S - 1; ++u)
    if (b + u < nb) iterate(b + u, u);

  // epilogue: lane holds column c of each strip, rows 4 quad + r of each tile;
  // with split-K the fp32 partial goes to part[z][m][n] (bias and rounding
  // happen in split_reduce)
  float* pz = part != nullptr ? part + split * M * N : nullptr;
#pragma unroll
  for (int nt = 0; nt < NS; ++nt) {
    const int64_t t = tw0 + nt;
    if (t >= T) continue;
    const int64_t n = t * kTileN + c;
    if (n >= N) continue;  // the padded half of the last strip
    const float bv = bias != nullptr && pz == nullptr ? act_to_f32<BF16>(bias[n]) : 0.f;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + 16 * i + 4 * quad + r;
        if (m >= M) continue;
        const float v = acc[i][nt][r] * s_prev[nt];
        if (pz != nullptr)
          pz[m * N + n] = v;
        else
          y[m * N + n] = f32_to_act<BF16>(v + bv);
      }
  }
  };

  if constexpr (GROUPED) {
    // A grouped launch walks every row tile of its expert in steps of
    // gridDim.y, so an expert with more rows than the launch height is
    // still computed whole (the loop bounds are uniform over the workgroup).
    // The weight bases pass through an opaque zero made inside the loop:
    // otherwise the compiler hoists the loop-invariant weight loads of the
    // pipeline prologue out of the loop, ahead of the activation loads,
    // and the counted vmcnt waits no longer cover the right loads.
    for (int64_t m0 = (int64_t)blockIdx.y * C::BM; m0 < M; m0 += (int64_t)gridDim.y * C::BM) {
      // (an element offset, not an integer round trip of the pointer, so the
      // loads stay global-memory loads)
      int64_t z0;
      asm volatile("s_mov_b64 %0, 0" : "=s"(z0));
      tile(m0, qw + z0, sc + z0, zs + z0);
      // the clamped prefetches of the last blocks may still be landing in
      // the LDS slots: drain them, and let every wave finish with the
      // slots, before the next row tile's prologue refills them
      wait_vmcnt<0>();
      lds_barrier();
    }
  } else {
    tile((int64_t)blockIdx.y * C::BM, qw, sc, zs);
  }
}

// y[m][n] = round(sum_z part[z][m][n] + bias[n]) for split-K launches; four
// consecutive columns per thread (N is a multiple of 16).
// SPLITS: the number of partial planes when known at compile time (all
// loads of an element are then in flight together); 0 reads `splits`.
template <bool BF16, int SPLITS>
__global__ void split_reduce(const float* __restrict__ part, const uint16_t* __restrict__ bias,
                             uint16_t* __restrict__ y, int64_t M, int64_t N, int splits) {
  const int64_t total4 = M * N / 4, plane4 = total4;
  const float4* p4 = reinterpret_cast<const float4*>(part);
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total4;
       idx += (int64_t)gridDim.x * blockDim.x) {
    float4 a;
    if constexpr (SPLITS > 0) {
      float4 v[SPLITS];
#pragma unroll
      for (int z = 0; z < SPLITS; ++z) v[z] = p4[z * plane4 + idx];
      a = v[0];
#pragma unroll
      for (int z = 1; z < SPLITS; ++z) {
        a.x += v[z].x;
        a.y += v[z].y;
        a.z += v[z].z;
        a.w += v[z].w;
      }
    } else {
      a = p4[idx];
      for (int z = 1; z < splits; ++z) {
        const float4 b = p4[z * plane4 + idx];
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
      }
    }
    const int64_t n = (idx * 4) % N;
    if (bias != nullptr) {
      a.x += act_to_f32<BF16>(bias[n]);
      a.y += act_to_f32<BF16>(bias[n + 1]);
      a.z += act_to_f32<BF16>(bias[n + 2]);
      a.w += act_to_f32<BF16>(bias[n + 3]);
    }
    const uint32_t lo = (uint32_t)f32_to_act<BF16>(a.x) | ((uint32_t)f32_to_act<BF16>(a.y) << 16);
    const uint32_t hi = (uint32_t)f32_to_act<BF16>(a.z) | ((uint32_t)f32_to_act<BF16>(a.w) << 16);
    uint32_t* y32 = reinterpret_cast<uint32_t*>(y) + 2 * idx;  // y is 4-byte aligned
    y32[0] = lo;
    y32[1] = hi;
  }
}

// xp[m][k] = k < K ? x[m][k] : 0 for k < Kp: the activations of a layer
// whose K is not a whole number of 128-row blocks, padded with zeros (the
// padded weight rows are zero too), eight halves per thread.
__global__ void pad_columns(const uint4* __restrict__ x, uint4* __restrict__ xp, int64_t M, int64_t K8,
                            int64_t Kp8) {
  const int64_t total = M * Kp8;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = idx / Kp8, k8 = idx - m * Kp8;
    xp[idx] = k8 < K8 ? x[m * K8 + k8] : make_uint4(0u, 0u, 0u, 0u);
  }
}

// x_perm[m][k'] = x[m][perm[k']]: the act-order activations of every path (perm entries
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

// The same gather, eight consecutive columns per thread: their perm entries
// in two 16-byte loads, one 16-byte store (K % 8 == 0; perm and xp 16-byte
// aligned).  Faster once there is work for many workgroups.
__global__ void gather_columns8(const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
                                uint16_t* __restrict__ xp, int64_t M, int64_t K) {
  const int64_t K8 = K / 8, total = M * K8;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = idx / K8, k8 = idx - m * K8;
    const int4 p0 = reinterpret_cast<const int4*>(perm)[2 * k8];
    const int4 p1 = reinterpret_cast<const int4*>(perm)[2 * k8 + 1];
    const uint32_t q[8] = {(uint32_t)p0.x, (uint32_t)p0.y, (uint32_t)p0.z, (uint32_t)p0.w,
                           (uint32_t)p1.x, (uint32_t)p1.y, (uint32_t)p1.z, (uint32_t)p1.w};
    const uint16_t* row = x + m * K;
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = row[q[e] < (uint32_t)K ? q[e] : 0u];
    reinterpret_cast<uint4*>(xp)[idx] =
        make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
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
  float* part;  // split-K partials [splits][M][N] (workspace), or nullptr
  int splits;   // K ranges (gridDim.z); 1 = no split
  const int32_t* offs;  // grouped launch: expert row offsets [groups + 1], or nullptr
  int groups;           // grouped launch: experts (gridDim.z)
  int64_t max_rows;     // grouped launch: rows of the largest expert (grid height)
  float* rsum;          // bf16 plain launches: workspace for the per-period row sums
                        // [K / L][M] (L = 128 / periods per block), or nullptr
  int64_t M, K, N;
  int G, gs;
};

// rs[pd][m] = sum of x[m][pd L .. pd L + L - 1] in fp32 (bf16 x): the
// zero-point term of the bf16 operand 128 + q, per scale period of L rows.
// One thread per (row, period); consecutive threads read consecutive
// periods of a row.
__global__ void row_sums_bf16(const uint16_t* __restrict__ x, float* __restrict__ rs, int64_t M, int64_t K,
                              int L) {
  const int64_t P = K / L, total = M * P;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = idx / P, pd = idx - m * P;
    const u4* src = reinterpret_cast<const u4*>(x + m * K + pd * L);
    float sum = 0.f;
    for (int c = 0; c < L / 8; ++c) {
      const u4 v = src[c];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) sum += bit_as<float>(w[h] << 16) + bit_as<float>(w[h] & 0xFFFF0000u);
    }
    rs[pd * M + m] = sum;
  }
}

// LDS bytes of a skinny launch: the reduction buffer, plus the staged
// activation rows (at most kXlRows, row stride K + kXPad halves) when XL.
constexpr size_t kMaxSkinnyLds = 128 * 1024;  // of the CU's 160 KiB

inline size_t skinny_lds_bytes(int mt, int nb, int kw, bool xl, int64_t M, int64_t K) {
  const size_t b = (size_t)kw * mt * nb * 4 * 64 * sizeof(float);
  if (!xl) return b;
  const size_t xb = (size_t)(M < kXlRows ? M : kXlRows) * (size_t)(K + kXPad) * sizeof(uint16_t);
  return b > xb ? b : xb;
}

// Ring depth of a skinny configuration (from timing sweeps): double
// buffering with LDS activations, where deeper rings measured slower; with
// the activations in registers, six blocks in flight for one strip and eight
// waves, three for sixteen waves or two strips.
template <int MT, int NB, int KW, bool XL>
constexpr int skinny_depth() {
  return XL ? 2 : (MT * NB == 1 ? (KW >= 16 ? 3 : 6) : (MT * NB == 2 ? 3 : 2));
}

template <int MT, int NB, int KW, int GM, bool BF16, bool HZ, bool XL, int D = skinny_depth<MT, NB, KW, XL>(),
          int AR = 0>
hipError_t run_skinny(const Args& a, hipStream_t st) {
  const int64_t T = (a.N + kTileN - 1) / kTileN;
  if (T % NB != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(T / NB), (unsigned)((a.M + 16 * MT - 1) / (16 * MT)));
  if (XL && a.M > kXlRows) return hipErrorInvalidValue;  // staging holds kXlRows rows
  const size_t lds = skinny_lds_bytes(MT, NB, KW, XL, a.M, a.K);
  if (lds > kMaxSkinnyLds) return hipErrorInvalidValue;
  // the AD ring is static LDS: D slots of KW 4 KiB copies, within the CU's 160 KiB with the rest
  constexpr size_t kAdBytes = (size_t)D * KW * AR * kTileK * sizeof(uint16_t);
  static_assert(kAdBytes + (size_t)KW * MT * NB * 4 * 64 * sizeof(float) <= 160 * 1024, "AD ring LDS");
  if (lds + kAdBytes > 160 * 1024) return hipErrorInvalidValue;
  if (lds > 64 * 1024) {
    // dynamic LDS beyond 64 KiB has to be allowed per kernel and device
    // (once each; devices past 64 are allowed on every call)
    static std::atomic<uint64_t> allowed{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev < 64 ? uint64_t(1) << dev : 0;
    if (bit == 0 || (allowed.load(std::memory_order_relaxed) & bit) == 0) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_skinny<MT, NB, KW, GM, BF16, HZ, XL, D, AR>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxSkinnyLds);
      if (e != hipSuccess) return e;
      allowed.fetch_or(bit, std::memory_order_relaxed);
    }
  }
  gemm_skinny<MT, NB, KW, GM, BF16, HZ, XL, D, AR><<<grid, 64 * KW, lds, st>>>(
      a.x, a.qw, a.sc, a.zs, a.bias, a.y, a.M, a.K, a.N, a.G);
  return hipGetLastError();
}

inline int group_mode(int gs, int64_t K) {
  if (gs == 32) return GM_32;
  if (gs == 64) return GM_64;
  if (gs == 128) return GM_128;
  return GM_CH;  // per-channel: one group of K rows
}

hipError_t launch_gather(const uint16_t* x, const int32_t* perm, uint16_t* xp, int64_t M, int64_t K, hipStream_t st) {
  const int64_t total = M * K;
  if (total / 8 >= 256 * 256) {
    // >= 256 workgroups of eight-column threads
    int64_t blocks = (total / 8 + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    gather_columns8<<<(unsigned)blocks, 256, 0, st>>>(x, perm, xp, M, K);
    return hipGetLastError();
  }
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  gather_columns<<<(unsigned)blocks, 256, 0, st>>>(x, perm, xp, M, K);
  return hipGetLastError();
}

template <int MT, int NS, int WN, int S, int GM, bool BF16, bool HZ, bool GR>
hipError_t run_wide(const Args& a, const uint16_t* x, hipStream_t st) {
  using C = WideCfg<MT, NS, WN, S>;
  const int64_t T = (a.N + kTileN - 1) / kTileN;
  const int splits = a.splits > 1 ? a.splits : 1;
  if (splits > 1 && (a.part == nullptr || splits > a.K / kTileK || a.offs != nullptr)) return hipErrorInvalidValue;
  const int64_t rows = a.offs != nullptr ? a.max_rows : a.M;
  const dim3 grid((unsigned)((T + NS * WN - 1) / (NS * WN)), (unsigned)((rows + C::BM - 1) / C::BM),
                  (unsigned)(a.offs != nullptr ? a.groups : splits));
  if (GR != (a.offs != nullptr)) return hipErrorInvalidValue;
  hipError_t e = hipSuccess;
  if constexpr (BF16 && !GR) {
    if (a.rsum != nullptr) {
      // the row sums of x per scale period first, then the kernel reads them
      const int L = kTileK / Groups<GM>::kPeriods;
      const int64_t total = a.M * (a.K / L);
      int64_t blocks = (total + 255) / 256;
      if (blocks > 65536) blocks = 65536;
      row_sums_bf16<<<(unsigned)blocks, 256, 0, st>>>(x, a.rsum, a.M, a.K, L);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      gemm_wide<MT, NS, WN, S, GM, BF16, HZ, GR, true><<<grid, 64 * WN, 0, st>>>(
          x, a.qw, a.sc, a.zs, a.bias, a.y, splits > 1 ? a.part : nullptr, a.offs, a.rsum, a.M, a.K, a.N, a.G);
    } else {
      gemm_wide<MT, NS, WN, S, GM, BF16, HZ, GR><<<grid, 64 * WN, 0, st>>>(
          x, a.qw, a.sc, a.zs, a.bias, a.y, splits > 1 ? a.part : nullptr, a.offs, nullptr, a.M, a.K, a.N, a.G);
    }
  } else {
    gemm_wide<MT, NS, WN, S, GM, BF16, HZ, GR><<<grid, 64 * WN, 0, st>>>(
        x, a.qw, a.sc, a.zs, a.bias, a.y, splits > 1 ? a.part : nullptr, a.offs, nullptr, a.M, a.K, a.N, a.G);
  }
  e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const int64_t total4 = a.M * a.N / 4;
  int64_t blocks = (total4 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  switch (splits) {
    case 2: split_reduce<BF16, 2><<<(unsigned)blocks, 256, 0, st>>>(a.part, a.bias, a.y, a.M, a.N, splits); break;
    case 4: split_reduce<BF16, 4><<<(unsigned)blocks, 256, 0, st>>>(a.part, a.bias, a.y, a.M, a.N, splits); break;
    case 8: split_reduce<BF16, 8><<<(unsigned)blocks, 256, 0, st>>>(a.part, a.bias, a.y, a.M, a.N, splits); break;
    default: split_reduce<BF16, 0><<<(unsigned)blocks, 256, 0, st>>>(a.part, a.bias, a.y, a.M, a.N, splits);
  }
  return hipGetLastError();
}

template <int MT, int NS, int WN, int S, bool BF16, bool HZ, bool GR>
hipError_t wide_gm(const Args& a, const uint16_t* x, hipStream_t st) {
  switch (group_mode(a.gs, a.K)) {
    case GM_32: return run_wide<MT, NS, WN, S, GM_32, BF16, HZ, GR>(a, x, st);
    case GM_64: return run_wide<MT, NS, WN, S, GM_64, BF16, HZ, GR>(a, x, st);
    case GM_128: return run_wide<MT, NS, WN, S, GM_128, BF16, HZ, GR>(a, x, st);
    default: return run_wide<MT, NS, WN, S, GM_CH, BF16, HZ, GR>(a, x, st);
  }
}

template <int MT, int NS, int WN, int S, bool GR>
hipError_t wide_flags(const Shape& s, const Args& a, const uint16_t* x, hipStream_t st) {
  if (s.bf16)
    return s.has_z ? wide_gm<MT, NS, WN, S, true, true, GR>(a, x, st)
                   : wide_gm<MT, NS, WN, S, true, false, GR>(a, x, st);
  return s.has_z ? wide_gm<MT, NS, WN, S, false, true, GR>(a, x, st)
                 : wide_gm<MT, NS, WN, S, false, false, GR>(a, x, st);
}

// Wide tile configurations: (MT, NS, WN, S) = row tiles per wave, strips per
// wave, waves per workgroup, pipeline depth, and the smallest M each is used
// for.  Chosen from timing sweeps of the prefill, mid-batch and act-order
// shapes on MI355X; largest tile first.  Prefill is bound by vector-ALU issue
// (dequantization plus the per-period rescale, ~4 VALU instructions per MFMA
// at 4 row tiles per wave), so its tile gives each wave 8 row tiles that
// share one dequantization of each strip.
struct WideChoice {
  int mt, ns, wn, st;
  int64_t min_m;
  const char* name;
};
constexpr WideChoice kWide[] = {
    {8, 2, 4, 2, 1024, "w4_wide_128x128"},
    {4, 4, 4, 3, 0, "w4_wide_64x256_s3"},
    {4, 2, 4, 4, 0, "w4_wide_64x128"},
    {2, 2, 4, 8, 0, "w4_wide_32x128"},
    {2, 2, 2, 8, 0, "w4_wide_32x64"},
    {2, 1, 2, 8, 0, "w4_wide_32x32"},
    // 16-row tiles: M <= 16 on wide layers and grouped (MoE) launches (below)
    {1, 1, 1, 8, 0, "w4_wide_16x16"},
    {1, 2, 1, 8, 0, "w4_wide_16x32"},
    {1, 1, 4, 8, 0, "w4_wide_16x64_w4"},
    {1, 1, 2, 6, 0, "w4_wide_16x32_w2"},
};
constexpr int kNumWide = 6;  // entries searched for M > 16
constexpr int kWide16x16 = 6, kWide16x32 = 7, kWide16x64w4 = 8, kWide16x32w2 = 9;

template <bool GR>
hipError_t wide_dispatch(int idx, const Shape& s, const Args& a, const uint16_t* x, hipStream_t st) {
  switch (idx) {
    case 0: return wide_flags<8, 2, 4, 2, GR>(s, a, x, st);
    case 1: return wide_flags<4, 4, 4, 3, GR>(s, a, x, st);
    case 2: return wide_flags<4, 2, 4, 4, GR>(s, a, x, st);
    case 3: return wide_flags<2, 2, 4, 8, GR>(s, a, x, st);
    case 4: return wide_flags<2, 2, 2, 8, GR>(s, a, x, st);
    case 5: return wide_flags<2, 1, 2, 8, GR>(s, a, x, st);
    case 6: return wide_flags<1, 1, 1, 8, GR>(s, a, x, st);
    case 7: return wide_flags<1, 2, 1, 8, GR>(s, a, x, st);
    case 8: return wide_flags<1, 1, 4, 8, GR>(s, a, x, st);
    default: return wide_flags<1, 1, 2, 6, GR>(s, a, x, st);
  }
}

}  // namespace
}  // namespace w4
