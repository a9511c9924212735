// INT4 weights x FP8 activations (W4A8-fp8) on gfx950.
//
// y = s_x * x_q W + bias, x_q = e4m3(clamp(x / s_x, +-448)) with a static
// per-tensor activation scale s_x, W[k, n] = (q - z[g(k), n]) s[g(k), n]
// (the W4AFp8 scheme of the SGLang quantization page, section 5, and the
// fp8-activation branch of the vLLM loading page, "Boundaries and failures").
//
// The weights keep the library's tile layout.  A 4-bit code written into a
// byte is the E4M3 value code * 2^-9 (codes 0..7 are the subnormals m 2^-9,
// 8..15 the exponent-1 values), so the B operand of the fp8 MFMA is the
// nibbles themselves, unpacked with two masks and a shift, and the MFMA's
// E8M0 scale of B (2^9) multiplies them back exactly: the 512 the pages
// apply to the scales.  The zero point is removed per group with the row
// sums of the quantized activations: the period sum of x_q (q - z) is
// P - z RS, with P the MFMA result and RS the row sum.
//
// v_mfma_scale_f32_16x16x128_f8f6f4 consumes 128 K values per instruction,
// exactly one group of 128 rows, so each block's product is one MFMA per
// 16 x 16 tile, folded into the fp32 total with the group's scale; per-channel
// layers accumulate all blocks in the MFMA and scale once.  Lane l supplies
// row (A) or column (B) l % 16 and 32 K values; lane l's B operand is its
// 16-byte chunk of the tile layout (column l % 16 at rows 32 j + 8 (l / 16) + e
// of the block, j = 0..3, K-offset e in nibble slot S[e], S = [0,4,1,5,2,6,3,7]),
// so the activations are quantized straight into that order ("operand
// order"): byte 32 q + 8 j + i of a 128-byte block holds column
// 32 j + 8 q + S[i] of the block.
#include "w4_kern.h"

namespace w4 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kE8m0One = 127;       // 2^0
constexpr int kE8m0Code = 127 + 9;  // 2^9: a code byte is worth code * 2^-9

__device__ __forceinline__ f4 mfma_f8(const v8i& a, const v8i& b, f4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, kE8m0One, 0, kE8m0Code);
}

// ---------------------------------------------------------------------------
// Activation quantization: one thread per 8 consecutive (sorted) columns.
// xq [M][Kp] in operand order; rs [Kp/128][Mr] fp32 block sums of the
// quantized values (the exact E4M3 values summed in fp32), Mr = M rounded up
// to a multiple of 4 (rows M .. Mr - 1 are zero); columns K .. Kp - 1 of a
// K tail are zero.
// ---------------------------------------------------------------------------
// VEC (no perm, K % 8 == 0, x 16-byte aligned): the 8 columns arrive in one
// 16-byte load; otherwise one 2-byte load per column.
template <bool BF16, bool PERM, bool VEC>
__global__ void quant_fp8(const uint16_t* __restrict__ x, const float* __restrict__ xscale,
                          const int32_t* __restrict__ perm, uint8_t* __restrict__ xq, float* __restrict__ rs,
                          int64_t M, int64_t Mr, int64_t K, int64_t Kp) {
  static_assert(!(VEC && PERM), "the gathered order has no contiguous 8-column chunks");
  const int64_t chunks = Kp / 8;  // per row; 16 per 128-column block
  const int64_t total = Mr * chunks;  // a multiple of 16
  const float s = xscale[0];
  // 16 consecutive threads cover one block of one row and leave the loop
  // together, so the block sum reduces inside a 16-lane group of a wave
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = idx / chunks, cc = idx - m * chunks;
    const int64_t k0 = 8 * cc;
    const uint16_t* row = x + m * K;
    // v[i]: column k0 + S[i] of the sorted order, S = [0,4,1,5,2,6,3,7]
    float v[8];
    if constexpr (VEC) {
      uint16_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (m < M && k0 < K) {
        const u4 raw = *reinterpret_cast<const u4*>(row + k0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          h[2 * j] = (uint16_t)(raw[j] & 0xFFFFu);
          h[2 * j + 1] = (uint16_t)(raw[j] >> 16);
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = (i & 1) ? 4 + (i >> 1) : (i >> 1);
        v[i] = act_to_f32<BF16>(h[j]) / s;  // IEEE fp32 division
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t k = k0 + ((i & 1) ? 4 + (i >> 1) : (i >> 1));
        v[i] = 0.f;
        if (m < M && k < K) {
          const uint32_t src = PERM ? (uint32_t)perm[k] : (uint32_t)k;
          v[i] = act_to_f32<BF16>(row[src < (uint32_t)K ? src : 0u]) / s;  // IEEE fp32 division
        }
      }
    }
    // codes two at a time (round to nearest even), four per 32-bit word
    uint32_t word[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      float c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = __builtin_fminf(__builtin_fmaxf(v[4 * w + i], -448.f), 448.f);
      const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
      word[w] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], lo, true);
    }
    // the exact E4M3 values, summed in the sorted order
    const int w0 = (int)word[0], w1 = (int)word[1];
    const float e[8] = {__builtin_amdgcn_cvt_f32_fp8(w0, 0), __builtin_amdgcn_cvt_f32_fp8(w0, 1),
                        __builtin_amdgcn_cvt_f32_fp8(w0, 2), __builtin_amdgcn_cvt_f32_fp8(w0, 3),
                        __builtin_amdgcn_cvt_f32_fp8(w1, 0), __builtin_amdgcn_cvt_f32_fp8(w1, 1),
                        __builtin_amdgcn_cvt_f32_fp8(w1, 2), __builtin_amdgcn_cvt_f32_fp8(w1, 3)};
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) sum += e[i];
    // operand order: chunk cc of its block -> (j, q) = (cc % 16 / 4, cc % 4)
    const int64_t b = cc / 16, c16 = cc % 16;
    if (m < M) *reinterpret_cast<uint2*>(xq + m * Kp + 128 * b + 32 * (c16 % 4) + 8 * (c16 / 4)) = make_uint2(word[0], word[1]);
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) sum += __shfl_xor(sum, d, 16);
    if (c16 == 0) rs[b * Mr + m] = sum;
  }
}

// ---------------------------------------------------------------------------
// Fused GEMM: WN waves side by side, each MT 16-row tiles x NS strips
// (workgroup tile 16 MT x 16 NS WN); K walked in 128-row blocks through an
// S-deep pipeline as in the wide kernel: the BM x 128-byte activation tile
// of block b in LDS slot b % S (direct global->LDS loads; 16-byte chunk c of
// row r at position c ^ swz(r), swz(r) = (r & 7) ^ ((r >> 3) & 1), so the 16
// rows one A read touches fall on distinct banks), the packed words, scales,
// zero words and row sums of block b in register slot b % S.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int MT, int NS, int WN, int S>
struct F8Cfg {
  static constexpr int BM = 16 * MT;
  static constexpr int BN = 16 * NS * WN;
  static constexpr int NA = BM * 128 / (1024 * WN);  // 1 KiB direct-to-LDS loads per wave per block
  static constexpr int kAfter = (S - 2) * (NS + NA);
  static_assert(NA >= 1 && NA * 1024 * WN == BM * 128, "the activation tile splits evenly over the waves");
  static_assert(S >= 2 && S <= 4 && kAfter < 64, "pipeline depth");
};

template <int MT, int NS, int WN, int S, bool PERCH, bool HAS_Z, bool BF16>
__global__ __launch_bounds__(64 * WN, 1) void gemm_f8(const uint8_t* __restrict__ xq, const float* __restrict__ rs,
                                                       const float* __restrict__ xscale,
                                                       const u4* __restrict__ qw, const uint16_t* __restrict__ sc,
                                                       const uint32_t* __restrict__ zs,
                                                       const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
                                                       int64_t M, int64_t Mr, int64_t K, int64_t N, int G) {
  using C = F8Cfg<MT, NS, WN, S>;
  constexpr int NA = C::NA;
  constexpr int kSlot = C::BM * 128, kNone = 16;
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kSlot];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kSlot];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[S > 2 ? kSlot : kNone];
  __shared__ __attribute__((aligned(1024))) uint8_t lds3[S > 3 ? kSlot : kNone];
  auto slot_lds = [&](int u) __attribute__((always_inline)) -> uint8_t* {
    switch (u) {
      case 0: return lds0;
      case 1: return lds1;
      case 2: return lds2;
      default: return lds3;
    }
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, quad = lane >> 4;
  const int64_t T = (N + kTileN - 1) / kTileN;
  const int64_t nblk = K / kTileK;
  const int64_t m0 = (int64_t)blockIdx.y * C::BM;
  const int64_t tw0 = ((int64_t)blockIdx.x * WN + wave) * NS;
  const uint32_t zshift = 4u * (uint32_t)(c & 7);

  // operand addresses: uniform bases (per strip, per row tile) plus 32-bit
  // per-lane byte offsets, so the loads take the scalar-base form; strips
  // past the end read strip 0
  const char* wb[NS];
  const char* sb[NS];
  const char* zb[NS];
#pragma unroll
  for (int nt = 0; nt < NS; ++nt) {
    const int64_t t = tw0 + nt;
    const int64_t tt = t < T ? t : 0;
    wb[nt] = reinterpret_cast<const char*>(qw + tt * nblk * 64);
    sb[nt] = reinterpret_cast<const char*>(sc + tt * G * kTileN);
    zb[nt] = reinterpret_cast<const char*>(HAS_Z ? zs + tt * G * 2 : zs);
  }
  const uint32_t wo = (uint32_t)lane * (uint32_t)sizeof(u4);
  const uint32_t so = (uint32_t)c * (uint32_t)sizeof(uint16_t);
  const uint32_t zo = (uint32_t)(c >> 3) * (uint32_t)sizeof(uint32_t);
  // staging: load i of this wave fills rows 8 (NA wave + i) .. + 7; lane l
  // lands at position l % 8 of row base + l / 8 and so loads logical chunk
  // (l % 8) ^ swz(row)
  const char* ab = reinterpret_cast<const char*>(xq + m0 * K);
  uint32_t ao[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int row = 8 * (NA * wave + i) + (lane >> 3);
    const int64_t r = m0 + row < M ? row : M - 1 - m0;
    ao[i] = (uint32_t)(r * K + 16 * ((lane & 7) ^ swz8(row)));
  }
  // the lane's four output rows of tile i: 16 i + 4 quad + 0..3 (their block
  // sums are one 16-byte load; groups of rows past Mr, never stored, read
  // the last group)
  uint32_t ro[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int64_t r = m0 + 16 * i + 4 * quad;
    ro[i] = (uint32_t)((r < Mr ? r : Mr - 4) * sizeof(float));
  }

  struct Slot {
    u4 w[NS];
    uint16_t s[NS];
    uint32_t z[NS];
    f4 rsum[MT];
  };
  Slot rg[S];

  auto issue = [&](int64_t b, Slot& r, int slot) __attribute__((always_inline)) {
    const uint32_t g = PERCH ? 0u : (uint32_t)b;
#pragma unroll
    for (int nt = 0; nt < NS; ++nt) {
      r.s[nt] = *reinterpret_cast<const uint16_t*>(sb[nt] + (so + g * (uint32_t)(kTileN * sizeof(uint16_t))));
      r.z[nt] = HAS_Z ? *reinterpret_cast<const uint32_t*>(zb[nt] + (zo + g * 8u)) : 0u;
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) r.rsum[i] = *reinterpret_cast<const f4*>(reinterpret_cast<const char*>(rs + b * Mr) + ro[i]);
#pragma unroll
    for (int nt = 0; nt < NS; ++nt) r.w[nt] = *reinterpret_cast<const u4*>(wb[nt] + (wo + (uint32_t)b * 1024u));
#pragma unroll
    for (int i = 0; i < NA; ++i)
      load_lds16(reinterpret_cast<const uint16_t*>(ab + (ao[i] + (uint32_t)b * 128u)),
                 reinterpret_cast<uint16_t*>(slot_lds(slot) + 8 * (NA * wave + i) * 128));
  };

  f4 tot[MT][NS];
  f4 rsacc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    rsacc[i] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NS; ++nt) tot[i][nt] = f4{0.f, 0.f, 0.f, 0.f};
  }

  auto compute = [&](const Slot& r, int slot) __attribute__((always_inline)) {
    const uint8_t* base = slot_lds(slot);
    // A: row 16 i + c of the tile, bytes 32 quad .. + 31 (chunks 2 quad, 2 quad + 1)
    v8i a[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int row = 16 * i + c;
      const uint8_t* rowp = base + row * 128;
      const u4 lo = *reinterpret_cast<const u4*>(rowp + 16 * ((2 * quad) ^ swz8(row)));
      const u4 hi = *reinterpret_cast<const u4*>(rowp + 16 * ((2 * quad + 1) ^ swz8(row)));
      a[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int nt = 0; nt < NS; ++nt) {
      // B: word j -> (w & 0x0F0F0F0F, (w >> 4) & 0x0F0F0F0F): the bytes of
      // K-offsets S[0..3] and S[4..7], in operand order
      v8i bq;
      const uint32_t w4[4] = {r.w[nt].x, r.w[nt].y, r.w[nt].z, r.w[nt].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bq[2 * j] = (int)(w4[j] & 0x0F0F0F0Fu);
        bq[2 * j + 1] = (int)((w4[j] >> 4) & 0x0F0F0F0Fu);
      }
      const float sf = act_to_f32<BF16>(r.s[nt]);
      const float z = HAS_Z ? (float)((r.z[nt] >> zshift) & 0xFu) : 8.f;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        if constexpr (PERCH) {
          tot[i][nt] = mfma_f8(a[i], bq, tot[i][nt]);
        } else {
          const f4 p = mfma_f8(a[i], bq, f4{0.f, 0.f, 0.f, 0.f});
          const float nsz = -sf * z;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            tot[i][nt][q] = __builtin_fmaf(sf, p[q], __builtin_fmaf(nsz, r.rsum[i][q], tot[i][nt][q]));
        }
      }
    }
    if constexpr (PERCH) {
#pragma unroll
      for (int i = 0; i < MT; ++i) rsacc[i] += r.rsum[i];
    }
  };

  auto iterate = [&](int64_t b, int u) __attribute__((always_inline)) {
    const int un = (u + S - 1) % S;
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<C::kAfter>();
    lds_barrier();
    const int64_t bn = b + S - 1 < nblk ? b + S - 1 : nblk - 1;
    issue(bn, rg[un], un);
    compute(rg[u], u);
  };

#pragma unroll
  for (int u = 0; u < S - 1; ++u) issue(u < nblk ? u : nblk - 1, rg[u], u);
  int64_t b = 0;
  for (; b + S <= nblk; b += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) iterate(b + u, u);
  }
#pragma unroll
  for (int u = 0; u < S - 1; ++u)
    if (b + u < nblk) iterate(b + u, u);

  const float sx = xscale[0];
#pragma unroll
  for (int nt = 0; nt < NS; ++nt) {
    const int64_t t = tw0 + nt;
    if (t >= T) continue;
    const int64_t n = t * kTileN + c;
    if (n >= N) continue;
    const float bv = bias != nullptr ? act_to_f32<BF16>(bias[n]) : 0.f;
    float s_ch = 1.f, z_ch = 0.f;
    if constexpr (PERCH) {
      s_ch = act_to_f32<BF16>(*reinterpret_cast<const uint16_t*>(sb[nt] + so));
      z_ch = HAS_Z ? (float)((*reinterpret_cast<const uint32_t*>(zb[nt] + zo) >> zshift) & 0xFu) : 8.f;
    }
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t m = m0 + 16 * i + 4 * quad + q;
        if (m >= M) continue;
        float v = tot[i][nt][q];
        if constexpr (PERCH) v = s_ch * (v - z_ch * rsacc[i][q]);
        y[m * N + n] = f32_to_act<BF16>(sx * v + bv);
      }
  }
}

// ---------------------------------------------------------------------------
// Decode kernel (M <= 16): one 16 x 16 output tile per workgroup, its KW
// waves splitting K into contiguous block ranges (as the W4A16 skinny
// kernel).  A wave loads each block's operands straight into registers --
// the lane's 32 activation bytes (row l % 16, bytes 32 (l / 16) .. + 31 of the
// block in operand order, 2 KiB per block: L2-resident), its 16 bytes of
// packed weights, the scale, the zero word and the four row sums -- through
// a D-deep ring (prefetch index clamped to the wave's last block, so the
// steady state has no branch), computes one fp8 MFMA per block and folds it
// into the fp32 total with the group's scale.  The KW partial tiles are
// summed in LDS in wave order (a fixed order: the result does not depend on
// timing).  Rows >= M read row M - 1 and are never stored.
// ---------------------------------------------------------------------------
template <int KW, int D, bool PERCH, bool HAS_Z, bool BF16, bool AD = false>
__global__ __launch_bounds__(64 * KW) void gemm_f8_skinny(const uint8_t* __restrict__ xq,
                                                           const float* __restrict__ rs,
                                                           const float* __restrict__ xscale,
                                                           const u4* __restrict__ qw, const uint16_t* __restrict__ sc,
                                                           const uint32_t* __restrict__ zs,
                                                           const uint16_t* __restrict__ bias,
                                                           uint16_t* __restrict__ y, int64_t M, int64_t Mr, int64_t K,
                                                           int64_t N, int G) {
  static_assert(D >= 2 && (!AD || D <= 6), "ring depth");
  static_assert(!AD || (D - 1) * 3 < 64, "vmcnt is six bits");
  constexpr int R = PERCH ? 8 : 4;  // partial tile (+ row-sum totals per channel)
  __shared__ float red[KW * R * 64];
  // AD: each wave copies every block's 16 x 128-byte activation tile into its
  // own slot of an LDS ring with two direct-to-LDS loads of eight whole rows
  // each (16-byte chunk j of row r at position j ^ swz8(r)); loaded straight
  // into registers, one A load touches 16 half-used cache lines
  constexpr int kAd = AD ? KW * 16 * 128 : 16;
  __shared__ __attribute__((aligned(1024))) uint8_t ad0[kAd];
  __shared__ __attribute__((aligned(1024))) uint8_t ad1[kAd];
  __shared__ __attribute__((aligned(1024))) uint8_t ad2[AD && D > 2 ? kAd : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t ad3[AD && D > 3 ? kAd : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t ad4[AD && D > 4 ? kAd : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t ad5[AD && D > 5 ? kAd : 16];
  auto slot_ad = [&](int u) __attribute__((always_inline)) -> uint8_t* {
    switch (u) {
      case 0: return ad0;
      case 1: return ad1;
      case 2: return ad2;
      case 3: return ad3;
      case 4: return ad4;
      default: return ad5;
    }
  };
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, quad = lane >> 4;
  const int64_t t = blockIdx.x;
  const int nblk = (int)(K / kTileK);
  const int lo = __builtin_amdgcn_readfirstlane((int)(((int64_t)nblk * wave) / KW));
  const int hi = __builtin_amdgcn_readfirstlane((int)(((int64_t)nblk * (wave + 1)) / KW));
  const uint32_t zshift = 4u * (uint32_t)(c & 7);

  const u4* wp = qw + t * nblk * 64 + lane;
  const uint16_t* sp = sc + t * G * kTileN + c;
  const uint32_t* zp = HAS_Z ? zs + t * G * 2 + (c >> 3) : nullptr;
  const int64_t m = c < M ? c : M - 1;
  const u4* ap = reinterpret_cast<const u4*>(xq + m * K + 32 * quad);
  const float* rp = rs + (4 * quad < Mr ? 4 * quad : Mr - 4);
  // AD: load i of a block fills rows 8 i .. 8 i + 7 of the wave's copy; lane l
  // lands at chunk position l % 8 of row 8 i + l / 8 and so loads logical
  // chunk (l % 8) ^ swz8(row) (rows >= M read row M - 1, never stored)
  const uint8_t* xd[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 8 * i + (lane >> 3);
    const int64_t mr = row < M ? row : M - 1;
    xd[i] = xq + mr * K + 16 * ((lane & 7) ^ swz8(row));
  }

  struct Blk {
    u4 w, a0, a1;
    f4 rsum;
    uint32_t z;
    uint16_t s;
  };
  auto load = [&](int b, Blk& r) __attribute__((always_inline)) {
    const int64_t g = PERCH ? 0 : b;
    r.w = wp[(int64_t)b * 64];
    r.s = sp[g * kTileN];
    r.z = HAS_Z ? zp[g * 2] : 0u;
    r.rsum = *reinterpret_cast<const f4*>(rp + (int64_t)b * Mr);
    if constexpr (!AD) {
      r.a0 = ap[(int64_t)b * 8];
      r.a1 = ap[(int64_t)b * 8 + 1];
    }
  };
  // the loads of block b into ring slot u, the activation copy last
  auto fill = [&](int b, Blk& r, int u) __attribute__((always_inline)) {
    load(b, r);
    if constexpr (AD) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        load_lds16(reinterpret_cast<const uint16_t*>(xd[i] + (int64_t)b * 128),
                   reinterpret_cast<uint16_t*>(slot_ad(u) + wave * 2048 + i * 1024));
    }
  };

  f4 tot = {0.f, 0.f, 0.f, 0.f}, rsacc = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const Blk& r, int u) __attribute__((always_inline)) {
    u4 a0 = r.a0, a1 = r.a1;
    if constexpr (AD) {
      // row c of the wave's copy, chunks 2 quad and 2 quad + 1
      const uint8_t* rowp = slot_ad(u) + wave * 2048 + c * 128;
      a0 = *reinterpret_cast<const u4*>(rowp + 16 * ((2 * quad) ^ swz8(c)));
      a1 = *reinterpret_cast<const u4*>(rowp + 16 * ((2 * quad + 1) ^ swz8(c)));
    }
    const v8i a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                   (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    const uint32_t w4[4] = {r.w.x, r.w.y, r.w.z, r.w.w};
    v8i bq;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bq[2 * j] = (int)(w4[j] & 0x0F0F0F0Fu);
      bq[2 * j + 1] = (int)((w4[j] >> 4) & 0x0F0F0F0Fu);
    }
    if constexpr (PERCH) {
      tot = mfma_f8(a, bq, tot);
      rsacc += r.rsum;
    } else {
      const float sf = act_to_f32<BF16>(r.s);
      const float z = HAS_Z ? (float)((r.z >> zshift) & 0xFu) : 8.f;
      const f4 p = mfma_f8(a, bq, f4{0.f, 0.f, 0.f, 0.f});
      const float nsz = -sf * z;
#pragma unroll
      for (int q = 0; q < 4; ++q) tot[q] = __builtin_fmaf(sf, p[q], __builtin_fmaf(nsz, r.rsum[q], tot[q]));
    }
  };

  if (lo < hi) {  // wave-uniform
    const int last = hi - 1;
    Blk ring[D];
#pragma unroll
    for (int u = 0; u < D - 1; ++u) {
      fill(lo + u < last ? lo + u : last, ring[u], u);
      if constexpr (AD) __builtin_amdgcn_sched_barrier(0);
    }
    int kb = lo;
    for (; kb + D <= hi; kb += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const int nb = kb + u + D - 1;
        fill(nb < last ? nb : last, ring[(u + D - 1) % D], (u + D - 1) % D);
        if constexpr (AD) {
          // block kb + u's copy has landed once at most the loads of the
          // D - 1 later fills are outstanding (a lower bound of 3 per fill:
          // the weight load and the two copies; fills stay in block order)
          __builtin_amdgcn_sched_barrier(0);
          wait_vmcnt<(D - 1) * 3>();
        }
        compute(ring[u], u);
        if constexpr (AD) __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int u = 0; u < D - 1; ++u)
      if (kb + u < hi) {
        if constexpr (AD) wait_vmcnt<0>();
        compute(ring[u], u);
      }
  }

#pragma unroll
  for (int q = 0; q < 4; ++q) {
    red[(wave * R + q) * 64 + lane] = tot[q];
    if constexpr (PERCH) red[(wave * R + 4 + q) * 64 + lane] = rsacc[q];
  }
  __syncthreads();
  if (wave != 0) return;
  const int64_t n = t * kTileN + c;
  if (n >= N) return;  // the padded half of the last strip
  const float sx = xscale[0];
  const float bv = bias != nullptr ? act_to_f32<BF16>(bias[n]) : 0.f;
  float s_ch = 1.f, z_ch = 0.f;
  if constexpr (PERCH) {
    s_ch = act_to_f32<BF16>(sp[0]);
    z_ch = HAS_Z ? (float)((zp[0] >> zshift) & 0xFu) : 8.f;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t mo = 4 * quad + q;
    if (mo >= M) continue;
    float v = 0.f, rsa = 0.f;
#pragma unroll
    for (int w = 0; w < KW; ++w) {
      v += red[(w * R + q) * 64 + lane];
      if constexpr (PERCH) rsa += red[(w * R + 4 + q) * 64 + lane];
    }
    if constexpr (PERCH) v = s_ch * (v - z_ch * rsa);
    y[mo * N + n] = f32_to_act<BF16>(sx * v + bv);
  }
}

template <int KW, int D, bool PERCH, bool HZ, bool BF16, bool AD>
hipError_t run_f8_skinny(const Shape& s, int64_t M, const uint8_t* xq, const float* rs, const float* xscale,
                         const int32_t* tw, const void* ts, const int32_t* tz, const void* bias, void* y,
                         hipStream_t st) {
  if (M < 1 || M > 16) return hipErrorInvalidValue;
  const int64_t T = s.Np / kTileN;
  gemm_f8_skinny<KW, D, PERCH, HZ, BF16, AD><<<(unsigned)T, 64 * KW, 0, st>>>(
      xq, rs, xscale, reinterpret_cast<const u4*>(tw), static_cast<const uint16_t*>(ts),
      reinterpret_cast<const uint32_t*>(tz), static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y), M,
      (int64_t)f8_rows(M), s.K, s.N, s.G);
  return hipGetLastError();
}

template <int KW, int D, bool AD = false>
hipError_t f8_skinny_flags(const Shape& s, int64_t M, const uint8_t* xq, const float* rs, const float* xscale,
                           const int32_t* tw, const void* ts, const int32_t* tz, const void* bias, void* y,
                           hipStream_t st) {
  const bool perch = s.Gp == 1;
#define W4_F8S(P, Z, B) run_f8_skinny<KW, D, P, Z, B, AD>(s, M, xq, rs, xscale, tw, ts, tz, bias, y, st)
  if (s.bf16) {
    if (perch) return s.has_z ? W4_F8S(true, true, true) : W4_F8S(true, false, true);
    return s.has_z ? W4_F8S(false, true, true) : W4_F8S(false, false, true);
  }
  if (perch) return s.has_z ? W4_F8S(true, true, false) : W4_F8S(true, false, false);
  return s.has_z ? W4_F8S(false, true, false) : W4_F8S(false, false, false);
#undef W4_F8S
}

template <int MT, int NS, int WN, int S, bool PERCH, bool HZ, bool BF16>
hipError_t run_f8(const Shape& s, int64_t M, const uint8_t* xq, const float* rs, const float* xscale,
                  const int32_t* tw, const void* ts, const int32_t* tz, const void* bias, void* y, hipStream_t st) {
  using C = F8Cfg<MT, NS, WN, S>;
  const int64_t T = s.Np / kTileN;
  const dim3 grid((unsigned)((T + NS * WN - 1) / (NS * WN)), (unsigned)((M + C::BM - 1) / C::BM));
  gemm_f8<MT, NS, WN, S, PERCH, HZ, BF16><<<grid, 64 * WN, 0, st>>>(
      xq, rs, xscale, reinterpret_cast<const u4*>(tw), static_cast<const uint16_t*>(ts),
      reinterpret_cast<const uint32_t*>(tz), static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y), M,
      (int64_t)f8_rows(M), s.K, s.N, s.G);
  return hipGetLastError();
}

template <int MT, int NS, int WN, int S>
hipError_t f8_flags(const Shape& s, int64_t M, const uint8_t* xq, const float* rs, const float* xscale,
                    const int32_t* tw, const void* ts, const int32_t* tz, const void* bias, void* y, hipStream_t st) {
  const bool perch = s.Gp == 1;
#define W4_F8(P, Z, B) run_f8<MT, NS, WN, S, P, Z, B>(s, M, xq, rs, xscale, tw, ts, tz, bias, y, st)
  if (s.bf16) {
    if (perch) return s.has_z ? W4_F8(true, true, true) : W4_F8(true, false, true);
    return s.has_z ? W4_F8(false, true, true) : W4_F8(false, false, true);
  }
  if (perch) return s.has_z ? W4_F8(true, true, false) : W4_F8(true, false, false);
  return s.has_z ? W4_F8(false, true, false) : W4_F8(false, false, false);
#undef W4_F8
}

}  // namespace

size_t f8_rows(int64_t M) { return (size_t)((M + 3) / 4 * 4); }

// Workspace of a W4A8 call: the quantized activations [M][Kp] (256-byte
// aligned), then the block row sums [Kp / 128][Mr] fp32.
size_t f8_xq_bytes(const Shape& s, int64_t M) { return ((size_t)M * (size_t)s.Kp + 255) / 256 * 256; }
size_t f8_workspace_bytes(const Shape& s, int64_t M) {
  return f8_xq_bytes(s, M) + (size_t)(s.Kp / kTileK) * f8_rows(M) * sizeof(float);
}

const char* f8_kernel_name(const Shape& s, int64_t M) {
  const int64_t T = s.Np / kTileN;
  if (M <= 4 && T <= 256) return s.K <= 4096 ? "w4a8_f8_skinny_k16" : "w4a8_f8_skinny_k16_r2";
  if (M <= 4 && T <= 1024) return "w4a8_f8_skinny_dma_k4";
  if (M <= 16 && T <= 256 && s.K <= 4096) return "w4a8_f8_skinny_dma_k16";
  if (M <= 16 && T <= 1024) return "w4a8_f8_skinny_dma_k8";
  if (M <= 16) return "w4a8_f8_16x16";
  if (M <= 128) return "w4a8_f8_64x128";
  return "w4a8_f8_64x256";
}

hipError_t launch_f8_quantize(const Shape& s, int64_t M, const void* x, const float* xscale, const int32_t* perm,
                              uint8_t* xq, float* rs, hipStream_t st) {
  // s: the unpadded shape (x rows are K long; xq rows are Kp long)
  const int64_t Mr = (int64_t)f8_rows(M);
  const int64_t total = Mr * (s.Kp / 8);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const uint16_t* xx = static_cast<const uint16_t*>(x);
  const bool vec = s.K % 8 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0;
#define W4_Q(B, P, V) quant_fp8<B, P, V><<<(unsigned)blocks, 256, 0, st>>>(xx, xscale, perm, xq, rs, M, Mr, s.K, s.Kp)
  if (s.bf16) {
    if (perm) W4_Q(true, true, false);
    else if (vec) W4_Q(true, false, true);
    else W4_Q(true, false, false);
  } else {
    if (perm) W4_Q(false, true, false);
    else if (vec) W4_Q(false, false, true);
    else W4_Q(false, false, false);
  }
#undef W4_Q
  return hipGetLastError();
}

hipError_t launch_f8_gemm(const Shape& s, int64_t M, const uint8_t* xq, const float* rs, const float* xscale,
                          const int32_t* tiled_w, const void* tiled_s, const int32_t* tiled_z, const void* bias,
                          void* y, hipStream_t st) {
  // Decode rows (M <= 16), from timing sweeps of the 7B-class decode layers:
  // up to 256 strips (N <= 4096), the K-split kernel (16 waves up to 4
  // rows); up to 1024 strips, the K-split kernel with 4 waves at M <= 4;
  // otherwise one wave walking all of K per 16 columns.  Prefill: 64 x 256 tiles of four waves (each 64 x 64), which
  // measured fastest among the 64- and 128-row shapes at 2048 and 8192 rows.
  // Above 4 rows the K-split kernels copy each block's activation tile into
  // LDS (whole rows per load): 13-19% faster at M = 16 than loading the
  // operands into registers.
  const int64_t T = s.Np / kTileN;
  if (M <= 4 && T <= 256) {
    // two blocks per wave at K = 4096 fit a 3-deep ring; longer K ran 6-7%
    // faster with a 2-deep one (11008 x 4096: 8.4 -> 7.8 us)
    if (s.K <= 4096) return f8_skinny_flags<16, 3>(s, M, xq, rs, xscale, tiled_w, tiled_s, tiled_z, bias, y, st);
    return f8_skinny_flags<16, 2>(s, M, xq, rs, xscale, tiled_w, tiled_s, tiled_z, bias, y, st);
  }
  if (M <= 4 && T <= 1024)  // four waves, activation tiles through LDS (4096 x 12288, M = 4: 9.8 -> 9.2 us)
    return f8_skinny_flags<4, 4, true>(s, M, xq, rs, xscale, tiled_w, tiled_s, tiled_z, bias, y, st);
  if (M <= 16 && T <= 256 && s.K <= 4096)
    return f8_skinny_flags<16, 3, true>(s, M, xq, rs, xscale, tiled_w, tiled_s, tiled_z, bias, y, st);
  if (M <= 16 && T <= 1024)
    return f8_skinny_flags<8, 3, true>(s, M, xq, rs, xscale, tiled_w, tiled_s, tiled_z, bias, y, st);
  if (M <= 16) return f8_flags<1, 1, 1, 4>(s, M, xq, rs, xscale, tiled_w, tiled_s, tiled_z, bias, y, st);
  if (M <= 128) return f8_flags<4, 2, 4, 3>(s, M, xq, rs, xscale, tiled_w, tiled_s, tiled_z, bias, y, st);
  return f8_flags<4, 4, 4, 2>(s, M, xq, rs, xscale, tiled_w, tiled_s, tiled_z, bias, y, st);
}

}  // namespace w4
