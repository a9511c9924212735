// Dense dequantization of a tiled layer (the unfused comparison path).
//
// W[k, n] = (q[k, n] - z[g(k), n]) * s[g(k), n], rounded once to the
// activation dtype, written row-major [K][N] in the original row order.  The
// pages' AWQ path switches, for large batches, from the fused kernel to
// "dequantize, then matmul" (vLLM AWQ practice page, section 5.3); this
// kernel is the first half of that unfused path, so the fused GEMM can be
// measured against it on this chip.  It is not used by w4a16_linear.
//
// One thread per lane-slice of a tiled block: the 16 bytes of lane l of
// block (t, b) hold column 16 t + l % 16, sorted rows
// 128 b + 32 j + 8 (l / 16) + e (j = 0..3, e = 0..7), K-offset e in nibble
// slot [0,4,1,5,2,6,3,7][e].  (q - z) is an integer of magnitude <= 15 and s
// has at most 11 significant bits, so the fp32 product is exact and the one
// rounding to fp16/bf16 is the only rounding.  Zero scales were replaced in
// the tile layout by a nonzero scale with codes equal to the zero point, so
// those weights come out as exact zeros.
#include "w4_internal.h"

namespace w4 {
namespace {

template <bool BF16>
__device__ __forceinline__ float act_f32(uint16_t bits) {
  if constexpr (BF16)
    return __builtin_bit_cast(float, (uint32_t)bits << 16);
  else
    return (float)__builtin_bit_cast(_Float16, bits);
}

template <bool BF16>
__device__ __forceinline__ uint16_t f32_act(float v) {
  if constexpr (BF16)
    return __builtin_bit_cast(uint16_t, (__bf16)v);
  else
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}

template <bool BF16, bool HAS_Z, bool HAS_PERM>
__global__ __launch_bounds__(256) void dequant_dense_kernel(const uint4* __restrict__ tw,
                                                              const uint16_t* __restrict__ ts,
                                                              const uint32_t* __restrict__ tz,
                                                              const int32_t* __restrict__ perm,
                                                              uint16_t* __restrict__ w, int64_t K, int64_t Kp,
                                                              int64_t N, int G, int gs) {
  // K, N: the layer; Kp, G, gs: the tile layout's padded rows and groups
  const int64_t nblk = Kp / kTileK;
  const int64_t total = ((N + kTileN - 1) / kTileN) * nblk * 64;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(idx & 63);
    const int64_t blk = idx >> 6;
    const int64_t t = blk / nblk, b = blk - t * nblk;
    const int c = lane & 15, quad = lane >> 4;
    const int64_t n = t * kTileN + c;
    if (n >= N) continue;  // the padded half of the last strip
    const uint4 v = tw[idx];
    const uint32_t words[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t k0 = b * kTileK + 32 * j + 8 * quad;  // sorted row of e = 0
      const int g = (int)(k0 / gs);                        // eight rows never straddle a group
      const float s = act_f32<BF16>(ts[(t * G + g) * kTileN + c]);
      const int z = HAS_Z ? (int)((tz[(t * G + g) * 2 + (c >> 3)] >> (4 * (c & 7))) & 0xFu) : 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t slot = (0x73625140u >> (4 * e)) & 0xFu;
        const int q = (int)((words[j] >> (4 * slot)) & 0xFu);
        const int64_t k = HAS_PERM ? (int64_t)perm[k0 + e] : k0 + e;
        if ((uint64_t)k >= (uint64_t)K) continue;  // a padded row, or a perm entry out of range: nothing written
        w[k * N + n] = f32_act<BF16>((float)(q - z) * s);
      }
    }
  }
}

template <bool BF16, bool HZ>
hipError_t launch_dq(const Shape& s, const uint4* tw, const uint16_t* ts, const uint32_t* tz, const int32_t* perm,
                     uint16_t* w, hipStream_t st) {
  const Shape p = padded_k(s);
  const int64_t total = (s.Np / kTileN) * (p.K / kTileK) * 64;
  int64_t blocks = (total + 255) / 256;
  if (blocks > (1 << 20)) blocks = 1 << 20;
  if (s.has_perm)
    dequant_dense_kernel<BF16, HZ, true><<<(unsigned)blocks, 256, 0, st>>>(tw, ts, tz, perm, w, s.K, p.K, s.N, p.G,
                                                                           p.gs);
  else
    dequant_dense_kernel<BF16, HZ, false><<<(unsigned)blocks, 256, 0, st>>>(tw, ts, tz, perm, w, s.K, p.K, s.N, p.G,
                                                                            p.gs);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant_dense(const Shape& s, const int32_t* tiled_w, const void* tiled_s, const int32_t* tiled_z,
                                const int32_t* perm, void* w, hipStream_t st) {
  const uint4* tw = reinterpret_cast<const uint4*>(tiled_w);
  const uint16_t* ts = static_cast<const uint16_t*>(tiled_s);
  const uint32_t* tz = reinterpret_cast<const uint32_t*>(tiled_z);
  uint16_t* out = static_cast<uint16_t*>(w);
  if (s.bf16) return s.has_z ? launch_dq<true, true>(s, tw, ts, tz, perm, out, st)
                             : launch_dq<true, false>(s, tw, ts, tz, perm, out, st);
  return s.has_z ? launch_dq<false, true>(s, tw, ts, tz, perm, out, st)
                 : launch_dq<false, false>(s, tw, ts, tz, perm, out, st);
}

}  // namespace w4
