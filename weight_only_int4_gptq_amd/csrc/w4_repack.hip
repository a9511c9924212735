// One-time weight re-layout kernels of libw4hip (gfx950).
//
//  * awq_to_std: AWQ words (eight output columns per word, logical column j
//    in nibble slot [0,4,1,5,2,6,3,7][j]; vLLM AWQ practice page, sections
//    5.1 and 5.3) -> standard words (eight input rows per word, row 8r+i in
//    slot i).  Each thread transposes one 8x8 nibble tile: it reads the 8
//    AWQ words of rows 8r..8r+7 at word column c and writes the 8 standard
//    words of columns 8c..8c+7 at row r (two 16-byte stores).
//  * actorder_perm: stable sort of the input rows by g_idx (GPTQ act-order,
//    loading page "Design motivation") by counting, one workgroup, with the
//    g_idx validation bits.
//  * tile_*: standard words / scales / zeros -> the gfx950 tile layout that
//    the GEMM kernels stream (layout stated in w4hip.h).
//
// All kernels are out-of-place, write every output element exactly once and
// use no atomics on global memory.
#include "w4_internal.h"

namespace w4 {
namespace {

__device__ __forceinline__ uint32_t awq_slot(int j) {
  // nibble slot of logical column j in an AWQ word
  return (0x73625140u >> (4 * j)) & 0xFu;
}

__device__ __forceinline__ uint32_t tile_slot(int e) {
  // nibble slot of K-offset e in a tiled word
  return (0x73625140u >> (4 * e)) & 0xFu;
}

__global__ void awq_to_std_weights(const uint32_t* __restrict__ aw, uint32_t* __restrict__ sw, int64_t K8,
                                   int64_t N8) {
  const int64_t total = K8 * N8;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = idx / N8, c = idx - r * N8;
    uint32_t in[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) in[i] = aw[(8 * r + i) * N8 + c];
    uint32_t out[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t sh = 4 * awq_slot(j);
      uint32_t v = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) v |= ((in[i] >> sh) & 0xFu) << (4 * i);
      out[j] = v;
    }
    uint4* dst = reinterpret_cast<uint4*>(sw + r * (8 * N8) + 8 * c);
    dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
    dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  }
}

__global__ void awq_to_std_zeros(const uint32_t* __restrict__ az, uint32_t* __restrict__ sz, int64_t total) {
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t w = az[idx];
    uint32_t v = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) v |= ((w >> (4 * awq_slot(j))) & 0xFu) << (4 * j);
    sz[idx] = v;
  }
}

// Single workgroup.  Phase 1 fills perm with the identity so that every
// entry is a valid row index whatever g_idx holds.  Phase 2: thread t owns
// groups t, t+1024, ...; g_idx is staged through LDS in chunks and each
// thread walks it in row order, so rows of one group keep their original
// order (stable).  A group that owns more than gs rows writes only gs of
// them.  status bit 0: entry outside [0, G); bit 1: a group size != gs.
constexpr int kPermThreads = 1024;
constexpr int kPermChunk = 8192;

__global__ __launch_bounds__(kPermThreads) void actorder_perm_kernel(const int32_t* __restrict__ g_idx,
                                                                     int32_t* __restrict__ perm,
                                                                     int32_t* __restrict__ status, int K, int G,
                                                                     int gs) {
  __shared__ int32_t chunk[kPermChunk];
  __shared__ int32_t st;
  const int tid = threadIdx.x;
  if (tid == 0) st = 0;
  for (int k = tid; k < K; k += kPermThreads) perm[k] = k;
  __syncthreads();

  int bad = 0;
  for (int k = tid; k < K; k += kPermThreads) {
    const int v = g_idx[k];
    if (v < 0 || v >= G) bad |= 1;
  }
  // Each thread handles up to kMaxGroupsPerThread groups per pass.
  constexpr int kMaxGroupsPerThread = 4;
  for (int gbase = 0; gbase < G; gbase += kPermThreads * kMaxGroupsPerThread) {
    int cnt[kMaxGroupsPerThread];
#pragma unroll
    for (int u = 0; u < kMaxGroupsPerThread; ++u) cnt[u] = 0;
    for (int k0 = 0; k0 < K; k0 += kPermChunk) {
      const int n = min(kPermChunk, K - k0);
      __syncthreads();
      for (int i = tid; i < n; i += kPermThreads) chunk[i] = g_idx[k0 + i];
      __syncthreads();
      for (int i = 0; i < n; ++i) {
        const int v = chunk[i];
#pragma unroll
        for (int u = 0; u < kMaxGroupsPerThread; ++u) {
          const int g = gbase + tid + u * kPermThreads;
          if (g < G && v == g) {
            if (cnt[u] < gs) perm[(int64_t)g * gs + cnt[u]] = k0 + i;
            ++cnt[u];
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kMaxGroupsPerThread; ++u) {
      const int g = gbase + tid + u * kPermThreads;
      if (g < G && cnt[u] != gs) bad |= 2;
    }
  }
  if (bad) atomicOr(&st, bad);
  __syncthreads();
  if (tid == 0 && status != nullptr) *status = st;
}

template <bool HAS_Z, bool HAS_PERM>
__global__ void tile_weights(const uint32_t* __restrict__ sw, const uint32_t* __restrict__ sz,
                             const uint16_t* __restrict__ scales, const int32_t* __restrict__ perm,
                             uint32_t* __restrict__ tw, int64_t K, int64_t Kp, int64_t N, int gs, int Gp) {
  // columns n >= N pad the last strip and rows k >= K (K % 128 != 0) pad the
  // last block: their codes equal their zero point (8, or the per-channel
  // zero point for padded rows of a per-channel layer; see tile_scales /
  // tile_zeros for the padded scales 1 and zero points 8), so the weight is 0
  const int64_t B = Kp / kTileK;
  const int64_t Np = (N + kTileN - 1) / kTileN * kTileN;
  const int64_t total = Kp * Np / 8;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(idx & 3);
    const int l = (int)((idx >> 2) & 63);
    const int64_t tb = idx >> 8;
    const int64_t t = tb / B, b = tb - t * B;
    const int64_t n = kTileN * t + (l & 15);
    const int64_t k0 = kTileK * b + 32 * j + 8 * (l >> 4);
    if (n >= N) {
      tw[idx] = 0x88888888u;
      continue;
    }
    if (k0 >= K) {
      // one group only (per-channel): the padded rows share its zero point
      const uint32_t z = HAS_Z && Gp == 1 ? (sz[n / 8] >> (4 * (n & 7))) & 0xFu : 8u;
      tw[idx] = z * 0x11111111u;
      continue;
    }
    const int64_t g = k0 / gs;
    const uint16_t sbits = scales[g * N + n];
    uint32_t word = 0;
    if ((sbits & 0x7FFFu) == 0) {
      const uint32_t z = HAS_Z ? (sz[g * (N / 8) + n / 8] >> (4 * (n & 7))) & 0xFu : 8u;
      word = z * 0x11111111u;
    } else if (!HAS_PERM) {
      const uint32_t src = sw[(k0 / 8) * N + n];
#pragma unroll
      for (int e = 0; e < 8; ++e) word |= ((src >> (4 * e)) & 0xFu) << (4 * tile_slot(e));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int64_t kk = perm[k0 + e];
        kk = (kk < 0 || kk >= K) ? 0 : kk;
        const uint32_t code = (sw[(kk / 8) * N + n] >> (4 * (kk & 7))) & 0xFu;
        word |= code << (4 * tile_slot(e));
      }
    }
    tw[idx] = word;
  }
}

// One thread per column: walks the groups in order so that a zero scale can
// take the previous group's stored scale.
__global__ void tile_scales(const uint16_t* __restrict__ s, uint16_t* __restrict__ ts, int64_t N, int G, int Gp,
                            uint16_t one_bits) {
  const int64_t Np = (N + kTileN - 1) / kTileN * kTileN;  // padded columns and groups get scale 1
  for (int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; n < Np; n += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = n / kTileN, c = n - t * kTileN;
    uint16_t prev = one_bits;
    for (int g = 0; g < Gp; ++g) {
      const uint16_t v = n < N && g < G ? s[(int64_t)g * N + n] : one_bits;
      const uint16_t out = (v & 0x7FFFu) == 0 ? prev : v;
      ts[(t * Gp + g) * kTileN + c] = out;
      prev = out;
    }
  }
}

// Tiled zero word (t, g, w) is the standard zero word [g, 2t + w] (eight
// padded columns, N % 16 == 8: zero points 8).
__global__ void tile_zeros(const uint32_t* __restrict__ sz, uint32_t* __restrict__ tz, int64_t N, int G, int Gp) {
  const int64_t T = (N + kTileN - 1) / kTileN;
  const int64_t total = T * Gp * 2;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int w = (int)(idx & 1);
    const int64_t tg = idx >> 1;
    const int64_t t = tg / Gp, g = tg - t * Gp;
    tz[idx] = 8 * (2 * t + w) < N && g < G ? sz[g * (N / 8) + 2 * t + w] : 0x88888888u;
  }
}

__global__ void write_zero_status(int32_t* __restrict__ status) {
  if (threadIdx.x == 0) *status = 0;
}

inline unsigned grid_for(int64_t total, int threads) {
  int64_t b = (total + threads - 1) / threads;
  if (b < 1) b = 1;
  if (b > 65536) b = 65536;
  return (unsigned)b;
}

}  // namespace

hipError_t launch_awq_to_std(const Shape& s, const int32_t* awq_w, const int32_t* awq_z, int32_t* std_w,
                             int32_t* std_z, hipStream_t st) {
  const int64_t K8 = s.K / 8, N8 = s.N / 8;
  awq_to_std_weights<<<grid_for(K8 * N8, 256), 256, 0, st>>>(reinterpret_cast<const uint32_t*>(awq_w),
                                                             reinterpret_cast<uint32_t*>(std_w), K8, N8);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nz = (int64_t)s.G * N8;
  awq_to_std_zeros<<<grid_for(nz, 256), 256, 0, st>>>(reinterpret_cast<const uint32_t*>(awq_z),
                                                      reinterpret_cast<uint32_t*>(std_z), nz);
  return hipGetLastError();
}

hipError_t launch_actorder_perm(const Shape& s, const int32_t* g_idx, int32_t* perm, int32_t* status,
                                hipStream_t st) {
  actorder_perm_kernel<<<1, kPermThreads, 0, st>>>(g_idx, perm, status, (int)s.K, s.G, s.gs);
  return hipGetLastError();
}

hipError_t launch_status_zero(int32_t* status, hipStream_t st) {
  write_zero_status<<<1, 64, 0, st>>>(status);
  return hipGetLastError();
}

hipError_t launch_tile(const Shape& s, const int32_t* std_w, const int32_t* std_z, const uint16_t* scales,
                       const int32_t* perm, int32_t* tiled_w, uint16_t* tiled_s, int32_t* tiled_z,
                       hipStream_t st) {
  const int64_t total = s.Kp * s.Np / 8;
  const unsigned grid = grid_for(total, 256);
  const uint32_t* sw = reinterpret_cast<const uint32_t*>(std_w);
  const uint32_t* sz = reinterpret_cast<const uint32_t*>(std_z);
  uint32_t* tw = reinterpret_cast<uint32_t*>(tiled_w);
  if (s.has_z && s.has_perm)
    tile_weights<true, true><<<grid, 256, 0, st>>>(sw, sz, scales, perm, tw, s.K, s.Kp, s.N, s.gs, s.Gp);
  else if (s.has_z)
    tile_weights<true, false><<<grid, 256, 0, st>>>(sw, sz, scales, perm, tw, s.K, s.Kp, s.N, s.gs, s.Gp);
  else if (s.has_perm)
    tile_weights<false, true><<<grid, 256, 0, st>>>(sw, sz, scales, perm, tw, s.K, s.Kp, s.N, s.gs, s.Gp);
  else
    tile_weights<false, false><<<grid, 256, 0, st>>>(sw, sz, scales, perm, tw, s.K, s.Kp, s.N, s.gs, s.Gp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  tile_scales<<<grid_for(s.Np, 256), 256, 0, st>>>(scales, tiled_s, s.N, s.G, s.Gp, s.bf16 ? 0x3F80 : 0x3C00);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (s.has_z) {
    tile_zeros<<<grid_for(s.Np / kTileN * s.Gp * 2, 256), 256, 0, st>>>(sz, reinterpret_cast<uint32_t*>(tiled_z),
                                                                        s.N, s.G, s.Gp);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace w4
