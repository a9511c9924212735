// libw4floor: comparison kernels for the memory-bound GEMM launches, built
// beside libw4hip but not part of it.  A decode-size GEMM streams a few to a
// few tens of MB; at that size the launch itself and the first memory
// latency are a large share of the time, so HBM peak alone says little about
// what a launch can reach.  These kernels give the two reference points on
// the GEMM's own grid:
//   w4floor_empty   a kernel that does nothing (launch and dispatch cost)
//   w4floor_stream  a plain streaming read of a byte count (every workgroup
//                   reads its contiguous share in 16-byte loads, eight per
//                   thread in flight, and keeps only an XOR of what it read)
// A GEMM that moves B algorithmic bytes can at best match w4floor_stream
// over B bytes on the same grid.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kInFlight = 8;

// TAG only makes the kernel name differ per caller-chosen case, so that a
// kernel trace tells the cases apart.
template <int TAG>
__global__ void stream_read(const uint4* __restrict__ src, uint64_t chunks, uint32_t* __restrict__ sink) {
  const uint64_t nwg = (uint64_t)gridDim.x * gridDim.y * gridDim.z;
  const uint64_t b = blockIdx.x + (uint64_t)gridDim.x * (blockIdx.y + (uint64_t)gridDim.y * blockIdx.z);
  const uint64_t lo = chunks * b / nwg, hi = chunks * (b + 1) / nwg;
  const uint64_t step = blockDim.x;
  uint32_t acc = 0;
  for (uint64_t i = lo + threadIdx.x; i < hi; i += kInFlight * step) {
    // unconditional loads (an index past the share re-reads chunk lo, which
    // is in bounds and cached), so all of them issue before the first use
    uint4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const uint64_t j = i + u * step;
      v[u] = src[j < hi ? j : lo];
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const uint32_t h = v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
      acc ^= (i + u * step < hi) ? h : 0u;
    }
  }
  // keeps the loads live; practically never taken (one word, vector store)
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

template <int TAG>
__global__ void empty_kernel() {}

constexpr int kTags = 16;

template <int T>
hipError_t stream_tag(int tag, dim3 g, unsigned threads, const uint4* src, uint64_t chunks, uint32_t* sink,
                      hipStream_t st) {
  if constexpr (T < kTags) {
    if (tag != T) return stream_tag<T + 1>(tag, g, threads, src, chunks, sink, st);
    stream_read<T><<<g, threads, 0, st>>>(src, chunks, sink);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <int T>
hipError_t empty_tag(int tag, dim3 g, unsigned threads, hipStream_t st) {
  if constexpr (T < kTags) {
    if (tag != T) return empty_tag<T + 1>(tag, g, threads, st);
    empty_kernel<T><<<g, threads, 0, st>>>();
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

bool dims_ok(const uint32_t* grid, uint32_t threads) {
  return grid != nullptr && grid[0] >= 1 && grid[1] >= 1 && grid[2] >= 1 && grid[1] <= 65535 &&
         grid[2] <= 65535 && threads >= 64 && threads <= 1024 && threads % 64 == 0;
}

}  // namespace

extern "C" {

// Streaming read of `bytes` bytes at `src` (device, 16-byte aligned, bytes a
// multiple of 16) on a grid[0] x grid[1] x grid[2] grid of `threads`-wide
// workgroups; `sink` is one device word that is written only if the XOR of
// the data equals a fixed constant.  tag in [0, 16) selects the kernel name
// (stream_read<tag>).  Returns a hipError_t value (0 = launched).
int w4floor_stream(const void* src, uint64_t bytes, const uint32_t* grid, uint32_t threads, uint32_t* sink, int tag,
                   void* stream) {
  if (src == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0 || (uintptr_t)src % 16 != 0 ||
      !dims_ok(grid, threads))
    return (int)hipErrorInvalidValue;
  return (int)stream_tag<0>(tag, dim3(grid[0], grid[1], grid[2]), threads, static_cast<const uint4*>(src), bytes / 16,
                            sink, static_cast<hipStream_t>(stream));
}

// An empty kernel on the same kind of grid (empty_kernel<tag>).
int w4floor_empty(const uint32_t* grid, uint32_t threads, int tag, void* stream) {
  if (!dims_ok(grid, threads)) return (int)hipErrorInvalidValue;
  return (int)empty_tag<0>(tag, dim3(grid[0], grid[1], grid[2]), threads, static_cast<hipStream_t>(stream));
}

}  // extern "C"
