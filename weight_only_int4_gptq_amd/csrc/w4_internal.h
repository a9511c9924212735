// Internal declarations shared by the libw4hip translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "w4hip.h"

namespace w4 {

// Tile geometry of the kernel weight layout: a block is 16 output columns
// (one "strip") by 128 input rows, 1 KiB of packed codes; each of the 64
// lanes of a wave owns 16 contiguous bytes (4 words) of a block.
constexpr int kTileN = 16;
constexpr int kTileK = 128;
constexpr int kWordsPerBlock = kTileN * kTileK / 8;  // 256

struct Shape {
  int64_t K, N;
  int64_t Np;  // N padded to whole 16-column strips (the tile layout's column count)
  int64_t Kp;  // K padded to whole 128-row blocks (the tile layout's row count)
  int Gp;      // groups of the padded rows (G, plus the groups of rows K .. Kp-1)
  int gs;  // effective group size (K for per-channel)
  int G;   // number of groups
  bool bf16, has_z, has_perm;
};

inline Shape shape_of(const w4_layer* L) {
  Shape s;
  s.K = L->K;
  s.N = L->N;
  s.Np = (L->N + kTileN - 1) / kTileN * kTileN;
  s.Kp = (L->K + kTileK - 1) / kTileK * kTileK;
  s.gs = L->group_size == -1 ? (int)L->K : L->group_size;
  s.G = (int)(L->K / s.gs);
  s.Gp = L->group_size == -1 ? 1 : (int)(s.Kp / s.gs);
  s.bf16 = L->act_dtype == W4_BF16;
  s.has_z = L->has_zero_points != 0;
  s.has_perm = L->has_g_idx != 0;
  return s;
}

// The shape the GEMM kernels run: K and the groups padded to whole blocks
// (padded rows carry zero weights; activations are padded with zeros).
inline Shape padded_k(const Shape& s) {
  Shape p = s;
  p.K = s.Kp;
  p.G = s.Gp;
  if (s.Gp == 1) p.gs = (int)s.Kp;  // per-channel: one group of all rows
  return p;
}

// ---- host-side checks shared by the entry points (w4_api.cpp) ----
w4_status device_status();  // W4_OK on a gfx950 device, cached per device
// argument checks of a linear call (descriptor, M, pointers, alignment)
w4_status linear_checks(const w4_layer* L, int64_t M, const void* x, const int32_t* tiled_qweight,
                        const void* tiled_scales, const int32_t* tiled_qzeros, const int32_t* perm, const void* bias,
                        const void* y);

// ---- repack launchers (w4_repack.hip) ----
hipError_t launch_awq_to_std(const Shape& s, const int32_t* awq_w, const int32_t* awq_z, int32_t* std_w,
                             int32_t* std_z, hipStream_t st);
hipError_t launch_actorder_perm(const Shape& s, const int32_t* g_idx, int32_t* perm, int32_t* status,
                                hipStream_t st);
hipError_t launch_status_zero(int32_t* status, hipStream_t st);
hipError_t launch_tile(const Shape& s, const int32_t* std_w, const int32_t* std_z, const uint16_t* scales,
                       const int32_t* perm, int32_t* tiled_w, uint16_t* tiled_s, int32_t* tiled_z,
                       hipStream_t st);

// ---- GEMM (w4_gemm.hip) ----
enum class GemmKind { kSkinny, kWide, kBig };

struct GemmPlan {
  GemmKind kind;
  int mt;        // 16-row M tiles per wave (skinny kernel)
  int nb;        // strips per workgroup
  int kw;        // waves splitting K inside a workgroup
  bool xl;       // activations staged in LDS
  const char* name;
  int wide = 0;    // wide tile configuration (index into the kernel's table)
  int splits = 1;  // wide kernel: K ranges reduced by a second kernel (1 = none)
  bool rsin = false;  // bf16 wide kernel: row sums from a pre-pass instead of ones-operand MFMAs
  bool h16 = false;   // bf16 layer on the large-M kernel: exact fp16 copy of x from a pre-pass
  int ar = 0;         // skinny kernel: rows of each block's activation tile copied into LDS
                      // by direct-to-LDS loads (4 or 16; 0 = none)
};

// bf16_big: let bf16 layers take the large-M kernel (which needs an fp16
// copy of x in the workspace)
GemmPlan plan_gemm(const Shape& s, int64_t M, bool bf16_big = true);
// ws_cap: the most workspace the call can have.  A bf16 plan whose fp16 copy
// of x would not fit falls back to the wide kernel (whose row sums need
// M K / 32 bytes at most); the other plans are the same at any cap.
size_t gemm_workspace_bytes(const Shape& s, int64_t M, size_t ws_cap = SIZE_MAX);
void gemm_launch_dims(const Shape& s, int64_t M, unsigned grid[3], unsigned* threads);
hipError_t launch_gemm(const Shape& s, int64_t M, const void* x, const int32_t* tiled_w, const void* tiled_s,
                       const int32_t* tiled_z, const int32_t* perm, const void* bias, void* y, void* ws,
                       hipStream_t st, size_t ws_cap = SIZE_MAX);

// ---- large-M GEMM on 32x32x16 MFMA tiles (w4_big.hip) ----
int64_t big_tile_rows();
int64_t big_tile_cols();
int big_threads();
// bf16 layers need xh ([M][K] fp16) and rowf ([M] fp32) in the workspace for
// the exact fp16 copy of x the kernel runs on; fp16 layers ignore them
hipError_t launch_big(const Shape& s, int64_t M, const uint16_t* x, const int32_t* tiled_w, const void* tiled_s,
                      const int32_t* tiled_z, const void* bias, void* y, uint16_t* xh, float* rowf,
                      hipStream_t st);
// the bf16 part of launch_big (w4_big_h16.hip)
hipError_t launch_big_h16(const Shape& s, int64_t M, const uint16_t* x, const int32_t* tiled_w, const void* tiled_s,
                          const int32_t* tiled_z, const void* bias, void* y, uint16_t* xh, float* rowf,
                          hipStream_t st);
// grouped (mixture-of-experts) launch of the same kernel, fp16 only
hipError_t launch_big_moe(const Shape& s, int experts, int64_t total_rows, int64_t max_rows, const void* x,
                          const int32_t* offsets, const int32_t* tiled_w, const void* tiled_s,
                          const int32_t* tiled_z, const void* bias, void* y, hipStream_t st);

// ---- INT4 weights x FP8 activations (w4_fp8.hip); the GEMM takes the padded shape ----
size_t f8_rows(int64_t M);  // rows of the row-sum array (M rounded up to 4)
size_t f8_xq_bytes(const Shape& s, int64_t M);
size_t f8_workspace_bytes(const Shape& s, int64_t M);
const char* f8_kernel_name(const Shape& s, int64_t M);  // s: the padded shape
hipError_t launch_f8_quantize(const Shape& s_unpadded, int64_t M, const void* x, const float* xscale,
                              const int32_t* perm, uint8_t* xq, float* rs, hipStream_t st);
hipError_t launch_f8_gemm(const Shape& s, int64_t M, const uint8_t* xq, const float* rs, const float* xscale,
                          const int32_t* tiled_w, const void* tiled_s, const int32_t* tiled_z, const void* bias,
                          void* y, hipStream_t st);

// ---- grouped (mixture-of-experts) GEMM (w4_moe.hip) ----
GemmPlan plan_moe(const Shape& s, int64_t max_rows, int experts);
hipError_t launch_moe(const Shape& s, int experts, int64_t total_rows, int64_t max_rows, const void* x,
                      const int32_t* offsets, const int32_t* tiled_w, const void* tiled_s, const int32_t* tiled_z,
                      const void* bias, void* y, hipStream_t st);

// ---- dense dequantization, the unfused comparison path (w4_dequant.hip) ----
hipError_t launch_dequant_dense(const Shape& s, const int32_t* tiled_w, const void* tiled_s, const int32_t* tiled_z,
                                const int32_t* perm, void* w, hipStream_t st);

}  // namespace w4
