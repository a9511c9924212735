/*
 * w4hip.h -- C ABI of libw4hip: weight-only INT4 group-quantized linear
 * layers (AWQ / GPTQ, W4A16) on AMD Instinct MI355X (gfx950).
 *
 * The calls follow the three-phase lifecycle of a quantized linear layer in
 * the vLLM / SGLang designs: create the parameters (here: validate the layer
 * and report buffer sizes; the caller allocates), post-process the weights
 * once after loading (AWQ -> standard repack, then standard -> kernel tile
 * repack), and apply the quantized GEMM on every forward pass.  See the
 * SGLang quantization design page, section 1 (three hooks), and the vLLM
 * "Quantized layer loading: AWQ / GPTQ / Marlin / fp8" page, sections
 * "Responsibilities" and "Data flow".
 *
 * Conventions for every call:
 *   - All buffers are owned by the caller.  The library never allocates or
 *     frees memory, keeps no per-layer state and is thread-safe.
 *   - Pointers named *_dev / weights / activations are device pointers;
 *     descriptor and size pointers are host pointers.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device work is enqueued asynchronously on it; no call synchronizes.
 *   - Arguments are validated on the host before any launch; an error
 *     return means nothing was enqueued.  W4_ERR_HIP means a launch failed.
 *   - Integers: int32 words hold eight 4-bit codes each ("packed words").
 *   - No C++ exception crosses this interface.
 */
#ifndef W4HIP_H
#define W4HIP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W4_OK = 0,
  W4_ERR_INVALID_ARGUMENT = 1, /* null / misaligned pointer, negative M, missing zeros or g_idx */
  W4_ERR_UNSUPPORTED = 2,      /* shape, group size, dtype or device the kernels do not handle */
  W4_ERR_WORKSPACE = 3,        /* workspace smaller than w4_workspace_size() */
  W4_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed */
} w4_status;

typedef enum { W4_FP16 = 0, W4_BF16 = 1 } w4_dtype;

/* Layer descriptor; the analogue of the MPLinearLayerConfig of the vLLM
 * "Quantized layer loading" page ("Design motivation"): weight shape, group
 * size, zero points, act-order, activation dtype.  4-bit weights only. */
typedef struct {
  int64_t K;               /* input features (rows of the weight)              */
  int64_t N;               /* output features (columns of the weight)          */
  int32_t group_size;      /* 32, 64, 128, or -1 = one group of K rows
                              (per-channel; "Boundaries and failures")        */
  int32_t has_zero_points; /* 0: symmetric, every zero point is 8              */
  int32_t has_g_idx;       /* 1: GPTQ act-order, a g_idx[K] gives each row's group */
  int32_t act_dtype;       /* w4_dtype of x, scales, bias and y               */
} w4_layer;

/* Byte sizes of the buffers of one layer (host-side arithmetic only). */
typedef struct {
  size_t awq_qweight;   /* int32 [K][N/8]   AWQ qweight (packed along N)          */
  size_t qzeros;        /* int32 [G][N/8]   AWQ or standard zero words (0 if none) */
  size_t scales;        /* act   [G][N]     scales as loaded                       */
  size_t std_qweight;   /* int32 [K/8][N]   standard qweight (packed along K)      */
  size_t tiled_qweight; /* int32 Kp*Np/8    tile layout (see w4_repack_gptq)       */
  size_t tiled_scales;  /* act   [Np/16][Gp][16]                                    */
  size_t tiled_qzeros;  /* int32 [Np/16][Gp][2] (0 if no zero points)              */
  /* Np = N rounded up to a multiple of 16 (the tile layout pads a last half
   * strip when N % 16 == 8); Kp = K rounded up to a multiple of 128 (padded
   * rows when K % 128 != 0); Gp = Kp / group_size (1 for group_size -1) */
  size_t perm;          /* int32 [K] act-order row permutation (0 without g_idx)   */
} w4_sizes_t;

/* Validate a layer descriptor (analogue of the support check that raises in
 * the vLLM "Boundaries and failures" section).  Returns
 *   W4_ERR_INVALID_ARGUMENT  layer == NULL, K <= 0, N <= 0;
 *   W4_ERR_UNSUPPORTED       group_size not in {-1, 32, 64, 128} (the group
 *                            sizes listed in section 5.3 of the vLLM AWQ
 *                            practice page), K % 32 != 0, N % 8 != 0,
 *                            K % group_size != 0, K % 128 != 0 with
 *                            group_size 128 or act-order (a K tail is
 *                            padded to whole 128-row blocks, which needs
 *                            whole groups and the natural row order),
 *                            act_dtype not fp16/bf16,
 *                            has_g_idx with group_size == -1, K > 2^20 or
 *                            N > 2^20.
 * Host only; never touches the GPU. */
w4_status w4_check_layer(const w4_layer* layer);

/* Fill *out with the byte sizes of the layer's buffers.  Host only. */
w4_status w4_sizes(const w4_layer* layer, w4_sizes_t* out);

/* Bytes of scratch device memory w4a16_linear needs for M rows, in
 * 256-byte-aligned parts: the activations gathered through perm (act-order,
 * M K 2 bytes) or zero-padded to whole 128-row blocks (K tails); split-K
 * fp32 partials [splits][M][N] (16 < M <= 256 on layers with N <= 16384);
 * for bf16 on the wide kernel from M = 256 (M = 64 on layers with
 * K >= 16384 or N > 16384), fp32 row sums of x per scale period [Kp / L][M]
 * (L = the group size, at most 128); and for bf16 on the large-M kernel
 * (at least 256 tiles of 128 x 256 outputs), an fp16 copy of x [M][Kp] and
 * fp32 row factors [M].  0 when none applies (fp16 with K % 128 == 0 and no
 * act-order outside the split-K range, for instance).  Host only. */
w4_status w4_workspace_size(const w4_layer* layer, int64_t M, size_t* bytes);

/* Name of the kernel w4a16_linear launches for M rows (the analogue of the
 * "Using ... kernel" log line of the vLLM learning-book page, Q1), or
 * "invalid" for a bad descriptor.  Static string; host only. */
const char* w4_kernel_name(const w4_layer* layer, int64_t M);

/* Launch dimensions of the GEMM kernel that w4a16_linear runs for M >= 1
 * rows (the kernel w4_kernel_name names): grid[0..2] workgroups along x, y,
 * z and *threads work-items per workgroup.  The act-order gather, K-tail
 * padding and split-K reduction launches are not included.  For sizing
 * comparison launches (a streaming-read or empty kernel on the same grid).
 * Host only; W4_ERR_INVALID_ARGUMENT for M < 1 or NULL outputs. */
w4_status w4_launch_dims(const w4_layer* layer, int64_t M, uint32_t grid[3], uint32_t* threads);

/* Static description of a status code. */
const char* w4_status_str(w4_status s);

/* AWQ -> standard repack (the vLLM AWQ practice page, section 5.1; the
 * "Design motivation" section of the loading page).  Each AWQ word holds
 * eight output columns, logical column j in nibble slot R[j] with
 * R = [0,4,1,5,2,6,3,7]; the output packs eight input rows per word along K
 * in the standard order (row 8r+i in slot i).
 *   awq_qweight  int32 [K][N/8]  (device, 4-byte aligned)
 *   awq_qzeros   int32 [G][N/8]  (device; AWQ always carries zero points)
 *   std_qweight  int32 [K/8][N]  (device, 16-byte aligned) -- written
 *   std_qzeros   int32 [G][N/8]  (device) -- written: same shape, standard
 *                nibble order (column 8c+i in slot i)
 * Out-of-place and re-runnable (a weight update re-runs it).  Requires
 * layer->has_zero_points and !layer->has_g_idx; otherwise
 * W4_ERR_UNSUPPORTED.  Bit-exact. */
w4_status w4_repack_awq(const w4_layer* layer, const int32_t* awq_qweight, const int32_t* awq_qzeros,
                        int32_t* std_qweight, int32_t* std_qzeros, void* stream);

/* Standard -> gfx950 tile repack (the kernel-specific re-layout of the
 * loading page's "Key files" / "Data flow"; act-order g_idx from its
 * "Design motivation").
 *   std_qweight    int32 [K/8][N]      (device)
 *   std_qzeros     int32 [G][N/8]      (device; NULL iff !has_zero_points)
 *   scales         act   [G][N]        (device)
 *   g_idx          int32 [K]           (device; NULL iff !has_g_idx)
 *   tiled_qweight  int32 [Kp*Np/8]     (device, 16-byte aligned) -- written
 *   tiled_scales   act   [Np/16][Gp][16] (device) -- written
 *   tiled_qzeros   int32 [Np/16][Gp][2] (device; NULL iff !has_zero_points) -- written
 *   perm           int32 [K]           (device; NULL iff !has_g_idx) -- written
 *   status_dev     int32 [1]           (device; may be NULL) -- written:
 *                  bit 0 = a g_idx entry outside [0, G); bit 1 = some group
 *                  does not own exactly group_size rows.  A nonzero status
 *                  means the tiled buffers are not valid for w4a16_linear.
 *                  perm always holds indices in [0, K).
 * Layout (bit-exact): with act-order, rows are sorted stably by group
 * (perm[k'] = original row of sorted row k'); a scale equal to zero is
 * replaced by the previous group's stored scale (1.0 for group 0) and the
 * codes of that group and column by its zero point; word [t][b][l][j]
 * (t < Np/16, b < Kp/128, l < 64, j < 4) holds column 16t + l%16 at sorted
 * rows 128b + 32j + 8(l/16) + e, e = 0..7, K-offset e in nibble slot
 * [0,4,1,5,2,6,3,7][e].  Columns N .. Np-1 (a padded half strip) hold codes
 * and zero points 8 and scale 1: their weights are 0 and no output column
 * is written for them.  Rows K .. Kp-1 (a padded last block) hold codes
 * equal to their zero point: the layer's zero point with group_size -1,
 * else 8 in the padded groups G .. Gp-1, whose scales are 1 and zero
 * points 8; their weights are 0. */
w4_status w4_repack_gptq(const w4_layer* layer, const int32_t* std_qweight, const int32_t* std_qzeros,
                         const void* scales, const int32_t* g_idx, int32_t* tiled_qweight,
                         void* tiled_scales, int32_t* tiled_qzeros, int32_t* perm, int32_t* status_dev,
                         void* stream);

/* y = x * W + bias with W[k][n] = (q[k][n] - z[g(k)][n]) * s[g(k)][n]
 * (dequantization of the vLLM AWQ practice page, section 5.3, fused into
 * the GEMM as in the learning-book page, section 5.3), for the tiled
 * buffers written by w4_repack_gptq.  fp32 accumulation; y rounded once
 * (round to nearest even) to the activation dtype.
 *   M              rows of x and y (M == 0: no launch, W4_OK)
 *   x              act [M][K] row-major (device, 16-byte aligned)
 *   tiled_qweight, tiled_scales, tiled_qzeros (NULL iff !has_zero_points),
 *   perm (NULL iff !has_g_idx): as written by w4_repack_gptq
 *   bias           act [N] (device) or NULL
 *   y              act [M][N] row-major (device, 4-byte aligned) -- written
 *   workspace      device scratch of >= w4_workspace_size() bytes (16-byte
 *                  aligned), or NULL when that size is 0; no initialization
 *                  needed.  With act-order it receives x with its columns
 *                  gathered through perm; with K % 128 != 0, x padded with
 *                  zero columns to Kp; for 16 < M <= 256 on layers with
 *                  N <= 16384 it also holds the fp32 split-K partials
 *                  [splits][M][N]; for bf16 the row sums or the fp16 copy
 *                  of x (w4_workspace_size).  Calls that overlap in time
 *                  must not share a workspace.
 * Accuracy: within max|y - ref| <= 1e-2 (1 + |ref|) elementwise and
 * relative Frobenius error <= 2e-3 of the float64 reference. */
w4_status w4a16_linear(const w4_layer* layer, int64_t M, const void* x, const int32_t* tiled_qweight,
                       const void* tiled_scales, const int32_t* tiled_qzeros, const int32_t* perm,
                       const void* bias, void* y, void* workspace, size_t workspace_bytes, void* stream);

/* w4a16_linear for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, result and accuracy as w4a16_linear without the workspace
 * pair: the workspace is a static device array of
 * w4_noalloc_scratch_bytes() bytes (64 MiB), one per device, held until the
 * process ends.  The call allocates nothing; its first call on a device
 * resolves that device's array address (hipGetSymbolAddress) with the device
 * current, so make the first call outside graph capture.
 *   W4_ERR_WORKSPACE  the call needs more than w4_noalloc_scratch_bytes()
 *                     (w4_workspace_size() tells how much it needs)
 * A bf16 call whose large-M kernel would need an fp16 copy of x larger than
 * the array runs the wide kernel instead (within the same accuracy bound;
 * its row sums need M K / 32 bytes at most), so only that call's kernel can
 * differ from w4a16_linear's.
 * Every call on a device shares that device's array, which keeps the last
 * call's contents (nothing in it needs to start at zero): calls that overlap
 * in time on one device race, whatever their streams. */
w4_status w4a16_linear_noalloc(const w4_layer* layer, int64_t M, const void* x, const int32_t* tiled_qweight,
                               const void* tiled_scales, const int32_t* tiled_qzeros, const int32_t* perm,
                               const void* bias, void* y, void* stream);

/* Bytes of the static workspace array of w4a16_linear_noalloc.  Host only. */
size_t w4_noalloc_scratch_bytes(void);

/* Grouped W4A16 linear for mixture-of-experts layers (the WNA16 MoE path of
 * the vLLM AWQ practice page, section 5.4, and of the SGLang quantization
 * page's MoE section): num_experts experts share one w4_layer description
 * (K, N, group size, zero points, dtype; act-order and K % 128 != 0 are
 * not supported and return W4_ERR_UNSUPPORTED), each with its own tiled weights, and
 *   y[r] = x[r] W_e (+ bias_e)   for every row r of expert e.
 *   x              act [total_rows][K] row-major (device, 16-byte aligned):
 *                  the rows routed to each expert, grouped by expert (the
 *                  routing and the gather/scatter of tokens belong to the
 *                  caller)
 *   expert_offsets int32 [num_experts + 1] (device): expert e owns rows
 *                  [expert_offsets[e], expert_offsets[e + 1]); nondecreasing,
 *                  from 0 to total_rows.  Entries are clamped into
 *                  [0, total_rows] (bad offsets give wrong rows, never an
 *                  access outside x or y).
 *   max_rows       host estimate of the rows of the largest expert, or 0 for
 *                  total_rows.  It sizes the launch only: every row of every
 *                  expert is computed whatever its value (workgroups walk
 *                  further row tiles when an expert has more rows), so a
 *                  low estimate costs time, never rows.
 *   tiled_qweight, tiled_scales, tiled_qzeros
 *                  the num_experts per-expert buffers of w4_repack_gptq,
 *                  each exactly w4_sizes() bytes, stacked in expert order
 *   bias           act [num_experts][N] or NULL
 *   y              act [total_rows][N] row-major (device) -- written
 * Asynchronous on `stream`; no workspace.  Accuracy as for w4a16_linear. */
w4_status w4a16_moe_linear(const w4_layer* layer, int32_t num_experts, int64_t total_rows, int64_t max_rows,
                           const void* x, const int32_t* expert_offsets, const int32_t* tiled_qweight,
                           const void* tiled_scales, const int32_t* tiled_qzeros, const void* bias, void* y,
                           void* stream);

/* ---- INT4 weights x FP8 activations (W4A8-fp8) ----
 * The W4AFp8 scheme of the SGLang quantization page (section 5: int4
 * weights, one scale per group of 128, fp8 activations with a static input
 * scale) and the fp8-activation branch of the vLLM loading page ("Boundaries
 * and failures": weights preprocessed for float8_e4m3fn activations, scales
 * times 512).  The weights are the tiled buffers of w4_repack_gptq (group
 * size 128 or -1; 32 and 64 return W4_ERR_UNSUPPORTED); the activations are
 * quantized per tensor:
 *   x_q = e4m3(clamp(x / s_x, -448, 448)),  x / s_x in fp32, round to
 *         nearest even, E4M3 = float8_e4m3fn (bias 7, largest 448)
 *   y   = s_x * x_q W + bias,  W[k][n] = (q - z) s as for w4a16_linear
 * computed with the fp8 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4): a 4-bit
 * code written into a byte is the E4M3 value code / 512, and the MFMA's
 * power-of-two block scale of the weight operand restores the 512 exactly. */

/* Quantize activations x [M][K] (act dtype, device) with the scale
 * x_scale[0] (fp32, device) into
 *   xq      uint8 [M][Kp] (device, 8-byte aligned): E4M3 codes in operand
 *           order: byte 32 q + 8 j + i of 128-byte block b of row m holds
 *           column 128 b + 32 j + 8 q + [0,4,1,5,2,6,3,7][i] of the row
 *           (with act-order: column perm[that index] of x); columns K .. Kp-1
 *           hold 0;
 *   rowsum  fp32 [Kp/128][Mr] (device), Mr = M rounded up to a multiple of
 *           4: the sum of the E4M3 values of each row's 128-column block
 *           (rows M .. Mr-1 hold 0).
 * perm: the act-order permutation written by w4_repack_gptq (NULL iff
 * !has_g_idx).  Asynchronous on `stream`. */
w4_status w4a8_quantize(const w4_layer* layer, int64_t M, const void* x, const float* x_scale, const int32_t* perm,
                        uint8_t* xq, float* rowsum, void* stream);

/* Bytes of workspace w4a8_linear needs for M rows (xq and rowsum above).
 * Host only. */
w4_status w4a8_workspace_size(const w4_layer* layer, int64_t M, size_t* bytes);

/* y [M][N] (act dtype) = s_x x_q W + bias for activations x [M][K] (act
 * dtype) and the per-tensor scale x_scale[0] (fp32, device): w4a8_quantize
 * into the workspace, then the fused int4 x fp8 GEMM.  Arguments as for
 * w4a16_linear; workspace >= w4a8_workspace_size() bytes (16-byte aligned,
 * no initialization needed).  fp32 accumulation, y rounded once.  Accuracy:
 * within max|y - ref| <= 1e-2 (1 + |ref|) elementwise and relative
 * Frobenius error <= 2e-3 of the float64 result of the same quantized
 * activations (the oracle's reference_w4a8_linear). */
w4_status w4a8_linear(const w4_layer* layer, int64_t M, const void* x, const float* x_scale,
                      const int32_t* tiled_qweight, const void* tiled_scales, const int32_t* tiled_qzeros,
                      const int32_t* perm, const void* bias, void* y, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Name of the kernel w4a8_linear launches for M rows ("invalid" for a bad
 * or unsupported descriptor).  Static string; host only. */
const char* w4a8_kernel_name(const w4_layer* layer, int64_t M);

/* Dense dequantization (the unfused path the fused GEMM is measured against).
 * The vLLM AWQ practice page (section 5.3) runs large batches as "dequantize,
 * then matmul" instead of the fused kernel; this call is the first half of
 * that path.  It is not used by w4a16_linear.
 *   tiled_*, perm  as written by w4_repack_gptq (perm NULL iff !has_g_idx)
 *   w              act [K][N] row-major (device, 2-byte aligned) -- written:
 *                  W[k][n] = (q[k][n] - z[g(k)][n]) * s[g(k)][n], computed
 *                  exactly and rounded once (round to nearest even) to the
 *                  activation dtype, rows in the original (unsorted) order.
 *                  Zero scales give +0.
 * Asynchronous on `stream`; every element of w is written once (a perm entry
 * outside [0, K) -- impossible after a successful repack -- writes nothing).
 * Errors as for w4a16_linear. */
w4_status w4_dequant_dense(const w4_layer* layer, const int32_t* tiled_qweight, const void* tiled_scales,
                           const int32_t* tiled_qzeros, const int32_t* perm, void* w, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4HIP_H */
