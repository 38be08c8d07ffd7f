/*
 * nvfp4.h — C ABI of the NVFP4 W4A4 linear-layer library for AMD MI355X (gfx950).
 *
 * The operations follow arXiv 2609.04098 ("Why Gated DeltaNet Survives 4-Bit
 * Quantization: NVFP4 W4A4 for the Recurrent Half of a Hybrid 27B LLM") as
 * described on these pages:
 *   - news article "Qwen3.8-27B最激进4bit量化开源，权重显存暴降2.9倍！",
 *     section 02 (NVFP4 format: E2M1 values, one E4M3 scale per 16 elements,
 *     one FP32 global scale per tensor; W4A4 = weights and activations both in
 *     that format, multiplied as 4-bit x 4-bit) and section 03 (fused-module
 *     global-scale repair, checkpoint side);
 *   - the paper's abstract (the same repair, and the FP8 KV remark).
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless the comment says "host".
 *   - The caller allocates and owns every buffer.  The library allocates no
 *     memory, keeps no pointer after a call returns and holds no global state
 *     besides a per-device cache of the compute-unit count.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream).  Results are visible after the caller synchronises.
 *   - All argument validation happens before any HIP call, so a rejected call
 *     writes nothing and launches nothing.  A launch failure returns
 *     NVFP4_ERR_DEVICE; faults during execution surface at the caller's next
 *     synchronisation, as with any HIP kernel.
 *   - NaN or Inf inputs are not detected: their outputs are unspecified, but
 *     every access stays inside the buffers described below.
 *   - Calls are reentrant and thread-safe; calls on different streams may run
 *     concurrently as long as their output buffers do not overlap.
 *
 * Data layout (the encoding)
 *   - A quantised [rows x cols] tensor (cols % 16 == 0) is three objects:
 *       codes  : uint8 [rows][cols/2], row-major, dense.  Byte j of a row holds
 *                element 2j in its low nibble and element 2j+1 in its high
 *                nibble.  A nibble is an E2M1 code s|e1e0|m (bias 1): 0..7 =
 *                0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 is the sign.
 *       scales : uint8 [rows][cols/16], row-major, dense.  One OCP E4M3FN
 *                byte (bias 7, max 448, no infinities) per 16 consecutive
 *                elements of a row.
 *       g      : one fp32, the ENCODE global scale.  Element value =
 *                e2m1(code) * e4m3(scale) / g.
 *   - Blocks run along the reduction axis K for both GEMM operands.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nvfp4_status {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,   /* a required pointer is NULL                                  */
  NVFP4_ERR_SHAPE = 2,  /* a size <= 0, cols/k not a multiple of 16, ld < row length   */
  NVFP4_ERR_ALIGN = 3,  /* a pointer or leading dimension breaks the alignment rules   */
  NVFP4_ERR_DTYPE = 4,  /* unknown dtype or mode value                                  */
  NVFP4_ERR_RANGE = 5,  /* a host global scale <= 0 or not finite; too many modules     */
  NVFP4_ERR_DEVICE = 6  /* no usable GPU, or a HIP launch failed                        */
} nvfp4_status;

typedef enum nvfp4_dtype { NVFP4_F32 = 0, NVFP4_BF16 = 1, NVFP4_F16 = 2 } nvfp4_dtype;

enum { NVFP4_GSCALE_STATIC = 0, NVFP4_GSCALE_DYNAMIC = 1 };

enum { NVFP4_MAX_FUSED_MODULES = 64 };

/*
 * nvfp4_quantize — online NVFP4 quantisation of a [rows x cols] tensor
 * (news article section 02: E2M1 elements, E4M3 scale per 16 elements,
 * FP32 global scale).
 *
 *   x        [rows][ldx] elements of type x_dtype (NVFP4_F32 / BF16 / F16);
 *            16-byte aligned, and ldx * sizeof(element) a multiple of 16.
 *   gscale   device fp32[1].  gscale_mode NVFP4_GSCALE_STATIC: read g from it
 *            (a calibrated activation scale).  NVFP4_GSCALE_DYNAMIC: the call
 *            first writes g = fp32(2688 / max|x|) there (1.0 when max|x| = 0),
 *            using the same word as its reduction buffer, then quantises.
 *   codes    [rows][cols/2] bytes, 4-byte aligned (output).
 *   scales   [rows][cols/16] bytes (output).
 *
 * Per 16-element block b of a row: s = fp32(fp32(max|x_b| / 6) * g); the scale
 * byte S is s rounded to E4M3 (nearest even, saturating at 448); every element
 * becomes the E2M1 code of y = fp32(x * fp32(g / e4m3(S))) (nearest, ties to
 * the even code, saturating at 6, sign bit from y), or a signed zero when S
 * encodes 0.  The result is a pure function of (x, g): bit-identical across
 * runs and launch configurations.
 *
 * Errors: NULL pointers -> ERR_NULL; rows <= 0, cols <= 0, cols % 16 != 0,
 * ldx < cols -> ERR_SHAPE; alignment -> ERR_ALIGN; bad x_dtype or gscale_mode
 * -> ERR_DTYPE.
 */
nvfp4_status nvfp4_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                            float* gscale, int32_t gscale_mode, uint8_t* codes, uint8_t* scales,
                            void* stream);

/*
 * nvfp4_amax_observe / nvfp4_gscale_from_amax — static activation global
 * scale from calibration data (the paper reading, section 四 4.1, and the news
 * article, section 03: the checkpoint is calibrated on 128 samples of 32K
 * tokens; the activation global scale then serves every later input).
 *
 * nvfp4_amax_observe folds max|x| of one batch into *amax_state:
 *   x           [rows][ldx] elements of type x_dtype (NVFP4_F32 / BF16 / F16),
 *               16-byte aligned, ldx * sizeof(element) a multiple of 16,
 *               cols a multiple of 8.
 *   amax_state  device fp32[1], owned by the caller, set to 0.0f (all bytes
 *               zero) before the first batch.  After any number of calls on
 *               the stream it holds the largest magnitude seen; max is exact
 *               and independent of order, so the result does not depend on
 *               batch order or launch configuration.  Calls may be
 *               concurrent on different streams.
 * nvfp4_gscale_from_amax writes *gscale = fp32(2688 / amax) (1.0 when amax is
 * 0): the encode global scale of the whole calibration set, ready for
 * nvfp4_quantize's static mode.  Both pointers are device fp32[1].
 *
 * Errors: NULL pointers -> ERR_NULL; rows <= 0, cols <= 0, cols % 8 != 0,
 * ldx < cols -> ERR_SHAPE; alignment -> ERR_ALIGN; bad x_dtype -> ERR_DTYPE.
 */
nvfp4_status nvfp4_amax_observe(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                                float* amax_state, void* stream);
nvfp4_status nvfp4_gscale_from_amax(const float* amax_state, float* gscale, void* stream);

/*
 * nvfp4_kv_quantize_fp8 / nvfp4_kv_scale_from_amax — static FP8 quantisation
 * of attention K/V activations (news article section 03: the "Minima+scales"
 * variant adds statically calibrated FP8 KV-cache scales; the abstract calls
 * them performance-free).  Not part of the W4A4 GEMM path; it sits next to
 * the attention layers.
 *
 * nvfp4_kv_quantize_fp8 writes one OCP E4M3FN byte per element:
 *   out[r][c] = sign(y) | E4M3(|y|),  y = fp32(x[r][c] * s),  s = *scale,
 * E4M3 rounding to nearest even and saturating at 448 (no NaN produced from
 * finite input); the dequantised value is e4m3(out) / s.
 *   x      [rows][ldx] of x_dtype (NVFP4_F32 / BF16 / F16), 16-byte aligned,
 *          ldx * sizeof(element) a multiple of 16, cols a multiple of 8.
 *   scale  device fp32[1], the ENCODE scale (448 / calibrated amax).
 *   out    [rows][cols] bytes, dense, 8-byte aligned (output).
 * nvfp4_kv_scale_from_amax writes *scale = fp32(448 / amax) (1.0 when amax is
 * 0) from an amax word filled by nvfp4_amax_observe.  Both device fp32[1].
 *
 * Errors: NULL pointers -> ERR_NULL; rows <= 0, cols <= 0, cols % 8 != 0,
 * ldx < cols -> ERR_SHAPE; alignment -> ERR_ALIGN; bad x_dtype -> ERR_DTYPE.
 */
nvfp4_status nvfp4_kv_quantize_fp8(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                                   const float* scale, uint8_t* out, void* stream);
nvfp4_status nvfp4_kv_scale_from_amax(const float* amax_state, float* scale, void* stream);

/*
 * nvfp4_fuse_rescale — checkpoint-side repair of a fused group of separately
 * calibrated modules (news article section 03: bring every tensor of the group
 * to one global scale and fold the ratio into its E4M3 block scales; the
 * abstract calls the defect a global-scale mismatch of fused GEMMs).
 *
 *   scales          [sum(module_rows)][k/16] E4M3 bytes of the modules stacked
 *                   in module order (the fused weight's scales), rewritten in
 *                   place.  Codes are not touched.
 *   k               the modules' common reduction length (k % 16 == 0).
 *   n_modules       1..NVFP4_MAX_FUSED_MODULES.
 *   module_rows     host int64[n_modules], each > 0.
 *   module_gscales  host fp32[n_modules], each module's encode global scale,
 *                   finite and > 0.
 *   shared_gscale   host fp32[1] (output): g* = min_i g_i, the group's largest
 *                   DEcode scale.  It is written before the call returns.
 *   lossy_blocks    device int64[1] or NULL (output): the number of blocks
 *                   whose dequantisation factor changed, i.e. where
 *                   e4m3(S') / g* != e4m3(S) / g_i.  Written on the stream.
 *
 * Rule per block of module i: rho_i = fp32(g* / g_i) (<= 1, so nothing can
 * saturate); S' = E4M3_nearest_even(fp32(e4m3(S) * rho_i)).  The module whose
 * g_i equals g* keeps its bytes exactly; power-of-two ratios are exact while
 * the folded scale stays normal.  After the call the fused GEMM uses g* as its
 * weight global scale.
 *
 * Errors: NULL scales/module_rows/module_gscales/shared_gscale -> ERR_NULL;
 * k <= 0, k % 16 != 0, module_rows[i] <= 0 -> ERR_SHAPE; n_modules out of
 * range or a bad global scale -> ERR_RANGE.
 */
nvfp4_status nvfp4_fuse_rescale(uint8_t* scales, int64_t k, int32_t n_modules, const int64_t* module_rows,
                                const float* module_gscales, float* shared_gscale, int64_t* lossy_blocks,
                                void* stream);

/*
 * nvfp4_gemm — block-scaled 4-bit x 4-bit GEMM with FP32 accumulation
 * (news article section 02: W4A4 computes on 4-bit operands):
 *
 *   C[m][n] = alpha * sum_k (e2m1(a)*e4m3(sa)) * (e2m1(w)*e4m3(sw)),
 *   alpha   = fp32(1 / fp32(g_a * g_w)),
 *
 * i.e. C = A_hat * W_hat^T with both operands in the encoding above (A is
 * [m x k], W is [n x k], nn.Linear layout, both K-contiguous).
 *
 *   a_codes  [m][k/2], a_scales [m][k/16], a_gscale device fp32[1]
 *   w_codes  [n][k/2], w_scales [n][k/16], w_gscale device fp32[1]
 *   c        [m][ldc] of c_dtype (NVFP4_F32, NVFP4_BF16 or NVFP4_F16), only
 *            the first n columns of each row are written; ldc >= n.
 *   Alignment: codes 16-byte aligned; c aligned to its element size.  Scales
 *            need no alignment; the prefill and decode-shaped kernels take
 *            4-byte aligned scale pointers (others go to a generic kernel),
 *            and the decode-shaped kernels stage scale rows in LDS with
 *            16-byte loads when the pointers are 16-byte aligned.
 *
 * Every decoded operand e2m1*e4m3 is exact in fp16 (at most 6 significant
 * bits, magnitudes 2^-10 .. 2688), every product is exact in fp32 and the sum
 * is accumulated in fp32.  The kernel, and with it the summation order, is
 * chosen from the shape, the operands' alignment and the device's CU count;
 * for a given choice it is fixed, so repeated calls give identical results.
 * A prefill-sized call whose last strip of columns (n % 256 of them) would
 * open another round of 256x256 tiles enqueues two kernels on `stream`: the
 * tiles over the first n - n % 256 columns, then the decode-shaped kernel
 * over the strip.  Each output element is computed by exactly one of them.
 * If the second launch fails, the call returns NVFP4_ERR_DEVICE and the
 * first part of C may already be written.
 * bf16/f16 outputs are the fp32 result rounded to nearest even.
 *
 * Errors: NULL pointers -> ERR_NULL; m, n, k <= 0, k % 16 != 0, ldc < n ->
 * ERR_SHAPE; alignment -> ERR_ALIGN; bad c_dtype -> ERR_DTYPE.
 */
nvfp4_status nvfp4_gemm(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                        const float* a_gscale, const uint8_t* w_codes, const uint8_t* w_scales,
                        const float* w_gscale, void* c, int32_t c_dtype, int64_t ldc, void* stream);

/* Static, NUL-terminated description of a status code ("unknown status" otherwise). */
const char* nvfp4_status_str(int32_t status);

/* ABI version of this header (incremented on any incompatible change). */
int32_t nvfp4_abi_version(void);

#define NVFP4_ABI_VERSION 1

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
