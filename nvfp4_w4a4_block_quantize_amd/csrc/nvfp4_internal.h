// Launchers shared between the C-ABI layer and the kernel translation units.
// Arguments are validated by the caller (nvfp4_abi.cpp); these only launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Quantiser: dtype 0 = f32, 1 = bf16, 2 = f16.  dynamic != 0 first writes g
// into *gscale (the word doubles as the amax reduction buffer).
hipError_t launch_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, float* gscale,
                           bool dynamic, uint8_t* codes, uint8_t* scales, hipStream_t stream);

// Calibration observer: atomically folds max|x| into the fp32 word *amax_state
// (non-negative floats order like their bit patterns); then g = 2688 / amax.
hipError_t launch_amax_observe(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, float* amax_state,
                               hipStream_t stream);
hipError_t launch_gscale_from_amax(const float* amax_state, float* gscale, hipStream_t stream);

// Static FP8 KV quantisation: out[e] = E4M3(x[e] * *scale), one byte per element.
hipError_t launch_kv_quantize_fp8(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                                  const float* scale, uint8_t* out, hipStream_t stream);
hipError_t launch_kv_scale_from_amax(const float* amax_state, float* scale, hipStream_t stream);

// Fold rho = g_star / g_module into `count` scale bytes starting at `scales`;
// adds the number of changed dequantisation factors to *lossy when non-null.
hipError_t launch_fuse_rescale(uint8_t* scales, int64_t count, float g_star, float g_module, int64_t* lossy,
                               hipStream_t stream);
hipError_t launch_zero_i64(int64_t* p, hipStream_t stream);

// GEMM C = alpha * A_hat W_hat^T; out_dtype 0 = f32, 1 = bf16, 2 = f16.
hipError_t launch_gemm(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                       const float* a_gscale, const uint8_t* w_codes, const uint8_t* w_scales,
                       const float* w_gscale, void* c, int out_dtype, int64_t ldc, hipStream_t stream);

// Main GEMM path (k % 128 == 0, m > 64, 16-byte aligned codes, 4-byte aligned scales, operands below 2 GiB).
bool gemm_fast_supported(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                         const uint8_t* w_codes, const uint8_t* w_scales);
// tile_n: 256 (256x256 tiles) or 128 (256x128 tiles, for the last round of a call)
hipError_t launch_gemm_fast(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                            const float* a_gscale, const uint8_t* w_codes, const uint8_t* w_scales,
                            const float* w_gscale, void* c, int out_dtype, int64_t ldc, hipStream_t stream,
                            int tile_n = 256);

// Decode-shaped path (m <= 256 in blocks of 64 rows, k % 128 == 0, 16-byte aligned codes, 4-byte aligned
// scales, operands below 2 GiB).  launch_gemm_decode itself takes any m up to 65535 blocks of 64 rows: the
// prefill dispatch hands it a ragged last column strip of a large-m GEMM.
bool gemm_decode_supported(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                           const uint8_t* w_codes, const uint8_t* w_scales);
hipError_t launch_gemm_decode(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                              const float* a_gscale, const uint8_t* w_codes, const uint8_t* w_scales,
                              const float* w_gscale, void* c, int out_dtype, int64_t ldc, hipStream_t stream);

// Weight-streaming path for up to 32 activation rows: k = 4096 or 5120, 16-byte aligned codes and scales,
// 80 to 144 weight rows per CU (one workgroup per CU streams a contiguous slab of the weight).
bool gemm_stream_supported(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                           const uint8_t* w_codes, const uint8_t* w_scales);
hipError_t launch_gemm_stream(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                              const float* a_gscale, const uint8_t* w_codes, const uint8_t* w_scales,
                              const float* w_gscale, void* c, int out_dtype, int64_t ldc, hipStream_t stream);

// Number of compute units of the current device (cached per device).
int device_cu_count();

}  // namespace nvfp4
