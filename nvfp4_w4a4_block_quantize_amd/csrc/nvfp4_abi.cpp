// C ABI of the NVFP4 W4A4 linear-layer library: argument validation (pure,
// before any HIP call) and dispatch onto the caller's stream.  The operations
// and their error behaviour are specified in include/nvfp4.h.
#include "nvfp4.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>

#include "nvfp4_internal.h"

namespace nvfp4 {

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev < 0 || dev >= 64) dev = 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

}  // namespace nvfp4

namespace {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int dtype_size(int32_t dt) { return dt == NVFP4_F32 ? 4 : (dt == NVFP4_BF16 || dt == NVFP4_F16) ? 2 : 0; }

// true when a GPU is usable from this thread (checked only after validation)
inline bool device_ok() {
  int dev = -1;
  return hipGetDevice(&dev) == hipSuccess && dev >= 0;
}

constexpr int64_t kMaxDim = (int64_t)1 << 31;  // rows / cols / m / n / k each below 2^31

}  // namespace

extern "C" {

int32_t nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

const char* nvfp4_status_str(int32_t s) {
  switch (s) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "invalid shape (sizes must be > 0, cols/k a multiple of 16, ld >= row length)";
    case NVFP4_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case NVFP4_ERR_DTYPE: return "unknown dtype or mode";
    case NVFP4_ERR_RANGE: return "global scale not finite and > 0, or module count out of range";
    case NVFP4_ERR_DEVICE: return "no usable GPU or a HIP launch failed";
    default: return "unknown status";
  }
}

nvfp4_status nvfp4_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ldx, float* gscale,
                            int32_t gscale_mode, uint8_t* codes, uint8_t* scales, void* stream) {
  if (!x || !gscale || !codes || !scales) return NVFP4_ERR_NULL;
  const int es = dtype_size(x_dtype);
  if (es == 0) return NVFP4_ERR_DTYPE;
  if (gscale_mode != NVFP4_GSCALE_STATIC && gscale_mode != NVFP4_GSCALE_DYNAMIC) return NVFP4_ERR_DTYPE;
  if (rows <= 0 || cols <= 0 || cols % 16 != 0 || ldx < cols || rows >= kMaxDim || cols >= kMaxDim ||
      ldx >= ((int64_t)1 << 40))
    return NVFP4_ERR_SHAPE;
  if (!aligned(x, 16) || (ldx * es) % 16 != 0 || !aligned(codes, 4) || !aligned(gscale, 4))
    return NVFP4_ERR_ALIGN;
  if (!device_ok()) return NVFP4_ERR_DEVICE;
  const hipError_t e = nvfp4::launch_quantize(x, x_dtype, rows, cols, ldx, gscale, gscale_mode == NVFP4_GSCALE_DYNAMIC,
                                              codes, scales, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_DEVICE;
}

nvfp4_status nvfp4_amax_observe(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                                float* amax_state, void* stream) {
  if (!x || !amax_state) return NVFP4_ERR_NULL;
  const int es = dtype_size(x_dtype);
  if (es == 0) return NVFP4_ERR_DTYPE;
  if (rows <= 0 || cols <= 0 || cols % 8 != 0 || ldx < cols || rows >= kMaxDim || cols >= kMaxDim ||
      ldx >= ((int64_t)1 << 40))
    return NVFP4_ERR_SHAPE;
  if (!aligned(x, 16) || (ldx * es) % 16 != 0 || !aligned(amax_state, 4)) return NVFP4_ERR_ALIGN;
  if (!device_ok()) return NVFP4_ERR_DEVICE;
  const hipError_t e =
      nvfp4::launch_amax_observe(x, x_dtype, rows, cols, ldx, amax_state, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_DEVICE;
}

nvfp4_status nvfp4_gscale_from_amax(const float* amax_state, float* gscale, void* stream) {
  if (!amax_state || !gscale) return NVFP4_ERR_NULL;
  if (!aligned(amax_state, 4) || !aligned(gscale, 4)) return NVFP4_ERR_ALIGN;
  if (!device_ok()) return NVFP4_ERR_DEVICE;
  const hipError_t e = nvfp4::launch_gscale_from_amax(amax_state, gscale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_DEVICE;
}

nvfp4_status nvfp4_kv_quantize_fp8(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                                   const float* scale, uint8_t* out, void* stream) {
  if (!x || !scale || !out) return NVFP4_ERR_NULL;
  const int es = dtype_size(x_dtype);
  if (es == 0) return NVFP4_ERR_DTYPE;
  if (rows <= 0 || cols <= 0 || cols % 8 != 0 || ldx < cols || rows >= kMaxDim || cols >= kMaxDim ||
      ldx >= ((int64_t)1 << 40))
    return NVFP4_ERR_SHAPE;
  if (!aligned(x, 16) || (ldx * es) % 16 != 0 || !aligned(out, 8) || !aligned(scale, 4)) return NVFP4_ERR_ALIGN;
  if (!device_ok()) return NVFP4_ERR_DEVICE;
  const hipError_t e =
      nvfp4::launch_kv_quantize_fp8(x, x_dtype, rows, cols, ldx, scale, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_DEVICE;
}

nvfp4_status nvfp4_kv_scale_from_amax(const float* amax_state, float* scale, void* stream) {
  if (!amax_state || !scale) return NVFP4_ERR_NULL;
  if (!aligned(amax_state, 4) || !aligned(scale, 4)) return NVFP4_ERR_ALIGN;
  if (!device_ok()) return NVFP4_ERR_DEVICE;
  const hipError_t e = nvfp4::launch_kv_scale_from_amax(amax_state, scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_DEVICE;
}

nvfp4_status nvfp4_fuse_rescale(uint8_t* scales, int64_t k, int32_t n_modules, const int64_t* module_rows,
                                const float* module_gscales, float* shared_gscale, int64_t* lossy_blocks,
                                void* stream) {
  if (!scales || !module_rows || !module_gscales || !shared_gscale) return NVFP4_ERR_NULL;
  if (k <= 0 || k % 16 != 0 || k >= kMaxDim) return NVFP4_ERR_SHAPE;
  if (n_modules < 1 || n_modules > NVFP4_MAX_FUSED_MODULES) return NVFP4_ERR_RANGE;
  float g_star = INFINITY;
  int64_t total_rows = 0;
  for (int32_t i = 0; i < n_modules; ++i) {
    if (module_rows[i] <= 0 || module_rows[i] >= kMaxDim) return NVFP4_ERR_SHAPE;
    const float g = module_gscales[i];
    if (!std::isfinite(g) || !(g > 0.0f)) return NVFP4_ERR_RANGE;
    if (g < g_star) g_star = g;
    total_rows += module_rows[i];
  }
  if (total_rows >= kMaxDim) return NVFP4_ERR_SHAPE;
  if (lossy_blocks && !aligned(lossy_blocks, 8)) return NVFP4_ERR_ALIGN;
  if (!device_ok()) return NVFP4_ERR_DEVICE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (lossy_blocks && nvfp4::launch_zero_i64(lossy_blocks, s) != hipSuccess) return NVFP4_ERR_DEVICE;
  const int64_t per_row = k / 16;
  int64_t r0 = 0;
  for (int32_t i = 0; i < n_modules; ++i) {
    const hipError_t e = nvfp4::launch_fuse_rescale(scales + r0 * per_row, module_rows[i] * per_row, g_star,
                                                    module_gscales[i], lossy_blocks, s);
    if (e != hipSuccess) return NVFP4_ERR_DEVICE;
    r0 += module_rows[i];
  }
  *shared_gscale = g_star;
  return NVFP4_OK;
}

nvfp4_status nvfp4_gemm(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                        const float* a_gscale, const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gscale,
                        void* c, int32_t c_dtype, int64_t ldc, void* stream) {
  if (!a_codes || !a_scales || !a_gscale || !w_codes || !w_scales || !w_gscale || !c) return NVFP4_ERR_NULL;
  const int es = dtype_size(c_dtype);
  if (es == 0) return NVFP4_ERR_DTYPE;
  if (m <= 0 || n <= 0 || k <= 0 || k % 16 != 0 || ldc < n || m >= kMaxDim || n >= kMaxDim || k >= kMaxDim ||
      ldc >= ((int64_t)1 << 40))
    return NVFP4_ERR_SHAPE;
  if (!aligned(a_codes, 16) || !aligned(w_codes, 16) || !aligned(c, es) || !aligned(a_gscale, 4) ||
      !aligned(w_gscale, 4))
    return NVFP4_ERR_ALIGN;
  if (!device_ok()) return NVFP4_ERR_DEVICE;
  const hipError_t e = nvfp4::launch_gemm(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c,
                                          c_dtype, ldc, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_DEVICE;
}

}  // extern "C"
