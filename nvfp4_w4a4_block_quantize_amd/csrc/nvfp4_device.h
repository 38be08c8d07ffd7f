// Device-side helpers for the NVFP4 kernels (gfx950).
//
// Element format (news article "Qwen3.8-27B最激进4bit量化开源，权重显存暴降2.9倍！",
// section 02): E2M1 codes s|e1e0|m with exponent bias 1, one OCP E4M3FN scale
// per 16 elements, one FP32 global scale per tensor.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));

// Largest magnitude in the E2M1 grid times the largest finite E4M3 value.
constexpr float kGlobalScaleNumerator = 2688.0f;

// OCP E4M3FN byte of a non-negative fp32 value: round to nearest even,
// saturating at 448 (0x7E).  Subnormal range [0, 2^-6): multiples of 2^-9.
__device__ __forceinline__ uint32_t e4m3_from_f32(float s) {
  if (!(s < 448.0f)) return 0x7Eu;
  if (s < 0x1p-6f) return (uint32_t)__builtin_rintf(s * 512.0f);  // 0..8; 8 is 0x08 = 2^-6
  const uint32_t u = __float_as_uint(s);
  // keep 3 fraction bits, ties to even; a carry moves into the exponent field
  const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
  return (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);  // fp32 bias 127 -> E4M3 bias 7
}

// Exact fp32 value of an E4M3FN byte (hardware conversion, OCP flavour on gfx950).
__device__ __forceinline__ float f32_from_e4m3(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

}  // namespace nvfp4
