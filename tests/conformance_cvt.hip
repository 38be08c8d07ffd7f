// Conformance check of the gfx950 conversion instructions the library relies
// on, against the rules they stand in for (written out here independently):
//
//  1. v_cvt_scalef32_pk_fp4_f32 with scale 1.0 (quantiser, element codes):
//     E2M1 nearest value, ties to the even code, |y| > 5 saturating to 6,
//     sign bit copied from y; compared for every non-NaN fp32 bit pattern.
//  2. v_cvt_scalef32_pk_f16_fp4 with scale 1.0 (GEMM decode): each of the 16
//     codes, in both nibble positions, gives the exact fp16 E2M1 value.
//  3. v_cvt_scalef32_pk_f16_fp8 with scale 1.0 (GEMM block scales) and
//     v_cvt_f32_fp8 (quantiser): each of the 254 finite E4M3FN bytes gives its
//     exact value (bias 7, subnormals m * 2^-9).
//  4. v_cvt_pk_bf16_f32 (GEMM epilogue, bf16 output): fp32 to bf16 nearest,
//     ties to even, compared for every non-NaN fp32 bit pattern.
//  5. v_cvt_pk_fp8_f32 after a clamp to [-448, 448] (FP8 KV quantiser):
//     E4M3FN nearest, ties to even, saturating at 448, sign bit copied from
//     y, in all four byte positions; compared for every non-NaN fp32 bit
//     pattern.
//
// Prints one line per check and exits 0 only when every count of mismatches
// is zero.  Built next to the library; run by the GPU test suite.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

namespace {

__device__ uint32_t e2m1_rule(float y) {
  const float a = __builtin_fabsf(y);
  const uint32_t mag = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return mag | ((__float_as_uint(y) >> 28) & 8u);
}

__device__ float e2m1_value(uint32_t code) {
  const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  return (code & 8u) ? -mag[code & 7u] : mag[code & 7u];
}

__device__ float e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float v = e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8u + m), (int)e - 10);
  return (b & 0x80u) ? -v : v;
}

__global__ void check_fp4_encode(unsigned long long* bad) {
  unsigned long long nb = 0;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 32); i += 2 * stride) {
    const uint32_t u0 = (uint32_t)i;
    const uint32_t u1 = (uint32_t)(i + stride);  // i + stride < 2^32: i < 2^32 - 2*stride at every step
    const float y0 = __uint_as_float(u0), y1 = __uint_as_float(u1);
    const uint32_t hw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y0, y1, 1.0f, 0);
    if ((u0 & 0x7FFFFFFFu) <= 0x7F800000u && (hw & 0xFu) != e2m1_rule(y0)) ++nb;
    if ((u1 & 0x7FFFFFFFu) <= 0x7F800000u && ((hw >> 4) & 0xFu) != e2m1_rule(y1)) ++nb;
  }
  if (nb) atomicAdd(bad, nb);
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// bf16 nearest-even of a finite or infinite fp32: add half a unit of the
// 16 dropped bits (less one when the kept part is even) and truncate
__device__ uint32_t bf16_rule(uint32_t u) { return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16; }

__global__ void check_bf16_pack(unsigned long long* bad) {
  unsigned long long nb = 0;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 32); i += 2 * stride) {
    const uint32_t u0 = (uint32_t)i;
    const uint32_t u1 = (uint32_t)(i + stride);  // i + stride < 2^32: i < 2^32 - 2*stride at every step
    const bf16x2_t v = {(__bf16)__uint_as_float(u0), (__bf16)__uint_as_float(u1)};
    const uint32_t hw = __builtin_bit_cast(uint32_t, v);
    if ((u0 & 0x7FFFFFFFu) <= 0x7F800000u && (hw & 0xFFFFu) != bf16_rule(u0)) ++nb;
    if ((u1 & 0x7FFFFFFFu) <= 0x7F800000u && (hw >> 16) != bf16_rule(u1)) ++nb;
  }
  if (nb) atomicAdd(bad, nb);
}

// E4M3FN of y: |y| clamped to 448, then nearest, ties to even, on the grid
// m * 2^-9 (m = 0..8) below 2^-6 and (1 + f/8) * 2^(e-7) above; sign from y
__device__ uint32_t e4m3_rule(float y) {
  const float a = fminf(__builtin_fabsf(y), 448.0f);
  uint32_t mag;
  if (a < 0x1p-6f) {
    mag = (uint32_t)rintf(a * 512.0f);  // 8 is the smallest normal, 0x08
  } else {
    int e;
    const float m = frexpf(a, &e);  // a = m * 2^e, m in [0.5, 1)
    uint32_t q = (uint32_t)rintf(m * 16.0f);  // 8..16: the significand with three fraction bits
    if (q == 16u) {
      q = 8u;
      ++e;
    }
    mag = ((uint32_t)(e + 6) << 3) | (q - 8u);  // biased exponent (e - 1) + 7
  }
  return mag | ((__float_as_uint(y) >> 24) & 0x80u);
}

__device__ float clamp448(float y) { return __builtin_amdgcn_fmed3f(y, -448.0f, 448.0f); }

__global__ void check_fp8_encode(unsigned long long* bad) {
  unsigned long long nb = 0;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 32); i += 2 * stride) {
    const uint32_t u0 = (uint32_t)i;
    const uint32_t u1 = (uint32_t)(i + stride);  // i + stride < 2^32: i < 2^32 - 2*stride at every step
    const float y0 = __uint_as_float(u0), y1 = __uint_as_float(u1);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(y0), clamp448(y1), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(y1), clamp448(y0), w, true);
    const uint32_t hw = (uint32_t)w;
    if ((u0 & 0x7FFFFFFFu) <= 0x7F800000u) {
      const uint32_t r = e4m3_rule(y0);
      nb += (hw & 0xFFu) != r;
      nb += ((hw >> 24) & 0xFFu) != r;
    }
    if ((u1 & 0x7FFFFFFFu) <= 0x7F800000u) {
      const uint32_t r = e4m3_rule(y1);
      nb += ((hw >> 8) & 0xFFu) != r;
      nb += ((hw >> 16) & 0xFFu) != r;
    }
  }
  if (nb) atomicAdd(bad, nb);
}

__global__ void check_decodes(unsigned long long* bad) {
  const uint32_t t = threadIdx.x;  // 0..255
  unsigned long long nb = 0;
  // fp4 pairs: byte t holds codes (t & 15, t >> 4)
  const half2_t p = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(t << 8, 1.0f, 1);
  if ((float)p[0] != e2m1_value(t & 15u) || (float)p[1] != e2m1_value(t >> 4)) ++nb;
  // E4M3 bytes, finite ones only (0x7F and 0xFF are NaN)
  if ((t & 0x7Fu) != 0x7Fu) {
    const half2_t q = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(t | (t << 8), 1.0f, false);
    if ((float)q[0] != e4m3_value(t) || (float)q[1] != e4m3_value(t)) ++nb;
    if (__builtin_amdgcn_cvt_f32_fp8((int)t, 0) != e4m3_value(t)) ++nb;
  }
  if (nb) atomicAdd(bad, nb);
}

}  // namespace

int main() {
  unsigned long long* bad = nullptr;
  if (hipMalloc(&bad, 4 * sizeof(unsigned long long)) != hipSuccess) return 2;
  if (hipMemset(bad, 0, 4 * sizeof(unsigned long long)) != hipSuccess) return 2;
  check_fp4_encode<<<4096, 256>>>(bad);
  check_decodes<<<1, 256>>>(bad + 1);
  check_bf16_pack<<<4096, 256>>>(bad + 2);
  check_fp8_encode<<<4096, 256>>>(bad + 3);
  unsigned long long h[4] = {1, 1, 1, 1};
  if (hipDeviceSynchronize() != hipSuccess) return 2;
  if (hipMemcpy(h, bad, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return 2;
  printf("fp4 encode (all non-NaN fp32 inputs): %llu mismatches\n", h[0]);
  printf("fp4->f16, e4m3->f16, e4m3->f32 decodes (all codes): %llu mismatches\n", h[1]);
  printf("fp32->bf16 pack (all non-NaN fp32 inputs): %llu mismatches\n", h[2]);
  printf("clamped fp32->e4m3 pack (all non-NaN fp32 inputs): %llu mismatches\n", h[3]);
  hipFree(bad);
  return (h[0] == 0 && h[1] == 0 && h[2] == 0 && h[3] == 0) ? 0 : 1;
}
