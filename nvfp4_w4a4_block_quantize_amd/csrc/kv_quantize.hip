// Static FP8 (E4M3) quantisation of attention K/V activations with one
// calibrated scale per tensor (news article "Qwen3.8-27B最激进4bit量化开源，
// 权重显存暴降2.9倍！", section 03: the "Minima+scales" variant adds statically
// calibrated FP8 KV-cache scales to the 16 attention layers, leaving the
// tensor arithmetic and the weight quantisation unchanged).
//
// Every element becomes q = sign(y) | E4M3FN_nearest_even_saturating(|y|) with
// y = fp32(x * s); s is the ENCODE scale (448 / calibrated amax), read from
// device memory, and the dequantised value is e4m3(q) / s.  The encode is
// v_cvt_pk_fp8_f32 on y clamped to [-448, 448] (two elements per
// instruction); that pair equals the rule above on every non-NaN fp32 input
// (checked exhaustively by conformance_cvt).  Bandwidth kernel: 2 B read +
// 1 B written per bf16 element; one lane owns 8 elements (16 B in, 8 B out),
// four such chunks in flight per thread.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int DT>
__device__ __forceinline__ void load8(const void* x, int64_t elem, float (&f)[8]) {
  if constexpr (DT == 0) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(static_cast<const float*>(x) + elem);
    const u32x4_t a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = __uint_as_float(a[i]);
      f[4 + i] = __uint_as_float(b[i]);
    }
  } else {
    const u32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(x) + elem));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == 1) {
        f[2 * i] = __uint_as_float(a[i] << 16);
        f[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
      } else {
        _Float16 lo, hi;
        const uint16_t l = (uint16_t)(a[i] & 0xFFFFu), h = (uint16_t)(a[i] >> 16);
        __builtin_memcpy(&lo, &l, 2);
        __builtin_memcpy(&hi, &h, 2);
        f[2 * i] = (float)lo;
        f[2 * i + 1] = (float)hi;
      }
    }
  }
}

// four E4M3 bytes of y[0..3], y[0] in the low byte
__device__ __forceinline__ uint32_t e4m3x4(float y0, float y1, float y2, float y3) {
  auto clamp = [](float y) { return __builtin_amdgcn_fmed3f(y, -448.0f, 448.0f); };
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(clamp(y0), clamp(y1), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp(y2), clamp(y3), lo, true);
}

template <int DT, bool DENSE>
__global__ __launch_bounds__(kThreads) void kv_quantize_kernel(const void* __restrict__ x, int64_t total_chunks,
                                                               uint32_t chunks_per_row, int64_t ldx,
                                                               const float* __restrict__ scale,
                                                               u32x2_t* __restrict__ out) {
  const float s = *scale;
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  float f[kUnroll][8];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t c = base + u * kThreads;
    const int64_t cc = c < total_chunks ? c : total_chunks - 1;  // past the end: reload the last chunk
    int64_t elem;
    if constexpr (DENSE) {
      elem = cc * 8;
    } else {
      const int64_t row = cc / chunks_per_row;
      elem = row * ldx + (cc - row * chunks_per_row) * 8;
    }
    load8<DT>(x, elem, f[u]);
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t c = base + u * kThreads;
    const u32x2_t w = {e4m3x4(f[u][0] * s, f[u][1] * s, f[u][2] * s, f[u][3] * s),
                       e4m3x4(f[u][4] * s, f[u][5] * s, f[u][6] * s, f[u][7] * s)};
    if (c < total_chunks) out[c] = w;
  }
}

template <int DT, bool DENSE>
hipError_t launch_kv_typed(const void* x, int64_t rows, int64_t cols, int64_t ldx, const float* scale, uint8_t* out,
                           hipStream_t stream) {
  const int64_t chunks_per_row = cols / 8;
  const int64_t total = rows * chunks_per_row;
  const int64_t per_block = (int64_t)kThreads * kUnroll;
  const int64_t blocks = (total + per_block - 1) / per_block;
  kv_quantize_kernel<DT, DENSE><<<(unsigned)blocks, kThreads, 0, stream>>>(
      x, total, (uint32_t)chunks_per_row, ldx, scale, reinterpret_cast<u32x2_t*>(out));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_quantize_fp8(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                                  const float* scale, uint8_t* out, hipStream_t stream) {
  const bool dense = (ldx == cols);
  switch (dtype) {
    case 0:
      return dense ? launch_kv_typed<0, true>(x, rows, cols, ldx, scale, out, stream)
                   : launch_kv_typed<0, false>(x, rows, cols, ldx, scale, out, stream);
    case 1:
      return dense ? launch_kv_typed<1, true>(x, rows, cols, ldx, scale, out, stream)
                   : launch_kv_typed<1, false>(x, rows, cols, ldx, scale, out, stream);
    default:
      return dense ? launch_kv_typed<2, true>(x, rows, cols, ldx, scale, out, stream)
                   : launch_kv_typed<2, false>(x, rows, cols, ldx, scale, out, stream);
  }
}

namespace {
__global__ void kv_scale_kernel(const float* amax_state, float* scale) {
  const float amax = *amax_state;
  *scale = amax > 0.0f ? 448.0f / amax : 1.0f;  // the largest magnitude lands on E4M3's 448
}
}  // namespace

hipError_t launch_kv_scale_from_amax(const float* amax_state, float* scale, hipStream_t stream) {
  kv_scale_kernel<<<1, 1, 0, stream>>>(amax_state, scale);
  return hipGetLastError();
}

}  // namespace nvfp4
