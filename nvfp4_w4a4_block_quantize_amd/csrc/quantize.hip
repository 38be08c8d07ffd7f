// Online NVFP4 quantisation (news article "Qwen3.8-27B最激进4bit量化开源，
// 权重显存暴降2.9倍！", section 02: E2M1 elements, one E4M3 scale per 16
// elements, FP32 global scale; W4A4 quantises activations as well as weights).
//
// One lane owns 8 consecutive elements (16 B of bf16/f16, 32 B of f32), so a
// 16-element block spans a lane pair and a wave covers 1 KiB of bf16 input
// contiguously.  The pair exchanges its partial block max with one lane swap,
// both lanes derive the same scale byte, each packs its 8 codes into one
// 32-bit word (coalesced stores) and the even lane stores the scale byte.
// The kernel is HBM-bound: 2 B read + 0.5625 B written per bf16 element.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
// independent 8-element chunks per thread, loads issued together; small
// tensors use one per thread so that more workgroups share the latency
constexpr int kUnrollLarge = 4;
constexpr int64_t kSmallChunks = (int64_t)1 << 18;

struct Raw {
  u32x4_t a;
  u32x4_t b;  // second half of an f32 chunk
};

template <int DT>
__device__ __forceinline__ Raw load_chunk(const void* x, int64_t elem) {
  Raw r;
  if constexpr (DT == 0) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(static_cast<const float*>(x) + elem);
    r.a = __builtin_nontemporal_load(p);
    r.b = __builtin_nontemporal_load(p + 1);
  } else {
    r.a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(x) + elem));
    r.b = u32x4_t{0, 0, 0, 0};
  }
  return r;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  _Float16 v;
  uint16_t hb = (uint16_t)h;
  __builtin_memcpy(&v, &hb, 2);
  return (float)v;
}

template <int DT>
__device__ __forceinline__ void widen(const Raw& r, float (&f)[8]) {
  const uint32_t w[4] = {r.a[0], r.a[1], r.a[2], r.a[3]};
  if constexpr (DT == 0) {
    const uint32_t w2[4] = {r.b[0], r.b[1], r.b[2], r.b[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = __uint_as_float(w[i]);
      f[4 + i] = __uint_as_float(w2[i]);
    }
  } else if constexpr (DT == 1) {  // bf16 -> f32 is a shift
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {  // f16 -> f32 is exact
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = f16_bits_to_f32(w[i] & 0xFFFFu);
      f[2 * i + 1] = f16_bits_to_f32(w[i] >> 16);
    }
  }
}

// Quantise one lane's 8 elements given the block max shared with its partner.
// The E2M1 rounding of y = fp32(x * r) is v_cvt_scalef32_pk_fp4_f32 with a
// scale of 1.0: nearest value, ties to the even code, saturation at 6, sign
// bit from y (so -0.0 gives 0x8).  That equals the element rule for every
// non-NaN fp32 input (checked exhaustively over all 2^32 bit patterns on
// gfx950), and each instruction writes two codes into one byte of the word,
// even element in the low nibble.
__device__ __forceinline__ uint32_t encode8(const float (&f)[8], float g, float amax_b, uint32_t* scale_out) {
  // s = fp32(fp32(amax_b / 6) * g); IEEE division (correctly rounded), no contraction
  const float s = (amax_b / 6.0f) * g;
  const uint32_t S = e4m3_from_f32(s);
  const float r = (S == 0u) ? 0.0f : g / f32_from_e4m3(S);
  uint32_t word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, f[0] * r, f[1] * r, 1.0f, 0);
  word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, f[2] * r, f[3] * r, 1.0f, 1);
  word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, f[4] * r, f[5] * r, 1.0f, 2);
  word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, f[6] * r, f[7] * r, 1.0f, 3);
  *scale_out = S;
  return word;
}

template <int DT, bool DENSE, int kUnroll>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const void* __restrict__ x, int64_t total_chunks,
                                                            uint32_t chunks_per_row, int64_t ldx,
                                                            const float* __restrict__ gscale,
                                                            uint32_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  const float g = *gscale;
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  Raw raw[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t c = base + u * kThreads;
    if (c < total_chunks) {
      int64_t elem;
      if constexpr (DENSE) {
        elem = c * 8;
      } else {
        const int64_t row = c / chunks_per_row;
        elem = row * ldx + (c - row * chunks_per_row) * 8;
      }
      raw[u] = load_chunk<DT>(x, elem);
    } else {
      raw[u].a = u32x4_t{0, 0, 0, 0};
      raw[u].b = u32x4_t{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t c = base + u * kThreads;
    float f[8];
    widen<DT>(raw[u], f);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(f[i]));
    // partner lane (c ^ 1) holds the other half of the block; every lane of the
    // wave takes part in the swap, in range or not (total_chunks is even)
    const float other = __shfl_xor(m, 1);
    const float amax_b = __builtin_fmaxf(m, other);
    uint32_t S;
    const uint32_t word = encode8(f, g, amax_b, &S);
    if (c < total_chunks) {
      codes[c] = word;  // regular store: the GEMM reads these bytes next
      if ((c & 1) == 0) scales[c >> 1] = (uint8_t)S;
    }
  }
}

// ---- dynamic global scale: amax reduction into the gscale word, then g = 2688 / amax
__global__ void zero_word_kernel(uint32_t* p) { *p = 0u; }

template <int DT, bool DENSE>
__global__ __launch_bounds__(kThreads) void amax_kernel(const void* __restrict__ x, int64_t total_chunks,
                                                        uint32_t chunks_per_row, int64_t ldx,
                                                        uint32_t* __restrict__ amax_bits) {
  // four chunks per thread and iteration, loads issued together
  constexpr int kU = 4;
  float m = 0.0f;
  const int64_t step = (int64_t)gridDim.x * kThreads * kU;
  for (int64_t c0 = (int64_t)blockIdx.x * kThreads * kU + threadIdx.x; c0 < total_chunks; c0 += step) {
    Raw raw[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t c = c0 + (int64_t)u * kThreads;
      if (c < total_chunks) {
        int64_t elem;
        if constexpr (DENSE) {
          elem = c * 8;
        } else {
          const int64_t row = c / chunks_per_row;
          elem = row * ldx + (c - row * chunks_per_row) * 8;
        }
        raw[u] = load_chunk<DT>(x, elem);
      } else {
        raw[u].a = u32x4_t{0, 0, 0, 0};
        raw[u].b = u32x4_t{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float f[8];
      widen<DT>(raw[u], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(f[i]));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
  // one value per workgroup, and an atomic only when it would raise the word:
  // thousands of atomics on one address serialise in the L2.  Non-negative
  // floats order like their bit patterns, so an integer max is exact.
  __shared__ float wave_max[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = wave_max[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) b = __builtin_fmaxf(b, wave_max[w]);
    const uint32_t bits = __float_as_uint(b);
    if (bits > __hip_atomic_load(amax_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(amax_bits, bits);
  }
}

__global__ void finalize_gscale_kernel(float* gscale) {
  const float amax = __uint_as_float(*reinterpret_cast<uint32_t*>(gscale));
  *gscale = amax > 0.0f ? kGlobalScaleNumerator / amax : 1.0f;
}

template <int DT, bool DENSE>
hipError_t launch_typed(const void* x, int64_t rows, int64_t cols, int64_t ldx, float* gscale, bool dynamic,
                        uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t chunks_per_row = cols / 8;
  const int64_t total = rows * chunks_per_row;
  if (dynamic) {
    zero_word_kernel<<<1, 1, 0, stream>>>(reinterpret_cast<uint32_t*>(gscale));
    int64_t blocks = (total + kThreads - 1) / kThreads;
    const int64_t cap = (int64_t)device_cu_count() * 8;
    if (blocks > cap) blocks = cap;
    amax_kernel<DT, DENSE><<<(unsigned)blocks, kThreads, 0, stream>>>(x, total, (uint32_t)chunks_per_row, ldx,
                                                                     reinterpret_cast<uint32_t*>(gscale));
    finalize_gscale_kernel<<<1, 1, 0, stream>>>(gscale);
  }
  if (total < kSmallChunks) {
    const int64_t blocks = (total + kThreads - 1) / kThreads;
    quantize_kernel<DT, DENSE, 1><<<(unsigned)blocks, kThreads, 0, stream>>>(
        x, total, (uint32_t)chunks_per_row, ldx, gscale, reinterpret_cast<uint32_t*>(codes), scales);
  } else {
    const int64_t per_block = (int64_t)kThreads * kUnrollLarge;
    const int64_t blocks = (total + per_block - 1) / per_block;
    quantize_kernel<DT, DENSE, kUnrollLarge><<<(unsigned)blocks, kThreads, 0, stream>>>(
        x, total, (uint32_t)chunks_per_row, ldx, gscale, reinterpret_cast<uint32_t*>(codes), scales);
  }
  return hipGetLastError();
}

__global__ void gscale_from_amax_kernel(const float* amax_state, float* gscale) {
  const float amax = *amax_state;
  *gscale = amax > 0.0f ? kGlobalScaleNumerator / amax : 1.0f;
}

template <int DT, bool DENSE>
hipError_t launch_observe_typed(const void* x, int64_t rows, int64_t cols, int64_t ldx, float* amax_state,
                                hipStream_t stream) {
  const int64_t chunks_per_row = cols / 8;
  const int64_t total = rows * chunks_per_row;
  int64_t blocks = (total + kThreads - 1) / kThreads;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (blocks > cap) blocks = cap;
  amax_kernel<DT, DENSE><<<(unsigned)blocks, kThreads, 0, stream>>>(x, total, (uint32_t)chunks_per_row, ldx,
                                                                   reinterpret_cast<uint32_t*>(amax_state));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_amax_observe(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, float* amax_state,
                               hipStream_t stream) {
  const bool dense = (ldx == cols);
  switch (dtype) {
    case 0:
      return dense ? launch_observe_typed<0, true>(x, rows, cols, ldx, amax_state, stream)
                   : launch_observe_typed<0, false>(x, rows, cols, ldx, amax_state, stream);
    case 1:
      return dense ? launch_observe_typed<1, true>(x, rows, cols, ldx, amax_state, stream)
                   : launch_observe_typed<1, false>(x, rows, cols, ldx, amax_state, stream);
    default:
      return dense ? launch_observe_typed<2, true>(x, rows, cols, ldx, amax_state, stream)
                   : launch_observe_typed<2, false>(x, rows, cols, ldx, amax_state, stream);
  }
}

hipError_t launch_gscale_from_amax(const float* amax_state, float* gscale, hipStream_t stream) {
  gscale_from_amax_kernel<<<1, 1, 0, stream>>>(amax_state, gscale);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, float* gscale,
                           bool dynamic, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const bool dense = (ldx == cols);
  switch (dtype) {
    case 0:
      return dense ? launch_typed<0, true>(x, rows, cols, ldx, gscale, dynamic, codes, scales, stream)
                   : launch_typed<0, false>(x, rows, cols, ldx, gscale, dynamic, codes, scales, stream);
    case 1:
      return dense ? launch_typed<1, true>(x, rows, cols, ldx, gscale, dynamic, codes, scales, stream)
                   : launch_typed<1, false>(x, rows, cols, ldx, gscale, dynamic, codes, scales, stream);
    default:
      return dense ? launch_typed<2, true>(x, rows, cols, ldx, gscale, dynamic, codes, scales, stream)
                   : launch_typed<2, false>(x, rows, cols, ldx, gscale, dynamic, codes, scales, stream);
  }
}

}  // namespace nvfp4
