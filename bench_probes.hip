// Measurement probes for the benchmark; not part of the NVFP4 library and not
// on its path.  They give the two ceilings the GEMMs are compared against,
// measured on the chip at hand rather than taken from its specification:
//
//  * probe_mfma_f16: waves that do nothing but v_mfma_f32_32x32x16_f16 (four
//    independent accumulator chains per wave, four waves per SIMD).  The rate
//    is the dense fp16 MFMA throughput at whatever clock the chip holds while
//    doing only that; a real GEMM also spends power and issue slots on loads,
//    LDS traffic and operand decode, so it runs at a lower clock.
//  * probe_stream_read: a grid-stride read of a buffer with 16-byte
//    non-temporal loads; the HBM read rate a streaming kernel can reach.
//
// Both are plain launches on the caller's stream; sink is a device uint32[1]
// that receives a value only when the data makes a never-taken branch true
// (it keeps the work from being removed).
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void mfma_loop_kernel(int iters, uint32_t* sink) {
  half8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.125f * (float)((threadIdx.x + i) & 7));
    b[i] = (_Float16)(0.0625f * (float)((threadIdx.x * 3 + i) & 7));
  }
  float16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (s == -1.0f) sink[0] = 1u;  // the sums are never negative
}

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4_t* __restrict__ p, size_t n16,
                                                                   uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_t v0 = __builtin_nontemporal_load(p + i);
    const u32x4_t v1 = __builtin_nontemporal_load(p + i + stride);
    const u32x4_t v2 = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4_t v3 = __builtin_nontemporal_load(p + i + 3 * stride);
    x ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
    x ^= v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(p + i);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (x == 0x9E3779B9u) sink[0] = x;
}

}  // namespace

extern "C" {

// flops = waves * iters * 4 * 32768; returns a hipError_t value
int probe_mfma_f16(int workgroups, int iters, uint32_t* sink, hipStream_t stream) {
  if (workgroups <= 0 || iters <= 0 || sink == nullptr) return (int)hipErrorInvalidValue;
  mfma_loop_kernel<<<workgroups, kProbeThreads, 0, stream>>>(iters, sink);
  return (int)hipGetLastError();
}

// reads bytes (a multiple of 16, 16-byte aligned) from p
int probe_stream_read(const void* p, size_t bytes, int workgroups, uint32_t* sink, hipStream_t stream) {
  if (p == nullptr || sink == nullptr || workgroups <= 0 || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return (int)hipErrorInvalidValue;
  stream_read_kernel<<<workgroups, kProbeThreads, 0, stream>>>(static_cast<const u32x4_t*>(p), bytes / 16, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
