// Fused-group global-scale repair (news article "Qwen3.8-27B最激进4bit量化开源，
// 权重显存暴降2.9倍！", section 03: unify the global scale of a fused group and
// fold each module's ratio into its E4M3 block scales, checkpoint side).
//
// One thread per scale byte of a module's rows: S' = E4M3(fp32(e4m3(S) * rho))
// with rho = fp32(g* / g_i).  The dequantisation factor changes exactly when
// e4m3(S') * g_i != e4m3(S) * g*; both products are exact in fp64 (4-bit by
// 24-bit significands), and the count of such blocks is accumulated per wave.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void fuse_rescale_kernel(uint8_t* __restrict__ scales, int64_t count,
                                                                float g_star, float g_module,
                                                                unsigned long long* __restrict__ lossy) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  bool changed = false;
  if (i < count) {
    const uint32_t S = scales[i];
    const float rho = g_star / g_module;  // IEEE division, identical in every thread
    const float d = f32_from_e4m3(S & 0x7Fu);
    const uint32_t S2 = e4m3_from_f32(d * rho);
    scales[i] = (uint8_t)S2;
    changed = (double)f32_from_e4m3(S2) * (double)g_module != (double)d * (double)g_star;
  }
  if (lossy != nullptr) {
    // one atomic per workgroup: thousands on one address serialise in the L2
    __shared__ unsigned int wave_count[kThreads / 64];
    const unsigned long long votes = __ballot(changed);
    if ((threadIdx.x & 63) == 0) wave_count[threadIdx.x >> 6] = (unsigned int)__popcll(votes);
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long total = 0;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) total += wave_count[w];
      if (total != 0ull) atomicAdd(lossy, total);
    }
  }
}

__global__ void zero_i64_kernel(int64_t* p) { *p = 0; }

}  // namespace

hipError_t launch_zero_i64(int64_t* p, hipStream_t stream) {
  zero_i64_kernel<<<1, 1, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_fuse_rescale(uint8_t* scales, int64_t count, float g_star, float g_module, int64_t* lossy,
                               hipStream_t stream) {
  const int64_t blocks = (count + kThreads - 1) / kThreads;
  fuse_rescale_kernel<<<(unsigned)blocks, kThreads, 0, stream>>>(scales, count, g_star, g_module,
                                                                reinterpret_cast<unsigned long long*>(lossy));
  return hipGetLastError();
}

}  // namespace nvfp4
