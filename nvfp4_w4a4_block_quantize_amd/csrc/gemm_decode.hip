// Decode-shaped W4A4 GEMM for gfx950 (M <= 256, in blocks of up to 64 activation
// rows): C = alpha * A_hat W_hat^T on
// NVFP4 operands (news article "Qwen3.8-27B最激进4bit量化开源，权重显存暴降2.9倍！",
// section 02: E2M1 codes, one E4M3 scale per 16 elements, one FP32 global
// scale per tensor, both operands 4-bit).
//
// With a few activation rows the product is bound by streaming the weight
// once from HBM (0.5625 B per weight element), not by MFMA.  What limits a
// stream on CDNA is the number of cache-line requests a CU can keep in
// flight, so every line a load instruction touches must be used whole:
//
//  * K is walked in super-groups of 256 elements: one 128-byte line of codes
//    and 16 scale bytes per row.  The 16x16x32 MFMA layout puts a row on 4
//    lanes (q = lane/16), so a lane owns 32 code bytes of the row (bytes
//    32q..32q+31, elements 64q..64q+63, blocks 4q..4q+3): two 16-byte buffer
//    loads issued back to back (offsets 32q and 32q+16) together read each
//    row's line once, and one 4-byte load reads the lane's four scale bytes
//    (the 4 lanes of a row read its 16 contiguous scale bytes).
//  * MFMA step s (0..7) of a super-group takes code word s of every lane:
//    lane q contributes elements 64q+8s..64q+8s+7 (block 4q + s/2) to the
//    K = 32 of v_mfma_f32_16x16x32_f16.  A and W use the same map, so every
//    k is summed exactly once.
//  * A workgroup of 4 waves owns R = 16*T weight rows over the whole of K.
//    Wave w takes super-groups w, w+4, w+8, ..., so the four waves read
//    adjacent lines of the same rows at about the same time (DRAM page
//    locality), and each wave multiplies every weight tile by the same
//    decoded activation fragment (the activation decode is shared T ways and
//    done once per workgroup).  The four partial sums are added in LDS at the
//    end in a fixed order (deterministic).
//  * The workgroup's scale rows (weight and activation, all of K) are staged
//    in LDS at the start with coalesced 16-byte loads when they fit; 4-byte
//    scale loads per row and super-group would cost as many cache-line
//    requests as the code lines themselves.
//  * Two super-groups of code loads per wave alternate in registers: the
//    loads of super-group j+2 are issued as soon as j has been multiplied.
//  * Decode as in the prefill kernel: v_cvt_scalef32_pk_f16_fp4 (scale 1.0)
//    then one v_pk_mul_f16 by the E4M3 block scale converted to fp16 (both
//    exact), products exact in fp32, FP32 accumulation in the MFMA.
//  * Up to 32 activation rows with K up to about 5.9K, a second kernel keeps
//    all activation codes and scale rows in LDS: a workgroup of three such
//    quads of waves (one per CU) stages them once, and its main loop issues
//    weight loads only.  The dispatch (launch_gemm_decode) picks between the
//    two, and the weight rows per workgroup, by how many workgroups the
//    shape gives against the chip's slots.
//  * K % 256 == 128 (e.g. a row-parallel shard) ends in half a super-group:
//    the first kernel zeroes the scales of its blocks past K.
#include "gemm_common.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

using namespace gemm;

constexpr int kWaves = 4;
constexpr int kSuperK = 256;  // K elements per super-group: one 128-byte code line per row
// LDS bytes for staged scale rows: at least 32 KiB, or all of what the
// partial-sum reduction takes anyway when that is more
template <int MT, int T>
constexpr int scale_lds_bytes() {
  return kWaves * 16 * MT * (16 * T + 4) * 4 > 32768 ? kWaves * 16 * MT * (16 * T + 4) * 4 : 32768;
}
constexpr int64_t kDecodeMaxRows = 256;  // up to four 64-row blocks of activations (grid.y)

typedef float float4_v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

#if defined(__HIP_DEVICE_COMPILE__)

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

__device__ __forceinline__ uint32_t word_at(const uint4 (&v)[2], int s) {
  const uint4& h = v[s >> 2];
  return (s & 3) == 0 ? h.x : (s & 3) == 1 ? h.y : (s & 3) == 2 ? h.z : h.w;
}

// one tile's share of a super-group: 32 code bytes and 4 scale bytes per lane
struct Frag {
  uint4 c[2];
  uint32_t s;
};

template <int MT, int T>
struct Super {
  Frag w[T];
  Frag a[MT];
};

// four consecutive outputs of row m from column n on (columns past N dropped)
template <int OUT>
__device__ __forceinline__ void store_run4(void* c, int64_t ldc, int64_t m, int64_t n, int64_t N, const float (&o)[4],
                                           bool vec_ok) {
  if constexpr (OUT == 0) {
    float* p = static_cast<float*>(c) + m * ldc + n;
    if (n + 3 < N && vec_ok) {
      *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < N) p[e] = o[e];
    }
  } else {
    uint16_t* p = static_cast<uint16_t*>(c) + m * ldc + n;
    uint16_t b[4];
    if constexpr (OUT == 1) {
      const uint32_t lo = bf16x2_rne_bits(o[0], o[1]), hi = bf16x2_rne_bits(o[2], o[3]);
      b[0] = (uint16_t)lo;
      b[1] = (uint16_t)(lo >> 16);
      b[2] = (uint16_t)hi;
      b[3] = (uint16_t)(hi >> 16);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const _Float16 hv = (_Float16)o[e];
        __builtin_memcpy(&b[e], &hv, 2);
      }
    }
    if (n + 3 < N && (reinterpret_cast<uintptr_t>(p) % 8) == 0) {
      *reinterpret_cast<uint2*>(p) = make_uint2((uint32_t)b[0] | ((uint32_t)b[1] << 16),
                                                (uint32_t)b[2] | ((uint32_t)b[3] << 16));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < N) p[e] = b[e];
    }
  }
}

#endif  // __HIP_DEVICE_COMPILE__

// MT activation tiles of 16 rows (M <= 16*MT), T weight tiles of 16 rows per
// workgroup, OCC waves per SIMD.  SL: the workgroup's scale rows (weight and
// activation, all of K) are staged in LDS once, with coalesced 16-byte loads,
// instead of 4 bytes per row and super-group from memory.
template <int MT, int T, int OCC, bool SL, bool KT, int OUT>
__global__ __launch_bounds__(kThreads, OCC) void gemm_decode_kernel(int64_t M_all, int64_t N, int64_t K,
                                                                  const uint8_t* __restrict__ a_codes,
                                                                  const uint8_t* __restrict__ a_scales,
                                                                  const float* __restrict__ a_gscale,
                                                                  const uint8_t* __restrict__ w_codes,
                                                                  const uint8_t* __restrict__ w_scales,
                                                                  const float* __restrict__ w_gscale,
                                                                  void* __restrict__ c, int64_t ldc) {
#if defined(__HIP_DEVICE_COMPILE__)
  // blockIdx.y picks a block of 16*MT activation rows (one block when M <= 16*MT;
  // the blocks stream the same weight rows at about the same time, so all but
  // the first read of a line come from the caches)
  const int64_t m0 = (int64_t)blockIdx.y * (16 * MT);
  const int64_t M = min((int64_t)(16 * MT), M_all - m0);
  a_codes += m0 * (K / 2);
  a_scales += m0 * (K / 16);
  c = static_cast<uint8_t*>(c) + m0 * ldc * (OUT == 0 ? 4 : 2);
  constexpr int R = 16 * T;      // weight rows per workgroup
  constexpr int kPitch = R + 4;  // fp32 words per staged partial row (pad breaks bank aliasing)
  constexpr int kRows = 16 * MT; // activation rows per workgroup
  constexpr int kPartBytes = kWaves * kRows * kPitch * 4;
  constexpr int kScaleLdsBytes = scale_lds_bytes<MT, T>();
  constexpr int kLdsBytes = SL ? (kPartBytes > kScaleLdsBytes ? kPartBytes : kScaleLdsBytes) : kPartBytes;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  float* const part = reinterpret_cast<float*>(lds);  // [kWaves][kRows * kPitch], after the main loop

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, q = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * R;

  const int64_t code_ld = K / 2, scale_ld = K / 16;
  const __amdgpu_buffer_rsrc_t wc_r =
      __builtin_amdgcn_make_buffer_rsrc((void*)w_codes, (short)0, (int)(N * code_ld), 0x00020000);
  const __amdgpu_buffer_rsrc_t ws_r =
      __builtin_amdgcn_make_buffer_rsrc((void*)w_scales, (short)0, (int)(N * scale_ld), 0x00020000);
  const __amdgpu_buffer_rsrc_t ac_r =
      __builtin_amdgcn_make_buffer_rsrc((void*)a_codes, (short)0, (int)(M * code_ld), 0x00020000);
  const __amdgpu_buffer_rsrc_t as_r =
      __builtin_amdgcn_make_buffer_rsrc((void*)a_scales, (short)0, (int)(M * scale_ld), 0x00020000);

  // per-lane row offsets; rows past the matrix repeat the last row (results never stored)
  uint32_t wc_off[T], ws_off[T], ac_off[MT], as_off[MT];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    int64_t r = n0 + 16 * t + lr;
    r = r < N ? r : N - 1;
    wc_off[t] = (uint32_t)(r * code_ld + 32 * q);
    ws_off[t] = (uint32_t)(r * scale_ld + 4 * q);
  }
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    int64_t r = 16 * i + lr;
    r = r < M ? r : M - 1;
    ac_off[i] = (uint32_t)(r * code_ld + 32 * q);
    as_off[i] = (uint32_t)(r * scale_ld + 4 * q);
  }

  // this wave's super-groups
  // KT: K % 256 == 128, the last super-group holds only its first 128 elements
  const int G = (int)((K + kSuperK - 1) / kSuperK);
  // super-groups wv, wv+4, wv+8, ...: the four waves read adjacent lines of
  // the same rows at about the same time (DRAM page locality)
  const int ng = (G - wv + kWaves - 1) / kWaves;
  auto gidx = [&](int jj) { return wv + kWaves * jj; };

  // scale rows in LDS: weight rows 0..R-1, then activation rows R..R+kRows-1
  const int srow = (int)scale_ld;  // bytes per scale row
  const int chunks_per_row = srow / 16;
  const int n_chunks = (R + kRows) * chunks_per_row;
  // row = chunk / chunks_per_row by a multiply with ceil(2^32 / chunks_per_row)
  // and a shift: exact for chunk < 2^14 and chunks_per_row < 2^12
  const uint64_t row_mag = (0xFFFFFFFFull + (uint64_t)chunks_per_row) / (uint64_t)chunks_per_row;
  auto chunk_row = [&](int f) { return (int)(((uint64_t)(uint32_t)f * row_mag) >> 32); };
  // chunks per thread: enough for every chunk the host lets through (n_chunks * 16 <= kScaleLdsBytes)
  constexpr int kChunksPer = (kScaleLdsBytes / 16 + kThreads - 1) / kThreads;

  // KT: in the last, half super-group the lanes with q >= 2 (blocks 8..15,
  // past the end of K) read the first half's bytes again, inside the row;
  // compute() zeroes their scale words, so they add nothing
  auto past_k = [&](int g) { return KT && g == G - 1 && q >= 2; };
  auto load = [&](Super<MT, T>& b, int g) {
    g = max(0, min(g, G - 1));
    const int cs = g * (kSuperK / 2), ss = g * (kSuperK / 16);
    const uint32_t back_c = past_k(g) ? 64u : 0u, back_s = past_k(g) ? 8u : 0u;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      b.w[t].c[0] = load16(wc_r, wc_off[t] - back_c, cs);
      b.w[t].c[1] = load16(wc_r, wc_off[t] - back_c, cs + 16);
      if constexpr (!SL) b.w[t].s = load4(ws_r, ws_off[t] - back_s, ss);
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      b.a[i].c[0] = load16(ac_r, ac_off[i] - back_c, cs);
      b.a[i].c[1] = load16(ac_r, ac_off[i] - back_c, cs + 16);
      if constexpr (!SL) b.a[i].s = load4(as_r, as_off[i] - back_s, ss);
    }
    // each super-group's loads stay together and in issue order (prologue and
    // loop alike), so the wait before its use counts only the one issued after it
    __builtin_amdgcn_sched_barrier(0);
  };

  float4_v acc[MT][T];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[i][t] = float4_v{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](Super<MT, T>& b, int g) {
    if constexpr (KT) {
      if (past_k(g)) {
#pragma unroll
        for (int t = 0; t < T; ++t) b.w[t].s = 0u;
#pragma unroll
        for (int i = 0; i < MT; ++i) b.a[i].s = 0u;
      }
    }
    if constexpr (SL) {
      // this lane's four scale bytes of super-group g (blocks 4q..4q+3)
      const int off = g * 16 + 4 * q;
#pragma unroll
      for (int t = 0; t < T; ++t) b.w[t].s = *reinterpret_cast<const uint32_t*>(lds + (16 * t + lr) * srow + off);
#pragma unroll
      for (int i = 0; i < MT; ++i)
        b.a[i].s = *reinterpret_cast<const uint32_t*>(lds + (R + 16 * i + lr) * srow + off);
    }
    // scale byte s/2 of a lane's four, as an fp16 pair (exact), broadcast
    auto scale_at = [&](uint32_t w, int s) {
      const half2_t sp = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w >> (16 * (s >> 2)), 1.0f, false);
      const _Float16 v = sp[(s >> 1) & 1];
      return half2_t{v, v};
    };
    // software pipeline over the 8*T (step, weight tile) regions, one weight
    // fragment per scheduling region: the MFMAs of region r are issued before
    // the decode of region r+1 (the activation fragments are decoded with the
    // first region of each step)
    half8_t fa[MT], fw;
#pragma unroll
    for (int i = 0; i < MT; ++i) fa[i] = decode8(word_at(b.a[i].c, 0), scale_at(b.a[i].s, 0));
    fw = decode8(word_at(b.w[0].c, 0), scale_at(b.w[0].s, 0));
#pragma unroll
    for (int r = 0; r < 8 * T; ++r) {
      const int t = r % T;
#pragma unroll
      for (int i = 0; i < MT; ++i) acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fw, fa[i], acc[i][t], 0, 0, 0);
      if (r + 1 < 8 * T) {
        const int s2 = (r + 1) / T, t2 = (r + 1) % T;
        const half8_t fw2 = decode8(word_at(b.w[t2].c, s2), scale_at(b.w[t2].s, s2));
        half8_t fa2[MT];
        if (t2 == 0) {
#pragma unroll
          for (int i = 0; i < MT; ++i) fa2[i] = decode8(word_at(b.a[i].c, s2), scale_at(b.a[i].s, s2));
        }
        __builtin_amdgcn_sched_barrier(0);
        fw = fw2;
        if (t2 == 0) {
#pragma unroll
          for (int i = 0; i < MT; ++i) fa[i] = fa2[i];
        }
      }
    }
  };

  // two super-groups in flight; loads past this wave's range re-read its last
  // super-group (cache hits, never multiplied)
  // the first two super-groups' code loads go out first, the scale-row
  // staging loads right behind them, so both latencies overlap
  Super<MT, T> b0, b1;
  load(b0, gidx(0));
  load(b1, gidx(min(1, max(ng - 1, 0))));
  if constexpr (SL) {
    // straight-line, clamped (always valid) chunk indices: every load is
    // issued before the first wait; a thread past the end repeats the last
    // chunk and writes the same bytes to the same place
    uint4 stage[kChunksPer];
#pragma unroll
    for (int u = 0; u < kChunksPer; ++u) {
      const int f = min(tid + u * kThreads, n_chunks - 1);
      const int row = chunk_row(f), ch = f - row * chunks_per_row;
      // both candidate rows computed, then selected (no branch around the load)
      const bool wrow = row < R;
      const int rw = (int)min(n0 + row, N - 1), ra = (int)min((int64_t)(row - R), M - 1);
      const uint8_t* base = wrow ? w_scales : a_scales;
      const int r = wrow ? rw : ra;
      stage[u] = *reinterpret_cast<const uint4*>(base + (int64_t)r * scale_ld + 16 * ch);
    }
#pragma unroll
    for (int u = 0; u < kChunksPer; ++u) {
      const int f = min(tid + u * kThreads, n_chunks - 1);
      const int row = chunk_row(f), ch = f - row * chunks_per_row;
      *reinterpret_cast<uint4*>(lds + row * srow + 16 * ch) = stage[u];
    }
    __syncthreads();
  }

  int j = 0;
  for (; j + 2 <= ng; j += 2) {
    compute(b0, gidx(j));
    load(b0, gidx(min(j + 2, ng - 1)));
    compute(b1, gidx(j + 1));
    load(b1, gidx(min(j + 3, ng - 1)));
  }
  if (j < ng) compute(b0, gidx(j));
  if constexpr (SL) __syncthreads();  // the partial sums reuse the scale rows' LDS

  // acc[i][t]: lane holds activation row 16i + lane%16 and weight rows
  // 16t + 4q + 0..3
  float* mine = part + wv * (kRows * kPitch);
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < T; ++t)
      *reinterpret_cast<float4_v*>(mine + (16 * i + lr) * kPitch + 16 * t + 4 * q) = acc[i][t];
  __syncthreads();

  // sum the four waves' partial sums in a fixed order, apply alpha, store 4 columns per thread
  const float alpha = 1.0f / (*a_gscale * *w_gscale);
  constexpr int kRuns = R / 4;  // runs of 4 columns per row
  const bool vec_ok = (reinterpret_cast<uintptr_t>(c) % 16) == 0 && (ldc * (OUT == 0 ? 4 : 2)) % 16 == 0;
  for (int f = tid; f < kRows * kRuns; f += kThreads) {
    const int row = f / kRuns, run = f % kRuns;
    const int64_t m = row;
    const int64_t n = n0 + 4 * run;
    if (m >= M || n >= N) continue;
    float4_v s = *reinterpret_cast<const float4_v*>(part + row * kPitch + 4 * run);
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
      s += *reinterpret_cast<const float4_v*>(part + w * (kRows * kPitch) + row * kPitch + 4 * run);
    const float o[4] = {s[0] * alpha, s[1] * alpha, s[2] * alpha, s[3] * alpha};
    store_run4<OUT>(c, ldc, m, n, N, o, vec_ok);
  }
#endif
}

// ---------------------------------------------------------------------------
// Activations resident in LDS.  A wave's vector loads complete in issue
// order, so in the kernel above an activation fragment load (an L2 hit)
// issued behind weight loads holds its place until those come back from HBM:
// two in five of the loads in flight carry no HBM bytes.  Here a workgroup of
// Q quads (four waves each; each quad owns one group of R = 16*T weight rows
// over all of K, as a workgroup above does) first copies all activation codes
// and every scale row it uses into LDS, once, with coalesced 16-byte loads.
// The main loop then issues weight loads only and reads the activation
// fragments from LDS.  Q quads share one copy of A, so A is read from L2 Q
// times less often as well.
constexpr int kAlLdsBytes = 160 * 1024;  // all of a CU's LDS: one workgroup per CU
__host__ __device__ constexpr int64_t kib_round(int64_t bytes) { return (bytes + 1023) / 1024 * 1024; }

typedef __attribute__((address_space(3))) uint8_t* lds_ptr_t;
typedef __attribute__((address_space(3))) void* lds_void_t;

#if defined(__HIP_DEVICE_COMPILE__)
// s_waitcnt vmcnt(N), LDS and export counters unconstrained (the 6-bit vmcnt
// field is split over bits 3:0 and 15:14)
template <int N>
__device__ __forceinline__ void al_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x0F70);
}
// workgroup barrier ordering LDS only (direct-to-LDS loads are ordered by the
// explicit vmcnt wait before it; the weight loads still in flight need not drain)
__device__ __forceinline__ void al_lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
#endif
constexpr int kAlPad = 16;  // bytes added to each staged row: rows r and r+1 start 4 banks apart
constexpr int kAlT = 3, kAlQ = 3;  // 3 weight tiles per quad, 3 quads (12 waves) per workgroup
constexpr int kAlD = 2;  // super-groups of weight loads in flight per wave
constexpr int64_t kAlRowsPerWg = 16 * kAlT * kAlQ;

template <int MT, int T, int Q, int D, int OUT>
__global__ __launch_bounds__(kThreads * Q, Q) void gemm_decode_al_kernel(int64_t M, int64_t N, int64_t K,
                                                                      const uint8_t* __restrict__ a_codes,
                                                                      const uint8_t* __restrict__ a_scales,
                                                                      const float* __restrict__ a_gscale,
                                                                      const uint8_t* __restrict__ w_codes,
                                                                      const uint8_t* __restrict__ w_scales,
                                                                      const float* __restrict__ w_gscale,
                                                                      void* __restrict__ c, int64_t ldc) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int R = 16 * T;       // weight rows per quad
  constexpr int kRows = 16 * MT;  // activation rows
  constexpr int kPitch = R + 4;   // fp32 words per staged partial row
  constexpr int kPartBytes = kWaves * kRows * kPitch * 4;  // one quad's partial sums
  static_assert(Q * kPartBytes <= kAlLdsBytes, "partial sums fit");
  __shared__ __attribute__((aligned(16))) uint8_t lds[kAlLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qd = wave >> 2, wv = wave & 3;  // quad, wave within the quad
  const int lr = lane & 15, q = lane >> 4;
  const int64_t wg_row0 = (int64_t)blockIdx.x * (Q * R);
  const int64_t n0 = wg_row0 + qd * R;

  const int64_t code_ld = K / 2, scale_ld = K / 16;
  const int apitch = (int)code_ld + kAlPad;   // LDS bytes per activation code row
  const int spitch = (int)scale_ld + kAlPad;  // LDS bytes per scale row
  // LDS: activation codes [kRows][apitch], weight scale rows [Q*R, quad-major]
  // [spitch], activation scale rows [kRows][spitch], each region rounded up to
  // whole KiB; after the main loop the quads' partial sums overwrite the front
  const int a_bytes = (int)kib_round((int64_t)kRows * apitch);
  const int sw_bytes = (int)kib_round((int64_t)(Q * R) * spitch);
  const int sa_bytes = (int)kib_round((int64_t)kRows * spitch);
  uint8_t* const lds_a = lds;
  uint8_t* const lds_sw = lds + a_bytes;
  uint8_t* const lds_sa = lds_sw + sw_bytes;

  const __amdgpu_buffer_rsrc_t wc_r =
      __builtin_amdgcn_make_buffer_rsrc((void*)w_codes, (short)0, (int)(N * code_ld), 0x00020000);
  uint32_t wc_off[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    int64_t r = n0 + 16 * t + lr;
    r = r < N ? r : N - 1;
    wc_off[t] = (uint32_t)(r * code_ld + 32 * q);
  }

  const int G = (int)(K / kSuperK);
  const int ng = (G - wv + kWaves - 1) / kWaves;
  auto gidx = [&](int jj) { return wv + kWaves * jj; };

  // one weight tile's code bytes of a super-group (32 per lane)
  struct WCodes {
    uint4 c[2];
  };
  auto load_w = [&](WCodes (&b)[T], int g) {
    g = max(0, min(g, G - 1));
    const int cs = g * (kSuperK / 2);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      b[t].c[0] = load16(wc_r, wc_off[t], cs);
      b[t].c[1] = load16(wc_r, wc_off[t], cs + 16);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  float4_v acc[MT][T];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[i][t] = float4_v{0.f, 0.f, 0.f, 0.f};

  // super-group g: activation fragments and all scale words from LDS, then
  // 8 MFMA steps per weight tile and activation tile
  auto compute = [&](const WCodes (&bw)[T], int g) {
    Frag a[MT];
    uint32_t ws[T];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const uint8_t* pa = lds_a + (16 * i + lr) * apitch + g * (kSuperK / 2) + 32 * q;
      a[i].c[0] = *reinterpret_cast<const uint4*>(pa);
      a[i].c[1] = *reinterpret_cast<const uint4*>(pa + 16);
      a[i].s = *reinterpret_cast<const uint32_t*>(lds_sa + (16 * i + lr) * spitch + g * 16 + 4 * q);
    }
#pragma unroll
    for (int t = 0; t < T; ++t)
      ws[t] = *reinterpret_cast<const uint32_t*>(lds_sw + (qd * R + 16 * t + lr) * spitch + g * 16 + 4 * q);
    auto scale_at = [&](uint32_t w, int s) {
      const half2_t sp = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w >> (16 * (s >> 2)), 1.0f, false);
      const _Float16 v = sp[(s >> 1) & 1];
      return half2_t{v, v};
    };
    // software pipeline over the 8*T (step, weight tile) regions: the MFMAs of
    // region r are issued before the decode of region r+1
    half8_t fa[MT], fw;
#pragma unroll
    for (int i = 0; i < MT; ++i) fa[i] = decode8(word_at(a[i].c, 0), scale_at(a[i].s, 0));
    fw = decode8(word_at(bw[0].c, 0), scale_at(ws[0], 0));
#pragma unroll
    for (int r = 0; r < 8 * T; ++r) {
      const int t = r % T;
#pragma unroll
      for (int i = 0; i < MT; ++i) acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fw, fa[i], acc[i][t], 0, 0, 0);
      if (r + 1 < 8 * T) {
        const int s2 = (r + 1) / T, t2 = (r + 1) % T;
        const half8_t fw2 = decode8(word_at(bw[t2].c, s2), scale_at(ws[t2], s2));
        half8_t fa2[MT];
        if (t2 == 0) {
#pragma unroll
          for (int i = 0; i < MT; ++i) fa2[i] = decode8(word_at(a[i].c, s2), scale_at(a[i].s, s2));
        }
        __builtin_amdgcn_sched_barrier(0);
        fw = fw2;
        if (t2 == 0) {
#pragma unroll
          for (int i = 0; i < MT; ++i) fa[i] = fa2[i];
        }
      }
    }
  };

  // Staging, with direct-to-LDS buffer loads: one instruction moves 64 lanes
  // x 16 bytes into 1 KiB of consecutive LDS, each lane fetching the global
  // chunk that belongs at its slot.  No register holds a staged byte, so the
  // weight loads of all D super-groups go out at the start, right behind the
  // staging loads (a wave's loads complete in issue order).  Three regions,
  // each a whole number of KiB: activation code rows (pitch apitch), weight
  // scale rows and activation scale rows (pitch spitch).  Slot byte P of a
  // region is row P / pitch (a multiply with ceil(2^32 / pitch), exact while
  // P * pitch < 2^32) and column P % pitch; pad columns, rows past M or N and
  // the rounding tail fetch bytes of an existing row, never read as data.
  const lds_ptr_t lbase = (lds_ptr_t)lds;
  auto stage_region = [&](lds_ptr_t dst, int bytes, __amdgpu_buffer_rsrc_t src, int pitch, int64_t row0,
                          int64_t rows, int64_t ld) {
    const uint64_t mag = (uint64_t)(0xFFFFFFFFu / (uint32_t)pitch) + 1;
    for (int i = wave; i < bytes / 1024; i += kWaves * Q) {
      const uint32_t pos = (uint32_t)(i * 1024 + lane * 16);
      const uint32_t r = (uint32_t)(((uint64_t)pos * mag) >> 32);
      const uint32_t col = pos - r * (uint32_t)pitch;
      const int64_t gr = min(row0 + (int64_t)r, rows - 1);
      const uint32_t off = (uint32_t)(gr * ld) + (col < (uint32_t)ld ? col : 0u);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void_t)(dst + i * 1024), 16, off, 0, 0, 0);
    }
  };
  stage_region(lbase, a_bytes,
               __builtin_amdgcn_make_buffer_rsrc((void*)a_codes, (short)0, (int)(M * code_ld), 0x00020000), apitch, 0,
               M, code_ld);
  stage_region(lbase + a_bytes, sw_bytes,
               __builtin_amdgcn_make_buffer_rsrc((void*)w_scales, (short)0, (int)(N * scale_ld), 0x00020000), spitch,
               wg_row0, N, scale_ld);
  stage_region(lbase + a_bytes + sw_bytes, sa_bytes,
               __builtin_amdgcn_make_buffer_rsrc((void*)a_scales, (short)0, (int)(M * scale_ld), 0x00020000), spitch, 0,
               M, scale_ld);
  __builtin_amdgcn_sched_barrier(0);
  WCodes b[D][T];
#pragma unroll
  for (int d = 0; d < D; ++d) load_w(b[d], gidx(min(d, max(ng - 1, 0))));
  // this wave's staging loads have landed once only its 2*T*D weight loads
  // may be outstanding; then every wave's have, after the barrier
  al_wait_vmcnt<2 * T * D>();
  al_lds_barrier();

  // D super-groups of weight loads in flight per wave
  int j = 0;
  for (; j + D <= ng; j += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      compute(b[d], gidx(j + d));
      load_w(b[d], gidx(min(j + d + D, ng - 1)));
    }
  }
#pragma unroll
  for (int d = 0; d < D - 1; ++d)
    if (j + d < ng) compute(b[d], gidx(j + d));
  // (weight loads issued past a wave's last super-group only target registers)
  __syncthreads();  // every quad is done reading the staged rows

  float* const part = reinterpret_cast<float*>(lds + qd * kPartBytes);  // [kWaves][kRows * kPitch]
  float* mine = part + wv * (kRows * kPitch);
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < T; ++t)
      *reinterpret_cast<float4_v*>(mine + (16 * i + lr) * kPitch + 16 * t + 4 * q) = acc[i][t];
  __syncthreads();

  const float alpha = 1.0f / (*a_gscale * *w_gscale);
  constexpr int kRuns = R / 4;
  const bool vec_ok = (reinterpret_cast<uintptr_t>(c) % 16) == 0 && (ldc * (OUT == 0 ? 4 : 2)) % 16 == 0;
  for (int f = tid & (kThreads - 1); f < kRows * kRuns; f += kThreads) {
    const int row = f / kRuns, run = f % kRuns;
    const int64_t n = n0 + 4 * run;
    if (row >= M || n >= N) continue;
    float4_v s = *reinterpret_cast<const float4_v*>(part + row * kPitch + 4 * run);
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
      s += *reinterpret_cast<const float4_v*>(part + w * (kRows * kPitch) + row * kPitch + 4 * run);
    const float o[4] = {s[0] * alpha, s[1] * alpha, s[2] * alpha, s[3] * alpha};
    store_run4<OUT>(c, ldc, row, n, N, o, vec_ok);
  }
#endif
}

// LDS bytes the kernel above stages for these sizes
template <int MT, int T, int Q>
constexpr int64_t al_lds_bytes(int64_t k) {
  return kib_round((int64_t)(16 * MT) * (k / 2 + kAlPad)) + kib_round((int64_t)(Q * 16 * T) * (k / 16 + kAlPad)) +
         kib_round((int64_t)(16 * MT) * (k / 16 + kAlPad));
}

// D super-groups of weight loads in flight per wave
template <int MT, int T, int Q, int D>
hipError_t launch_decode_al(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                            const float* a_gscale, const uint8_t* w_codes, const uint8_t* w_scales,
                            const float* w_gscale, void* c, int out_dtype, int64_t ldc, hipStream_t stream) {
  const dim3 grid((unsigned)((n + Q * 16 * T - 1) / (Q * 16 * T)));
#define NVFP4_LAUNCH_AL(OUT)                                                                                 \
  gemm_decode_al_kernel<MT, T, Q, D, OUT><<<grid, kThreads * Q, 0, stream>>>(m, n, k, a_codes, a_scales, \
                                                                               a_gscale, w_codes, w_scales, \
                                                                               w_gscale, c, ldc)
  if (out_dtype == 0)
    NVFP4_LAUNCH_AL(0);
  else if (out_dtype == 1)
    NVFP4_LAUNCH_AL(1);
  else
    NVFP4_LAUNCH_AL(2);
#undef NVFP4_LAUNCH_AL
  return hipGetLastError();
}

template <int MT, int T, int OCC>
hipError_t launch_decode_cfg(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                             const float* a_gscale, const uint8_t* w_codes, const uint8_t* w_scales,
                             const float* w_gscale, void* c, int out_dtype, int64_t ldc, hipStream_t stream) {
  const dim3 grid((unsigned)((n + 16 * T - 1) / (16 * T)), (unsigned)((m + 16 * MT - 1) / (16 * MT)));
  // staged scale rows: all of them must fit, and 16-byte loads need 16-byte aligned rows
  const bool sl = (int64_t)(16 * T + 16 * MT) * (k / 16) <= scale_lds_bytes<MT, T>() &&
                  (reinterpret_cast<uintptr_t>(a_scales) % 16) == 0 && (reinterpret_cast<uintptr_t>(w_scales) % 16) == 0;
#define NVFP4_LAUNCH(SLV, KTV, OUT)                                                                            \
  gemm_decode_kernel<MT, T, OCC, SLV, KTV, OUT><<<grid, kThreads, 0, stream>>>(m, n, k, a_codes, a_scales,      \
                                                                              a_gscale, w_codes, w_scales,     \
                                                                              w_gscale, c, ldc)
#define NVFP4_LAUNCH_OUT(SLV, KTV)   \
  if (out_dtype == 0)                \
    NVFP4_LAUNCH(SLV, KTV, 0);       \
  else if (out_dtype == 1)           \
    NVFP4_LAUNCH(SLV, KTV, 1);       \
  else                               \
    NVFP4_LAUNCH(SLV, KTV, 2);
  // K % 256 == 128: a last half super-group, scales read from memory (the
  // scale rows are then not whole 16-byte chunks for the LDS staging)
  if (k % kSuperK != 0) {
    NVFP4_LAUNCH_OUT(false, true)
  } else if (sl) {
    NVFP4_LAUNCH_OUT(true, false)
  } else {
    NVFP4_LAUNCH_OUT(false, false)
  }
#undef NVFP4_LAUNCH_OUT
#undef NVFP4_LAUNCH
  return hipGetLastError();
}

}  // namespace

bool gemm_decode_supported(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                           const uint8_t* w_codes, const uint8_t* w_scales) {
  const bool aligned = (reinterpret_cast<uintptr_t>(a_codes) % 16) == 0 &&
                       (reinterpret_cast<uintptr_t>(w_codes) % 16) == 0 &&
                       (reinterpret_cast<uintptr_t>(a_scales) % 4) == 0 &&
                       (reinterpret_cast<uintptr_t>(w_scales) % 4) == 0;
  // buffer offsets and sizes are 32-bit
  const bool fits = n * (k / 2) < ((int64_t)1 << 31) && m * (k / 2) < ((int64_t)1 << 31);
  return aligned && fits && m <= kDecodeMaxRows && k % (kSuperK / 2) == 0;
}

hipError_t launch_gemm_decode(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                              const float* a_gscale, const uint8_t* w_codes, const uint8_t* w_scales,
                              const float* w_gscale, void* c, int out_dtype, int64_t ldc, hipStream_t stream) {
  // Up to 32 activation rows.  The time of a decode-shaped call is set by how
  // many weight rows each CU streams and by the serial chain of each wave's
  // super-groups, so the kernel is chosen by how many workgroups the shape
  // gives against the chip's slots (3 per CU for the first kernel):
  //  * the activations resident in LDS, 2 quads of 3, 2 or 1 weight tiles,
  //    with the fewest tiles that give at most one workgroup per CU;
  //  * else 2 weight tiles per workgroup when that fits one round of slots;
  //  * else the activations resident in LDS (one workgroup of 144 rows per
  //    CU) when it fits, the operands are 16-byte aligned and its grid fills
  //    one round (or, for 17-32 rows, ends in a round at least half full);
  //  * else 3 weight tiles per workgroup (4 for up to 16 rows).
  if (m <= 32) {
    const int64_t cus = device_cu_count();
    // Activations resident in LDS in smaller workgroups (2 quads, 96, 64 or
    // 32 weight rows) when that gives at most one workgroup per CU: the
    // weight loads then never queue behind activation loads.  Up to 24576
    // weight rows; 5-30% faster than the first kernel at M = 1-32.
    const bool al2_ok = (reinterpret_cast<uintptr_t>(a_codes) % 16) == 0 &&
                        (reinterpret_cast<uintptr_t>(a_scales) % 16) == 0 &&
                        (reinterpret_cast<uintptr_t>(w_scales) % 16) == 0 && k % kSuperK == 0;
    if (al2_ok && (n + 95) / 96 <= cus && (n + 63) / 64 > cus) {
      if (m <= 16 && al_lds_bytes<1, 3, 2>(k) <= kAlLdsBytes)
        return launch_decode_al<1, 3, 2, kAlD>(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c,
                                               out_dtype, ldc, stream);
      if (m > 16 && al_lds_bytes<2, 3, 2>(k) <= kAlLdsBytes)
        return launch_decode_al<2, 3, 2, kAlD>(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c,
                                               out_dtype, ldc, stream);
    }
    if (al2_ok && (n + 63) / 64 <= cus && 2 * ((n + 63) / 64) > cus) {
      if (m <= 16 && al_lds_bytes<1, 2, 2>(k) <= kAlLdsBytes)
        return launch_decode_al<1, 2, 2, kAlD>(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c,
                                               out_dtype, ldc, stream);
      if (m > 16 && al_lds_bytes<2, 2, 2>(k) <= kAlLdsBytes)
        return launch_decode_al<2, 2, 2, kAlD>(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c,
                                               out_dtype, ldc, stream);
    }
    if (al2_ok && (n + 31) / 32 <= cus) {
      if (m <= 16 && al_lds_bytes<1, 1, 2>(k) <= kAlLdsBytes)
        return launch_decode_al<1, 1, 2, kAlD>(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c,
                                               out_dtype, ldc, stream);
      if (m > 16 && al_lds_bytes<2, 1, 2>(k) <= kAlLdsBytes)
        return launch_decode_al<2, 1, 2, kAlD>(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c,
                                               out_dtype, ldc, stream);
    }
    if ((n + 31) / 32 <= 3 * cus) {
      if (m <= 16)
        return launch_decode_cfg<1, 2, 3>(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c,
                                          out_dtype, ldc, stream);
      return launch_decode_cfg<2, 2, 3>(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c,
                                        out_dtype, ldc, stream);
    }
    const bool al_ok = (reinterpret_cast<uintptr_t>(a_codes) % 16) == 0 &&
                       (reinterpret_cast<uintptr_t>(a_scales) % 16) == 0 &&
                       (reinterpret_cast<uintptr_t>(w_scales) % 16) == 0 && k % kSuperK == 0;
    // one round of its one-per-CU grid; for 17-32 rows also several rounds
    // when the last one is at least half full (an emptier last round, or 16
    // rows or fewer, is faster on the first kernel)
    const int64_t al_wgs = (n + kAlRowsPerWg - 1) / kAlRowsPerWg;
    const bool al_rounds_ok = al_wgs <= cus || (m > 16 && 2 * (al_wgs % cus) >= cus) || (m > 16 && al_wgs % cus == 0);
    if (m <= 16) {
      if (al_ok && al_wgs <= cus && al_lds_bytes<1, kAlT, kAlQ>(k) <= kAlLdsBytes)
        return launch_decode_al<1, kAlT, kAlQ, kAlD>(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales,
                                                     w_gscale, c, out_dtype, ldc, stream);
      return launch_decode_cfg<1, 4, 3>(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c,
                                        out_dtype, ldc, stream);
    }
    if (al_ok && al_rounds_ok && al_lds_bytes<2, kAlT, kAlQ>(k) <= kAlLdsBytes)
      return launch_decode_al<2, kAlT, kAlQ, kAlD>(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale,
                                                   c, out_dtype, ldc, stream);
    return launch_decode_cfg<2, 3, 3>(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c, out_dtype,
                                      ldc, stream);
  }
  // 64 activation rows per workgroup (more in 64-row blocks along grid.y,
  // which stream the same weight rows again, mostly from the caches): one
  // workgroup reads each weight line once for all of them, at 2 waves per
  // SIMD (3 would spill).  3 weight tiles per workgroup when that gives every
  // CU at most one workgroup and 2 would not (with 2, the CUs that get a
  // second workgroup set the time); else 2 when a block's workgroups fit one
  // round of slots (2 per CU), else 3
  const int64_t cus = device_cu_count(), blocks = (m + 63) / 64;
  if ((n + 31) / 32 * blocks > cus && (n + 47) / 48 * blocks <= cus)
    return launch_decode_cfg<4, 3, 2>(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c, out_dtype,
                                      ldc, stream);
  if ((n + 31) / 32 <= 2 * cus)
    return launch_decode_cfg<4, 2, 2>(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c, out_dtype,
                                      ldc, stream);
  return launch_decode_cfg<4, 3, 2>(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c, out_dtype,
                                    ldc, stream);
}

}  // namespace nvfp4
