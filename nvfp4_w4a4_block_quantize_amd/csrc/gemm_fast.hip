// Main GEMM path for gfx950: C = alpha * A_hat W_hat^T on NVFP4 operands
// (news article "Qwen3.8-27B最激进4bit量化开源，权重显存暴降2.9倍！", section 02:
// the W4A4 product of E2M1 codes with E4M3 scales per 16 elements and an FP32
// global scale per tensor), for k % 256 == 0.
//
// Tile: 256 x 256 per workgroup of 4 waves (2 x 2), 128 x 128 per wave = 4 x 4
// MFMA 32x32x16 tiles, 256 FP32 accumulators per lane.  One stage = 128 K
// elements = 8 MFMA steps of K 16.
//
// Data movement.  Global -> LDS uses buffer loads that write LDS directly: one
// instruction moves 64 lanes x 16 B of codes (or 64 x 4 B of scale words) into
// 1 KiB (256 B) of consecutive LDS, each lane fetching the global chunk that
// belongs at its slot; this produces the swizzled code rows and the
// [half][row] scale words without staging registers.  Two LDS buffers; the
// fragments of a stage (32 code bytes + one scale word per row and lane half)
// are double-buffered in registers, so a stage's LDS buffer is free as soon as
// its fragments have been read.
//
// Per stage kt (fragments of kt already in registers, step 0 decoded):
//   steps 0-3: MFMAs of step s, interleaved with the decode of step s+1;
//   wait for this wave's loads of stage kt+1, one workgroup barrier;
//   step 4: MFMAs interleaved with the LDS reads of stage kt+1's fragments and
//           the global loads of stage kt+2 (into buffer kt%2);
//   steps 5-7: as 0-3; step 7 decodes step 0 of stage kt+1.
// Interleaving is fixed in source: every MFMA is followed by half a fragment's
// decode (2 x v_cvt_scalef32_pk_f16_fp4 + 2 x v_pk_mul_f16) and a scheduling
// fence, which keeps the VALU work under the MFMA shadow.
#include "gemm_common.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

using namespace gemm;

constexpr int BM = 256, BN = 256, TM = 128, TN = 128, FM = 4, FN = 4;
using L = Layout<BM, BN>;

typedef __attribute__((address_space(3))) uint8_t* lds_ptr_t;
typedef __attribute__((address_space(3))) void* lds_void_t;

#if defined(__HIP_DEVICE_COMPILE__)

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);  // vmcnt(N); lgkm and exp counters unconstrained
}

__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

template <int ROWS>
struct DirectLoader {
  static constexpr int kCodeInstr = ROWS / 64;    // per wave: ROWS*4 chunks / 64 lanes / 4 waves
  static constexpr int kScaleInstr = ROWS / 128;  // per wave: 2*ROWS words / 64 lanes / 4 waves
  static_assert(ROWS % 128 == 0, "rows per tile");
  __amdgpu_buffer_rsrc_t codes_rsrc, scales_rsrc;
  uint32_t code_off[kCodeInstr];
  uint32_t scale_off[kScaleInstr];

  __device__ __forceinline__ void init(const uint8_t* codes, const uint8_t* scales, int64_t row0, int64_t rows,
                                       int64_t k, int wave, int lane) {
    codes_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)codes, (short)0, (int)(rows * (k / 2)), 0x00020000);
    scales_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)scales, (short)0, (int)(rows * (k / 16)), 0x00020000);
#pragma unroll
    for (int i = 0; i < kCodeInstr; ++i) {
      const int p = (wave * kCodeInstr + i) * 64 + lane;  // 16-byte LDS slot of this lane
      const int row = p >> 2;
      const int chunk = (p & 3) ^ swz(row);
      int64_t r = row0 + row;
      r = r < rows ? r : rows - 1;  // rows past the matrix repeat the last one (never stored)
      code_off[i] = (uint32_t)(r * (k / 2) + chunk * 16);
    }
#pragma unroll
    for (int i = 0; i < kScaleInstr; ++i) {
      const int p = (wave * kScaleInstr + i) * 64 + lane;  // scale word slot, [half][row]
      const int h = p >= ROWS ? 1 : 0;
      const int row = p - h * ROWS;
      int64_t r = row0 + row;
      r = r < rows ? r : rows - 1;
      scale_off[i] = (uint32_t)(r * (k / 16) + h * 4);
    }
  }

  __device__ __forceinline__ void issue_code(lds_ptr_t lds_codes, int i, int kt, int wave) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(codes_rsrc, (lds_void_t)(lds_codes + (wave * kCodeInstr + i) * 1024), 16,
                                             code_off[i], kt * kRowBytes, 0, 0);
  }
  __device__ __forceinline__ void issue_scale(lds_ptr_t lds_scales, int i, int kt, int wave) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(scales_rsrc, (lds_void_t)(lds_scales + (wave * kScaleInstr + i) * 256),
                                             4, scale_off[i], kt * kBlocksPerStage, 0, 0);
  }
};

constexpr int kLoadsPerStage = 2 * (DirectLoader<BM>::kCodeInstr + DirectLoader<BM>::kScaleInstr);  // A and W

struct Frags {
  uint4 a[FM][2], w[FN][2];
  uint32_t sa[FM], sw[FN];
};

__device__ __forceinline__ uint32_t word_of(const uint4 (&q)[2], int s) {
  const uint4& v = q[s >> 2];
  return (s & 3) == 0 ? v.x : (s & 3) == 1 ? v.y : (s & 3) == 2 ? v.z : v.w;
}

// (S_q, S_q) as fp16 for block q (0..3) of a scale word
__device__ __forceinline__ half2_t scale_pair(uint32_t w, int q) {
  const uint32_t dup = __builtin_amdgcn_perm(w, w, 0x0C0C0000u | (uint32_t)(q * 0x0101));
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(dup, 1.0f, false);
}

// elements 4*HALF .. 4*HALF+3 of a fragment
template <int HALF>
__device__ __forceinline__ void decode_half(uint32_t word, half2_t pair, half8_t& dst) {
  const half2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2 * HALF) * pair;
  const half2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2 * HALF + 1) * pair;
  dst[4 * HALF + 0] = v0[0];
  dst[4 * HALF + 1] = v0[1];
  dst[4 * HALF + 2] = v1[0];
  dst[4 * HALF + 3] = v1[1];
}

struct Tile {
  DirectLoader<BM> la;
  DirectLoader<BN> lw;
  lds_ptr_t lds;
  const uint8_t* smem;
  int wave, wm, wn, lr, h;
  float16_t acc[FM][FN];
  half8_t fa[FM], fw[FN];  // decoded operands of the current step
  half8_t ga[FM], gw[FN];  // decoded operands of the next step
  half2_t pa[FM], pw[FN];  // block-scale pairs for the next step

  __device__ __forceinline__ void issue_all(int kt) {
    const lds_ptr_t b = lds + (kt & 1) * L::stage_bytes;
#pragma unroll
    for (int i = 0; i < DirectLoader<BM>::kCodeInstr; ++i) la.issue_code(b + L::a_codes, i, kt, wave);
#pragma unroll
    for (int i = 0; i < DirectLoader<BM>::kScaleInstr; ++i) la.issue_scale(b + L::a_scales, i, kt, wave);
#pragma unroll
    for (int i = 0; i < DirectLoader<BN>::kCodeInstr; ++i) lw.issue_code(b + L::w_codes, i, kt, wave);
#pragma unroll
    for (int i = 0; i < DirectLoader<BN>::kScaleInstr; ++i) lw.issue_scale(b + L::w_scales, i, kt, wave);
  }

  // the g-th of 12 global loads of stage kt (interleaved issue)
  __device__ __forceinline__ void issue_one(int kt, int g) {
    const lds_ptr_t b = lds + (kt & 1) * L::stage_bytes;
    constexpr int C = DirectLoader<BM>::kCodeInstr, S = DirectLoader<BM>::kScaleInstr;
    if (g < C) la.issue_code(b + L::a_codes, g, kt, wave);
    else if (g < C + S) la.issue_scale(b + L::a_scales, g - C, kt, wave);
    else if (g < 2 * C + S) lw.issue_code(b + L::w_codes, g - C - S, kt, wave);
    else lw.issue_scale(b + L::w_scales, g - 2 * C - S, kt, wave);
  }

  // LDS reads of fragment f (0..3 = A, 4..7 = W) of the stage held in buffer `st`
  __device__ __forceinline__ void read_frag(Frags& fr, const uint8_t* st, int f) const {
    if (f < FM) {
      const int row = wm * TM + f * 32 + lr;
      const uint8_t* base = st + L::a_codes + row * kRowBytes;
      fr.a[f][0] = *reinterpret_cast<const uint4*>(base + (((2 * h) ^ swz(row)) << 4));
      fr.a[f][1] = *reinterpret_cast<const uint4*>(base + (((2 * h + 1) ^ swz(row)) << 4));
      fr.sa[f] = reinterpret_cast<const uint32_t*>(st + L::a_scales)[h * BM + row];
    } else {
      const int j = f - FM;
      const int row = wn * TN + j * 32 + lr;
      const uint8_t* base = st + L::w_codes + row * kRowBytes;
      fr.w[j][0] = *reinterpret_cast<const uint4*>(base + (((2 * h) ^ swz(row)) << 4));
      fr.w[j][1] = *reinterpret_cast<const uint4*>(base + (((2 * h + 1) ^ swz(row)) << 4));
      fr.sw[j] = reinterpret_cast<const uint32_t*>(st + L::w_scales)[h * BN + row];
    }
  }

  // chunk q (0..15) of the decode of step s of `src` into ga/gw
  __device__ __forceinline__ void decode_chunk(const Frags& src, int s, int q) {
    const int f = q >> 1;
    if (f < FM) {
      if ((q & 1) == 0) {
        pa[f] = scale_pair(src.sa[f], s >> 1);
        decode_half<0>(word_of(src.a[f], s), pa[f], ga[f]);
      } else {
        decode_half<1>(word_of(src.a[f], s), pa[f], ga[f]);
      }
    } else {
      const int j = f - FM;
      if ((q & 1) == 0) {
        pw[j] = scale_pair(src.sw[j], s >> 1);
        decode_half<0>(word_of(src.w[j], s), pw[j], gw[j]);
      } else {
        decode_half<1>(word_of(src.w[j], s), pw[j], gw[j]);
      }
    }
  }

  __device__ __forceinline__ void mfma(int q) {
    const int i = q / FN, j = q % FN;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fw[j], acc[i][j], 0, 0, 0);
  }

  __device__ __forceinline__ void advance() {
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = ga[i];
#pragma unroll
    for (int j = 0; j < FN; ++j) fw[j] = gw[j];
  }

  // one MFMA step on fa/fw while decoding step s_next of `src` (DECODE) into ga/gw
  template <bool DECODE>
  __device__ __forceinline__ void step(const Frags& src, int s_next) {
#pragma unroll
    for (int q = 0; q < FM * FN; ++q) {
      mfma(q);
      if constexpr (DECODE) decode_chunk(src, s_next, q);
      fence();
    }
    advance();
  }

  // step 4 after the barrier: also read the next stage's fragments and start
  // the global loads of the stage after it
  template <bool ISSUE>
  __device__ __forceinline__ void step_with_loads(const Frags& cur, Frags& nxt, const uint8_t* nxt_st, int kt_issue) {
#pragma unroll
    for (int q = 0; q < FM * FN; ++q) {
      if (q < FM + FN) read_frag(nxt, nxt_st, q);
      mfma(q);
      decode_chunk(cur, 5, q);
      // all fragment reads (q < 8) precede the first load into LDS, so no read
      // has to wait behind the new loads
      if constexpr (ISSUE) {
        if (q >= 8 && 2 * (q - 8) < kLoadsPerStage) issue_one(kt_issue, 2 * (q - 8));
        if (q >= 8 && 2 * (q - 8) + 1 < kLoadsPerStage) issue_one(kt_issue, 2 * (q - 8) + 1);
      }
      fence();
    }
    advance();
  }

  // One stage.  MORE: a next stage exists (read it into `nxt` after the
  // barrier and decode its step 0 at the end).  ISSUE: also start the global
  // loads of stage kt+2.
  template <bool MORE, bool ISSUE>
  __device__ __forceinline__ void stage(int kt, const Frags& cur, Frags& nxt) {
    step<true>(cur, 1);
    step<true>(cur, 2);
    step<true>(cur, 3);
    step<true>(cur, 4);
    if constexpr (MORE) {
      wait_vmcnt<0>();
      __syncthreads();
      step_with_loads<ISSUE>(cur, nxt, smem + ((kt + 1) & 1) * L::stage_bytes, kt + 2);
    } else {
      step<true>(cur, 5);
    }
    step<true>(cur, 6);
    step<true>(cur, 7);
    if constexpr (MORE) {
      step<true>(nxt, 0);
    } else {
      step<false>(nxt, 0);
    }
  }
};

#endif  // __HIP_DEVICE_COMPILE__

// XCD-aware tile id: consecutive workgroup ids go round-robin over the 8 XCDs;
// remap so that tiles adjacent in the grouped order share an XCD (and its L2).
__device__ __forceinline__ int xcd_remap(int pid, int total) {
  constexpr int kXcd = 8;
  const int xcd = pid % kXcd, local = pid / kXcd;
  const int per = total / kXcd, rem = total % kXcd;
  return xcd * per + min(xcd, rem) + local;
}

template <int OUT>
__global__ __launch_bounds__(kThreads, 1) void gemm_fast_kernel(int64_t M, int64_t N, int64_t K,
                                                                const uint8_t* __restrict__ a_codes,
                                                                const uint8_t* __restrict__ a_scales,
                                                                const float* __restrict__ a_gscale,
                                                                const uint8_t* __restrict__ w_codes,
                                                                const uint8_t* __restrict__ w_scales,
                                                                const float* __restrict__ w_gscale,
                                                                void* __restrict__ c, int64_t ldc, int tiles_m,
                                                                int tiles_n) {
#if defined(__HIP_DEVICE_COMPILE__)  // device-only types below; the host pass needs only the launch stub
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * L::stage_bytes];

  Tile t;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  t.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  t.wm = t.wave >> 1;
  t.wn = t.wave & 1;
  t.lr = lane & 31;
  t.h = lane >> 5;
  t.lds = (lds_ptr_t)smem;
  t.smem = smem;

  // grouped tile order (8 tile rows walk the N tiles together) on the XCD-remapped id
  const int total = tiles_m * tiles_n;
  const int tile = xcd_remap((int)blockIdx.x, total);
  constexpr int kGroup = 8;
  const int group_size = kGroup * tiles_n;
  const int first_m = (tile / group_size) * kGroup;
  const int gm_count = min(tiles_m - first_m, kGroup);
  const int tm = first_m + (tile % group_size) % gm_count;
  const int tn = (tile % group_size) / gm_count;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  t.la.init(a_codes, a_scales, m0, M, K, t.wave, lane);
  t.lw.init(w_codes, w_scales, n0, N, K, t.wave, lane);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) t.acc[i][j] = float16_t{};

  const int nk = (int)(K / kBK);
  t.issue_all(0);
  t.issue_all(1);
  wait_vmcnt<kLoadsPerStage>();  // stage 0 landed; stage 1 may still be in flight
  __syncthreads();

  Frags fx, fy;  // the two fragment register sets, used in turn
#pragma unroll
  for (int f = 0; f < FM + FN; ++f) t.read_frag(fx, smem, f);
#pragma unroll
  for (int q = 0; q < 16; ++q) t.decode_chunk(fx, 0, q);
  t.advance();

  // nk is even and >= 2: pairs of stages alternate the two register sets
  for (int kt = 0; kt + 2 < nk; kt += 2) {
    t.stage<true, true>(kt, fx, fy);
    t.stage<true, true>(kt + 1, fy, fx);
  }
  t.stage<true, false>(nk - 2, fx, fy);
  t.stage<false, false>(nk - 1, fy, fx);

  // epilogue: alpha applied once, fp32 or RNE-narrowed store
  const float alpha = 1.0f / (*a_gscale * *w_gscale);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = n0 + t.wn * TN + j * 32 + t.lr;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + t.wm * TM + i * 32 + 8 * (e >> 2) + 4 * t.h + (e & 3);
        if (row < M && col < N) store_out<OUT>(c, row * ldc + col, t.acc[i][j][e] * alpha);
      }
    }
#endif
}

}  // namespace

bool gemm_fast_supported(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                         const uint8_t* w_codes, const uint8_t* w_scales) {
  const bool aligned = (reinterpret_cast<uintptr_t>(a_codes) % 16) == 0 &&
                       (reinterpret_cast<uintptr_t>(w_codes) % 16) == 0 &&
                       (reinterpret_cast<uintptr_t>(a_scales) % 4) == 0 &&
                       (reinterpret_cast<uintptr_t>(w_scales) % 4) == 0;
  // buffer offsets are 32-bit: each operand's code bytes must stay below 2^31
  const bool fits = m * (k / 2) < ((int64_t)1 << 31) && n * (k / 2) < ((int64_t)1 << 31);
  return aligned && fits && k % (2 * kBK) == 0 && m > 64;  // an even number of stages
}

hipError_t launch_gemm_fast(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                            const float* a_gscale, const uint8_t* w_codes, const uint8_t* w_scales,
                            const float* w_gscale, void* c, int out_dtype, int64_t ldc, hipStream_t stream) {
  const int tiles_m = (int)((m + BM - 1) / BM), tiles_n = (int)((n + BN - 1) / BN);
  const unsigned grid = (unsigned)tiles_m * (unsigned)tiles_n;
#define NVFP4_LAUNCH(OUT)                                                                                        \
  gemm_fast_kernel<OUT><<<grid, kThreads, 0, stream>>>(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, \
                                                       w_gscale, c, ldc, tiles_m, tiles_n)
  if (out_dtype == 0)
    NVFP4_LAUNCH(0);
  else if (out_dtype == 1)
    NVFP4_LAUNCH(1);
  else
    NVFP4_LAUNCH(2);
#undef NVFP4_LAUNCH
  return hipGetLastError();
}

}  // namespace nvfp4
