// Main GEMM path for gfx950: C = alpha * A_hat W_hat^T on NVFP4 operands
// (news article "Qwen3.8-27B最激进4bit量化开源，权重显存暴降2.9倍！", section 02:
// the W4A4 product of E2M1 codes with E4M3 scales per 16 elements and an FP32
// global scale per tensor), for k % 128 == 0.
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
// are double-buffered in registers; four LDS stage buffers (separate objects,
// so the compiler never waits on a direct load into one before reading
// another) keep the loads of stage kt+3 in flight while stage kt runs.
//
// Per stage kt (fragments of kt already in registers, step 0 decoded):
//   every step: MFMAs of step s interleaved with the decode of step s+1;
//   steps 0-5: also two of the global loads of stage kt+3 each;
//   after step 1: wait for this wave's loads of stage kt+1, one barrier;
//   steps 2-5: also the LDS reads of stage kt+1's fragments (two per step);
//   step 7 decodes step 0 of stage kt+1.
// Interleaving is fixed in source: every MFMA is followed by half a fragment's
// decode (two v_cvt_scalef32_pk_f16_fp4 for this chunk, two v_pk_mul_f16 for
// the previous chunk, so no multiply waits on the conversion just issued) and
// a scheduling fence, which keeps the VALU work under the MFMA shadow.
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

// s_waitcnt vmcnt(N) with the LDS and export counters unconstrained; the
// 6-bit vmcnt field is split over bits 3:0 and 15:14
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// Workgroup barrier for the stage buffers.  Each wave's direct-to-LDS loads of
// the stage about to be read are complete once the explicit vmcnt wait before
// the barrier returns (loads complete in issue order), so the loads of later
// stages may stay in flight across it.  A workgroup-scope release fence on LDS
// cannot be used here: direct-to-LDS loads count as LDS writes, so it waits
// for every one in flight (vmcnt(0)), which would drain the prefetch at every
// stage.  Instead the wave waits for its own LDS reads (lgkmcnt(0): no buffer
// is refilled while a read of it is pending), and the wavefront-scope fences
// only keep the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int ROWS>
struct DirectLoader {
  static constexpr int kCodeInstr = ROWS / 64;    // per wave: ROWS*4 chunks / 64 lanes / 4 waves
  static constexpr int kScaleInstr = ROWS / 128;  // per wave: 2*ROWS words / 64 lanes / 4 waves
  static_assert(ROWS % 128 == 0, "rows per tile");
  __amdgpu_buffer_rsrc_t codes_rsrc, scales_rsrc;
  uint32_t code_off[kCodeInstr];
  uint32_t scale_off[kScaleInstr];
  int nk;  // stages of K

  __device__ __forceinline__ void init(const uint8_t* codes, const uint8_t* scales, int64_t row0, int64_t rows,
                                       int64_t k, int wave, int lane) {
    nk = (int)(k / kBK);
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
  // A stage past the end of K (the loop runs whole groups of four stages)
  // gets zero block scales instead, so every operand it decodes is zero; its
  // code bytes are loaded as usual and multiplied by those zeros.
  template <bool TAIL = true>
  __device__ __forceinline__ void issue_scale(lds_ptr_t lds_scales, int i, int kt, int wave) const {
    const lds_ptr_t dst = lds_scales + (wave * kScaleInstr + i) * 256;
    if (!TAIL || kt < nk) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(scales_rsrc, (lds_void_t)dst, 4, scale_off[i], kt * kBlocksPerStage, 0,
                                               0);
    } else {
      reinterpret_cast<__attribute__((address_space(3))) uint32_t*>(dst)[__lane_id()] = 0u;
    }
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

struct Tile {
  DirectLoader<BM> la;
  DirectLoader<BN> lw;
  int wave, wm, wn, lr, h;
  float16_t acc[FM][FN];
  // decoded operands by step parity: F[p][0..3] = A fragments, F[p][4..7] = W
  half8_t F[2][FM + FN];
  // fp16 block-scale pairs (S_2b, S_2b+1) of the half stage being decoded
  half2_t SP[FM + FN];
  // converted-but-unscaled codes, double-buffered by chunk parity
  half2_t T[2][2];

  __device__ __forceinline__ void issue_all(lds_ptr_t b, int kt) {
#pragma unroll
    for (int i = 0; i < DirectLoader<BM>::kCodeInstr; ++i) la.issue_code(b + L::a_codes, i, kt, wave);
#pragma unroll
    for (int i = 0; i < DirectLoader<BM>::kScaleInstr; ++i) la.issue_scale(b + L::a_scales, i, kt, wave);
#pragma unroll
    for (int i = 0; i < DirectLoader<BN>::kCodeInstr; ++i) lw.issue_code(b + L::w_codes, i, kt, wave);
#pragma unroll
    for (int i = 0; i < DirectLoader<BN>::kScaleInstr; ++i) lw.issue_scale(b + L::w_scales, i, kt, wave);
  }

  // the g-th of the stage's global loads (interleaved issue)
  template <bool TAIL>
  __device__ __forceinline__ void issue_one(lds_ptr_t b, int kt, int g) {
    constexpr int C = DirectLoader<BM>::kCodeInstr, S = DirectLoader<BM>::kScaleInstr;
    if (g < C) la.issue_code(b + L::a_codes, g, kt, wave);
    else if (g < C + S) la.template issue_scale<TAIL>(b + L::a_scales, g - C, kt, wave);
    else if (g < 2 * C + S) lw.issue_code(b + L::w_codes, g - C - S, kt, wave);
    else lw.template issue_scale<TAIL>(b + L::w_scales, g - 2 * C - S, kt, wave);
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

  // Decode of step s is split in 16 chunks, chunk q = half (q & 1) of fragment
  // q >> 1.  start(): two code->fp16 conversions into T[q&1] (and, on the
  // first chunk of a fragment in a half stage, its scale pair).  finish():
  // the two block-scale multiplies into F[s&1], one chunk later.
  __device__ __forceinline__ void start(const Frags& src, int s, int q) {
    const int f = q >> 1, hf = q & 1;
    const uint32_t word = f < FM ? word_of(src.a[f], s) : word_of(src.w[f - FM], s);
    if (hf == 0 && (s & 3) == 0) {
      const uint32_t sw = f < FM ? src.sa[f] : src.sw[f - FM];
      SP[f] = s >= 4 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, true)
                     : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
    }
    if (hf == 0) {
      T[q & 1][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0);
      T[q & 1][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1);
    } else {
      T[q & 1][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2);
      T[q & 1][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3);
    }
  }
  __device__ __forceinline__ void finish(int s, int q) {
    const int f = q >> 1, hf = q & 1;
    const _Float16 sv = ((s >> 1) & 1) ? SP[f][1] : SP[f][0];
    const half2_t pair = {sv, sv};
    const half2_t v0 = T[q & 1][0] * pair;
    const half2_t v1 = T[q & 1][1] * pair;
    half8_t& d = F[s & 1][f];
    d[4 * hf + 0] = v0[0];
    d[4 * hf + 1] = v0[1];
    d[4 * hf + 2] = v1[0];
    d[4 * hf + 3] = v1[1];
  }

  // acc[i][j] = W fragment j times A fragment i: the MFMA tile's rows are
  // output columns, so each lane ends with four runs of four consecutive
  // output columns of one output row (lane l: row i*32 + l%32, columns
  // j*32 + 8g + 4*(l/32) + 0..3 for g = 0..3)
  __device__ __forceinline__ void mfma(int s, int q) {
    const int i = q / FN, j = q % FN;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(F[s & 1][FM + j], F[s & 1][i], acc[i][j], 0, 0, 0);
  }

  // Step S of a stage: the MFMAs of step S while decoding step S+1 of `cur`
  // (step 0 of `nxt` when S == 7).  Steps 0-5 also issue two of the twelve
  // global loads of stage kt+3 (slots 5 and 13); steps 2-5, after the barrier,
  // read two of the next stage's fragments from LDS (slots 0 and 8).
  template <int S, bool TAIL>
  __device__ __forceinline__ void step_s(const Frags& cur, Frags& nxt, const uint8_t* rd, lds_ptr_t ld, int kt_load) {
#pragma unroll
    for (int q = 0; q < FM * FN; ++q) {
      mfma(S, q);
      if (q == 0) finish(S, 15);
      if (q > 0) finish((S + 1) & 7, q - 1);
      if constexpr (S < 7) {
        start(cur, S + 1, q);
      } else {
        start(nxt, 0, q);
      }
      if constexpr (S >= 2 && S <= 5) {
        if ((q & 7) == 0) read_frag(nxt, rd, 2 * (S - 2) + (q >> 3));
      }
      if constexpr (S <= 5) {
        if ((q & 7) == 5) issue_one<TAIL>(ld, kt_load, 2 * S + (q >> 3));
      }
      fence();
    }
  }

  // One stage; `cur` holds stage kt (step 0 decoded but for chunk 15), stage
  // kt+1 sits in LDS buffer `rd` once every wave's loads of it have landed,
  // and `ld` (the buffer of stage kt-1, whose fragments every wave read during
  // stage kt-2) takes the global loads of stage kt+3.  Loads and reads issued
  // for stages past the end of K fetch data that is never multiplied.
  // TAIL: some stage this one loads or waits for may lie past the end of K
  // (only in the last iterations of the loop); it then checks.
  template <bool TAIL>
  __device__ __forceinline__ void stage(int kt, const Frags& cur, Frags& nxt, const uint8_t* rd, lds_ptr_t ld) {
    step_s<0, TAIL>(cur, nxt, rd, ld, kt + 3);
    step_s<1, TAIL>(cur, nxt, rd, ld, kt + 3);
    // stage kt+1 landed once at most stage kt+2's twelve loads and the four
    // of stage kt+3 issued in steps 0-1 are outstanding; a stage past the end
    // of K issues fewer loads (no scale loads), so near the end wait for all
    if (TAIL && kt + 2 >= la.nk) {
      wait_vmcnt<0>();
    } else {
      wait_vmcnt<kLoadsPerStage + 4>();
    }
    lds_barrier();
    step_s<2, TAIL>(cur, nxt, rd, ld, kt + 3);
    step_s<3, TAIL>(cur, nxt, rd, ld, kt + 3);
    step_s<4, TAIL>(cur, nxt, rd, ld, kt + 3);
    step_s<5, TAIL>(cur, nxt, rd, ld, kt + 3);
    step_s<6, TAIL>(cur, nxt, rd, ld, kt + 3);
    step_s<7, TAIL>(cur, nxt, rd, ld, kt + 3);
  }
};

#endif  // __HIP_DEVICE_COMPILE__

// two outputs rounded to nearest even bf16 / f16, packed low-first
template <int OUT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (OUT == 1) {
    return bf16x2_rne_bits(a, b);
  } else {
    const _Float16 ha = (_Float16)a, hb = (_Float16)b;
    uint16_t ua, ub;
    __builtin_memcpy(&ua, &ha, 2);
    __builtin_memcpy(&ub, &hb, 2);
    return (uint32_t)ua | ((uint32_t)ub << 16);
  }
}

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
  // four stage buffers as separate objects: the compiler can then tell that
  // a read of one never depends on a direct-to-LDS load into another
  __shared__ __attribute__((aligned(1024))) uint8_t buf0[L::stage_bytes];
  __shared__ __attribute__((aligned(1024))) uint8_t buf1[L::stage_bytes];
  __shared__ __attribute__((aligned(1024))) uint8_t buf2[L::stage_bytes];
  __shared__ __attribute__((aligned(1024))) uint8_t buf3[L::stage_bytes];
  const lds_ptr_t l0 = (lds_ptr_t)buf0, l1 = (lds_ptr_t)buf1, l2 = (lds_ptr_t)buf2, l3 = (lds_ptr_t)buf3;

  Tile t;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  t.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  t.wm = t.wave >> 1;
  t.wn = t.wave & 1;
  t.lr = lane & 31;
  t.h = lane >> 5;

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
  t.issue_all(l0, 0);
  t.issue_all(l1, 1);
  t.issue_all(l2, 2);
  // stage 0 landed (a stage past the end of K issues no scale loads: wait for all then)
  if (nk < 3) {
    wait_vmcnt<0>();
  } else {
    wait_vmcnt<2 * kLoadsPerStage>();
  }
  lds_barrier();

  Frags fx, fy;  // the two fragment register sets, used in turn
#pragma unroll
  for (int f = 0; f < FM + FN; ++f) t.read_frag(fx, buf0, f);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    t.start(fx, 0, q);
    if (q < 15) t.finish(0, q);  // chunk 15 is finished in the first slot of stage 0
  }

  // Four stages per iteration (stages past nk, up to the next multiple of
  // four, multiply zeros): two register sets x four LDS buffers, all static.  Stage kt reads stage kt+1 from buffer (kt+1)%4 and
  // loads stage kt+3 into buffer (kt+3)%4, which held stage kt-1 (already in
  // every wave's registers by the barrier of stage kt).
  // Iterations whose loads (stages kt+3 .. kt+6) all lie inside K take no
  // checks, and so does every iteration when K is a whole number of groups
  // of four stages (then no stage past the end is multiplied); otherwise the
  // last one or two check every load and wait.
  const int kt_plain = (nk & 3) == 0 ? nk : nk - 6;
  int kt = 0;
  for (; kt < kt_plain; kt += 4) {
    t.stage<false>(kt + 0, fx, fy, buf1, l3);
    t.stage<false>(kt + 1, fy, fx, buf2, l0);
    t.stage<false>(kt + 2, fx, fy, buf3, l1);
    t.stage<false>(kt + 3, fy, fx, buf0, l2);
  }
  for (; kt < nk; kt += 4) {
    t.stage<true>(kt + 0, fx, fy, buf1, l3);
    t.stage<true>(kt + 1, fy, fx, buf2, l0);
    t.stage<true>(kt + 2, fx, fy, buf3, l1);
    t.stage<true>(kt + 3, fy, fx, buf0, l2);
  }
  wait_vmcnt<0>();  // loads issued for stages past the end

  // Epilogue: alpha applied once.  16-bit outputs go through LDS (rows of
  // 128 values + 16 B pad, two passes of 64 rows per wave) so that each lane
  // stores 16 contiguous bytes and 16 lanes cover a 256-byte row segment;
  // fp32 output stores each run of four columns directly.
  const float alpha = 1.0f / (*a_gscale * *w_gscale);
  const bool vec_ok = (reinterpret_cast<uintptr_t>(c) % 16) == 0 && (ldc * (OUT == 0 ? 4 : 2)) % 16 == 0;
  const int64_t row_base = m0 + t.wm * TM, col_base = n0 + t.wn * TN;
  if constexpr (OUT == 0) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t row = row_base + i * 32 + t.lr;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t col = col_base + j * 32 + 8 * g + 4 * t.h;
          const float4 v = make_float4(t.acc[i][j][4 * g] * alpha, t.acc[i][j][4 * g + 1] * alpha,
                                       t.acc[i][j][4 * g + 2] * alpha, t.acc[i][j][4 * g + 3] * alpha);
          if (row < M) {
            float* p = static_cast<float*>(c) + row * ldc + col;
            if (col + 3 < N && vec_ok) {
              *reinterpret_cast<float4*>(p) = v;
            } else {
              if (col < N) p[0] = v.x;
              if (col + 1 < N) p[1] = v.y;
              if (col + 2 < N) p[2] = v.z;
              if (col + 3 < N) p[3] = v.w;
            }
          }
        }
    }
  } else {
    wait_vmcnt<0>();  // loads issued for stages past the end may still target LDS
    __syncthreads();  // every wave is done reading the stage buffers
    constexpr int kPitch = TN * 2 + 16;  // bytes per staged row
    static_assert(64 * kPitch <= L::stage_bytes, "a wave's staging rows fit in one stage buffer");
    // each wave stages in a stage buffer of its own (64 rows x kPitch fit in one)
    uint8_t* const stg = t.wave < 2 ? (t.wave == 0 ? buf0 : buf1) : (t.wave == 2 ? buf2 : buf3);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * half + ii;
        const int r = ii * 32 + t.lr;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            uint2 w;
            w.x = pack2<OUT>(t.acc[i][j][4 * g] * alpha, t.acc[i][j][4 * g + 1] * alpha);
            w.y = pack2<OUT>(t.acc[i][j][4 * g + 2] * alpha, t.acc[i][j][4 * g + 3] * alpha);
            *reinterpret_cast<uint2*>(stg + r * kPitch + (j * 32 + 8 * g + 4 * t.h) * 2) = w;
          }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are done
      __builtin_amdgcn_wave_barrier();
      // 64 rows x 256 B: lane reads 16 B; 16 lanes per row, 4 rows per pass
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        const int r = p * 4 + (lane >> 4);
        const int cb = (lane & 15) * 8;  // first of 8 columns
        const uint4 v = *reinterpret_cast<const uint4*>(stg + r * kPitch + cb * 2);
        const int64_t row = row_base + half * 64 + r;
        const int64_t col = col_base + cb;
        if (row < M) {
          uint16_t* q = static_cast<uint16_t*>(c) + row * ldc + col;
          if (col + 7 < N && vec_ok) {
            *reinterpret_cast<uint4*>(q) = v;
          } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (col + e < N) q[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
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
  return aligned && fits && k % kBK == 0 && m > 64;
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
