// Block-scaled 4-bit x 4-bit GEMM with FP32 accumulation for gfx950
// (news article "Qwen3.8-27B最激进4bit量化开源，权重显存暴降2.9倍！", section 02:
// W4A4 multiplies E2M1 operands carrying E4M3 scales per 16 elements and an
// FP32 global scale per tensor).
//
//   C[m][n] = alpha * sum_k (e2m1(a_mk) e4m3(sa)) (e2m1(w_nk) e4m3(sw)),
//   alpha = fp32(1 / fp32(g_a * g_w)).
//
// Design (MI355X / CDNA4):
//  * A workgroup of 4 waves owns a BM x BN tile of C; each wave a
//    (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA tiles with FP32
//    accumulators.
//  * The K loop walks stages of 128 elements.  A stage of packed codes (64 B
//    per row) and scale bytes (8 per row) for both operands is staged in LDS,
//    double-buffered, with one barrier per stage; the next stage's global
//    loads are in flight while the current one is multiplied.
//  * Decode happens in registers: every decoded operand e2m1(code)*e4m3(S)
//    has at most 6 significant bits and lies in [2^-10, 2688], so it is exact
//    in fp16.  v_cvt_scalef32_pk_f16_fp4 turns two codes into two fp16 values
//    (scale 1.0; the instruction applies only a power-of-two scale), and one
//    v_pk_mul_f16 by the block scale (converted exactly from E4M3 to fp16)
//    finishes two elements.  Products of two decoded operands are exact in
//    fp32, so v_mfma_f32_32x32x16_f16 accumulates exact products in FP32.
//  * K permutation: the 64 code bytes of a row and stage are split in two
//    32-byte halves; lane half h (lanes 0-31 / 32-63) reads half h with two
//    16-byte LDS reads, and MFMA step j (0..7) takes the j-th 32-bit word of
//    each half (elements 8j..8j+7 and 64+8j..64+8j+7).  A and W use the same
//    map, so every k of the stage is summed exactly once; each lane's 8
//    elements lie in one 16-element block, so one scale byte covers them.
//  * LDS code rows are 64 B with the 16-byte chunk index XOR-swizzled by
//    (row >> 1) & 3, so 8 lanes reading 8 consecutive rows hit 8 distinct
//    16-byte bank groups; scale words are stored [half][row] so a wave reads
//    128 contiguous bytes per half.
#include "gemm_common.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

using namespace gemm;

// ---------------------------------------------------------------- global -> LDS
// FAST: k % 128 == 0, codes 16-byte aligned rows (k % 32 == 0 follows), scale
// rows 8-byte aligned.  Every stage is full.
template <int ROWS>
struct FastLoader {
  static constexpr int kCodeChunks = ROWS * 4;  // 16-byte chunks per stage
  static constexpr int kCodeIters = (kCodeChunks + kThreads - 1) / kThreads;
  static constexpr int kScaleIters = (ROWS + kThreads - 1) / kThreads;
  uint4 code[kCodeIters];
  uint2 scale[kScaleIters];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                       int64_t row0, int64_t rows, int64_t k, int kt, int tid) {
    const int64_t code_ld = k / 2, scale_ld = k / 16;
#pragma unroll
    for (int i = 0; i < kCodeIters; ++i) {
      const int q = i * kThreads + tid;
      if (kCodeChunks % kThreads == 0 || q < kCodeChunks) {
        int64_t r = row0 + (q >> 2);
        r = r < rows ? r : rows - 1;
        code[i] = *reinterpret_cast<const uint4*>(codes + r * code_ld + (int64_t)kt * kRowBytes + (q & 3) * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < kScaleIters; ++i) {
      const int q = i * kThreads + tid;
      if (ROWS % kThreads == 0 || q < ROWS) {
        int64_t r = row0 + q;
        r = r < rows ? r : rows - 1;
        scale[i] = *reinterpret_cast<const uint2*>(scales + r * scale_ld + (int64_t)kt * kBlocksPerStage);
      }
    }
  }

  __device__ __forceinline__ void store(uint8_t* lds_codes, uint32_t* lds_scales, int tid) const {
#pragma unroll
    for (int i = 0; i < kCodeIters; ++i) {
      const int q = i * kThreads + tid;
      if (kCodeChunks % kThreads == 0 || q < kCodeChunks) {
        const int row = q >> 2;
        *reinterpret_cast<uint4*>(lds_codes + row * kRowBytes + (((q & 3) ^ swz(row)) << 4)) = code[i];
      }
    }
#pragma unroll
    for (int i = 0; i < kScaleIters; ++i) {
      const int q = i * kThreads + tid;
      if (ROWS % kThreads == 0 || q < ROWS) {
        lds_scales[q] = scale[i].x;
        lds_scales[ROWS + q] = scale[i].y;
      }
    }
  }
};

// GENERIC: k % 16 == 0 only.  Code rows are 8-byte aligned; one 8-byte unit is
// one 16-element block.  Units and scale bytes past k are zero (decode to 0).
template <int ROWS>
struct GenericLoader {
  static constexpr int kUnits = ROWS * kBlocksPerStage;
  static constexpr int kIters = (kUnits + kThreads - 1) / kThreads;
  uint2 code[kIters];
  uint32_t scale[kIters];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                       int64_t row0, int64_t rows, int64_t k, int kt, int tid) {
    const int64_t code_ld = k / 2, scale_ld = k / 16, nblocks = k / 16;
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int q = i * kThreads + tid;
      code[i] = make_uint2(0, 0);
      scale[i] = 0;
      if (kUnits % kThreads == 0 || q < kUnits) {
        int64_t r = row0 + (q >> 3);
        r = r < rows ? r : rows - 1;
        const int64_t blk = (int64_t)kt * kBlocksPerStage + (q & 7);
        if (blk < nblocks) {
          code[i] = *reinterpret_cast<const uint2*>(codes + r * code_ld + blk * 8);
          scale[i] = scales[r * scale_ld + blk];
        }
      }
    }
  }

  __device__ __forceinline__ void store(uint8_t* lds_codes, uint32_t* lds_scales, int tid) const {
    uint8_t* sc = reinterpret_cast<uint8_t*>(lds_scales);
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int q = i * kThreads + tid;
      if (kUnits % kThreads == 0 || q < kUnits) {
        const int row = q >> 3, u = q & 7;  // unit u = chunk u/2, half u%2
        *reinterpret_cast<uint2*>(lds_codes + row * kRowBytes + ((((u >> 1) ^ swz(row)) << 4) | ((u & 1) << 3))) =
            code[i];
        // scale word layout [half][row]: block u lives in half u/4, byte u%4
        sc[(((u >> 2) * ROWS + row) << 2) | (u & 3)] = (uint8_t)scale[i];
      }
    }
  }
};

// ---------------------------------------------------------------- kernel
template <int BM, int BN, int WM, int WN, bool FAST, int OUT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(int64_t M, int64_t N, int64_t K,
                                                        const uint8_t* __restrict__ a_codes,
                                                        const uint8_t* __restrict__ a_scales,
                                                        const float* __restrict__ a_gscale,
                                                        const uint8_t* __restrict__ w_codes,
                                                        const uint8_t* __restrict__ w_scales,
                                                        const float* __restrict__ w_gscale, void* __restrict__ c,
                                                        int64_t ldc, int tiles_m, int tiles_n) {
  static_assert(WM * WN == 4, "four waves");
  constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 MFMA tiles per wave
  static_assert(FM >= 1 && FN >= 1 && TM % 32 == 0 && TN % 32 == 0, "wave tile");
  using L = Layout<BM, BN>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * L::stage_bytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 31, h = lane >> 5;

  // grouped tile order: 8 tile rows per group walk the N tiles together (L2 reuse of W)
  const int tile = blockIdx.x;
  constexpr int kGroup = 8;
  const int group_size = kGroup * tiles_n;
  const int first_m = (tile / group_size) * kGroup;
  const int gm_count = min(tiles_m - first_m, kGroup);
  const int tm = first_m + (tile % group_size) % gm_count;
  const int tn = (tile % group_size) / gm_count;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  using LoaderA = typename std::conditional<FAST, FastLoader<BM>, GenericLoader<BM>>::type;
  using LoaderW = typename std::conditional<FAST, FastLoader<BN>, GenericLoader<BN>>::type;
  LoaderA ldA;
  LoaderW ldW;

  float16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = float16_t{};

  const int nk = (int)((K + kBK - 1) / kBK);
  ldA.load(a_codes, a_scales, m0, M, K, 0, tid);
  ldW.load(w_codes, w_scales, n0, N, K, 0, tid);
  ldA.store(smem + L::a_codes, reinterpret_cast<uint32_t*>(smem + L::a_scales), tid);
  ldW.store(smem + L::w_codes, reinterpret_cast<uint32_t*>(smem + L::w_scales), tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    uint8_t* st = smem + (kt & 1) * L::stage_bytes;
    // the next stage's loads (the last iteration loads its own stage again
    // into the buffer nobody reads after the loop: no branch around the
    // loader registers, which then stay in registers)
    const int kn = min(kt + 1, nk - 1);
    ldA.load(a_codes, a_scales, m0, M, K, kn, tid);
    ldW.load(w_codes, w_scales, n0, N, K, kn, tid);
    // fragments of this stage: 32 code bytes + one scale word per row
    uint4 ca[FM][2], cw[FN][2];
    half2_t sa[FM][4], sw[FN][4];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = wm * TM + i * 32 + lr;
      const uint8_t* base = st + L::a_codes + row * kRowBytes;
      ca[i][0] = *reinterpret_cast<const uint4*>(base + (((2 * h) ^ swz(row)) << 4));
      ca[i][1] = *reinterpret_cast<const uint4*>(base + (((2 * h + 1) ^ swz(row)) << 4));
      scale_pairs(reinterpret_cast<const uint32_t*>(st + L::a_scales)[h * BM + row], sa[i]);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int row = wn * TN + j * 32 + lr;
      const uint8_t* base = st + L::w_codes + row * kRowBytes;
      cw[j][0] = *reinterpret_cast<const uint4*>(base + (((2 * h) ^ swz(row)) << 4));
      cw[j][1] = *reinterpret_cast<const uint4*>(base + (((2 * h + 1) ^ swz(row)) << 4));
      scale_pairs(reinterpret_cast<const uint32_t*>(st + L::w_scales)[h * BN + row], sw[j]);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      half8_t fa[FM], fw[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint4& q = ca[i][s >> 2];
        const uint32_t word = (s & 3) == 0 ? q.x : (s & 3) == 1 ? q.y : (s & 3) == 2 ? q.z : q.w;
        fa[i] = decode8(word, sa[i][s >> 1]);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint4& q = cw[j][s >> 2];
        const uint32_t word = (s & 3) == 0 ? q.x : (s & 3) == 1 ? q.y : (s & 3) == 2 ? q.z : q.w;
        fw[j] = decode8(word, sw[j][s >> 1]);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fw[j], acc[i][j], 0, 0, 0);
    }
    {
      uint8_t* nx = smem + ((kt + 1) & 1) * L::stage_bytes;
      ldA.store(nx + L::a_codes, reinterpret_cast<uint32_t*>(nx + L::a_scales), tid);
      ldW.store(nx + L::w_codes, reinterpret_cast<uint32_t*>(nx + L::w_scales), tid);
    }
    __syncthreads();
  }

  // epilogue: alpha applied once, fp32 or RNE-narrowed store
  const float alpha = 1.0f / (*a_gscale * *w_gscale);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = n0 + wn * TN + j * 32 + lr;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * TM + i * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
        if (row < M && col < N) {
          const float v = acc[i][j][e] * alpha;
          if constexpr (OUT == 0) {
            static_cast<float*>(c)[row * ldc + col] = v;
          } else if constexpr (OUT == 1) {
            static_cast<uint16_t*>(c)[row * ldc + col] = (uint16_t)bf16_rne_bits(v);
          } else {
            static_cast<_Float16*>(c)[row * ldc + col] = (_Float16)v;
          }
        }
      }
    }
}

template <int BM, int BN, int WM, int WN, bool FAST>
hipError_t launch_cfg(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                      const float* a_gscale, const uint8_t* w_codes, const uint8_t* w_scales,
                      const float* w_gscale, void* c, int out_dtype, int64_t ldc, hipStream_t stream) {
  const int tiles_m = (int)((m + BM - 1) / BM), tiles_n = (int)((n + BN - 1) / BN);
  const unsigned grid = (unsigned)tiles_m * (unsigned)tiles_n;
#define NVFP4_LAUNCH(OUT)                                                                                     \
  gemm_kernel<BM, BN, WM, WN, FAST, OUT><<<grid, kThreads, 0, stream>>>(                                    \
      m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c, ldc, tiles_m, tiles_n)
  if (out_dtype == 0)
    NVFP4_LAUNCH(0);
  else if (out_dtype == 1)
    NVFP4_LAUNCH(1);
  else
    NVFP4_LAUNCH(2);
#undef NVFP4_LAUNCH
  return hipGetLastError();
}

}  // namespace

namespace {

// Between 65 and 256 activation rows both the prefill and the decode-shaped
// kernels apply.  Estimated times, from measurements of both on MI355X:
//  * prefill: rounds of 256x256 tiles over the CUs, about 0.0205 us per K
//    element of a tile (105 us at K = 5120), however few rows a tile holds;
//  * decode-shaped: one pass per 64-row block of activations, each streaming
//    the weight at about 4.1e6 weight elements per us, at least 10 us.
// The prefill kernel wins once its tiles fill the chip; with few tiles (small
// N, or a single 256-row tile row at large K) the decode-shaped passes do.
bool decode_beats_prefill(int64_t m, int64_t n, int64_t k) {
  const int64_t cus = device_cu_count();
  const int64_t tiles = ((m + 255) / 256) * ((n + 255) / 256);
  const double prefill_us = (double)((tiles + cus - 1) / cus) * 0.0205 * (double)k;
  const double pass_us = (double)n * (double)k / 4.1e6;
  const double decode_us = (double)((m + 63) / 64) * (pass_us > 10.0 ? pass_us : 10.0);
  return decode_us < prefill_us;
}

// A ragged last column strip (n % 256 in 1..128) of the prefill grid is a
// column of tm mostly empty 256x256 tiles.  When those tiles are what opens
// one more round of tiles on the CUs, that round (the strip alone) costs
// about a third of a full one (about 0.0205 * k / 3 us: with few CUs busy the
// chip holds a higher clock).  The decode-shaped kernel then takes the strip
// instead, in 64-row blocks (grid.y) spread over the whole chip, at about
// 330 TFLOP/s for these narrow shapes, right after the full columns.
bool split_ragged_strip(int64_t m, int64_t n, int64_t k) {
  const int64_t strip = n % 256;
  if (strip == 0 || strip > 128 || n < 256 || (m + 63) / 64 > 65535) return false;
  const int64_t cus = device_cu_count();
  const int64_t tm = (m + 255) / 256, tn = (n + 255) / 256;
  if ((tm * tn + cus - 1) / cus == (tm * (tn - 1) + cus - 1) / cus) return false;  // the strip adds no round
  const double tail_us = 0.0205 * (double)k / 3.0;
  const double strip_us = 2.0 * (double)m * (double)strip * (double)k / 3.3e8;
  return strip_us < tail_us;
}

// A call whose 256x256 tiles leave the last round of tiles over the CUs
// part-empty (MLP down, 8192x5120x17408: 640 tiles, 2.5 rounds of 256) gives
// the columns of that round to 256x128 tiles, twice as many, so that more CUs
// take part in it.  Returns how many 256-wide tile columns move to the
// 128-wide tiles, the fewest that leave the 256x256 part whole rounds, or 0
// when that is not estimated faster.  Fitted to same-box measurements: a
// round of 256x128 tiles takes about 0.82 of a round of full tiles (half the
// MFMAs each, but 1.5 times the decode per MFMA), and a part-empty round of
// full tiles about 0.95 (the chip clocks higher with fewer CUs busy).  Below
// K = 1024 a round is too short to pay for the second launch.  Only for n a
// multiple of 256.
int64_t half_tile_columns(int64_t m, int64_t n, int64_t k) {
  if (n % 256 != 0 || k < 1024) return 0;
  const int64_t cus = device_cu_count();
  const int64_t tm = (m + 255) / 256, tn = n / 256;
  if ((tm * tn) % cus == 0) return 0;
  const double unsplit = (double)((tm * tn) / cus) + 0.95;
  for (int64_t kk = 1; kk < tn; ++kk) {
    const int64_t main = tm * (tn - kk);
    if (main % cus != 0) continue;
    const int64_t half_rounds = (2 * tm * kk + cus - 1) / cus;
    const double split = (double)(main / cus) + 0.82 * (double)half_rounds;
    return split < unsplit ? kk : 0;
  }
  return 0;
}

}  // namespace

hipError_t launch_gemm(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                       const float* a_gscale, const uint8_t* w_codes, const uint8_t* w_scales,
                       const float* w_gscale, void* c, int out_dtype, int64_t ldc, hipStream_t stream) {
  // up to 32 activation rows against a large weight: the weight-streaming kernel
  if (gemm_stream_supported(m, n, k, a_codes, a_scales, w_codes, w_scales))
    return launch_gemm_stream(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c, out_dtype, ldc,
                              stream);
  const bool decode = gemm_decode_supported(m, n, k, a_codes, a_scales, w_codes, w_scales);
  const bool prefill = gemm_fast_supported(m, n, k, a_codes, a_scales, w_codes, w_scales);
  if (decode && (m <= 64 || !prefill || decode_beats_prefill(m, n, k)))
    return launch_gemm_decode(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c, out_dtype, ldc,
                              stream);
  if (prefill && split_ragged_strip(m, n, k)) {
    // full 256-column tiles, then the strip's weight rows and output columns
    const int64_t n_main = n - n % 256;
    const hipError_t e = launch_gemm_fast(m, n_main, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c,
                                          out_dtype, ldc, stream);
    if (e != hipSuccess) return e;
    const int64_t es = out_dtype == 0 ? 4 : 2;
    return launch_gemm_decode(m, n - n_main, k, a_codes, a_scales, a_gscale, w_codes + n_main * (k / 2),
                              w_scales + n_main * (k / 16), w_gscale, static_cast<uint8_t*>(c) + n_main * es,
                              out_dtype, ldc, stream);
  }
  if (prefill) {
    const int64_t kk = half_tile_columns(m, n, k);
    if (kk > 0) {
      // whole rounds of 256x256 tiles, then the last columns in 256x128 tiles
      const int64_t n_main = n - 256 * kk;
      const hipError_t e = launch_gemm_fast(m, n_main, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale,
                                            c, out_dtype, ldc, stream);
      if (e != hipSuccess) return e;
      const int64_t es = out_dtype == 0 ? 4 : 2;
      return launch_gemm_fast(m, n - n_main, k, a_codes, a_scales, a_gscale, w_codes + n_main * (k / 2),
                              w_scales + n_main * (k / 16), w_gscale, static_cast<uint8_t*>(c) + n_main * es,
                              out_dtype, ldc, stream, 128);
    }
    return launch_gemm_fast(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c, out_dtype, ldc,
                            stream);
  }
  const bool fast = (k % kBK) == 0 && (reinterpret_cast<uintptr_t>(a_codes) % 16) == 0 &&
                    (reinterpret_cast<uintptr_t>(w_codes) % 16) == 0 &&
                    (reinterpret_cast<uintptr_t>(a_scales) % 8) == 0 &&
                    (reinterpret_cast<uintptr_t>(w_scales) % 8) == 0;
  if (m <= 64) {
    if (fast)
      return launch_cfg<32, 256, 1, 4, true>(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c,
                                            out_dtype, ldc, stream);
    return launch_cfg<32, 256, 1, 4, false>(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c,
                                           out_dtype, ldc, stream);
  }
  if (fast)
    return launch_cfg<256, 256, 2, 2, true>(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c,
                                           out_dtype, ldc, stream);
  return launch_cfg<256, 256, 2, 2, false>(m, n, k, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c,
                                          out_dtype, ldc, stream);
}

}  // namespace nvfp4
