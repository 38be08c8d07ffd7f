// Main GEMM path for gfx950: C = alpha * A_hat W_hat^T on NVFP4 operands
// (news article "Qwen3.8-27B最激进4bit量化开源，权重显存暴降2.9倍！", section 02:
// the W4A4 product of E2M1 codes with E4M3 scales per 16 elements and an FP32
// global scale per tensor), for k % 128 == 0.
//
// Tile: 256 x BN per workgroup of 4 waves (2 x 2), 128 x BN/2 per wave = 4 x
// BN/64 MFMA 32x32x16 tiles (BN = 256: 256 FP32 accumulators per lane).  One
// stage = 128 K elements = 8 MFMA steps of K 16.  BN = 128 is for the last
// round of tiles of a call whose 256 x 256 tiles would leave it part-empty.
//
// Data movement.  Global -> LDS uses buffer loads that write LDS directly: one
// instruction moves 64 lanes x 16 B of codes (or 64 x 4 B of scale words) into
// 1 KiB (256 B) of consecutive LDS, each lane fetching the global chunk that
// belongs at its slot; this produces the swizzled code rows and the
// [half][row] scale words without staging registers.  The fragments of a
// stage (32 code bytes + one scale word per row and lane half) are
// double-buffered in registers, and four LDS stage buffers (separate objects,
// so the compiler never waits on a direct load into one before reading
// another) keep the loads of stage kt+3 in flight while stage kt runs.
//
// Per stage kt (fragments of kt already in registers, step 0 decoded):
//   every step: MFMAs of step s interleaved with the decode of step s+1;
//   steps 0-5: also two of the global loads of stage kt+3 each;
//   after step 1: wait for this wave's loads of stage kt+1, one barrier;
//   steps 2-5 (2-4 at BN = 128): also the LDS reads of stage kt+1's fragments
//   (two per step);
//   step 7 decodes step 0 of stage kt+1.
// Interleaving is fixed in source: the decode of a step is cut in chunks of
// half a fragment, spread evenly over the step's MFMAs (one per MFMA at
// BN = 256, one or two at BN = 128); a chunk's two v_cvt_scalef32_pk_f16_fp4
// are issued after one MFMA and its two v_pk_mul_f16 after the next, so no
// multiply waits on the conversion just issued, and a scheduling fence after
// each MFMA's share keeps the VALU work under the MFMA shadow.
#include "gemm_common.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

using namespace gemm;

constexpr int BM = 256, TM = 128, FM = 4;

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

  // this lane's source offsets within a tile's rows (the same for every tile)
  __device__ __forceinline__ void init_lanes(int64_t k, int wave, int lane) {
    nk = (int)(k / kBK);
#pragma unroll
    for (int i = 0; i < kCodeInstr; ++i) {
      const int p = (wave * kCodeInstr + i) * 64 + lane;  // 16-byte LDS slot of this lane
      const int row = p >> 2;
      const int chunk = (p & 3) ^ swz(row);
      code_off[i] = (uint32_t)(row * (k / 2) + chunk * 16);
    }
#pragma unroll
    for (int i = 0; i < kScaleInstr; ++i) {
      const int p = (wave * kScaleInstr + i) * 64 + lane;  // scale word slot, [half][row]
      const int h = p >= ROWS ? 1 : 0;
      const int row = p - h * ROWS;
      scale_off[i] = (uint32_t)(row * (k / 16) + h * 4);
    }
  }
  // the tile's first row: the resources start there and end with the
  // matrix, so rows past it read zeros (never stored); rows <= row0 leaves
  // the resources empty and every load reads nothing
  __device__ __forceinline__ void target(const uint8_t* codes, const uint8_t* scales, int64_t row0, int64_t rows,
                                         int64_t k) {
    const int64_t valid = rows > row0 ? rows - row0 : 0;
    codes_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(codes + row0 * (k / 2)), (short)0, (int)(valid * (k / 2)),
                                                   0x00020000);
    scales_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(scales + row0 * (k / 16)), (short)0,
                                                    (int)(valid * (k / 16)), 0x00020000);
  }
  // The whole matrix instead (the persistent kernel, whose tiles are all
  // whole): the tile is chosen by `tile_off`, a scalar byte offset of its
  // first row that every load adds (no record check needed: all rows exist).
  __device__ __forceinline__ void target_matrix(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                                int64_t k) {
    codes_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)codes, (short)0, (int)(rows * (k / 2)), 0x00020000);
    scales_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)scales, (short)0, (int)(rows * (k / 16)), 0x00020000);
  }
  // code bytes of the tile's first row; its scale bytes are 1/8 of that
  uint32_t tile_off = 0;

  __device__ __forceinline__ void issue_code(lds_ptr_t lds_codes, int i, int kt, int wave) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(codes_rsrc, (lds_void_t)(lds_codes + (wave * kCodeInstr + i) * 1024), 16,
                                             code_off[i], tile_off + kt * kRowBytes, 0, 0);
  }
  // A stage past the end of K (the loop runs whole groups of four stages)
  // gets zero block scales instead, so every operand it decodes is zero; its
  // code bytes are loaded as usual and multiplied by those zeros.
  template <bool TAIL = true>
  __device__ __forceinline__ void issue_scale(lds_ptr_t lds_scales, int i, int kt, int wave) const {
    const lds_ptr_t dst = lds_scales + (wave * kScaleInstr + i) * 256;
    if (!TAIL || kt < nk) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(scales_rsrc, (lds_void_t)dst, 4, scale_off[i],
                                               (tile_off >> 3) + kt * kBlocksPerStage, 0, 0);
    } else {
      reinterpret_cast<__attribute__((address_space(3))) uint32_t*>(dst)[__lane_id()] = 0u;
    }
  }
};

template <int FN>
struct Frags {
  uint4 a[FM][2], w[FN][2];
  uint32_t sa[FM], sw[FN];
};

__device__ __forceinline__ uint32_t word_of(const uint4 (&q)[2], int s) {
  const uint4& v = q[s >> 2];
  return (s & 3) == 0 ? v.x : (s & 3) == 1 ? v.y : (s & 3) == 2 ? v.z : v.w;
}

template <int BN>
struct Tile {
  static constexpr int TN = BN / 2, FN = TN / 32;
  static constexpr int NF = FM + FN;     // fragments decoded per step
  static constexpr int NQ = FM * FN;     // MFMAs per step
  static constexpr int NCH = 2 * NF;     // decode chunks per step
  using L = Layout<BM, BN>;
  using LA = DirectLoader<BM>;
  using LW = DirectLoader<BN>;
  using Fr = Frags<FN>;
  static constexpr int kLoads = LA::kCodeInstr + LA::kScaleInstr + LW::kCodeInstr + LW::kScaleInstr;
  static_assert(kLoads <= 12, "two load slots in each of steps 0-5");
  // the decode chunks started after MFMA q of a step: [first_chunk(q), first_chunk(q+1))
  static constexpr int first_chunk(int q) { return (q * NCH + NQ - 1) / NQ; }
  LA la;
  LW lw;
  int wave, wm, wn, lr, h;
  // this lane's LDS read offsets within a stage buffer, for fragment 0 of
  // each operand: code chunks 2h and 2h+1 of its row (swizzled) and its
  // scale word.  Fragment f's row is 32 f rows further and has the same
  // swizzle (it depends on row bits 1-3 only), so its offsets differ by
  // compile-time constants.
  uint32_t ra0, ra1, rsa, rw0, rw1, rsw;
  float16_t acc[FM][FN];
  // decoded operands by step parity: F[p][0..FM-1] = A fragments, F[p][FM..] = W
  half8_t F[2][NF];
  // fp16 block-scale pairs (S_2b, S_2b+1) of the half stage being decoded
  half2_t SP[NF];
  // converted-but-unscaled codes by chunk parity (at most two chunks wait)
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
    constexpr int CA = LA::kCodeInstr, SA = LA::kScaleInstr, CW = LW::kCodeInstr;
    if (g < CA) la.issue_code(b + L::a_codes, g, kt, wave);
    else if (g < CA + SA) la.template issue_scale<TAIL>(b + L::a_scales, g - CA, kt, wave);
    else if (g < CA + SA + CW) lw.issue_code(b + L::w_codes, g - CA - SA, kt, wave);
    else lw.template issue_scale<TAIL>(b + L::w_scales, g - CA - SA - CW, kt, wave);
  }

  __device__ __forceinline__ void init_reads() {
    const int s = swz(lr);
    const uint32_t arow = (uint32_t)((wm * TM + lr) * kRowBytes), wrow = (uint32_t)((wn * TN + lr) * kRowBytes);
    ra0 = arow + (uint32_t)(((2 * h) ^ s) << 4);
    ra1 = arow + (uint32_t)(((2 * h + 1) ^ s) << 4);
    rsa = (uint32_t)((h * BM + wm * TM + lr) * 4);
    rw0 = wrow + (uint32_t)(((2 * h) ^ s) << 4);
    rw1 = wrow + (uint32_t)(((2 * h + 1) ^ s) << 4);
    rsw = (uint32_t)((h * BN + wn * TN + lr) * 4);
  }

  // LDS reads of fragment f (0..FM-1 = A, FM.. = W) of the stage held in buffer `st`
  __device__ __forceinline__ void read_frag(Fr& fr, const uint8_t* st, int f) const {
    if (f < FM) {
      const uint8_t* base = st + L::a_codes + f * 32 * kRowBytes;
      fr.a[f][0] = *reinterpret_cast<const uint4*>(base + ra0);
      fr.a[f][1] = *reinterpret_cast<const uint4*>(base + ra1);
      fr.sa[f] = *reinterpret_cast<const uint32_t*>(st + L::a_scales + f * 32 * 4 + rsa);
    } else {
      const int j = f - FM;
      const uint8_t* base = st + L::w_codes + j * 32 * kRowBytes;
      fr.w[j][0] = *reinterpret_cast<const uint4*>(base + rw0);
      fr.w[j][1] = *reinterpret_cast<const uint4*>(base + rw1);
      fr.sw[j] = *reinterpret_cast<const uint32_t*>(st + L::w_scales + j * 32 * 4 + rsw);
    }
  }

  // Decode of step s is split in NCH chunks, chunk q = half (q & 1) of
  // fragment q >> 1.  start(): two code->fp16 conversions into T[q&1] (and,
  // on the first chunk of a fragment in a half stage, its scale pair).
  // finish(): the two block-scale multiplies into F[s&1], one MFMA later.
  __device__ __forceinline__ void start(const Fr& src, int s, int q) {
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
  // (step 0 of `nxt` when S == 7).  Steps 0-5 also issue two of the stage
  // kt+3 global loads (after MFMAs NQ/2-3 and NQ-3); from step 2, after the
  // barrier, two of the next stage's fragments are read from LDS per step
  // (after MFMAs 0 and NQ/2).
  // NEXT = false: the stage is the last before an epilogue, and neither
  // reads the next stage's fragments nor starts decoding them
  template <int S, bool TAIL, bool NEXT = true>
  __device__ __forceinline__ void step_s(const Fr& cur, Fr& nxt, const uint8_t* rd, lds_ptr_t ld, int kt_load) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      mfma(S, q);
      if (q == 0) {
#pragma unroll
        for (int c = first_chunk(NQ - 1); c < NCH; ++c) finish(S, c);
      } else if (S < 7 || NEXT) {
#pragma unroll
        for (int c = first_chunk(q - 1); c < first_chunk(q); ++c) finish((S + 1) & 7, c);
      }
#pragma unroll
      for (int c = first_chunk(q); c < first_chunk(q + 1); ++c) {
        if constexpr (S < 7) {
          start(cur, S + 1, c);
        } else if constexpr (NEXT) {
          start(nxt, 0, c);
        }
      }
      if constexpr (S >= 2 && NEXT) {
        if (q == 0 || q == NQ / 2) {
          const int f = 2 * (S - 2) + (q == 0 ? 0 : 1);
          if (f < NF) read_frag(nxt, rd, f);
        }
      }
      if constexpr (S <= 5) {
        if (q == NQ / 2 - 3 || q == NQ - 3) {
          const int g = 2 * S + (q < NQ / 2 ? 0 : 1);
          if (g < kLoads) issue_one<TAIL>(ld, kt_load, g);
        }
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
  template <bool TAIL, bool NEXT = true>
  __device__ __forceinline__ void stage(int kt, const Fr& cur, Fr& nxt, const uint8_t* rd, lds_ptr_t ld) {
    stage_loading<TAIL, NEXT>(kt, kt + 3, cur, nxt, rd, ld);
  }
  // the same, with the stage the global loads fetch given apart (the
  // persistent kernel's last stages of a tile load the next tile's first)
  template <bool TAIL, bool NEXT = true>
  __device__ __forceinline__ void stage_loading(int kt, int kl, const Fr& cur, Fr& nxt, const uint8_t* rd,
                                                lds_ptr_t ld) {
    step_s<0, TAIL, NEXT>(cur, nxt, rd, ld, kl);
    step_s<1, TAIL, NEXT>(cur, nxt, rd, ld, kl);
    // stage kt+1 landed once at most stage kt+2's loads and the (up to) four
    // of stage kt+3 issued in steps 0-1 are outstanding; a stage past the end
    // of K issues fewer loads (no scale loads), so near the end wait for all
    if (TAIL && kt + 2 >= la.nk) {
      wait_vmcnt<0>();
    } else {
      wait_vmcnt<kLoads + (kLoads < 4 ? kLoads : 4)>();
    }
    lds_barrier();
    step_s<2, TAIL, NEXT>(cur, nxt, rd, ld, kl);
    step_s<3, TAIL, NEXT>(cur, nxt, rd, ld, kl);
    step_s<4, TAIL, NEXT>(cur, nxt, rd, ld, kl);
    step_s<5, TAIL, NEXT>(cur, nxt, rd, ld, kl);
    step_s<6, TAIL, NEXT>(cur, nxt, rd, ld, kl);
    step_s<7, TAIL, NEXT>(cur, nxt, rd, ld, kl);
  }

  // the fragments of the stage in buffer `st` read, and its step 0 decoded
  // but for the chunks of the last MFMA (finished in the stage's first step)
  __device__ __forceinline__ void begin(Fr& fr, const uint8_t* st) {
#pragma unroll
    for (int f = 0; f < NF; ++f) read_frag(fr, st, f);
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      start(fr, 0, q);
      if (q < first_chunk(NQ - 1)) finish(0, q);
    }
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

#if defined(__HIP_DEVICE_COMPILE__)

// First output row and column of tile `pid` of the grid: grouped tile order
// (8 tile rows walk the N tiles together) on the XCD-remapped id.
template <int BN>
__device__ __forceinline__ void tile_origin(int pid, int tiles_m, int tiles_n, int64_t& m0, int64_t& n0) {
  const int total = tiles_m * tiles_n;
  const int tile = xcd_remap(pid, total);
  constexpr int kGroup = 8;
  const int group_size = kGroup * tiles_n;
  const int first_m = (tile / group_size) * kGroup;
  const int gm_count = min(tiles_m - first_m, kGroup);
  const int tm = first_m + (tile % group_size) % gm_count;
  const int tn = (tile % group_size) / gm_count;
  m0 = (int64_t)tm * BM;
  n0 = (int64_t)tn * BN;
}

// Epilogue of one tile: alpha applied once.  16-bit outputs go through the
// wave's LDS staging area `stg` (PASS_ROWS rows of TN values + 16 B pad, in
// passes over the wave's 128 rows) so that each lane stores 16 contiguous
// bytes and TN/8 lanes cover a row segment; fp32 output stores each run of
// four columns directly (`stg` unused).
template <int BN, int OUT, int PASS_ROWS = 64>
__device__ __forceinline__ void store_tile(const Tile<BN>& t, void* __restrict__ c, int64_t ldc, int64_t M,
                                           int64_t N, int64_t m0, int64_t n0, float alpha, bool vec_ok,
                                           uint8_t* stg) {
  constexpr int TN = Tile<BN>::TN, FN = Tile<BN>::FN;
  // the lane id and what derives from it are computed here (a volatile
  // block cannot be hoisted out of a caller's tile loop, where the values
  // would only take registers across the main loop)
  int lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  const int lr = lane & 31, lh = lane >> 5;
  const int64_t row_base = m0 + t.wm * TM, col_base = n0 + t.wn * TN;
  if constexpr (OUT == 0) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t row = row_base + i * 32 + lr;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t col = col_base + j * 32 + 8 * g + 4 * lh;
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
    constexpr int kPitch = TN * 2 + 16;                  // bytes per staged row
    constexpr int kLanesPerRow = TN / 8;                 // 16 bytes (8 outputs) per lane
    constexpr int kRowsPerPass = 64 / kLanesPerRow;      // rows one read instruction covers
    constexpr int kFragsPerPass = PASS_ROWS / 32;
    static_assert(PASS_ROWS == 32 || PASS_ROWS == 64, "whole 32-row fragments per pass");
#pragma unroll
    for (int half = 0; half < FM / kFragsPerPass; ++half) {
#pragma unroll
      for (int ii = 0; ii < kFragsPerPass; ++ii) {
        const int i = kFragsPerPass * half + ii;
        const int r = ii * 32 + lr;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            uint2 w;
            w.x = pack2<OUT>(t.acc[i][j][4 * g] * alpha, t.acc[i][j][4 * g + 1] * alpha);
            w.y = pack2<OUT>(t.acc[i][j][4 * g + 2] * alpha, t.acc[i][j][4 * g + 3] * alpha);
            *reinterpret_cast<uint2*>(stg + r * kPitch + (j * 32 + 8 * g + 4 * lh) * 2) = w;
          }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are done
      __builtin_amdgcn_wave_barrier();
      // PASS_ROWS rows x 2 TN bytes: lane reads 16 B; TN/8 lanes per row
#pragma unroll
      for (int p = 0; p < PASS_ROWS / kRowsPerPass; ++p) {
        const int r = p * kRowsPerPass + lane / kLanesPerRow;
        const int cb = (lane % kLanesPerRow) * 8;  // first of 8 columns
        const uint4 v = *reinterpret_cast<const uint4*>(stg + r * kPitch + cb * 2);
        const int64_t row = row_base + half * PASS_ROWS + r;
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
}

#endif  // __HIP_DEVICE_COMPILE__

template <int BN, int OUT>
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
  using TileT = Tile<BN>;
  using L = typename TileT::L;
  constexpr int TN = TileT::TN, FN = TileT::FN;
  // four stage buffers as separate objects: the compiler can then tell that
  // a read of one never depends on a direct-to-LDS load into another
  __shared__ __attribute__((aligned(1024))) uint8_t buf0[L::stage_bytes];
  __shared__ __attribute__((aligned(1024))) uint8_t buf1[L::stage_bytes];
  __shared__ __attribute__((aligned(1024))) uint8_t buf2[L::stage_bytes];
  __shared__ __attribute__((aligned(1024))) uint8_t buf3[L::stage_bytes];
  const lds_ptr_t l0 = (lds_ptr_t)buf0, l1 = (lds_ptr_t)buf1, l2 = (lds_ptr_t)buf2, l3 = (lds_ptr_t)buf3;

  TileT t;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  t.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  t.wm = t.wave >> 1;
  t.wn = t.wave & 1;
  t.lr = lane & 31;
  t.h = lane >> 5;
  t.init_reads();

  int64_t m0, n0;
  tile_origin<BN>((int)blockIdx.x, tiles_m, tiles_n, m0, n0);
  // the global scales are read here, long before the epilogue needs alpha
  const float alpha = 1.0f / (*a_gscale * *w_gscale);

  t.la.init_lanes(K, t.wave, lane);
  t.lw.init_lanes(K, t.wave, lane);
  t.la.target(a_codes, a_scales, m0, M, K);
  t.lw.target(w_codes, w_scales, n0, N, K);
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
    wait_vmcnt<2 * TileT::kLoads>();
  }
  lds_barrier();

  typename TileT::Fr fx, fy;  // the two fragment register sets, used in turn
  t.begin(fx, buf0);

  // Four stages per iteration (stages past nk, up to the next multiple of
  // four, multiply zeros): two register sets x four LDS buffers, all static.
  // Stage kt reads stage kt+1 from buffer (kt+1)%4 and loads stage kt+3 into
  // buffer (kt+3)%4, which held stage kt-1 (already in every wave's registers
  // by the barrier of stage kt).
  // Iterations whose loads (stages kt+3 .. kt+6) all lie inside K take no
  // checks, and so does every iteration when K is a whole number of groups
  // of four stages (then no stage past the end is multiplied); otherwise the
  // last one or two check every load and wait.
  const int kt_plain = (nk & 3) == 0 ? nk : nk - 6;
  int kt = 0;
  for (; kt < kt_plain; kt += 4) {
    t.template stage<false>(kt + 0, fx, fy, buf1, l3);
    t.template stage<false>(kt + 1, fy, fx, buf2, l0);
    t.template stage<false>(kt + 2, fx, fy, buf3, l1);
    t.template stage<false>(kt + 3, fy, fx, buf0, l2);
  }
  for (; kt < nk; kt += 4) {
    t.template stage<true>(kt + 0, fx, fy, buf1, l3);
    t.template stage<true>(kt + 1, fy, fx, buf2, l0);
    t.template stage<true>(kt + 2, fx, fy, buf3, l1);
    t.template stage<true>(kt + 3, fy, fx, buf0, l2);
  }
  wait_vmcnt<0>();  // loads issued for stages past the end

  const bool vec_ok = (reinterpret_cast<uintptr_t>(c) % 16) == 0 && (ldc * (OUT == 0 ? 4 : 2)) % 16 == 0;
  if constexpr (OUT != 0) __syncthreads();  // every wave is done reading the stage buffers
  // each wave stages its 16-bit outputs in a stage buffer of its own
  static_assert(64 * (TN * 2 + 16) <= L::stage_bytes, "a wave's staging rows fit in one stage buffer");
  uint8_t* const stg = t.wave < 2 ? (t.wave == 0 ? buf0 : buf1) : (t.wave == 2 ? buf2 : buf3);
  store_tile<BN, OUT>(t, c, ldc, M, N, m0, n0, alpha, vec_ok, stg);
#endif
}

// Persistent form of the 256x256 kernel, for whole tiles, K a multiple of 512
// (a whole number of groups of four stages) and at least one tile per
// workgroup (the dispatch uses it from three tiles per CU on).  One workgroup
// per CU takes tiles pid, pid + G, pid + 2G, ... (G workgroups, a multiple of
// the 8 XCDs, so that every tile keeps the XCD the one-tile kernel would give
// it).  The load pipeline runs on across tiles: the last three stages of a
// tile, whose loads would lie past its end of K, load the next tile's first
// three stages (moving to the next tile changes only the loaders' scalar
// offset).  The next tile therefore starts with its operands in LDS, and no
// workgroup launch separates the tiles.  The tile's last stage reads the next
// tile's first stage and decodes its first step, as any stage does for the
// one after it, so those fragments stay in registers through the epilogue.
// The epilogue stages 16-bit outputs in the buffer of the tile's last stage
// (32 rows per wave and pass), the one buffer no load targets at that point.
template <int OUT>
__global__ __launch_bounds__(kThreads, 1) void gemm_fast_persistent_kernel(
    int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ a_gscale, const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales,
    const float* __restrict__ w_gscale, void* __restrict__ c, int64_t ldc, int tiles_m, int tiles_n) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BN = 256;
  using TileT = Tile<BN>;
  using L = typename TileT::L;
  constexpr int TN = TileT::TN, FN = TileT::FN;
  __shared__ __attribute__((aligned(1024))) uint8_t buf0[L::stage_bytes];
  __shared__ __attribute__((aligned(1024))) uint8_t buf1[L::stage_bytes];
  __shared__ __attribute__((aligned(1024))) uint8_t buf2[L::stage_bytes];
  __shared__ __attribute__((aligned(1024))) uint8_t buf3[L::stage_bytes];
  const lds_ptr_t l0 = (lds_ptr_t)buf0, l1 = (lds_ptr_t)buf1, l2 = (lds_ptr_t)buf2, l3 = (lds_ptr_t)buf3;

  TileT t;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  t.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  t.wm = t.wave >> 1;
  t.wn = t.wave & 1;
  t.lr = lane & 31;
  t.h = lane >> 5;
  t.init_reads();

  // this tile's and the next one's origins (the next one's is computed a
  // tile ahead, at the tile boundary, not inside the K loop where registers
  // are scarce)
  const int total = tiles_m * tiles_n;
  int pid = (int)blockIdx.x;
  int64_t m0, n0, nm0 = 0, nn0 = 0;
  tile_origin<BN>(pid, tiles_m, tiles_n, m0, n0);
  int next = pid + (int)gridDim.x;
  bool has_next = next < total;
  if (has_next) tile_origin<BN>(next, tiles_m, tiles_n, nm0, nn0);
  const float alpha = 1.0f / (*a_gscale * *w_gscale);
  const bool vec_ok = (reinterpret_cast<uintptr_t>(c) % 16) == 0 && (ldc * (OUT == 0 ? 4 : 2)) % 16 == 0;
  // 16-bit staging: 32 rows per wave in buf3
  constexpr int kStageRows = 32 * (TN * 2 + 16);
  static_assert(4 * kStageRows <= L::stage_bytes, "four waves' staging rows fit in one stage buffer");
  uint8_t* const stg = buf3 + t.wave * kStageRows;

  t.la.init_lanes(K, t.wave, lane);
  t.lw.init_lanes(K, t.wave, lane);
  t.la.target_matrix(a_codes, a_scales, M, K);
  t.lw.target_matrix(w_codes, w_scales, N, K);
  // byte offsets of this tile's and the next tile's first code rows (with
  // no next tile, this one's: the last stages then reload its first ones)
  const uint32_t row_bytes = (uint32_t)(K / 2);
  uint32_t a_off = (uint32_t)m0 * row_bytes, w_off = (uint32_t)n0 * row_bytes;
  uint32_t a_next = has_next ? (uint32_t)nm0 * row_bytes : a_off;
  uint32_t w_next = has_next ? (uint32_t)nn0 * row_bytes : w_off;
  t.la.tile_off = a_off;
  t.lw.tile_off = w_off;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) t.acc[i][j] = float16_t{};

  const int nk = (int)(K / kBK);  // a multiple of 4
  t.issue_all(l0, 0);
  t.issue_all(l1, 1);
  t.issue_all(l2, 2);
  wait_vmcnt<2 * TileT::kLoads>();  // stage 0 landed
  lds_barrier();

  typename TileT::Fr fx, fy;  // the two fragment register sets, used in turn
  t.begin(fx, buf0);

  for (;;) {
    // The last group of four stages is the loop's last iteration (the same
    // code, so the same address registers): after its first stage, which
    // loads the tile's last stage, the loaders move to the next tile, and
    // stages nk-3 .. nk-1 load its stages 0 .. 2.  The tile's last stage
    // reads the next tile's first stage and decodes its first step, as
    // within a tile.
    for (int kt = 0; kt < nk; kt += 4) {
      t.la.tile_off = a_off;
      t.lw.tile_off = w_off;
      t.template stage_loading<false>(kt, kt + 3, fx, fy, buf1, l3);
      const bool last = kt + 4 == nk;
      t.la.tile_off = last ? a_next : a_off;
      t.lw.tile_off = last ? w_next : w_off;
      const int kl = last ? 0 : kt + 4;
      t.template stage_loading<false>(kt + 1, kl, fy, fx, buf2, l0);
      t.template stage_loading<false>(kt + 2, kl + 1, fx, fy, buf3, l1);
      t.template stage_loading<false>(kt + 3, kl + 2, fy, fx, buf0, l2);
    }

    // buf3 held the tile's last stage, read by every wave before the barrier
    // of stage nk-1; loads into buf1 and buf2 (and the next tile's first
    // stage, landed, in buf0) stay where they are
    store_tile<BN, OUT, 32>(t, c, ldc, M, N, m0, n0, alpha, vec_ok, stg);
    if (!has_next) {
      wait_vmcnt<0>();  // the last three stages' loads (this tile's first ones again) still target LDS
      break;
    }
    // the staging reads are done before the next tile's first stage loads into buf3
    if constexpr (OUT != 0) lds_barrier();
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) t.acc[i][j] = float16_t{};
    pid = next;
    m0 = nm0;
    n0 = nn0;
    a_off = a_next;
    w_off = w_next;
    next = pid + (int)gridDim.x;
    has_next = next < total;
    if (has_next) tile_origin<BN>(next, tiles_m, tiles_n, nm0, nn0);
    a_next = has_next ? (uint32_t)nm0 * row_bytes : a_off;
    w_next = has_next ? (uint32_t)nn0 * row_bytes : w_off;
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
                            const float* w_gscale, void* c, int out_dtype, int64_t ldc, hipStream_t stream,
                            int tile_n) {
  const int bn = tile_n == 128 ? 128 : 256;
  const int tiles_m = (int)((m + BM - 1) / BM), tiles_n = (int)((n + bn - 1) / bn);
  const unsigned grid = (unsigned)tiles_m * (unsigned)tiles_n;
  // whole 256x256 tiles only, at least three per CU, and K a whole number of
  // four-stage groups: the persistent form, one workgroup per CU (a whole
  // number per XCD).  With about two tiles per CU it measured no faster.
  const int cus = device_cu_count();
  if (bn == 256 && m % BM == 0 && n % 256 == 0 && (k / kBK) % 4 == 0 && cus >= 8 && cus % 8 == 0 &&
      (int64_t)grid >= 3 * (int64_t)cus) {
    const unsigned pgrid = (unsigned)cus;
    if (out_dtype == 0)
      gemm_fast_persistent_kernel<0><<<pgrid, kThreads, 0, stream>>>(m, n, k, a_codes, a_scales, a_gscale, w_codes,
                                                                     w_scales, w_gscale, c, ldc, tiles_m, tiles_n);
    else if (out_dtype == 1)
      gemm_fast_persistent_kernel<1><<<pgrid, kThreads, 0, stream>>>(m, n, k, a_codes, a_scales, a_gscale, w_codes,
                                                                     w_scales, w_gscale, c, ldc, tiles_m, tiles_n);
    else
      gemm_fast_persistent_kernel<2><<<pgrid, kThreads, 0, stream>>>(m, n, k, a_codes, a_scales, a_gscale, w_codes,
                                                                     w_scales, w_gscale, c, ldc, tiles_m, tiles_n);
    return hipGetLastError();
  }
#define NVFP4_LAUNCH(BN, OUT)                                                                                  \
  gemm_fast_kernel<BN, OUT><<<grid, kThreads, 0, stream>>>(m, n, k, a_codes, a_scales, a_gscale, w_codes,    \
                                                           w_scales, w_gscale, c, ldc, tiles_m, tiles_n)
  if (bn == 256) {
    if (out_dtype == 0)
      NVFP4_LAUNCH(256, 0);
    else if (out_dtype == 1)
      NVFP4_LAUNCH(256, 1);
    else
      NVFP4_LAUNCH(256, 2);
  } else {
    if (out_dtype == 0)
      NVFP4_LAUNCH(128, 0);
    else if (out_dtype == 1)
      NVFP4_LAUNCH(128, 1);
    else
      NVFP4_LAUNCH(128, 2);
  }
#undef NVFP4_LAUNCH
  return hipGetLastError();
}

}  // namespace nvfp4
