// Weight-streaming W4A4 GEMM for few activation rows (M <= 32) and large N:
// C = alpha * A_hat W_hat^T on NVFP4 operands (news article
// "Qwen3.8-27B最激进4bit量化开源，权重显存暴降2.9倍！", section 02: E2M1 codes, one
// E4M3 scale per 16 elements, one FP32 global scale per tensor, both
// operands 4-bit).
//
// A decode-shaped call reads every weight byte once (0.5625 B per element)
// and is bound by how steadily the weight streams from HBM.  The design:
//
//  * One workgroup per CU owns a contiguous slab of at most 144 weight rows
//    (N / CUs rounded up to 8), so every CU streams the same number of bytes
//    and the slab's codes and scale rows are contiguous in memory.
//  * The slab goes through a ring of three LDS slots, one 16-row tile (all of
//    K: 16 * K/2 code bytes and 16 * K/16 scale bytes) per slot, with
//    direct-to-LDS buffer loads of 16 bytes per lane: one instruction moves
//    1 KiB of consecutive memory (8 whole cache lines), non-temporal.  Code
//    rows are stored with their 16-byte chunks XOR-swizzled by row within
//    each 256-byte window (each lane fetches the chunk that belongs at its
//    slot), so 16 lanes reading 16 rows at one K offset hit 16 distinct bank
//    groups.
//  * Eight waves (two per SIMD) split K: wave w owns elements
//    [w K/8, (w+1) K/8).  Its eighth of the activations is decoded once, at
//    the start, into registers (MT x K/1024 x 4 fp16 fragments), so the main
//    loop decodes only weights.  Activations are staged through slots 1 and 2
//    with the same loads before the weight stream starts.
//  * Per tile: wait for this wave's loads of the tile (vmcnt), one barrier,
//    issue the loads of tile t+2 into the slot read in the previous tile,
//    copy this wave's slice (16 rows x K/8) into registers, decode (exact
//    fp4 -> fp16 times the E4M3 block scale converted to fp16) and
//    v_mfma_f32_16x16x32_f16, then the eight partial sums of the tile are
//    added in LDS in a fixed order (deterministic) and alpha applied.
//  * Outputs are staged in LDS and stored after the loop with 16-byte
//    stores (fp32 output of 32 rows does not fit and is stored per tile).
//
// The weight loads are issued from inline asm (no register outputs), so the
// compiler does not treat them as pending LDS writes; every read of a slot is
// ordered after its loads by an explicit vmcnt wait (a wave's loads complete
// in issue order) and a workgroup barrier.  Any other global access in the
// loop is a store, which never makes those waits wait for less.
#include <type_traits>

#include "gemm_common.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

using namespace gemm;

constexpr int kSWaves = 8;  // two per SIMD
constexpr int kSThreads = 64 * kSWaves;
constexpr int kSlots = 3;
constexpr int kMaxRowsPerWg = 144;  // 9 tiles: the output stage holds a workgroup's outputs
constexpr int kOutStageBytes = 9216;
constexpr uint32_t kOob = 0x80000000u;  // a buffer offset past any record count: the load reads nothing

typedef float float4_v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t* lds_ptr_t;

// HG: 128-element groups of K per wave (K = 1024 HG); MT: 16-row activation tiles
template <int HG, int MT>
struct StreamCfg {
  static constexpr int K = 128 * kSWaves * HG;
  static constexpr int kRowCode = K / 2;
  static constexpr int kRowScale = K / 16;
  static constexpr int kCodeBytes = 16 * kRowCode;  // a tile's codes (a whole number of KiB)
  static constexpr int kScaleBytes = (16 * kRowScale + 1023) / 1024 * 1024;
  static constexpr int kSlotBytes = kCodeBytes + kScaleBytes;
  static constexpr int kCodeInst = kCodeBytes / 1024;  // 1 KiB load instructions per tile
  static constexpr int kInst = kCodeInst + kScaleBytes / 1024;
  static constexpr int kInstMax = (kInst + kSWaves - 1) / kSWaves;  // per wave
  static constexpr int kInstMin = kInst / kSWaves;
  static constexpr int kPartBytes = kSWaves * MT * 64 * 16;
  static constexpr int kLdsBytes = kSlots * kSlotBytes + kPartBytes + kOutStageBytes;
  static_assert(kLdsBytes <= 160 * 1024, "ring, partial sums and output stage fit the LDS");
};

#if defined(__HIP_DEVICE_COMPILE__)
template <int N>
__device__ __forceinline__ void s_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x0F70);
}
// workgroup barrier for LDS: the wave's own LDS accesses are done
// (lgkmcnt(0)); loads still in flight to other slots need not drain
__device__ __forceinline__ void s_lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
// One direct-to-LDS load: lane l's 16 bytes at voffset go to LDS byte
// lds_addr + 16 l.  M0 is set in the same asm block, one wait state before
// the load reads it.  NT: non-temporal (streamed weights).
template <bool NT>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_addr, uint32_t voffset) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :
                 : "s"(lds_addr), "v"(voffset), "s"(rsrc)
                 : "memory");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr), "v"(voffset), "s"(rsrc)
                 : "memory");
}
#endif

template <int HG, int MT, int OUT>
__global__ __launch_bounds__(kSThreads, 1) void gemm_stream_kernel(int M, int N, int rows_per_wg,
                                                                    const uint8_t* __restrict__ a_codes,
                                                                    const uint8_t* __restrict__ a_scales,
                                                                    const float* __restrict__ a_gscale,
                                                                    const uint8_t* __restrict__ w_codes,
                                                                    const uint8_t* __restrict__ w_scales,
                                                                    const float* __restrict__ w_gscale,
                                                                    void* __restrict__ c, int64_t ldc) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = StreamCfg<HG, MT>;
  constexpr int K = C::K;
  constexpr int kOutBytes = OUT == 0 ? 4 : 2;
  constexpr bool kStage = 16 * MT * kMaxRowsPerWg * kOutBytes <= kOutStageBytes;
  constexpr int kOutPitch = kMaxRowsPerWg * kOutBytes;  // bytes per staged output row
  // the ring slots and the partial sums as separate objects
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[C::kSlotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[C::kSlotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t slot2[C::kSlotBytes];
  __shared__ __attribute__((aligned(16))) float4_v part[kSWaves * MT * 64];
  __shared__ __attribute__((aligned(16))) uint8_t outst[kStage ? 16 * MT * kOutPitch : 16];
  const lds_ptr_t slots[3] = {(lds_ptr_t)slot0, (lds_ptr_t)slot1, (lds_ptr_t)slot2};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, q = lane >> 4;
  const int r0 = __builtin_amdgcn_readfirstlane(blockIdx.x * rows_per_wg);
  const int nrows = __builtin_amdgcn_readfirstlane(min(rows_per_wg, N - r0));
  const int nt = (nrows + 15) / 16;

  // block-local source offsets of this wave's loads: instruction u = wv + 8v
  // of a 16-row block (code chunks first, then scale chunks)
  uint32_t voff[C::kInstMax];
#pragma unroll
  for (int v = 0; v < C::kInstMax; ++v) {
    const int u = wv + kSWaves * v;
    if (u < C::kCodeInst) {
      const uint32_t o = (uint32_t)(u * 1024 + 16 * lane);
      const uint32_t row = o / C::kRowCode, col = o - row * C::kRowCode;
      const uint32_t colg = (col & ~255u) | ((((col >> 4) & 15u) ^ (row & 15u)) << 4);
      voff[v] = row * C::kRowCode + colg;
    } else {
      const uint32_t o = (uint32_t)((u - C::kCodeInst) * 1024 + 16 * lane);
      voff[v] = o < (uint32_t)(16 * C::kRowScale) ? o : kOob;
    }
  }
  // one 16-row block (all of K) of a row-major operand into a slot; rows
  // past `valid` read nothing (the resource has no records for them)
  auto issue_rows = [&](auto nt_tag, const uint8_t* codes, const uint8_t* scales, int64_t row0, int valid,
                        lds_ptr_t slot) {
    constexpr bool kNt = decltype(nt_tag)::value;
    valid = __builtin_amdgcn_readfirstlane(max(0, min(16, valid)));
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(codes + row0 * C::kRowCode), (short)0, valid * C::kRowCode, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(scales + row0 * C::kRowScale), (short)0, valid * C::kRowScale, 0x00020000);
#pragma unroll
    for (int v = 0; v < C::kInstMax; ++v) {
      const int u = wv + kSWaves * v;
      const uint32_t dst_c = (uint32_t)(uintptr_t)(slot + u * 1024);
      const uint32_t dst_s = (uint32_t)(uintptr_t)(slot + C::kCodeBytes + (u - C::kCodeInst) * 1024);
      if (kSWaves * v + kSWaves - 1 < C::kCodeInst) {  // a code chunk for every wave
        dma16<kNt>(rc, dst_c, voff[v]);
      } else if (kSWaves * v >= C::kCodeInst && kSWaves * v + kSWaves - 1 < C::kInst) {  // a scale chunk for every wave
        dma16<kNt>(rs, dst_s, voff[v]);
      } else if (u < C::kCodeInst) {
        dma16<kNt>(rc, dst_c, voff[v]);
      } else if (u < C::kInst) {
        dma16<kNt>(rs, dst_s, voff[v]);
      }
    }
  };
  auto issue_tile = [&](int t, lds_ptr_t slot) {
    const int tu = __builtin_amdgcn_readfirstlane(t);
    issue_rows(std::true_type{}, w_codes, w_scales, (int64_t)(r0 + 16 * tu), nrows - 16 * tu, slot);
  };
  // this wave's slice of a 16-row block in a slot: per 128-element group j,
  // 16 code bytes of row lr (elements 32q .. 32q+31 of the group) and the
  // scale bytes of its blocks 2q and 2q+1
  auto read_slice = [&](lds_ptr_t sl, uint4 (&wc)[HG], uint32_t (&wsc)[HG]) {
#pragma unroll
    for (int j = 0; j < HG; ++j) {
      const uint32_t col = (uint32_t)(wv * (K / 16) + 64 * j + 16 * q);
      uint32_t off = (uint32_t)(lr * C::kRowCode) + (col & ~255u) + ((((col >> 4) & 15u) ^ (uint32_t)lr) << 4);
      asm volatile("" : "+v"(off));  // each read keeps its own address (no folded offsets)
      wc[j] = *reinterpret_cast<const __attribute__((address_space(3))) uint4*>(sl + off);
      uint32_t soff = (uint32_t)(C::kCodeBytes + lr * C::kRowScale + wv * (K / 128) + 8 * j + 2 * q);
      asm volatile("" : "+v"(soff));
      wsc[j] = (uint32_t) * reinterpret_cast<const __attribute__((address_space(3))) uint16_t*>(sl + soff);
    }
  };

  // Activations: this wave's eighth of K for all rows, decoded once.  The
  // MFMA step s of group j takes word s of the lane's 16 code bytes (elements
  // 32q + 8s .. +7 of the group, block 2q + s/2) for A and W alike, so every
  // k is summed exactly once.
  half8_t fa[MT][HG][4];
  {
    issue_rows(std::false_type{}, a_codes, a_scales, 0, M, slots[1]);
    if constexpr (MT == 2) issue_rows(std::false_type{}, a_codes, a_scales, 16, M - 16, slots[2]);
    s_wait_vmcnt<0>();
    s_lds_barrier();
    uint4 ac[MT][HG];
    uint32_t as[MT][HG];
    read_slice(slots[1], ac[0], as[0]);
    if constexpr (MT == 2) read_slice(slots[2], ac[MT - 1], as[MT - 1]);
    s_lds_barrier();  // every wave has its slice: slots 1 and 2 take weight tiles now
    issue_tile(0, slots[0]);
    issue_tile(1, slots[1]);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < HG; ++j) {
        const half2_t sp = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(as[i][j], 1.0f, false);
        const half2_t s0 = {sp[0], sp[0]}, s1 = {sp[1], sp[1]};
        fa[i][j][0] = decode8(ac[i][j].x, s0);
        fa[i][j][1] = decode8(ac[i][j].y, s0);
        fa[i][j][2] = decode8(ac[i][j].z, s1);
        fa[i][j][3] = decode8(ac[i][j].w, s1);
      }
  }

  const float alpha = 1.0f / (*a_gscale * *w_gscale);
  // the eight waves' partial sums of tile t in a fixed order, times alpha:
  // activation row 16i + ln%16, weight rows 16t + 4(ln/16) .. +3 of the slab
  auto reduce = [&](int t) {
    if (tid < MT * 64) {
      const int i = tid >> 6, ln = tid & 63;
      float4_v s = part[i * 64 + ln];
#pragma unroll
      for (int w = 1; w < kSWaves; ++w) s += part[(w * MT + i) * 64 + ln];
      const int m = 16 * i + (ln & 15);
      const int nl = 16 * t + 4 * (ln >> 4);
      const float o0 = s[0] * alpha, o1 = s[1] * alpha, o2 = s[2] * alpha, o3 = s[3] * alpha;
      if constexpr (kStage) {
        auto* dst = outst + m * kOutPitch + nl * kOutBytes;
        if constexpr (OUT == 0) {
          *reinterpret_cast<float4_v*>(dst) = float4_v{o0, o1, o2, o3};
        } else if constexpr (OUT == 1) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(bf16x2_rne_bits(o0, o1), bf16x2_rne_bits(o2, o3));
        } else {
          typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
          *reinterpret_cast<half4_t*>(dst) = half4_t{(_Float16)o0, (_Float16)o1, (_Float16)o2, (_Float16)o3};
        }
      } else if (m < M && nl < nrows) {
        float* p = static_cast<float*>(c) + m * ldc + r0 + nl;
        const float o[4] = {o0, o1, o2, o3};
        for (int e = 0; e < 4 && nl + e < nrows; ++e) p[e] = o[e];
      }
    }
  };

  // one tile: S is its ring slot (t % 3), a compile-time value
  auto body = [&](auto slot_tag, int t) {
    constexpr int S = decltype(slot_tag)::value;
    // tile t's loads are done once only tile t+1's may be in flight (every
    // body issues exactly one tile, so this holds on every path)
    s_wait_vmcnt<C::kInstMin>();
    s_lds_barrier();
    issue_tile(t + 2, slots[(S + 2) % 3]);  // read in the previous tile, before this barrier
    uint4 wc[HG];
    uint32_t wsc[HG];
    read_slice(slots[S], wc, wsc);

    float4_v acc[2][MT];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < MT; ++i) acc[h][i] = float4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < HG; ++j) {
      const half2_t sp = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wsc[j], 1.0f, false);
      const half2_t s0 = {sp[0], sp[0]}, s1 = {sp[1], sp[1]};
      const uint32_t wd[4] = {wc[j].x, wc[j].y, wc[j].z, wc[j].w};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const half8_t fw = decode8(wd[s], s < 2 ? s0 : s1);
#pragma unroll
        for (int i = 0; i < MT; ++i)
          acc[s & 1][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fw, fa[i][j][s], acc[s & 1][i], 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) part[(wv * MT + i) * 64 + lane] = acc[0][i] + acc[1][i];
    s_lds_barrier();  // every wave's partial sums of tile t are written
    reduce(t);        // (the next tile's barrier orders these reads before the next writes)
  };
  // the loop closes only after a third body, so every path into a body has
  // the same loads in flight
  for (int t = 0;;) {
    body(std::integral_constant<int, 0>{}, t);
    if (++t == nt) break;
    body(std::integral_constant<int, 1>{}, t);
    if (++t == nt) break;
    body(std::integral_constant<int, 2>{}, t);
    if (++t == nt) break;
  }
  s_wait_vmcnt<0>();  // loads issued past the last tile read nothing but still target LDS
  if constexpr (kStage) {
    s_lds_barrier();
    // staged outputs to C: 16-byte pieces of each activation row's run of the slab
    const bool vec = (reinterpret_cast<uintptr_t>(c) % 16) == 0 && (ldc * kOutBytes) % 16 == 0 &&
                     ((int64_t)r0 * kOutBytes) % 16 == 0;
    constexpr int kPer = 16 / kOutBytes;  // outputs per piece
    const int pieces = (nrows + kPer - 1) / kPer;
    for (int f = tid; f < M * pieces && f < 16 * MT * pieces; f += kSThreads) {
      const int m = f / pieces, pc = f - m * pieces;
      const int nl = pc * kPer;
      uint8_t* dst = static_cast<uint8_t*>(c) + ((int64_t)m * ldc + r0 + nl) * kOutBytes;
      const uint8_t* src = outst + m * kOutPitch + nl * kOutBytes;
      if (vec && nl + kPer <= nrows) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
      } else {
        for (int e = 0; e < kPer && nl + e < nrows; ++e)
          for (int b = 0; b < kOutBytes; ++b) dst[e * kOutBytes + b] = src[e * kOutBytes + b];
      }
    }
  }
#endif
}

template <int HG, int MT>
hipError_t launch_stream_cfg(int64_t m, int64_t n, int rows, int grid, const uint8_t* a_codes,
                             const uint8_t* a_scales, const float* a_gscale, const uint8_t* w_codes,
                             const uint8_t* w_scales, const float* w_gscale, void* c, int out_dtype, int64_t ldc,
                             hipStream_t stream) {
#define NVFP4_LAUNCH_STREAM(OUT)                                                                           \
  gemm_stream_kernel<HG, MT, OUT><<<grid, kSThreads, 0, stream>>>((int)m, (int)n, rows, a_codes, a_scales, \
                                                                  a_gscale, w_codes, w_scales, w_gscale, c, ldc)
  if (out_dtype == 0)
    NVFP4_LAUNCH_STREAM(0);
  else if (out_dtype == 1)
    NVFP4_LAUNCH_STREAM(1);
  else
    NVFP4_LAUNCH_STREAM(2);
#undef NVFP4_LAUNCH_STREAM
  return hipGetLastError();
}

// weight rows per workgroup: N over the CUs, rounded up to 8
int64_t stream_rows_per_wg(int64_t n, int64_t cus) { return ((n + cus - 1) / cus + 7) / 8 * 8; }

}  // namespace

bool gemm_stream_supported(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                           const uint8_t* w_codes, const uint8_t* w_scales) {
  const bool aligned = (reinterpret_cast<uintptr_t>(a_codes) % 16) == 0 &&
                       (reinterpret_cast<uintptr_t>(a_scales) % 16) == 0 &&
                       (reinterpret_cast<uintptr_t>(w_codes) % 16) == 0 &&
                       (reinterpret_cast<uintptr_t>(w_scales) % 16) == 0;
  if (!aligned || m < 1 || m > 32 || (k != 4096 && k != 5120) || n >= ((int64_t)1 << 30)) return false;
  // one round of one workgroup per CU, each with enough tiles that the
  // stream, not the start-up (activation staging and the first tiles'
  // latency), sets the time: 80 to 144 weight rows per CU
  const int64_t cus = device_cu_count();
  const int64_t rows = stream_rows_per_wg(n, cus);
  return rows >= 80 && rows <= kMaxRowsPerWg;
}

hipError_t launch_gemm_stream(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                              const float* a_gscale, const uint8_t* w_codes, const uint8_t* w_scales,
                              const float* w_gscale, void* c, int out_dtype, int64_t ldc, hipStream_t stream) {
  const int64_t cus = device_cu_count();
  const int rows = (int)stream_rows_per_wg(n, cus);
  const int grid = (int)((n + rows - 1) / rows);
  if (k == 5120)
    return m <= 16 ? launch_stream_cfg<5, 1>(m, n, rows, grid, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale,
                                             c, out_dtype, ldc, stream)
                   : launch_stream_cfg<5, 2>(m, n, rows, grid, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale,
                                             c, out_dtype, ldc, stream);
  return m <= 16 ? launch_stream_cfg<4, 1>(m, n, rows, grid, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c,
                                           out_dtype, ldc, stream)
                 : launch_stream_cfg<4, 2>(m, n, rows, grid, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, c,
                                           out_dtype, ldc, stream);
}

}  // namespace nvfp4
