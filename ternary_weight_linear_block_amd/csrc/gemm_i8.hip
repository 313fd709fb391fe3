// Prefill ternary linear: int8 MFMA GEMM with the 2-bit weight unpack fused
// into the operand path, int32 accumulation and a fused per-token/per-row
// rescale.
//
// Method ([P1] "Ternary-Bonsai-2-27B on 2x RTX 5070 with vLLM TP=2", section 4,
// prefill linear layers to an int8 GEMM): with q[n,g] = round(127 s / smax) the
// weight W_int8[n,k] = code[n,k] * q[n, k/128] is exactly int8, so
//   acc[t,n] = sum_k x_i8[t,k] * W_int8[n,k]        (int32, exact)
//   y[t,n]   = acc[t,n] * a_scale[t] * smax[n] / 127
// The pages expand W_int8 in a separate pass every step (section 6 timing
// table: 31 of 83 ms) before a library int8 GEMM.  Here W_int8 never exists in
// memory: each lane turns one packed 32-bit word (16 codes) into the 16 int8
// bytes of its MFMA B operand with 1 shift, 4 ANDs and 4 byte-permutes
// against tables built from {-q, +q, 0}.
//
// gfx950 mapping
//   * v_mfma_i32_32x32x32_i8 (measured full rate on gfx950: 32 cycles per
//     32x32x32; the 16x16x64 form is markedly slower per MAC).  Each lane
//     supplies 16 bytes of A (one row) and 16 bytes of B (one column) per
//     instruction.  Integer accumulation is exact, so the k values assigned to
//     (lane half h, byte) only have to agree between A and B: in a 128-k
//     pipeline stage (one scale group), lane half h at k-step s covers
//     k = 16 (4 h + s) .. +15, so a lane's B data for a whole stage is 16
//     contiguous packed bytes (4 words) and its scale is q[n, g].
//   * Workgroup: 2 WN x 2 waves (8 for WN = 2, two per SIMD; 12 for WN = 3,
//     three per SIMD).  Block tile BM = 64 RM rows x BN = 32 FN columns split
//     2 along M x WN along N; wave (wm, wn) owns RM row fragments and
//     ceil(FN/WN) column fragments (a remainder leaves the last wn padding
//     fragments), and the two waves (wk = 0, 1) of each (wm, wn) take k-steps
//     {0,1} and {2,3} of every stage.  At the end the pair splits the output
//     by fragment rows (accumulator registers 0-7 / 8-15) and each wave adds
//     its partner's int32 partials for its half through LDS (exact), so all
//     waves store.  With two or more waves per SIMD one wave's unpack VALU
//     and LDS reads run while another's MFMAs execute (the MFMA clusters run
//     at raised wave priority).
//   * Multi-stage pipeline (4 stages; 3 for 256-row tiles) of direct
//     global->LDS loads (global_load_lds dwordx4: no VGPR staging).  A stage
//     holds BM x 128 bytes of x_i8 (8 lanes per row; 16-byte chunks
//     XOR-swizzled by row so the column-wise ds_read_b128 hits distinct banks)
//     and BN x 32 bytes of packed weights (2 lanes per weight row, the two
//     16-byte halves parity-swizzled by column; in the tiled weight layout
//     these are whole 2 KB tiles of 64 rows, contiguous in memory).  Each load instruction thus
//     touches few cache lines; the q block of the tile is copied to LDS once
//     up front.  Every wave issues the same static set of loads per stage,
//     waits only for its own (vmcnt), and a bare s_barrier publishes the
//     stage.  No load into VGPRs happens inside the loop, so the compiler
//     never has to drain vmcnt.
//   * Optional split-K over stages: each split stores its exact int32 partial
//     tile (lane-major, fully coalesced) to a workspace slot and a second
//     kernel, one wave per output fragment, adds the splits and runs the
//     epilogue.  (A device-scope
//     fence + counter scheme in one kernel was measured to cost far more: on
//     this multi-XCD part each fence writes back the L2.)
//   * Tiles are ordered so that the workgroups sharing a column block (the
//     same weights) land on the same XCD and its L2.
//   * The stage loop is unrolled by the pipeline depth, so buffer offsets are
//     constants and the packed words alternate between two register sets.
//   * Output: each kept 16x32 half fragment is transposed through a per-wave
//     LDS scratch (two buffers, alternated) so that every lane writes 16
//     contiguous bytes (fp32 / int32 y: 4 columns; bf16 y: 8 columns): the
//     output phase is bound by the number of store transactions, not by
//     bytes.
#include "twl_internal.h"

#include <algorithm>
#include <cstdio>
#include <cstdlib>

namespace twl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kStages = 4;       // pipeline depth
constexpr int kStageK = 128;     // k per stage = one scale group
constexpr int kXcds = 8;         // MI355X: 8 XCDs, workgroups dispatched round robin

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] + vmcnt_hi[15:14], expcnt[6:4], lgkmcnt[11:8]
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait for this wave's outstanding LDS reads (and scalar loads).  Issued as
// the builtin, not inline asm: the compiler then knows those reads have
// landed and does not wait for them again before their first use, which it
// would do behind the reads issued later (and so wait for those too).
__device__ __forceinline__ void wait_lgkm0() {
  // vmcnt 63 and expcnt 7 (no wait), lgkmcnt 0
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
}

// Workgroup barrier without the memory fence __syncthreads implies: LDS
// visibility is established by each wave's explicit vmcnt wait before it.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct global->LDS loads (lane i writes LDS[lds_base + i * size]) at
// address sbase (wave-uniform, SGPR pair) + voff (per lane, 32 bit).  Issued
// as inline asm on purpose: the compiler then does not see these LDS writes
// and does not drain vmcnt before every LDS read of the other stages; the
// kernel orders them itself (wait_vmcnt on its own loads + bare_barrier).
// M0 is set inside the same statement; the compiler does not use M0 in this
// kernel (checked by a test on the generated code).
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_base) : "memory", "m0");
}

__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_base) : "memory", "m0");
}

// A wave-uniform pointer forced into SGPRs (the inline-asm loads take their
// base address as an SGPR pair; 64-bit address arithmetic may otherwise be
// left in VGPRs).
__device__ __forceinline__ const void* sgpr_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// LDS byte offset of a __shared__ object (generic -> local address space).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)(p)));
}

// 16-byte chunk swizzle inside a 128-byte LDS row: distinct chunks for any 8
// consecutive rows (32-bank view) and for the even / odd rows of any 16
// consecutive rows (64-bank view).
__device__ __forceinline__ int chunk_swizzle(int row) { return (row ^ (row >> 3)) & 7; }

// The 16 int8 weights {code * q} of one packed word (16 codes), as the four
// dwords of an MFMA / dot4 operand (dword i = codes 4i .. 4i+3 of the word).
// Fields at bits 0-1 / 4-5 of each byte are selectors {0,1,2} into
// ta = [-q, +q, 0, 0]; fields at bits 2-3 / 6-7, masked in place, are
// selectors {0,4,8}: byte 0 of tb1 (-q), byte 0 of tb0 (+q), or the sign fill
// of tb1's byte 1, which is 0.  9 VALU operations per 16 codes.
struct QTables {
  uint32_t ta, tb0, tb1;
};

__device__ __forceinline__ QTables make_tables(int qv) {
  // ta = [-q, +q, 0, 0]; tb0 = q (only its byte 0 is ever selected);
  // tb1 = [-q, 0, 0, 0] (byte 0, and the zero sign bit of byte 1)
  const uint32_t q = static_cast<uint32_t>(qv);
  const uint32_t neg = 0u - q;
  return QTables{__builtin_amdgcn_perm(q, neg, 0x0C0C0400u), q, __builtin_amdgcn_perm(0u, neg, 0x0C0C0C00u)};
}

__device__ __forceinline__ v4i unpack16(uint32_t w, const QTables& t) {
  const uint32_t w4 = w >> 4;
  v4i b;
  b.x = static_cast<int>(__builtin_amdgcn_perm(0u, t.ta, w & 0x03030303u));
  b.y = static_cast<int>(__builtin_amdgcn_perm(t.tb0, t.tb1, w & 0x0C0C0C0Cu));
  b.z = static_cast<int>(__builtin_amdgcn_perm(0u, t.ta, w4 & 0x03030303u));
  b.w = static_cast<int>(__builtin_amdgcn_perm(t.tb0, t.tb1, w4 & 0x0C0C0C0Cu));
  return b;
}

constexpr int kQTileBytes = 16384;  // q of a block tile: BN columns x its groups

// Block tile of 2 RM x FN fragments (BM = 64 RM rows, BN = 32 FN columns)
// computed by 2 WN WK waves: (wm, wn) split the tile 2 x WN and, with WK = 2,
// a pair of waves splits each stage's four k-steps.
template <int RM, int FN, int WK, int WN = 2>
struct Tile {
  static constexpr int RN = (FN + WN - 1) / WN;  // column fragments per wave
  static constexpr int BM = 64 * RM;
  static constexpr int BN = 32 * FN;
  static constexpr int NW = 2 * WN * WK;       // waves per workgroup
  static constexpr int THREADS = 64 * NW;
  static constexpr int KS = 4 / WK;            // k-steps of a stage per wave
  static constexpr int STAGES = RM >= 4 ? 3 : kStages;
  static constexpr int A_BYTES = BM * kStageK; // x_i8 of one stage
  static constexpr int B_BYTES = BN * 32;      // BN columns x 2 half-planes x 16 B
  static constexpr int A_INSTR = A_BYTES / 1024;   // 1 KB per load instruction
  static constexpr int B_INSTR = B_BYTES / 1024;
  static constexpr int A_PER_WAVE = (A_INSTR + NW - 1) / NW;
  static constexpr int B_PER_WAVE = (B_INSTR + NW - 1) / NW;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr int LOADS_PER_STAGE = A_PER_WAVE + B_PER_WAVE;
  static constexpr int SLOT_INTS = 2 * WN * RM * RN * 64 * 16;  // one split's partial tile
  static_assert((STAGES - 1) * LOADS_PER_STAGE < 64, "vmcnt range");
};

struct GemmArgs {
  const int8_t* x;
  const float* a_scale;
  const uint8_t* packed;
  const int8_t* q;
  const float* smax;
  void* out;
  int32_t* ws_part;    // [tiles][splits][SLOT_INTS] split-K partial tiles
  int M, N, K;
  int tiles_m, tiles_n, splits, stages_per_split;
  int tile_sn;         // column stride between block tiles: a tile computes
                       // BN columns and stores the first tile_sn (the
                       // planner sets tile_sn = BN)
};

// Writes one wave's RM x RN fragments of the output tile: fp32 y with the
// per-row / per-column scales (staged in LDS) or the raw int32 accumulators.
// 32x32 accumulator layout: lane holds column l32 of a fragment; register r
// holds row 8 (r / 4) + 4 half + (r % 4).
// Writes one wave's RM x RN fragments of the output tile: fp32 or bf16 y with
// the per-row / per-column scales (staged in LDS), or the raw int32
// accumulators.  32x32 accumulator layout: lane holds column l32 of a
// fragment; register r holds row 8 (r / 4) + 4 half + (r % 4).  Stored as is,
// every store instruction would cover only two 128-byte row pieces, and the
// output phase is bound by the number of store transactions (halving the
// bytes with bf16 was measured not to shorten it).  So when N % 4 == 0 each
// fragment goes through this wave's LDS scratch `tr` (32 rows x kTrStride
// words; the stride puts the two lane halves' writes on different banks) and
// comes back as 4 consecutive columns per lane: one 16-byte (8 for bf16)
// store per lane covers 8 rows of the fragment.
constexpr int kTrStride = 40;

// two fp32 values (as bit patterns) -> two bf16 in one dword, low one first
__device__ __forceinline__ uint32_t bf16_pair(int lo_bits, int hi_bits) {
  return f32_to_bf16_rne(__int_as_float(lo_bits)) |
         (static_cast<uint32_t>(f32_to_bf16_rne(__int_as_float(hi_bits))) << 16);
}

__device__ __forceinline__ void lds_wave_sync() {
  // LDS operations of one wave execute in order; the fences only keep the
  // compiler from moving the reads of other lanes' data above the writes (or
  // the next writes above these reads)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Stores one 32x32 fragment of one wave (MFMA layout: lane l32 = column,
// register r = row 8 (r / 4) + 4 (lane / 32) + r % 4) with its epilogue.
// row0/col0: the fragment's first output row and column; rs/cs: the scales of
// its 32 rows and 32 columns.  With N % 4 == 0 it goes through the wave's LDS
// transpose buffer tr and leaves as 16-byte stores of 4 columns (8 for bf16
// when N % 8 == 0); otherwise element by element.  Rows past M and columns
// past N are not stored.
template <int OUT>
__device__ __forceinline__ void store_frag(const v16i& acc, void* out, const float* rs, const float* cs,
                                           int M, int N, int row0, int col0, int lane, int32_t* tr) {
  const int l32 = lane & 31, half = lane >> 5;
  const float cscale = OUT == kOutAcc ? 0.0f : cs[l32] * (1.0f / 127.0f);
  if ((N & 3) != 0) {
    const int col = col0 + l32;
    if (col >= N) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rr = 8 * (r >> 2) + 4 * half + (r & 3);
      if (row0 + rr < M)
        store_out(out, static_cast<size_t>(row0 + rr) * N + col, OUT, acc[r],
                  OUT == kOutAcc ? 0.0f : static_cast<float>(acc[r]) * rs[rr] * cscale);
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rr = 8 * (r >> 2) + 4 * half + (r & 3);
    tr[rr * kTrStride + l32] =
        OUT == kOutAcc ? acc[r] : __float_as_int(static_cast<float>(acc[r]) * rs[rr] * cscale);
  }
  lds_wave_sync();
  if (OUT == kOutBf16 && (N & 7) == 0) {
    // 8 columns per lane: one 16-byte store covers 16 rows of the fragment
    const int c8 = 8 * (lane & 3);
    const int gcol = col0 + c8;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int rr = 16 * k + (lane >> 2);
      const v4i a = *reinterpret_cast<const v4i*>(tr + rr * kTrStride + c8);
      const v4i b = *reinterpret_cast<const v4i*>(tr + rr * kTrStride + c8 + 4);
      const int grow = row0 + rr;
      if (grow < M && gcol < N) {  // N % 8 == 0: all eight columns are in range
        const uint4 w = make_uint4(bf16_pair(a.x, a.y), bf16_pair(a.z, a.w), bf16_pair(b.x, b.y),
                                   bf16_pair(b.z, b.w));
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + static_cast<size_t>(grow) * N + gcol) = w;
      }
    }
    return;
  }
  const int c4 = 4 * (lane & 7);
  const int gcol = col0 + c4;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rr = 8 * k + (lane >> 3);
    const v4i v = *reinterpret_cast<const v4i*>(tr + rr * kTrStride + c4);
    const int grow = row0 + rr;
    if (grow < M && gcol < N) {  // N % 4 == 0: all four columns are in range
      const size_t o = static_cast<size_t>(grow) * N + gcol;
      if (OUT == kOutBf16)
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + o) =
            make_uint2(bf16_pair(v.x, v.y), bf16_pair(v.z, v.w));
      else
        *reinterpret_cast<v4i*>(static_cast<int32_t*>(out) + o) = v;
    }
  }
}

// Work item of a workgroup: XCD-aware order (consecutive items share a column
// block, i.e. the same weights, and land on one XCD), then (column block, row
// block, split).
struct WorkItem {
  int tile, split, m0, n0;
};

__device__ __forceinline__ WorkItem work_item(int bid, int tiles_m, int tiles_n, int splits,
                                              int bm, int sn) {
  const int total = tiles_m * tiles_n * splits;
  const int per = total / kXcds, rem = total % kXcds;
  const int xcd = bid % kXcds;
  const int lin = xcd * per + min(xcd, rem) + bid / kXcds;
  WorkItem w;
  w.split = lin % splits;
  w.tile = lin / splits;
  w.m0 = (w.tile % tiles_m) * bm;
  w.n0 = (w.tile / tiles_m) * sn;
  return w;
}

// LDS-only workgroup barrier: this wave's LDS operations have completed, then
// the waves meet (outstanding global stores are not waited for).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Register half of an accumulator fragment: in the 32x32 layout register r
// holds row 8 (r / 4) + 4 half + (r % 4), so registers 0-7 are rows 0-15 and
// registers 8-15 rows 16-31.
__device__ __forceinline__ v8i reg_half(const v16i& a, bool upper) {
  const v8i lo = __builtin_shufflevector(a, a, 0, 1, 2, 3, 4, 5, 6, 7);
  const v8i hi = __builtin_shufflevector(a, a, 8, 9, 10, 11, 12, 13, 14, 15);
  return upper ? hi : lo;
}

// Everything after the main loop for one wave.
//
// Wave-pair exchange (WK = 2): both waves of a pair hold int32 partials of the
// same RM x RN fragments over complementary k-steps.  Wave wk keeps rows
// [16 wk, 16 wk + 16) of every fragment (register half wk) and hands the
// other half to its partner through the idle pipeline buffers, XR fragments
// per round; the received half is added (exact).  wk only selects registers
// and offsets, so the code has no per-fragment branches and each round is one
// burst of LDS writes, a barrier and one burst of reads.
//
// Output: each kept half-fragment (16 rows x 32 columns) goes through a
// per-wave LDS transpose (two buffers, alternated, so that one fragment is
// written and read back while the stores of the previous one issue) and comes
// back as 4 consecutive columns per lane (8 for bf16 when N % 8 == 0): one
// 16-byte store covers 8 rows (bf16: 16).  Rows past M and columns past N are
// not stored (per-store predicates); with N % 4 != 0 the values are stored one
// by one straight from the registers.
//
// Split-K: the split's exact partial tile goes to the workspace instead, in
// the layout splitk_reduce_kernel reads (fragment, 16-byte chunk, lane).
template <int RM, int FN, int WK, int WN, int OUT>
__device__ __forceinline__ void finish_tile(v16i (&acc)[RM][(FN + WN - 1) / WN], const GemmArgs& p,
                                            const WorkItem& w, int8_t* smem, const float* row_scale,
                                            const float* col_scale, int wave, int wk, int lane) {
  using T = Tile<RM, FN, WK, WN>;
  constexpr int RN = T::RN, NF = RM * RN, NP = 2 * WN;  // NP: (wm, wn) pairs
  const int wm = wave & 1, wn = (wave >> 1) % WN, pair = wave % NP;
  const bool upper = WK == 2 && wk == 1;
  v8i kept[NF];
#pragma unroll
  for (int q = 0; q < NF; ++q) kept[q] = reg_half(acc[q / RN][q % RN], upper);
  if (WK == 2) {
    constexpr int XR = T::LDS_BYTES / (T::NW * 2 * 1024) < NF ? T::LDS_BYTES / (T::NW * 2 * 1024) : NF;
    static_assert(XR >= 1, "LDS too small for the wave-pair exchange");
    int32_t* xch = reinterpret_cast<int32_t*>(smem);
    // 16-byte chunk c (0, 1) of fragment slot k sent by wave (pair, sender)
    const auto slot = [&](int k, int sender, int c) {
      return xch + ((((k * 2 + sender) * NP + pair) * 2 + c) * 64 + lane) * 4;
    };
#pragma unroll
    for (int r0 = 0; r0 < NF; r0 += XR) {
      bare_barrier();  // the buffers are free (stage reads / previous round done)
#pragma unroll
      for (int k = 0; k < XR && r0 + k < NF; ++k) {
        const v8i s = reg_half(acc[(r0 + k) / RN][(r0 + k) % RN], !upper);
        *reinterpret_cast<v4i*>(slot(k, wk, 0)) = __builtin_shufflevector(s, s, 0, 1, 2, 3);
        *reinterpret_cast<v4i*>(slot(k, wk, 1)) = __builtin_shufflevector(s, s, 4, 5, 6, 7);
      }
      lds_barrier();
#pragma unroll
      for (int k = 0; k < XR && r0 + k < NF; ++k) {
        const v4i i0 = *reinterpret_cast<const v4i*>(slot(k, wk ^ 1, 0));
        const v4i i1 = *reinterpret_cast<const v4i*>(slot(k, wk ^ 1, 1));
        kept[r0 + k] += __builtin_shufflevector(i0, i1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
  }
  // every wave is past the exchange (or its last stage) before the buffers
  // become transposes
  lds_barrier();
  const int l32 = lane & 31, half = lane >> 5;
  const int row_off = upper ? 16 : 0;  // first fragment row this wave outputs
  if (p.splits > 1) {
    int32_t* mine = p.ws_part + (static_cast<size_t>(w.tile) * p.splits + w.split) * T::SLOT_INTS;
#pragma unroll
    for (int q = 0; q < NF; ++q) {
      const int i = q / RN, j = q % RN;
      const int c0 = WK == 2 ? 2 * wk : 0;
      int32_t* dst = mine + ((((pair * RM + i) * RN + j) * 4 + c0) * 64 + lane) * 4;
      *reinterpret_cast<v4i*>(dst) = __builtin_shufflevector(kept[q], kept[q], 0, 1, 2, 3);
      *reinterpret_cast<v4i*>(dst + 256) = __builtin_shufflevector(kept[q], kept[q], 4, 5, 6, 7);
      if (WK == 1) {
        const v8i hi = reg_half(acc[i][j], true);
        *reinterpret_cast<v4i*>(dst + 512) = __builtin_shufflevector(hi, hi, 0, 1, 2, 3);
        *reinterpret_cast<v4i*>(dst + 768) = __builtin_shufflevector(hi, hi, 4, 5, 6, 7);
      }
    }
    return;
  }
  static_assert(WK == 2, "the output path covers one register half per wave (wave pairs)");
  const int M = p.M, N = p.N, m0 = w.m0, n0 = w.n0;
  const int n_end = min(N, n0 + p.tile_sn);  // columns this tile stores
  if ((N & 3) != 0) {
    // rare shapes: element stores straight from the registers
#pragma unroll
    for (int q = 0; q < NF; ++q) {
      const int f = wn * RN + q % RN;
      const int col = n0 + 32 * f + l32;
      if ((FN % WN != 0 && f >= FN) || col >= n_end) continue;
      const float cscale = OUT == kOutAcc ? 0.0f : col_scale[32 * f + l32] * (1.0f / 127.0f);
      const int rbase = wm * 32 * RM + 32 * (q / RN) + row_off;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int rl = rbase + 8 * (r >> 2) + 4 * half + (r & 3);
        if (m0 + rl < M)
          store_out(p.out, static_cast<size_t>(m0 + rl) * N + col, OUT, kept[q][r],
                    OUT == kOutAcc ? 0.0f : static_cast<float>(kept[q][r]) * row_scale[rl] * cscale);
      }
    }
    return;
  }
  constexpr int kHalfWords = 16 * kTrStride;  // one transpose buffer
  static_assert(T::LDS_BYTES >= T::NW * 2 * kHalfWords * 4, "LDS too small for the output transposes");
  int32_t* tr0 = reinterpret_cast<int32_t*>(smem) + wave * 2 * kHalfWords;
  const bool bf16x8 = OUT == kOutBf16 && (N & 7) == 0;
  v4i rd[2][2];
  // transpose kept half-fragment q through buffer b into rd[b]
  const auto stage = [&](int q, int b) {
    const int f = wn * RN + q % RN;
    const int rbase = wm * 32 * RM + 32 * (q / RN) + row_off;
    const float cscale = OUT == kOutAcc ? 0.0f : col_scale[32 * f + l32] * (1.0f / 127.0f);
    int32_t* tr = tr0 + b * kHalfWords;
    lds_wave_sync();  // earlier reads of this buffer stay ahead of these writes
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int rr = 8 * (r >> 2) + 4 * half + (r & 3);
      tr[rr * kTrStride + l32] =
          OUT == kOutAcc ? kept[q][r]
                         : __float_as_int(static_cast<float>(kept[q][r]) * row_scale[rbase + rr] * cscale);
    }
    lds_wave_sync();
    if (bf16x8) {
      const int rr = lane >> 2, c8 = 8 * (lane & 3);
      rd[b][0] = *reinterpret_cast<const v4i*>(tr + rr * kTrStride + c8);
      rd[b][1] = *reinterpret_cast<const v4i*>(tr + rr * kTrStride + c8 + 4);
    } else {
      const int c4 = 4 * (lane & 7);
#pragma unroll
      for (int k = 0; k < 2; ++k) rd[b][k] = *reinterpret_cast<const v4i*>(tr + (8 * k + (lane >> 3)) * kTrStride + c4);
    }
  };
  const auto emit = [&](int q, int b) {
    const int f = wn * RN + q % RN;
    if (FN % WN != 0 && f >= FN) return;  // padding fragment (wave-uniform)
    const int grow0 = m0 + wm * 32 * RM + 32 * (q / RN) + row_off;
    if (bf16x8) {
      const int grow = grow0 + (lane >> 2), gcol = n0 + 32 * f + 8 * (lane & 3);
      if (grow < M && gcol < n_end)
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + static_cast<size_t>(grow) * N + gcol) =
            make_uint4(bf16_pair(rd[b][0].x, rd[b][0].y), bf16_pair(rd[b][0].z, rd[b][0].w),
                       bf16_pair(rd[b][1].x, rd[b][1].y), bf16_pair(rd[b][1].z, rd[b][1].w));
      return;
    }
    const int gcol = n0 + 32 * f + 4 * (lane & 7);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int grow = grow0 + 8 * k + (lane >> 3);
      if (grow < M && gcol < n_end) {  // n_end % 4 == 0: all four columns are in range
        const size_t o = static_cast<size_t>(grow) * N + gcol;
        if (OUT == kOutBf16)
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + o) =
              make_uint2(bf16_pair(rd[b][k].x, rd[b][k].y), bf16_pair(rd[b][k].z, rd[b][k].w));
        else
          *reinterpret_cast<v4i*>(static_cast<int32_t*>(p.out) + o) = rd[b][k];
      }
    }
  };
  stage(0, 0);
#pragma unroll
  for (int q = 1; q < NF; ++q) {
    __builtin_amdgcn_sched_barrier(0);
    stage(q, q & 1);
    emit(q - 1, (q - 1) & 1);
  }
  __builtin_amdgcn_sched_barrier(0);
  emit(NF - 1, (NF - 1) & 1);
}

template <int RM, int FN, int WK, int WN, int OUT>
__global__ __launch_bounds__(64 * 2 * WN * WK, 1) void gemm_kernel(GemmArgs p) {
  using T = Tile<RM, FN, WK, WN>;
  constexpr int RN = T::RN, BN = T::BN;
  __shared__ __attribute__((aligned(1024))) int8_t smem[T::LDS_BYTES];
  __shared__ __attribute__((aligned(16))) int8_t q_lds[kQTileBytes + 256];
  // epilogue scales of this tile, staged once: a_scale of its rows and
  // smax / 127 of its columns (reading them from global memory next to the
  // output stores would order every load behind the stores before it)
  __shared__ __attribute__((aligned(16))) float row_scale[T::BM];
  __shared__ __attribute__((aligned(16))) float col_scale[(T::BN + 63) / 64 * 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1;
  const int wn = (wave >> 1) % WN;
  const int wk = WK == 1 ? 0 : wave / (2 * WN);  // which k-steps of each stage
  const int l32 = lane & 31;
  const int half = lane >> 5;

  const WorkItem w = work_item(blockIdx.x, p.tiles_m, p.tiles_n, p.splits, T::BM, p.tile_sn);
  const int m0 = w.m0, n0 = w.n0;
  const int M = p.M, N = p.N, K = p.K;
  const int G = K >> 7;
  const int st_begin = w.split * p.stages_per_split;
  const int st_end = min(G, st_begin + p.stages_per_split);

  // ---- once per tile, loaded straight into LDS by the DMA path (no VGPR
  // staging, so the compiler never waits on these loads): the q block
  // [BN columns] x [groups g0 .. g0 + qw) (qw a multiple of 4, rows of q
  // contiguous: dword copies), and the epilogue scales -- a_scale of the rows
  // and smax of the columns.  Issued before the first stages' loads; the
  // first pipeline wait covers them.  The planner keeps BN * qw <= kQTileBytes
  // (q_lds has 256 spare bytes for the last, partly used instruction).
  const int g0 = st_begin & ~3;
  const int qw = (st_end - g0 + 3) & ~3;
  {
    const int qd = qw >> 2;
    const int q_dwords = BN * qd;
    const uint32_t q_base = lds_addr(q_lds);
    const int8_t* q_tile = p.q + static_cast<size_t>(n0) * G;
    for (int ii = wave; ii < (q_dwords + 63) / 64; ii += T::NW) {
      const int idx = min(ii * 64 + lane, q_dwords - 1);
      const int c = idx / qd, d = idx - c * qd;
      dma4(sgpr_ptr(q_tile), static_cast<uint32_t>((min(n0 + c, N - 1) - n0) * G + g0 + 4 * d),
           __builtin_amdgcn_readfirstlane(q_base + ii * 256));
    }
    if (OUT != kOutAcc) {
      const uint32_t r_base = lds_addr(row_scale), c_base = lds_addr(col_scale);
      for (int ii = wave; ii < T::BM / 64; ii += T::NW)
        dma4(sgpr_ptr(p.a_scale + m0), static_cast<uint32_t>((min(m0 + ii * 64 + lane, M - 1) - m0) * 4),
             __builtin_amdgcn_readfirstlane(r_base + ii * 256));
      for (int ii = wave; ii < (BN + 63) / 64; ii += T::NW)
        dma4(sgpr_ptr(p.smax + n0), static_cast<uint32_t>((min(n0 + ii * 64 + lane, N - 1) - n0) * 4),
             __builtin_amdgcn_readfirstlane(c_base + ii * 256));
    }
  }

  // ---- this wave's direct-to-LDS load slots.  Global addresses are a
  // wave-uniform tile base (SGPRs) plus a 32-bit per-lane offset; rows and
  // columns past M / N are clamped to the last one (computed, never stored).
  // Load instructions are dealt round robin to the waves; every wave issues
  // the same number per stage (a wave past the last instruction of a kind
  // repeats an earlier one: same data to the same LDS bytes), which keeps the
  // per-stage load count static for the vmcnt bookkeeping.
  const int8_t* x_tile = p.x + static_cast<size_t>(m0) * K;
  // weights: tiled layout, tile (row block r, group g) of 64 rows x 32 bytes at
  // byte (r * G + g) * 2048; the tile base is this workgroup's first row block
  const uint8_t* w_tile = p.packed + static_cast<size_t>(n0 >> 6) * G * 2048;
  // A: instruction ia covers rows 8 ia .. 8 ia + 7 (1 KB, 8 lanes per 128-byte
  // row); lane -> row, 16-B slot, holding chunk slot ^ swizzle(row)
  uint32_t a_off[T::A_PER_WAVE];
  int a_lds[T::A_PER_WAVE];
#pragma unroll
  for (int i = 0; i < T::A_PER_WAVE; ++i) {
    const int ia = (wave + T::NW * i) % T::A_INSTR;
    const int r = 8 * ia + (lane >> 3);
    const int chunk = (lane & 7) ^ chunk_swizzle(r);
    a_off[i] = static_cast<uint32_t>((min(m0 + r, M - 1) - m0) * K + 16 * chunk);
    a_lds[i] = ia * 1024;
  }
  // B: instruction ib covers columns 32 ib .. 32 ib + 31 (2 lanes per column:
  // its 32 bytes of the stage); LDS slot 2 col + p holds half-plane
  // h = p ^ ((col >> 3) & 1), which spreads a fragment read over all banks.
  uint32_t b_off[T::B_PER_WAVE];
  int b_lds[T::B_PER_WAVE];
#pragma unroll
  for (int i = 0; i < T::B_PER_WAVE; ++i) {
    const int ib = (wave + T::NW * i) % T::B_INSTR;
    const int col = 32 * ib + (lane >> 1);
    const int h = (lane & 1) ^ ((col >> 3) & 1);
    const int nc = min(n0 + col, N - 1);
    b_off[i] = static_cast<uint32_t>(((nc >> 6) - (n0 >> 6)) * G * 2048 + (nc & 63) * 32 + 16 * h);
    b_lds[i] = T::A_BYTES + ib * 1024;
  }

  const uint32_t smem_base = lds_addr(smem);
  // load instruction `i` (A first, then B) of stage `st` into buffer `buf`
  auto issue_one = [&](int i, int st, int buf) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(smem_base + buf * T::STAGE_BYTES);
    if (i < T::A_PER_WAVE)
      dma16(x_tile + static_cast<size_t>(st) * kStageK, a_off[i], base + a_lds[i]);
    else
      dma16(sgpr_ptr(w_tile + static_cast<size_t>(st) * 2048), b_off[i - T::A_PER_WAVE],
            base + b_lds[i - T::A_PER_WAVE]);
  };
  auto issue = [&](int st, int buf) {
#pragma unroll
    for (int i = 0; i < T::LOADS_PER_STAGE; ++i) issue_one(i, st, buf);
  };

  // ---- operand fragments of this lane
  int a_row[RM];
#pragma unroll
  for (int i = 0; i < RM; ++i) a_row[i] = wm * 32 * RM + 32 * i + l32;
  int b_slot[RN];  // LDS byte offset of this lane's B words in a stage
  int q_pos[RN];   // offset of this lane's column in the q block
#pragma unroll
  for (int j = 0; j < RN; ++j) {
    const int c = min(32 * (wn * RN + j) + l32, BN - 1);  // padding fragment clamped
    b_slot[j] = (2 * c + (half ^ ((c >> 3) & 1))) * 16 + 4 * T::KS * wk;
    q_pos[j] = c * qw - g0;
  }

  v16i acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j) acc[i][j] = v16i{0};

  // ---- pipeline.  STAGES buffers, all in flight.  Per stage the wave runs KS
  // k-steps (k-step index 4 wk / WK .. ), in two halves.  The operands of a
  // stage are read from LDS ahead of the MFMAs that use them, so LDS latency
  // hides behind matrix work: A of the second half while the first half's
  // MFMAs run, and A of the next stage's first half, its packed words and q
  // bytes (after the stage barrier) while the second half's MFMAs run.
  // Loop body for stage st:
  //   MFMAs(first half) | wait own DMA of st+1, barrier | read next stage |
  //   MFMAs(second half) interleaved with the DMA of stage st+STAGES into the
  //   buffer of st (free: the barrier proves every wave is past its reads).
  constexpr int KS = T::KS, KH = KS / 2;
  typedef unsigned int words_t __attribute__((ext_vector_type(KS)));
  const int s0 = KS * wk;  // first k-step of this wave
  const auto read_a = [&](int b, int h, v4i (&a)[RM][KH]) {
    const int8_t* As = smem + b * T::STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int t = 0; t < KH; ++t)
        a[i][t] = *reinterpret_cast<const v4i*>(
            As + a_row[i] * kStageK + 16 * ((4 * half + s0 + KH * h + t) ^ chunk_swizzle(a_row[i])));
  };
  const auto read_b = [&](int b, int st, words_t (&bw)[RN], int (&qb)[RN]) {
    const int8_t* Bs = smem + b * T::STAGE_BYTES + T::A_BYTES;
#pragma unroll
    for (int j = 0; j < RN; ++j) {
      bw[j] = *reinterpret_cast<const words_t*>(Bs + b_slot[j]);
      qb[j] = q_lds[q_pos[j] + st];
    }
  };
  constexpr int S = T::STAGES;
  constexpr int SLOTS = RN * KH;  // DMA issue slots in the second half
#pragma unroll
  for (int k = 0; k < S; ++k) issue(min(st_begin + k, st_end - 1), k);
  wait_vmcnt<(S - 1) * T::LOADS_PER_STAGE>();  // own loads of the first stage done
  bare_barrier();
  v4i a0[RM][KH], a1[RM][KH];
  // The stage loop is unrolled by U (a multiple of S and of 2), so that the
  // buffer of every stage is a compile-time constant (LDS addresses fold into
  // the instructions' offsets) and the packed words alternate between two
  // register sets instead of being copied.
  constexpr int U = S % 2 == 0 ? S : 2 * S;
  words_t bwv[2][RN];
  int qbv[2][RN];
  read_a(0, 0, a0);
  read_b(0, st_begin, bwv[0], qbv[0]);
  for (int st0 = st_begin; st0 < st_end; st0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int st = st0 + u;
      if (st >= st_end) break;
      const int buf = u % S, nbuf = (u + 1) % S;
      const int cur = u & 1, nxt = cur ^ 1;
      const int dst = min(st + S, st_end - 1);  // stage whose DMA reuses this buffer
      QTables tab[RN];
#pragma unroll
      for (int j = 0; j < RN; ++j) tab[j] = make_tables(qbv[cur][j]);
      read_a(buf, 1, a1);
      __builtin_amdgcn_sched_barrier(0);  // keep these reads ahead of the first half's MFMAs
      // first half; the MFMA clusters run at raised wave priority, so that a
      // wave issuing MFMAs is not held back by the unpack and LDS work of the
      // other waves of its SIMD (measured 2-4% faster on the 512-token
      // prefill of 5120 -> 17408)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int t = 0; t < KH; ++t)
#pragma unroll
        for (int j = 0; j < RN; ++j) {
          const v4i b = unpack16(bwv[cur][j][t], tab[j]);
#pragma unroll
          for (int i = 0; i < RM; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0[i][t], b, acc[i][j], 0, 0, 0);
        }
      __builtin_amdgcn_s_setprio(0);
      // this wave's reads of buffer `buf` have landed, on both paths below
      // (so that at the join the compiler does not wait for them again)
      wait_lgkm0();
      if (st + 1 < st_end) {
        wait_vmcnt<(S - 2) * T::LOADS_PER_STAGE>();  // own loads of stage st+1 done
        bare_barrier();  // everyone's stage st+1 is in LDS; everyone is past buffer `buf`
        read_a(nbuf, 0, a0);
        read_b(nbuf, st + 1, bwv[nxt], qbv[nxt]);
        __builtin_amdgcn_sched_barrier(0);  // and these ahead of the second half's
      }
      // second half, with this stage's DMA into the freed buffer
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int t = 0; t < KH; ++t)
#pragma unroll
        for (int j = 0; j < RN; ++j) {
          const v4i b = unpack16(bwv[cur][j][KH + t], tab[j]);
#pragma unroll
          for (int i = 0; i < RM; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1[i][t], b, acc[i][j], 0, 0, 0);
#pragma unroll
          for (int k = 0; k < T::LOADS_PER_STAGE; ++k)
            if ((k * SLOTS) / T::LOADS_PER_STAGE == t * RN + j) issue_one(k, dst, buf);
        }
      __builtin_amdgcn_s_setprio(0);
    }
  }
  wait_vmcnt<0>();  // drain the padding loads of the tail before the LDS is reused
  finish_tile<RM, FN, WK, WN, OUT>(acc, p, w, smem, row_scale, col_scale, wave, wk, lane);
}

// Split-K second pass: one wave per output fragment (block tile, wave role
// (wm, wn) of the GEMM's wk = 0 waves, fragment i * RN + j), so that the
// partial tiles are read by a grid that spans the chip; adds the splits'
// partial fragments in split order (exact int32) and runs the same epilogue.
template <int RM, int FN, int OUT>
__global__ __launch_bounds__(64) void splitk_reduce_kernel(GemmArgs p) {
  using T = Tile<RM, FN, 1>;
  constexpr int RN = T::RN, NF = RM * RN, NP = 4;  // NP: wave roles (wm, wn)
  __shared__ float scales[64];  // the fragment's 32 row scales, then its 32 column scales
  __shared__ __attribute__((aligned(16))) int32_t tr_lds[32 * kTrStride];
  const int lane = threadIdx.x;
  const int unit = blockIdx.x;
  const int q = unit % NF, pair = (unit / NF) % NP, tile = unit / (NF * NP);
  const int i = q / RN, j = q % RN, wm = pair & 1, wn = pair >> 1;
  const int f = wn * RN + j;  // column fragment within the tile
  if (f >= FN) return;        // padding fragment: nothing to store
  const int m0 = (tile % p.tiles_m) * T::BM, n0 = (tile / p.tiles_m) * p.tile_sn;
  const int row0 = m0 + wm * 32 * RM + 32 * i, col0 = n0 + 32 * f;
  // one scale per lane (lanes 0-31: rows, 32-63: columns), loaded branch-free
  // ahead of the partials and written to LDS after them
  float sv = 0.0f;
  if (OUT != kOutAcc) {
    const float rsv = p.a_scale[min(row0 + (lane & 31), p.M - 1)];
    const float csv = p.smax[min(col0 + (lane & 31), p.N - 1)];
    sv = lane < 32 ? rsv : csv;
  }
  v16i acc = v16i{0};
  const int32_t* part = p.ws_part + static_cast<size_t>(tile) * p.splits * T::SLOT_INTS +
                        (static_cast<size_t>((pair * RM + i) * RN + j) * 256 + lane) * 4;
  // four splits' loads in flight at a time; a split index past the last is
  // clamped to it (an in-bounds re-read) and its values are not added
  for (int sp = 0; sp < p.splits; sp += 4) {
    v4i v[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int su = min(sp + u, p.splits - 1);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        v[u][c] = *reinterpret_cast<const v4i*>(part + static_cast<size_t>(su) * T::SLOT_INTS + c * 256);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool use = sp + u < p.splits;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[4 * c] += use ? v[u][c].x : 0;
        acc[4 * c + 1] += use ? v[u][c].y : 0;
        acc[4 * c + 2] += use ? v[u][c].z : 0;
        acc[4 * c + 3] += use ? v[u][c].w : 0;
      }
    }
  }
  scales[lane] = sv;
  __syncthreads();
  store_frag<OUT>(acc, p.out, scales, scales + 32, p.M, p.N, row0, col0, lane, tr_lds);
}

// ---------------------------------------------------------------- planner

struct Plan {
  int rm = 0, fn = 0, wk = 2, wn = 2, sn = 0, splits = 1, stages_per_split = 0, tiles_m = 0, tiles_n = 0;
  size_t slot_ints = 0;
};

struct Cfg {
  int rm, fn, wk, wn;
};
// (RM, FN, WK, WN): 2 WN WK waves.  The three-column-wave shapes (12 waves,
// three per SIMD) exist for widths such as 17408 = 17 x 1024, where a
// 128 x 288 tile advanced by 272 columns gives exactly 256 tiles.
constexpr Cfg kCfgs[] = {{1, 4, 2, 2}, {1, 8, 2, 2}, {1, 10, 2, 2}, {2, 4, 2, 2}, {2, 5, 2, 2},
                         {2, 8, 2, 2}, {2, 9, 2, 2}, {2, 10, 2, 2}, {4, 2, 2, 2}, {4, 4, 2, 2},
                         {2, 9, 2, 3}};

// Estimated cycles of one block tile on one CU.  Per 128-k stage and SIMD
// (NW / 4 waves, each running 4 / WK k-steps of RM x RN MFMAs): MFMA issue
// (32 cycles per 32x32x32, ~10% lost), unpack VALU (9 ops x 4 cycles per
// column fragment and k-step, plus per-stage overhead), LDS traffic (fragment
// reads of all waves plus the DMA writes, 128 B/clk) and L2->CU traffic
// (64 B/clk); a stage costs the largest of these plus a fixed barrier/wait
// overhead.  Then pipeline fill, epilogue stores and, with split-K, the
// partial-tile traffic.
double tile_cycles(int rm, int fn, int wn, int stages, int splits) {
  const int rn = (fn + wn - 1) / wn, bm = 64 * rm, bn = 32 * fn;
  const int nw = 4 * wn;                 // waves (WK = 2)
  const double wps = nw / 4.0;           // waves per SIMD
  const double mfma = wps * 2.0 * rm * rn * 32.0 * 1.1;
  const double valu = wps * (2.0 * rn * 9 * 4 + rn * 12.0 + 20.0);
  const double dma = static_cast<double>(bm) * 128 + bn * 32.0;
  const double lds = nw * (2.0 * rm * 1024 + rn * 512.0) / 128.0 + dma / 128.0;
  const double l2 = dma / 64.0;
  const double stage = std::max(std::max(mfma, valu), std::max(lds, l2)) + 250.0;
  double t = stages * stage + 2500.0 + bm * bn * 4.0 / 32.0;
  if (splits > 1) {
    // partial tile out, and the reduce kernel's reads of all splits
    const double slot = 4.0 * 4 * rm * rn * 1024;
    t += slot / 32.0 + slot / 32.0 + 1500.0;
  }
  return t;
}

// Choose the block tile and the split count that minimise the estimated
// makespan (tiles are spread evenly, so the busiest CU runs ceil(units / CUs)
// tiles).  Tiles advance by their full width (a stride 16 columns short, the
// last half fragment recomputed by the next tile, was measured no faster for
// N = 17408); the three-column-wave shapes are used without split-K only.
Plan make_plan(int64_t M, int64_t N, int64_t K, int cus) {
  Plan best;
  double best_t = 1e300;
  const int n_stages = static_cast<int>(K / kStageK);
  for (const Cfg& c : kCfgs) {
    const int bm = 64 * c.rm, bn = 32 * c.fn, rn = (c.fn + c.wn - 1) / c.wn;
    for (int sn : {bn}) {
      const int64_t tm = (M + bm - 1) / bm, tn = (N + sn - 1) / sn;
      for (int s = 1; s <= 32; ++s) {
        if (s > 1 && (sn != bn || c.wn != 2)) break;
        const int sps = (n_stages + s - 1) / s;
        const int splits = (n_stages + sps - 1) / sps;
        if (splits != s) continue;
        const int64_t units = tm * tn * splits;
        if (units > (int64_t{1} << 31) - 1) continue;
        if (static_cast<int64_t>(bn) * (((sps + 3) & ~3) + 4) > kQTileBytes) continue;
        const int64_t rounds = (units + cus - 1) / cus;
        const double tc = tile_cycles(c.rm, c.fn, c.wn, sps, splits);
        // makespan, plus a small charge for the total work (padding fragments,
        // recomputed columns, shared L2/HBM traffic) so that of two plans with
        // the same number of rounds the one with fewer, fuller tiles wins
        const double t = static_cast<double>(rounds) * tc +
                         0.15 * tc * static_cast<double>(units) / cus *
                             (static_cast<double>(c.wn * rn) / c.fn) * (static_cast<double>(bn) / sn);
        if (t < best_t * 0.995) {
          best_t = t;
          best.rm = c.rm;
          best.fn = c.fn;
          best.wk = c.wk;
          best.wn = c.wn;
          best.sn = sn;
          best.splits = splits;
          best.stages_per_split = sps;
          best.tiles_m = static_cast<int>(tm);
          best.tiles_n = static_cast<int>(tn);
          best.slot_ints = static_cast<size_t>(2 * c.wn) * c.rm * rn * 64 * 16;
        }
      }
    }
  }
  return best;
}

size_t plan_workspace_bytes(const Plan& pl) {
  if (pl.splits <= 1) return 0;
  const size_t tiles = static_cast<size_t>(pl.tiles_m) * pl.tiles_n;
  return tiles * pl.splits * pl.slot_ints * sizeof(int32_t);
}

template <int RM, int FN, int WK, int WN, int OUT>
hipError_t launch_cfg_out(const GemmArgs& a, hipStream_t stream) {
  using T = Tile<RM, FN, WK, WN>;
  const unsigned tiles = static_cast<unsigned>(a.tiles_m) * a.tiles_n;
  const unsigned grid = tiles * a.splits;
  hipLaunchKernelGGL((gemm_kernel<RM, FN, WK, WN, OUT>), dim3(grid), dim3(T::THREADS), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits <= 1) return e;
  if (WN != 2) return hipErrorInvalidConfiguration;  // split-K is planned for WN = 2 only
  const unsigned units = tiles * 4u * static_cast<unsigned>(RM * T::RN);  // one wave per fragment
  hipLaunchKernelGGL((splitk_reduce_kernel<RM, FN, OUT>), dim3(units), dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <int RM, int FN, int WK, int WN>
hipError_t launch_cfg(const GemmArgs& a, OutKind out_kind, hipStream_t stream) {
  switch (out_kind) {
    case kOutAcc: return launch_cfg_out<RM, FN, WK, WN, kOutAcc>(a, stream);
    case kOutBf16: return launch_cfg_out<RM, FN, WK, WN, kOutBf16>(a, stream);
    default: return launch_cfg_out<RM, FN, WK, WN, kOutF32>(a, stream);
  }
}

}  // namespace

void gemm_plan_info(int64_t M, int64_t N, int64_t K, const DeviceInfo& dev, int64_t* info) {
  const Plan pl = make_plan(M, N, K, std::max(1, dev.cu_count));
  info[0] = 1;
  info[1] = 64 * pl.rm;
  info[2] = 32 * pl.fn;
  info[3] = pl.splits;
  info[4] = static_cast<int64_t>(pl.tiles_m) * pl.tiles_n * pl.splits;
  info[5] = 2 * pl.wn * pl.wk;
  info[6] = pl.splits > 1 ? 1 : 0;
  info[7] = static_cast<int64_t>(plan_workspace_bytes(pl));
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, const DeviceInfo& dev) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return plan_workspace_bytes(make_plan(M, N, K, std::max(1, dev.cu_count)));
}

hipError_t launch_gemm(const int8_t* x_i8, const float* a_scale, const uint8_t* packed,
                       const int8_t* q, const float* smax, int64_t M, int64_t N, int64_t K,
                       void* out, OutKind out_kind, void* workspace, size_t, const DeviceInfo& dev,
                       hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const Plan pl = make_plan(M, N, K, std::max(1, dev.cu_count));
  if (pl.rm == 0 || 32 * pl.fn * (((pl.stages_per_split + 3) & ~3) + 4) > kQTileBytes)
    return hipErrorInvalidConfiguration;  // no plan fits the q block in LDS
  if (std::getenv("TWL_LOG"))
    std::fprintf(stderr, "[twl] gemm M=%lld N=%lld K=%lld -> tile %dx%d (stride %d), %d waves, splits=%d (%d groups each) grid=%d\n",
                 static_cast<long long>(M), static_cast<long long>(N), static_cast<long long>(K),
                 64 * pl.rm, 32 * pl.fn, pl.sn, 2 * pl.wn * pl.wk, pl.splits, pl.stages_per_split,
                 pl.tiles_m * pl.tiles_n * pl.splits);
  GemmArgs a;
  a.x = x_i8;
  a.a_scale = a_scale;
  a.packed = packed;
  a.q = q;
  a.smax = smax;
  a.out = out;
  a.ws_part = static_cast<int32_t*>(workspace);
  a.M = static_cast<int>(M);
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  a.tiles_m = pl.tiles_m;
  a.tiles_n = pl.tiles_n;
  a.splits = pl.splits;
  a.stages_per_split = pl.stages_per_split;
  a.tile_sn = pl.sn;
#define TWL_CFG(RM_, FN_, WK_, WN_)                                 \
  if (pl.rm == RM_ && pl.fn == FN_ && pl.wk == WK_ && pl.wn == WN_) \
    return launch_cfg<RM_, FN_, WK_, WN_>(a, out_kind, stream);
  TWL_CFG(1, 4, 2, 2)
  TWL_CFG(1, 8, 2, 2)
  TWL_CFG(1, 10, 2, 2)
  TWL_CFG(2, 4, 2, 2)
  TWL_CFG(2, 5, 2, 2)
  TWL_CFG(2, 8, 2, 2)
  TWL_CFG(2, 9, 2, 2)
  TWL_CFG(2, 10, 2, 2)
  TWL_CFG(4, 2, 2, 2)
  TWL_CFG(4, 4, 2, 2)
  TWL_CFG(2, 9, 2, 3)
#undef TWL_CFG
  return hipErrorInvalidValue;
}

}  // namespace twl
