// Decode ternary linear (M <= 24 tokens): two HBM-streaming kernels over the
// packed 2-bit weights, a VALU int8 dot-product GEMV for the smallest batches
// and a matrix-core variant for the rest.
//
// Method ([P1] "Ternary-Bonsai-2-27B on 2x RTX 5070 with vLLM TP=2", section 4
// for the arithmetic, section 5 for the prior art): the same exact int32
// accumulator as the prefill GEMM,
//   acc[t,n] = sum_k x_i8[t,k] * code[n,k] * q[n, k/128],
//   y[t,n]   = acc[t,n] * a_scale[t] * smax[n] / 127.
// The pages tried a dp4a decode GEMV on their GPU (section 5 table: 2.1x as a
// kernel, +2% end to end, rejected because its error grew); here both decode
// kernels are bit-exact with the GEMM because all compute the same integer sum.
//
// gfx950 mapping (both kernels)
//   * A workgroup holds one 64-row block and one K range; each wave takes a
//     run of at most GMAX consecutive 128-groups of that range and issues the
//     loads of its whole run up front (up to GMAX x 2 KB per wave in flight),
//     so the memory system sees the matrix as one burst instead of a
//     latency-bound sequence of small reads.  In the tiled weight layout a
//     wave's group is one contiguous 2 KB tile, read with two 1 KB loads.
//   * Per packed word: 1 shift, 4 ANDs, 4 byte-permutes against tables built
//     from {-q, +q, 0} give the 16 int8 weights code * q.
//   * The waves' partial sums meet in LDS through integer atomics (exact).
//     Streaming is bound per CU (about 22 GB/s each, measured), so every CU
//     needs an equal share: when there are too few row blocks, K is also split
//     across workgroups ("slices"), each slice writes its int32 partial sums to
//     the workspace and a second kernel adds them in slice order and rescales.
// dot4 kernel (gemv_kernel): lane l owns row n0 + l; one half-wave swap
//   (v_permlane32_swap) gives each lane its row's 8 words, then 4 v_dot4 per
//   word and token, with the activations read at wave-uniform addresses
//   through the constant address space (scalar loads, one copy per wave).
//   Its VALU work grows with M: it is used for M < 4 on layers too narrow
//   for the row-balanced kernel.
// MFMA kernels: the tokens padded to 32 form the B operand of
//   v_mfma_i32_32x32x32_i8 (in gemv_rows_kernel at up to 16 tokens: padded to
//   16, v_mfma_i32_16x16x64_i8; above 16 tokens, where 16-row subtiles pad the
//   rows less, two 16-token operands of that instruction) and the unpacked
//   weights the A operand, which makes the work nearly independent of M.
//   gemv_rows_kernel gives every CU an equal contiguous range of rows over all
//   of K (no partial sums leave the workgroup) and is used at every M whenever
//   each CU gets at least 16 rows;
//   gemv_mfma_kernel keeps the 64-row-block split with K slices (4 <= M <= 24)
//   for layers with fewer rows per CU.
#include "rotate_block.h"

#include <algorithm>
#include <type_traits>
#include <cstdio>
#include <cstdlib>

namespace twl {
namespace {

constexpr int kMaxWaves = 16;

// Activations are read at wave-uniform addresses; reading them through the
// constant address space makes them scalar loads (one copy in SGPRs for the
// whole wave) instead of 64 identical vector loads.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(4))) const u32x4 const_u32x4;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i_t __attribute__((ext_vector_type(16)));

// The 16 int8 weights {code * q} of one packed word (16 codes), as the four
// dwords of a dot4 operand (dword i = codes 4i .. 4i+3 of the word).  Fields
// at bits 0-1 / 4-5 of each byte are selectors {0,1,2} into ta = [-q, +q, 0,
// 0]; fields at bits 2-3 / 6-7, masked in place, are selectors {0,4,8}: byte 0
// of tb1 (-q), byte 0 of tb0 (+q), or the sign fill of tb1's byte 1, which is
// 0.  9 VALU operations per 16 codes.
struct QTables {
  uint32_t ta, tb0, tb1;
};

__device__ __forceinline__ QTables make_tables(int qv) {
  const uint32_t neg = static_cast<uint32_t>(-qv) & 0xFFu;
  const uint32_t pos = static_cast<uint32_t>(qv) & 0xFFu;
  return QTables{neg | (pos << 8), pos, neg};
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

struct GemvArgs {
  const int8_t* x;
  const float* a_scale;
  const uint8_t* packed;
  const int8_t* q;
  const float* smax;
  void* out;          // y [M,N] (fp32 or bf16) or int32 acc [M,N]
  int32_t* part;      // [slices][M][N] int32 partial sums when slices > 1
  int N, K, G;        // G = K / 128
  int n_rb;           // 64-row blocks
  int slices;         // workgroups per row block (K split across workgroups)
  int out_kind;       // OutKind
  // fused rotation (gemv_rows_kernel with ROT): the kernel quantises its own
  // activations from bf16 x [M, K] (with silu, [gate | up] [M, 2K]) and writes
  // x_i8 [M, K] and a_scale [M] from workgroup 0
  const uint16_t* xb;
  const int8_t* sign;
  int8_t* x_i8_out;
  float* a_scale_out;
  int silu;
};

// v_permlane32_swap_b32 exchanges lanes 32..63 of its first operand with lanes
// 0..31 of its second: applied to each dword of two 16-byte values it moves
// lo's upper-lane half into hi's lower lanes and back.
__device__ __forceinline__ void swap_halves(uint4& lo, uint4& hi) {
  auto r0 = __builtin_amdgcn_permlane32_swap(lo.x, hi.x, false, false);
  auto r1 = __builtin_amdgcn_permlane32_swap(lo.y, hi.y, false, false);
  auto r2 = __builtin_amdgcn_permlane32_swap(lo.z, hi.z, false, false);
  auto r3 = __builtin_amdgcn_permlane32_swap(lo.w, hi.w, false, false);
  lo = make_uint4(r0[0], r1[0], r2[0], r3[0]);
  hi = make_uint4(r0[1], r1[1], r2[1], r3[1]);
}

// Direct global->LDS loads for the activations of the row-balanced kernel.
// Three 1 KB instructions (lane i writes LDS[lds + 1024 k + 16 i]) at address
// sbase (wave-uniform, SGPR pair) + voff_k (per lane).  Issued from inline asm
// so that the compiler does not drain vmcnt before every LDS read; the kernel
// waits for them itself.  The LDS reads of the slot being refilled are
// complete first (lgkmcnt(0)).
// `n` (1 .. 3, wave-uniform) instructions are issued: tokens 8 n .. 23 of a
// slot are not loaded when M <= 8 n.
__device__ __forceinline__ void dma16xn(int n, const void* sbase, uint32_t v0, uint32_t v1, uint32_t v2,
                                        uint32_t lds0, uint32_t lds1, uint32_t lds2) {
  if (n >= 3)
    asm volatile(
        "s_waitcnt lgkmcnt(0)\n\t"
        "s_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %0, %6\n\t"
        "s_mov_b32 m0, %4\n\tglobal_load_lds_dwordx4 %1, %6\n\t"
        "s_mov_b32 m0, %5\n\tglobal_load_lds_dwordx4 %2, %6"
        :: "v"(v0), "v"(v1), "v"(v2), "s"(lds0), "s"(lds1), "s"(lds2), "s"(sbase) : "memory", "m0");
  else if (n == 2)
    asm volatile(
        "s_waitcnt lgkmcnt(0)\n\t"
        "s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %4\n\t"
        "s_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %4"
        :: "v"(v0), "v"(v1), "s"(lds0), "s"(lds1), "s"(sbase) : "memory", "m0");
  else
    asm volatile(
        "s_waitcnt lgkmcnt(0)\n\t"
        "s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, %2"
        :: "v"(v0), "s"(lds0), "s"(sbase) : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] + vmcnt_hi[15:14], expcnt[6:4], lgkmcnt[11:8]
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ const void* sgpr_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)(p)));
}

// 16-byte chunk swizzle inside a 128-byte LDS row (distinct chunks for any 8
// consecutive rows, so the column-wise 16-byte reads hit distinct banks).
__device__ __forceinline__ int chunk_swizzle(int row) { return (row ^ (row >> 3)) & 7; }

// Wait until at most `later` groups of PER loads each are outstanding (a
// constant once the caller's loop is unrolled; later <= 4).
template <int PER>
__device__ __forceinline__ void wait_groups_after(int later) {
  switch (later) {
    case 1: wait_vmcnt<PER>(); break;
    case 2: wait_vmcnt<2 * PER>(); break;
    case 3: wait_vmcnt<3 * PER>(); break;
    case 4: wait_vmcnt<4 * PER>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

// MT is the exact number of tokens (1 .. 24).  A workgroup of nw waves covers
// one 64-row block and one K slice; its waves split the slice's groups as
// evenly as possible, at most GMAX each.  Static LDS: MT x 64 ints for the
// cross-wave sums.
template <int MT, int GMAX>
__global__ __launch_bounds__(1024) void gemv_kernel(GemvArgs a) {
  __shared__ int red[MT * 64];
  const int lane = threadIdx.x & 63;
  // wave index as a scalar: everything derived from it (the K range, the
  // activation addresses) is then known to be wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int rb = blockIdx.x % a.n_rb;
  const int slice = blockIdx.x / a.n_rb;
  const int n0 = rb * 64;
  const int N = a.N, K = a.K, G = a.G;

  for (int i = threadIdx.x; i < MT * 64; i += blockDim.x) red[i] = 0;
  __syncthreads();

  const int s_lo = (slice * G) / a.slices;
  const int s_n = ((slice + 1) * G) / a.slices - s_lo;
  const int g0 = s_lo + (wave * s_n) / nw;
  const int ng = s_lo + ((wave + 1) * s_n) / nw - g0;   // 0 .. GMAX

  if (ng > 0) {
    // The group's weights are one contiguous 2 KB tile (64 rows x 32 bytes;
    // rows past N are code-0 padding), read with two 1 KB loads: in load A
    // lane l < 32 takes bytes 0-15 of row l and lane l >= 32 bytes 16-31 of
    // row l - 32; load B the same for rows 32..63.  One half-swap (lanes
    // 32..63 of A with lanes 0..31 of B) then leaves lane l with bytes 0-15
    // (A) and 16-31 (B) of its own row n0 + l.
    const int hsel = lane >> 5;
    const int rlo = lane & 31;
    const uint8_t* srcA = a.packed + static_cast<size_t>(rb) * G * 2048 + rlo * 32 + hsel * 16;
    const uint8_t* srcB = srcA + 1024;
    const int8_t* qrow = a.q + static_cast<size_t>(min(n0 + lane, N - 1)) * G;

    // all of this wave's groups in flight at once (slots past ng re-read the
    // last group, which is already on its way: no extra HBM traffic)
    uint4 dA[GMAX], dB[GMAX];
#pragma unroll
    for (int j = 0; j < GMAX; ++j) {
      const size_t g = static_cast<size_t>(g0 + min(j, ng - 1));
      dA[j] = *reinterpret_cast<const uint4*>(srcA + g * 2048);
      dB[j] = *reinterpret_cast<const uint4*>(srcB + g * 2048);
    }
    int qv[GMAX];
#pragma unroll
    for (int j = 0; j < GMAX; ++j) qv[j] = qrow[g0 + min(j, ng - 1)];

    // small M: two accumulator chains per token so consecutive dot4s do not
    // wait on each other
    constexpr int NA = MT <= 4 ? 2 : 1;
    int acc[NA][MT];
#pragma unroll
    for (int c = 0; c < NA; ++c)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[c][t] = 0;

#pragma unroll
    for (int j = 0; j < GMAX; ++j) {
      if (j != 0 && j >= ng) continue;   // ng >= 1: group 0 always runs
      uint4 lo = dA[j], hi = dB[j];
      swap_halves(lo, hi);
      const uint32_t words[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      const QTables tab = make_tables(qv[j]);
      const int8_t* xg = a.x + static_cast<size_t>(g0 + j) * 128;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const v4i wq = unpack16(words[w], tab);
        const int wq0 = wq.x, wq1 = wq.y, wq2 = wq.z, wq3 = wq.w;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const u32x4 xv = *(const const_u32x4*)(xg + static_cast<size_t>(t) * K + 16 * w);
          int s = acc[w % NA][t];
          s = __builtin_amdgcn_sdot4(wq0, static_cast<int>(xv.x), s, false);
          s = __builtin_amdgcn_sdot4(wq1, static_cast<int>(xv.y), s, false);
          s = __builtin_amdgcn_sdot4(wq2, static_cast<int>(xv.z), s, false);
          s = __builtin_amdgcn_sdot4(wq3, static_cast<int>(xv.w), s, false);
          acc[w % NA][t] = s;
        }
      }
    }
    // exact cross-wave reduction (integer LDS atomics, order independent)
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      int s = acc[0][t];
#pragma unroll
      for (int c = 1; c < NA; ++c) s += acc[c][t];
      atomicAdd(&red[t * 64 + lane], s);
    }
  }
  __syncthreads();

  const int n = n0 + lane;
  auto finish = [&](int t, int s) {
    const size_t o = static_cast<size_t>(t) * N + n;
    const float v = a.out_kind == kOutAcc
                        ? 0.0f
                        : static_cast<float>(s) * a.a_scale[t] * (a.smax[n] * (1.0f / 127.0f));
    store_out(a.out, o, a.out_kind, s, v);
  };
  if (a.slices == 1) {
    if (n < N)
      for (int t = wave; t < MT; t += nw) finish(t, red[t * 64 + lane]);
    return;
  }

  // K is split across workgroups: this slice's partial sums go to the
  // workspace; gemv_reduce_kernel adds the slices in order and rescales.  (A
  // last-arriver scheme inside this kernel needs device-scope fences, which
  // write back the L2 on this multi-XCD part and were measured to cost far
  // more than the second launch.)
  if (n < N)
    for (int t = wave; t < MT; t += nw)
      a.part[(static_cast<size_t>(slice) * MT + t) * N + n] = red[t * 64 + lane];
}

// Decode with the matrix cores (M = 2 .. 32 tokens, padded to 32).  Same
// work split as gemv_kernel (one 64-row block and one K slice per workgroup,
// a run of at most GMAX groups per wave), but each group is 8 MFMAs
// v_mfma_i32_32x32x32_i8: A = the unpacked weights of 32 rows x 32 k
// (subtile s = rows 32 s .. 32 s + 31 of the block, k-step t), B = 32 k x 32
// tokens of x_i8.  The k values of a (lane half h, k-step t) pair only have to
// agree between A and B: lane half h at k-step t covers k = 16 (4 h + t) ..
// +15 of the group, so a lane's weights for the whole group are the 16
// contiguous packed bytes [16 h, 16 h + 16) of its row (one load per subtile,
// no lane exchange), and its activations are the 64 contiguous bytes
// [64 h, 64 h + 64) of token row j of the group.  Columns j >= M re-read row
// M - 1 and are never reduced.
constexpr int kRedStride = 40;  // [n][m] int32 sums: 64 rows, 32 tokens, padded

template <int GMAX, int MAXT>
__global__ __launch_bounds__(MAXT) void gemv_mfma_kernel(GemvArgs a, int M) {
  __shared__ int red[64 * kRedStride];
  typedef int v16i __attribute__((ext_vector_type(16)));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int rb = blockIdx.x % a.n_rb;
  const int slice = blockIdx.x / a.n_rb;
  const int n0 = rb * 64;
  const int N = a.N, K = a.K, G = a.G;

  for (int i = threadIdx.x; i < 64 * kRedStride; i += blockDim.x) red[i] = 0;
  __syncthreads();

  const int s_lo = (slice * G) / a.slices;
  const int s_n = ((slice + 1) * G) / a.slices - s_lo;
  const int g0 = s_lo + (wave * s_n) / nw;
  const int ng = s_lo + ((wave + 1) * s_n) / nw - g0;   // 0 .. GMAX

  if (ng > 0) {
    const int j = lane & 31;   // A: weight row in the subtile; B: token column
    const int h = lane >> 5;   // lane half
    const uint8_t* srcA = a.packed + static_cast<size_t>(rb) * G * 2048 + j * 32 + h * 16;
    const uint8_t* srcB = srcA + 1024;
    const int8_t* qrowA = a.q + static_cast<size_t>(min(n0 + j, N - 1)) * G;
    const int8_t* qrowB = a.q + static_cast<size_t>(min(n0 + 32 + j, N - 1)) * G;
    const int8_t* xrow = a.x + static_cast<size_t>(min(j, M - 1)) * K + h * 64;

    uint4 dA[GMAX], dB[GMAX];
    v4i xv[GMAX][4];
#pragma unroll
    for (int jj = 0; jj < GMAX; ++jj) {
      const size_t g = static_cast<size_t>(g0 + min(jj, ng - 1));
      dA[jj] = *reinterpret_cast<const uint4*>(srcA + g * 2048);
      dB[jj] = *reinterpret_cast<const uint4*>(srcB + g * 2048);
#pragma unroll
      for (int t = 0; t < 4; ++t) xv[jj][t] = *reinterpret_cast<const v4i*>(xrow + g * 128 + 16 * t);
    }
    int qa[GMAX], qb[GMAX];
#pragma unroll
    for (int jj = 0; jj < GMAX; ++jj) {
      qa[jj] = qrowA[g0 + min(jj, ng - 1)];
      qb[jj] = qrowB[g0 + min(jj, ng - 1)];
    }

    v16i acc0 = {}, acc1 = {};
#pragma unroll
    for (int jj = 0; jj < GMAX; ++jj) {
      if (jj != 0 && jj >= ng) continue;   // ng >= 1: group 0 always runs
      const QTables ta = make_tables(qa[jj]);
      const QTables tb = make_tables(qb[jj]);
      const uint32_t wa[4] = {dA[jj].x, dA[jj].y, dA[jj].z, dA[jj].w};
      const uint32_t wb[4] = {dB[jj].x, dB[jj].y, dB[jj].z, dB[jj].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(unpack16(wa[t], ta), xv[jj][t], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(unpack16(wb[t], tb), xv[jj][t], acc1, 0, 0, 0);
      }
    }
    // exact cross-wave reduction.  32x32 accumulator layout: lane (j, h) holds
    // column j (token) and, in register r, row 8 (r / 4) + 4 h + (r % 4)
    if (j < M) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * h + (r & 3);
        atomicAdd(&red[row * kRedStride + j], acc0[r]);
        atomicAdd(&red[(32 + row) * kRedStride + j], acc1[r]);
      }
    }
  }
  __syncthreads();

  const int n = n0 + lane;
  if (n >= N) return;
  for (int t = wave; t < M; t += nw) {
    const int s = red[lane * kRedStride + t];
    const size_t o = static_cast<size_t>(t) * N + n;
    if (a.slices > 1)
      a.part[static_cast<size_t>(slice) * M * N + o] = s;
    else
      store_out(a.out, o, a.out_kind, s,
                a.out_kind == kOutAcc ? 0.0f
                                      : static_cast<float>(s) * a.a_scale[t] * (a.smax[n] * (1.0f / 127.0f)));
  }
}

// Row-balanced matrix-core decode (M <= 24 tokens, N >= 16 rows per CU).
// Streaming is bound per CU, so each workgroup takes an equal contiguous range
// of rows [r0, r1) (any length up to RS NS) over the whole of K: every CU
// streams the same number of bytes and no partial sums leave the workgroup.
// The rows form NS subtiles of RS rows, the A operand of the MFMA (rows past
// r1 are computed and dropped):
//   RS = 32 (17..24 tokens): v_mfma_i32_32x32x32_i8, lane (j, h) = (row or
//     token j = lane % 32, half h = lane / 32); per 128-k group a lane holds
//     16 packed bytes of its row (k = 64 h .. 64 h + 63), four MFMAs;
//   RS = 16 (up to 16 tokens): v_mfma_i32_16x16x64_i8, lane (j, h) = (row or
//     token j = lane % 16, quarter h = lane / 16); per group a lane holds 8
//     packed bytes (k = 32 h .. 32 h + 31), two MFMAs.  Tokens pad to 16
//     instead of 32 and rows to a multiple of 16.
// Integer sums are exact, so A and B only have to agree on which k each
// (lane group, byte) covers.  The waves split K into runs of at
// most GMAX groups and keep P groups of loads in flight: group jj + P is issued
// as soon as group jj has been consumed (EARLY: as soon as group jj has
// landed, into a (P + 1)-th buffer and activation slot, before group jj is
// computed), so the stream and the unpack / MFMA work overlap.  Loads are
// issued unconditionally (slots past the wave's run re-read its last group)
// so that the compiler's vmcnt waits stay static.
// The activations of a group (at most kXRows tokens x 128 bytes) go to LDS
// by direct loads with 8 lanes per 128-byte row, so each 1 KB load touches 16
// cache lines; read as MFMA operands (16 bytes of one token per lane) they
// would touch 64 per instruction, and the address unit, not HBM, would bound
// the kernel.  Each wave owns P slots (P + 1 with EARLY), one per group in
// flight.
constexpr int kXRows = 24;              // the decode paths take M <= 24
// Word 3 of a raw buffer resource on gfx9-family parts: 32-bit data format
// (DATA_FORMAT = 4 in bits 15..18), no swizzle, no index stride, so the
// range check is a plain byte count.
constexpr int kRawBufferWord3 = 0x00020000;
// cache-policy operand of the buffer loads: nontemporal (the weights are read
// once per call)
constexpr int kCacheNonTemporal = 2;
constexpr int kXSlot = kXRows * 128;    // bytes per group slot
constexpr int kRowsMaxWaves = 8;
// Fused rotation (ROT): at most kRotMaxM tokens of at most kRotMaxK, each wave
// rotating at most kRotBlocksPerWave 1024-blocks; all of x_i8 then stays in
// LDS, rows padded by 16 bytes (so that the tokens' 16-byte reads fall on
// different banks).
constexpr int kRotMaxM = 2;
constexpr int kRotMaxK = 17408;
constexpr int kRotBlocksPerWave = 3;
constexpr int kRotXBytes = kRotMaxM * (kRotMaxK + 16);
// Up to this many tokens the row-balanced kernel uses 16-row subtiles and
// v_mfma_i32_16x16x64_i8 (the tokens are one 16-wide operand); above, 32-row
// subtiles and v_mfma_i32_32x32x32_i8.  Measured 0.1-0.7 us faster per call
// on the decode layers at M = 1, 8 and 16 (5120 -> 17408: 8.62 -> 8.48 us at
// M = 1, 11.10 -> 10.60 at M = 16; 17408 -> 5120: 10.50 -> 9.76 at M = 1).
constexpr int kRows16MaxM = 16;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
template <int NS, int RS>
struct RowGroup {
  // RS = 32: 16 packed bytes of row 32 s + j, half h; RS = 16: 8 bytes of row 16 s + j, quarter h
  typename std::conditional<RS == 32, uint4, uint2>::type w[NS];
};

// ROT: the workgroup first rotates and quantises the M <= kRotMaxM tokens
// itself (every workgroup, redundantly: at most kRotBlocksPerWave blocks per
// wave), while its first P groups of weights are already in flight; x_i8 then
// stays in LDS for the whole K and no activation is loaded per group.  The
// rotation and the quantiser are those of rotate_quant_act (rotate_block.h),
// so x_i8, a_scale and y equal the two-step result bit for bit.
//
// TH = 2 (16-row subtiles, more than 16 tokens): the tokens form two 16-wide
// B operands (tokens 0-15 and 16-31), so each unpacked weight operand feeds
// two v_mfma_i32_16x16x64_i8 and the rows of a workgroup pad to a multiple
// of 16, not 32.
template <int NS, int GMAX, int P, int MAXT, bool ROT = false, int RS = 32, bool EARLY = false, int TH = 1>
__global__ __launch_bounds__(MAXT) void gemv_rows_kernel(GemvArgs a, int M) {
  static_assert(P >= 1 && P <= GMAX, "prefetch depth");
  static_assert(TH == 1 || (TH == 2 && RS == 16 && !ROT), "token halves");
  static_assert(MAXT <= 64 * kRowsMaxWaves, "x slots are sized for 8 waves");
  static_assert(RS == 32 || RS == 16, "subtile rows");
  typedef typename std::conditional<RS == 32, v16i_t, v4i>::type acc_t;
  __shared__ int red[RS * NS * kRedStride];
  // per-wave group slots, or (ROT) all of x_i8: token t at t * (K + 16)
  // EARLY: group jj + P is issued as soon as group jj has landed, before
  // group jj is computed, into a (P + 1)-th buffer and slot
  constexpr int NB = EARLY ? P + 1 : P;
  __shared__ __attribute__((aligned(1024))) int8_t xs[ROT ? kRotXBytes : kRowsMaxWaves * NB * kXSlot];
  __shared__ float rot_buf[ROT ? kRowsMaxWaves * rot::kWaveBufWords : 1];  // rotation transposes
  __shared__ unsigned tok_max[kRotMaxM];  // ROT: absmax bits of each token
  __shared__ float row_scale[32];        // a_scale of the tokens
  __shared__ float col_scale[RS * NS];   // smax of the rows
  // QLDS: the workgroup's rows of q (R x G bytes, contiguous in q, G <= 8
  // GMAX) staged in LDS by coalesced loads, instead of per-lane gathers of
  // the lane's rows (measured, µs: 5120 <- 17408 9.58 -> 8.78 at M = 1 and
  // 13.61 -> 13.18 at M = 24, 5120 -> 17408 8.49 -> 8.25 at M = 1; with
  // 32-row subtiles on 5-group waves, one group in flight, the barrier that
  // publishes the staged rows cost more than it saved: 11.83 -> 12.12 at M =
  // 24 on 5120 -> 17408, so those keep the gathers; the fused kernels
  // publish the rows with the barriers their rotation already has)
  constexpr bool QLDS = GMAX <= 17 && (ROT || !(GMAX == 5 && RS == 32));
  __shared__ __attribute__((aligned(16))) int8_t qs[QLDS ? RS * NS * GMAX * 8 : 4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int N = a.N, K = a.K, G = a.G;
  // rows of this workgroup: an even share of N (gridDim.x shares)
  const int r0 = static_cast<int>((static_cast<int64_t>(blockIdx.x) * N) / gridDim.x);
  const int r1 = static_cast<int>((static_cast<int64_t>(blockIdx.x + 1) * N) / gridDim.x);
  const int R = r1 - r0;  // 1 .. 32 NS (checked by the planner)

  for (int i = threadIdx.x; i < RS * NS * kRedStride; i += blockDim.x) red[i] = 0;
  if (ROT && threadIdx.x < kRotMaxM) tok_max[threadIdx.x] = 0u;
  __syncthreads();

  const int g0 = (wave * G) / nw;
  const int ng = ((wave + 1) * G) / nw - g0;  // 0 .. GMAX

  // the epilogue's scales, loaded by the last wave now and used after the
  // main loop, so that their latency hides behind the weight stream (clamped
  // indices and no per-lane branch: a divergent load here made the compiler
  // wait for it before the stream was issued)
  const bool scale_wave = wave == nw - 1 && a.out_kind != kOutAcc;
  float sc_row = 0.0f, sc_col0 = 0.0f, sc_col1 = 0.0f;
  if (scale_wave) {
    if (!ROT) sc_row = a.a_scale[min(lane, M - 1)];
    sc_col0 = a.smax[r0 + min(lane, R - 1)];
    sc_col1 = a.smax[r0 + min(lane + 64, R - 1)];
  }

  if (ng > 0) {
    const int j = lane & (RS - 1), h = lane / RS;
    // lanes past the last row of this workgroup re-read that row: the same
    // cache lines, so no bytes beyond the workgroup's own rows are fetched
    // weights through a buffer resource: its base is the workgroup's first
    // row block and its range the row blocks the workgroup's rows touch (at
    // most three of G x 2 KB; a load outside it would return zeros instead of
    // reading another workgroup's rows).  A load then takes its lane offset
    // from a VGPR and the group's offset from an SGPR: no address arithmetic
    // per load.
    const int rb0 = r0 >> 6;
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.packed) + static_cast<size_t>(rb0) * G * 2048, 0,
        (((r1 - 1) >> 6) - rb0 + 1) * G * 2048, kRawBufferWord3);
    uint32_t wbase[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int n = min(r0 + RS * s + j, r1 - 1);
      wbase[s] = static_cast<uint32_t>(((n >> 6) - (r0 >> 6)) * G * 2048 + (n & 63) * 32 + h * (RS == 32 ? 16 : 8));
    }
    // ROT: this wave's blocks of x (block bi = wave + i nw of the M x K/1024
    // blocks is token bi / nblk, block bi % nblk), loaded first: waits complete
    // in issue order, so behind the q and weight loads the rotation would wait
    // for those too
    const int nblk = K >> 10;
    const int nbt = ROT ? M * nblk : 0;  // <= kRotBlocksPerWave * nw (checked by the host)
    rot::BlockIn rin[ROT ? kRotBlocksPerWave : 1];
    if (ROT) {
      // no branch around the loads (a join with loads in flight makes the
      // compiler wait for them): slots past the last block re-load it
#pragma unroll
      for (int i = 0; i < kRotBlocksPerWave; ++i) {
        const int bi = min(wave + i * nw, nbt - 1);
        const int t = bi / nblk, b = bi - t * nblk;
        rin[i] = rot::load_block_rt(a.xb + static_cast<size_t>(t) * (a.silu ? 2 * K : K), a.sign,
                                    a.silu ? K : 0, b, lane);
      }
      __builtin_amdgcn_sched_barrier(0);  // all of them ahead of the q and weight loads
    }
    // q of this lane's rows for all of the wave's groups: QD dwords from the
    // 4-aligned start q[n, g0 & ~3] (rows of q are G bytes, G % 8 == 0, so no
    // dword straddles a row end; dwords past the row end are clamped), loaded
    // once up front instead of one byte gather per group
    // (held in vector registers: as a plain array the compiler may move it to
    // LDS, which then waits on the loads before the other groups are issued)
    constexpr int QD = GMAX / 4 + 2;
    constexpr int QV = QD <= 4 ? 4 : (QD <= 8 ? 8 : 16);
    static_assert(QD <= QV, "q dwords");
    typedef uint32_t qvec __attribute__((ext_vector_type(QV)));
    const int qa = g0 & ~3, qsh = g0 & 3;
    const int qd_last = (G - qa) / 4 - 1;
    qvec qw[QLDS ? 1 : NS];  // indexed by constants only (unrolled), so kept in registers
    // QLDS: dwords t, t + MAXT, ... of the workgroup's R x G bytes of q (from
    // q[r0, 0]: G % 8 == 0, so dword aligned), clamped so that every slot
    // loads (no branch around loads in flight), issued ahead of the weights
    // and written to LDS once the first group has landed (fused: before the
    // rotation's first barrier)
    constexpr int QI = QLDS ? (RS * NS * GMAX * 2 + MAXT - 1) / MAXT : 1;
    const int qdw = R * G / 4;
    uint32_t qr[QI];
    if constexpr (QLDS) {
      const uint32_t* qsrc = reinterpret_cast<const uint32_t*>(a.q + static_cast<size_t>(r0) * G);
#pragma unroll
      for (int i = 0; i < QI; ++i) qr[i] = qsrc[min(static_cast<int>(threadIdx.x) + i * MAXT, qdw - 1)];
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int n = min(r0 + RS * s + j, r1 - 1);
        const uint32_t* qrow = reinterpret_cast<const uint32_t*>(a.q + static_cast<size_t>(n) * G + qa);
        qvec v = {};
#pragma unroll
        for (int d = 0; d < QD; ++d) v[d] = qrow[min(d, qd_last)];
        qw[s] = v;
      }
    }
    // q[n, g0 + jj]: QLDS, one byte of the staged rows; else byte qsh + jj of
    // the lane's run (jj is a constant once unrolled): a 64-bit shift of two
    // dwords picked by constant indices
    const auto qbyte = [&](int s, int jj) {
      if constexpr (QLDS) {
        return static_cast<int>(qs[min(RS * s + j, R - 1) * G + g0 + min(jj, ng - 1)]);
      } else {
        const qvec& v = qw[s];
        const uint64_t w = (static_cast<uint64_t>(v[(jj >> 2) + 1]) << 32) | v[jj >> 2];
        return static_cast<int>(static_cast<int8_t>(w >> (8 * (qsh + (jj & 3)))));
      }
    };
    // activation DMA: instruction i, lane l -> LDS row r = 8 i + l / 8 (token
    // min(r, M - 1)), LDS chunk l % 8 holding global chunk (l % 8) ^ swizzle(r);
    // xi = ceil(M / 8) instructions per group
    const int xi = (M + 7) >> 3;
    uint32_t xoff[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int r = 8 * i + (lane >> 3);
      // 24-bit multiply (tokens < 24, K <= 2^16): a 32-bit result, so the
      // compiler does not form a 64-bit multiply-add whose unused high half
      // could be a register still waiting on a load
      xoff[i] = __umul24(static_cast<uint32_t>(min(r, M - 1)), static_cast<uint32_t>(K)) +
                static_cast<uint32_t>(16 * ((lane & 7) ^ chunk_swizzle(r)));
    }
    const void* xbase = sgpr_ptr(a.x);
    const uint32_t xs_wave = lds_addr(xs) + static_cast<uint32_t>(wave * NB * kXSlot);
    // this lane's operand row in a slot (tokens past kXRows are never reduced)
    const int jr = min(j, kXRows - 1);

    // per group: NS weight loads (VGPR), then the xi activation DMAs; the
    // activation wait below counts on exactly this order.  The weights are
    // read once per call: nontemporal loads (measured 2-3% faster)
    RowGroup<NS, RS> buf[NB];
    auto issue = [&](RowGroup<NS, RS>& d, int jj) {
      const int g = g0 + min(jj, ng - 1);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if constexpr (RS == 32) {
          const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(wres, wbase[s], g * 2048, kCacheNonTemporal);
          d.w[s] = make_uint4(t.x, t.y, t.z, t.w);
        } else {
          const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(wres, wbase[s], g * 2048, kCacheNonTemporal);
          d.w[s] = make_uint2(t.x, t.y);
        }
      }
      if (!ROT) {
        const uint32_t slot = __builtin_amdgcn_readfirstlane(xs_wave + (jj % NB) * kXSlot);
        const uint32_t gx = static_cast<uint32_t>(g) * 128;
        dma16xn(xi, xbase, xoff[0] + gx, xoff[1] + gx, xoff[2] + gx, slot, slot + 1024, slot + 2048);
      }
    };
#pragma unroll
    for (int jj = 0; jj < P; ++jj) issue(buf[jj], jj);

    if (ROT) {
      // Every wave has groups here (the planner keeps nw <= G), so all of them
      // reach the two barriers.
      float* wb = rot_buf + wave * rot::kWaveBufWords;
      float rv[kRotBlocksPerWave][16];
#pragma unroll
      for (int i = 0; i < kRotBlocksPerWave; ++i) {
        const int bi = wave + i * nw;
        if (bi < nbt) {
          const int t = bi / nblk;
          if (a.silu)
            rot::rotate_loaded<true>(rin[i], lane, wb, rv[i]);
          else
            rot::rotate_loaded<false>(rin[i], lane, wb, rv[i]);
          float m = 0.0f;
#pragma unroll
          for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(rv[i][e]));
#pragma unroll
          for (int sh = 32; sh >= 1; sh >>= 1) m = fmaxf(m, __shfl_xor(m, sh));
          // non-negative floats order like their bit patterns
          if (lane == 0) atomicMax(&tok_max[t], __float_as_uint(m));
        }
      }
      if constexpr (QLDS) {
        // the staged q rows, published by the barriers of the rotation
#pragma unroll
        for (int i = 0; i < QI; ++i) {
          const int d = static_cast<int>(threadIdx.x) + i * MAXT;
          if (d < qdw) reinterpret_cast<uint32_t*>(qs)[d] = qr[i];
        }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kRotBlocksPerWave; ++i) {
        const int bi = wave + i * nw;
        if (bi < nbt) {
          const int t = bi / nblk, b = bi - t * nblk;
          const rot::TokenQuant tq = rot::token_quant(__uint_as_float(tok_max[t]));
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint32_t word = rot::quant_run(rv[i], c, tq);
            const int k = b * rot::kBlock + 256 * c + 4 * lane;
            *reinterpret_cast<uint32_t*>(xs + t * (K + 16) + k) = word;
            if (blockIdx.x == 0) *reinterpret_cast<uint32_t*>(a.x_i8_out + static_cast<size_t>(t) * K + k) = word;
          }
        }
      }
      if (wave == 0 && lane < M) {
        const float sc = rot::token_quant(__uint_as_float(tok_max[lane])).scale;
        row_scale[lane] = sc;
        if (blockIdx.x == 0) a.a_scale_out[lane] = sc;
      }
      __syncthreads();
    }

    acc_t acc[NS];
    acc_t acc2[TH == 2 ? NS : 1];  // TH = 2: tokens 16 .. 31
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[s] = acc_t{0};
#pragma unroll
    for (int s = 0; s < (TH == 2 ? NS : 1); ++s) acc2[s] = acc_t{0};
#pragma unroll
    for (int jj = 0; jj < GMAX; ++jj) {
      RowGroup<NS, RS>& d = buf[jj % NB];
      // this group's activation DMAs are done once at most the loads of the
      // groups issued after it are outstanding (NS + xi per group; counting
      // NS + 1 only makes the wait stricter)
      if (!ROT) wait_groups_after<NS + 1>(min(P - 1, GMAX - 1 - jj));
      asm volatile("" ::: "memory");
      if (EARLY && jj + P < GMAX) issue(buf[(jj + P) % NB], jj + P);
      if (QLDS && !ROT && jj == 0) {
        // the q loads were issued before the weights, so they have landed;
        // every wave has groups (the planner keeps nw <= G), so all reach
        // the barrier
#pragma unroll
        for (int i = 0; i < QI; ++i) {
          const int d = static_cast<int>(threadIdx.x) + i * MAXT;
          if (d < qdw) reinterpret_cast<uint32_t*>(qs)[d] = qr[i];
        }
        __syncthreads();
      }
      if (jj == 0 || jj < ng) {
        // k-chunks (16 bytes) of the group this lane supplies: RS = 32, chunk
        // 4 h + t for MFMA t = 0..3; RS = 16, chunk 2 h + t for MFMA t = 0, 1
        constexpr int NT = RS == 32 ? 4 : 2;
        v4i xv[NT];
        v4i xv2[TH == 2 ? NT : 1];
        if (ROT) {
          const int8_t* xr = xs + min(j, M - 1) * (K + 16) + (g0 + min(jj, ng - 1)) * 128 + 16 * NT * h;
#pragma unroll
          for (int t = 0; t < NT; ++t) xv[t] = *reinterpret_cast<const v4i*>(xr + 16 * t);
        } else {
          const int8_t* xr = xs + (wave * NB + jj % NB) * kXSlot + jr * 128;
#pragma unroll
          for (int t = 0; t < NT; ++t)
            xv[t] = *reinterpret_cast<const v4i*>(xr + 16 * ((NT * h + t) ^ chunk_swizzle(jr)));
          if constexpr (TH == 2) {
            const int jr2 = min(j + 16, kXRows - 1);
            const int8_t* xr2 = xs + (wave * NB + jj % NB) * kXSlot + jr2 * 128;
#pragma unroll
            for (int t = 0; t < NT; ++t)
              xv2[t] = *reinterpret_cast<const v4i*>(xr2 + 16 * ((NT * h + t) ^ chunk_swizzle(jr2)));
          }
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const QTables tab = make_tables(qbyte(s, jj));
          if constexpr (RS == 32) {
            const uint32_t wv[4] = {d.w[s].x, d.w[s].y, d.w[s].z, d.w[s].w};
#pragma unroll
            for (int t = 0; t < 4; ++t)
              acc[s] = __builtin_amdgcn_mfma_i32_32x32x32_i8(unpack16(wv[t], tab), xv[t], acc[s], 0, 0, 0);
          } else {
            const uint32_t wv[2] = {d.w[s].x, d.w[s].y};
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const v4i wop = unpack16(wv[t], tab);
              acc[s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wop, xv[t], acc[s], 0, 0, 0);
              if constexpr (TH == 2) acc2[s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wop, xv2[t], acc2[s], 0, 0, 0);
            }
          }
        }
      }
      if (!EARLY && jj + P < GMAX) issue(d, jj + P);
    }
    // exact cross-wave reduction; lane (j, h) holds token j and, in register
    // r, row 8 (r / 4) + 4 h + (r % 4) of each subtile
    if (j < M) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int r = 0; r < (RS == 32 ? 16 : 4); ++r) {
          // RS = 32: register r holds row 8 (r / 4) + 4 h + (r % 4); RS = 16: row 4 h + r
          const int row = RS * s + (RS == 32 ? 8 * (r >> 2) + 4 * h + (r & 3) : 4 * h + r);
          atomicAdd(&red[row * kRedStride + j], acc[s][r]);
        }
    }
    if (TH == 2 && j + 16 < M) {
#pragma unroll
      for (int s = 0; s < (TH == 2 ? NS : 1); ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) atomicAdd(&red[(RS * s + 4 * h + r) * kRedStride + j + 16], acc2[s][r]);
    }
  }
  if (scale_wave) {
    if (!ROT && lane < M) row_scale[lane] = sc_row;
    if (lane < R) col_scale[lane] = sc_col0;
    if (lane + 64 < R) col_scale[lane + 64] = sc_col1;
  }
  __syncthreads();

  for (int i = threadIdx.x; i < M * R; i += blockDim.x) {
    const int t = i / R, rr = i - t * R;
    const int sum = red[rr * kRedStride + t];
    const size_t o = static_cast<size_t>(t) * N + r0 + rr;
    store_out(a.out, o, a.out_kind, sum,
              a.out_kind == kOutAcc ? 0.0f
                                    : static_cast<float>(sum) * row_scale[t] * (col_scale[rr] * (1.0f / 127.0f)));
  }
}

// Sum of the slices' partial sums in slice order, then the rescale.
__global__ __launch_bounds__(256) void gemv_reduce_kernel(const int32_t* __restrict__ part,
                                                          int slices, int M, int N,
                                                          const float* __restrict__ a_scale,
                                                          const float* __restrict__ smax,
                                                          void* __restrict__ out, int out_kind) {
  const size_t total = static_cast<size_t>(M) * N;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += stride) {
    int s = 0;
    for (int sl = 0; sl < slices; ++sl) s += part[static_cast<size_t>(sl) * total + i];
    float v = 0.0f;
    if (out_kind != kOutAcc) {
      const int t = static_cast<int>(i / static_cast<size_t>(N));
      const int n = static_cast<int>(i - static_cast<size_t>(t) * N);
      v = static_cast<float>(s) * a_scale[t] * (smax[n] * (1.0f / 127.0f));
    }
    store_out(out, i, out_kind, s, v);
  }
}

struct GemvPlan {
  int gmax = 2;    // compile-time bound on groups per wave
  int nw = 1;      // waves per workgroup
  int slices = 1;  // workgroups per 64-row block (K split across workgroups)
  int n_rb = 1;
  bool mfma = false;
  // row-balanced MFMA kernel: `rows_wgs` workgroups of an even share of N
  int rows_ns = 0;   // subtiles of rows_rs rows per workgroup (0: not this kernel)
  int rows_rs = 32;
  int rows_wgs = 0;
  int rows_p = 2;    // groups of loads in flight per wave when gmax is 5 or 17
  bool rows_early = false;  // issue a group's successor before computing it
  int rows_th = 1;   // 2: 16-row subtiles with the tokens as two 16-wide operands
};

// From this many tokens on, the matrix-core kernel beats the dot4 kernel
// (measured on both decode shapes: at 4 tokens they are about even, at 8 the
// MFMA kernel is 1.3-1.6x faster, at 24 2.6-3.5x).
constexpr int kMfmaMinM = 4;

constexpr int kGmaxChoices[] = {2, 3, 5, 9};

// Streaming cost model (measured on MI355X): each CU moves about 22 GB/s, so
// the busiest CU's bytes set the time; splitting K over several workgroups per
// row block evens the CUs out but costs a second launch (about 3.5 us).
constexpr double kCuBytesPerUs = 22.0e3;
constexpr double kReduceUs = 3.5;

GemvPlan make_plan_for(int64_t M, int64_t N, int64_t K, const DeviceInfo& dev, bool mfma) {
  const int G = static_cast<int>(K >> 7);
  const int cus = std::max(1, dev.cu_count);
  GemvPlan best;
  best.slices = 0;  // none found yet
  double best_t = 1e30;
  for (int slices = 1; slices <= 32 && slices <= G; ++slices) {
    GemvPlan p;
    p.mfma = mfma;
    p.n_rb = static_cast<int>((N + 63) / 64);
    p.slices = slices;
    const int per_slice = (G + slices - 1) / slices;
    // two or three groups per wave keeps many waves in flight; at most 16
    // waves, at most 9 groups each (MFMA kernel, for its register budget: at
    // most 3 groups with 16 waves, 5 with 8)
    p.nw = std::min(kMaxWaves, std::max(1, per_slice / 2));
    int gw = (per_slice + p.nw - 1) / p.nw;
    if (mfma && gw > 3 && p.nw > 8) {
      p.nw = 8;
      gw = (per_slice + p.nw - 1) / p.nw;
    }
    if (gw > (mfma ? 5 : 9)) continue;
    for (int c : kGmaxChoices)
      if (c >= gw) { p.gmax = c; break; }
    const int64_t wgs = static_cast<int64_t>(p.n_rb) * slices;
    const double per_cu = static_cast<double>((wgs + cus - 1) / cus) * 64.0 * per_slice * 32.0;
    // partial sums: written once, read once by the reduce kernel (~4 TB/s)
    const double part_us = slices > 1 ? 2.0 * slices * static_cast<double>(M) * N * 4 / 4.0e6 : 0.0;
    const double t = per_cu / kCuBytesPerUs + (slices > 1 ? kReduceUs + part_us : 0.0);
    if (t < best_t - 1e-9) { best_t = t; best = p; }
  }
  return best;
}

constexpr int kRowsGmaxChoices[] = {3, 5, 9, 17, 33};

// Row-balanced plan: an even share of rows for every CU (a multiple of the CU
// count of workgroups), at most 3 subtiles of 32 rows each, the whole of K
// split over the waves.  Every workgroup reads all of x_i8 (M x K bytes, by
// coalesced direct loads into LDS) next to its R x K / 4 bytes of weights; the
// plan is taken when each workgroup has at least 16 rows.  Measured against
// the K-split kernel and its second launch: 17408 -> 5120 (20 rows per CU)
// 10.1 against 12.1 us at M = 4, 13.6 against 15.2 us at M = 24; and, for
// these shapes, faster than the dot4 kernel from M = 1 on.
GemvPlan make_rows_plan(int64_t N, int64_t K, const DeviceInfo& dev) {
  GemvPlan p;
  p.slices = 0;
  const int cus = std::max(1, dev.cu_count);
  const int G = static_cast<int>(K >> 7);
  const int64_t per_round = static_cast<int64_t>(cus) * 96;
  const int64_t rounds = (N + per_round - 1) / per_round;
  const int64_t wgs = rounds * cus;
  if (N < 16 * wgs) return p;
  const int64_t rmax = (N + wgs - 1) / wgs;
  p.rows_ns = static_cast<int>((rmax + 31) / 32);
  p.rows_wgs = static_cast<int>(wgs);
  p.n_rb = static_cast<int>((N + 63) / 64);
  p.mfma = true;
  p.slices = 1;
  p.nw = std::min(8, std::max(1, G));
  const int gw = (G + p.nw - 1) / p.nw;
  p.gmax = 0;
  for (int c : kRowsGmaxChoices)
    if (c >= gw) { p.gmax = c; break; }
  if (p.gmax == 0) p.slices = 0;
  return p;
}

// Always returns a valid plan for 1 <= M <= 24 and K <= the library's limit:
// the dot4 kernel takes up to 16 waves x 9 groups x 32 slices.
// Automatic choice: the row-balanced matrix-core kernel whenever its plan
// applies (at every M), else the dot4 kernel below kMfmaMinM tokens and the
// K-split matrix-core kernel from there on.
GemvPlan make_plan(int64_t M, int64_t N, int64_t K, GemvKind kind, const DeviceInfo& dev) {
  if (kind != kGemvDot4 && M <= kXRows) {
    GemvPlan r = make_rows_plan(N, K, dev);
    if (r.slices > 0 && M <= kRows16MaxM) {
      // 16-row subtiles and v_mfma_i32_16x16x64_i8: tokens padded to 16, not
      // 32, and the rows of a workgroup to a multiple of 16
      const int64_t rmax = (N + r.rows_wgs - 1) / r.rows_wgs;
      r.rows_rs = 16;
      r.rows_ns = static_cast<int>((rmax + 15) / 16);
    } else if (r.slices > 0 && r.gmax == 5) {
      // more than 16 tokens on 5-group waves: 16-row subtiles with two
      // 16-token operands where they pad the rows less than 32-row subtiles
      // (68 rows: 80, not 96), each unpacked weight operand feeding two
      // MFMAs.  Measured against the 32-row form, one group in flight and
      // issued early in both (µs, alternating on one box, bit-identical y):
      // 5120 -> 17408 10.43 -> 10.09 at M = 24, 10.20 -> 9.82 at M = 17;
      // 5120 -> 34816 17.32 -> 16.31 at M = 24, 17.23 -> 15.66 at M = 20.
      // Deeper prefetch was slower (three groups early: 10.80 and 20.18 at
      // M = 24; two, not early: 10.81 and 16.76).
      const int64_t rmax = (N + r.rows_wgs - 1) / r.rows_wgs;
      const int ns16 = static_cast<int>((rmax + 15) / 16);
      if (ns16 * 16 < r.rows_ns * 32 && ns16 <= 6) {
        r.rows_rs = 16;
        r.rows_ns = ns16;
        r.rows_th = 2;
      }
    }
    if (r.slices > 0) {
      // Loads in flight per wave, measured (µs, alternating on one box):
      // - 5-group waves (K = 5120) keep two by default (the workgroup then
      //   needs 65 KB of LDS, so two share a CU where N needs two rounds of
      //   workgroups, 5120 -> 34816).
      // - With 32-row subtiles (17..24 tokens) one group in flight, the next
      //   issued as soon as it has landed, before it is computed ("early"),
      //   is faster: 10.59 -> 9.66 on 5120 -> 17408, 16.94 -> 15.96 on
      //   5120 -> 34816, 6.57 -> 6.45 on 5120 -> 5120 at M = 24.
      // - With one round of workgroups and 16-row subtiles: all five, not
      //   early, on one subtile (4096 rows: 4.21 against 4.28 us with three
      //   early at M = 1); three, early, on two (5120 -> 5120, 20 rows: 5.22
      //   -> 5.00 at M = 1, 6.08 -> 5.67 at M = 16, against all five);
      //   with more subtiles two, early, up to 8 tokens and one above
      //   (5120 -> 17408: 8.23 -> 7.86 at M = 1, 8.57 -> 8.21 at M = 8,
      //   8.88 -> 8.42 at M = 12, 9.19 -> 8.65 at M = 16, against three).
      // - Two rounds of workgroups (5120 -> 34816) with 16-row subtiles keep
      //   two up to 8 tokens (one early: 11.43 -> 11.64 at M = 1) and one,
      //   early, above (14.20 -> 13.58 at M = 16).
      // - 17-group waves (K = 17408) keep five; with 16-row subtiles three
      //   early are faster (5120 <- 17408: 9.71 -> 9.49 at M = 1, 9.79 ->
      //   9.60 at M = 8), with 32-row subtiles slower (13.36 -> 15.08).
      const bool one_round = r.rows_wgs <= dev.cu_count;
      if (r.gmax == 5) {
        if (r.rows_rs == 32 || r.rows_th == 2) {
          r.rows_p = 1;
          r.rows_early = true;
        } else if (one_round) {
          r.rows_p = r.rows_ns == 1 ? 5 : r.rows_ns == 2 ? 3 : (M <= 8 ? 2 : 1);
          r.rows_early = r.rows_ns > 1;
        } else if (M > 8) {
          r.rows_p = 1;
          r.rows_early = true;
        }
      } else if (r.gmax == 17 && r.rows_rs == 16 && one_round) {
        r.rows_p = 3;
        r.rows_early = true;
      }
      return r;
    }
  }
  const bool want_mfma = kind == kGemvMfma || (kind == kGemvAuto && M >= kMfmaMinM);
  if (want_mfma && M <= 32) {
    const GemvPlan p = make_plan_for(M, N, K, dev, true);
    if (p.slices > 0) return p;
  }
  return make_plan_for(M, N, K, dev, false);
}

template <int NS, int MAXT, bool ROT = false, int RS = 32>
hipError_t launch_rows_ns(GemvArgs a, int M, const GemvPlan& pl, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(pl.rows_wgs));
  const dim3 block(64 * pl.nw);
  // the kernel stages q with MAXT threads (nw = 8 whenever K >= 1024)
  if (64 * pl.nw != MAXT) return hipErrorInvalidValue;
  // groups of loads in flight per wave, within the register budget: the
  // plan's rows_p and rows_early for 5- and 17-group waves, else 5 (3 for
  // 3-group waves)
  constexpr int PM = 5;
  switch (pl.gmax) {
    case 3: hipLaunchKernelGGL((gemv_rows_kernel<NS, 3, 3, MAXT, ROT, RS>), grid, block, 0, stream, a, M); break;
    case 5:
      if constexpr (!ROT) {
        if (pl.rows_early) {
          if (pl.rows_p == 1) {
            hipLaunchKernelGGL((gemv_rows_kernel<NS, 5, 1, MAXT, false, RS, true>), grid, block, 0, stream, a, M);
            break;
          }
          if constexpr (RS == 16) {
            if (pl.rows_p == 2) {
              hipLaunchKernelGGL((gemv_rows_kernel<NS, 5, 2, MAXT, false, RS, true>), grid, block, 0, stream, a, M);
              break;
            }
            if (pl.rows_p == 3) {
              hipLaunchKernelGGL((gemv_rows_kernel<NS, 5, 3, MAXT, false, RS, true>), grid, block, 0, stream, a, M);
              break;
            }
          }
          return hipErrorInvalidValue;
        }
        if constexpr (RS == 16 && NS == 1) {
          if (pl.rows_p == 5) {
            hipLaunchKernelGGL((gemv_rows_kernel<NS, 5, 5, MAXT, false, RS>), grid, block, 0, stream, a, M);
            break;
          }
        }
      }
      // the fused kernels (their x_i8 fills the LDS) on at most two subtiles:
      // two groups, early (5120 -> 5120: 7.24 -> 7.00 us at M = 1, 8.23 ->
      // 7.97 at M = 2; one early, or two early on more subtiles, was slower)
      if constexpr (ROT && NS <= 2) {
        hipLaunchKernelGGL((gemv_rows_kernel<NS, 5, 2, MAXT, ROT, RS, true>), grid, block, 0, stream, a, M);
        break;
      }
      // two groups in flight, not early: two rounds of workgroups up to 8
      // tokens, and the other fused kernels
      hipLaunchKernelGGL((gemv_rows_kernel<NS, 5, 2, MAXT, ROT, RS>), grid, block, 0, stream, a, M);
      break;
    case 9: hipLaunchKernelGGL((gemv_rows_kernel<NS, 9, PM, MAXT, ROT, RS>), grid, block, 0, stream, a, M); break;
    case 17:
      if constexpr (!ROT && RS == 16) {
        if (pl.rows_early && pl.rows_p == 3) {
          hipLaunchKernelGGL((gemv_rows_kernel<NS, 17, 3, MAXT, false, RS, true>), grid, block, 0, stream, a, M);
          break;
        }
      }
      hipLaunchKernelGGL((gemv_rows_kernel<NS, 17, PM, MAXT, ROT, RS>), grid, block, 0, stream, a, M);
      break;
    case 33:
      // K > kRotMaxK: never planned with ROT
      if (ROT) return hipErrorInvalidValue;
      hipLaunchKernelGGL((gemv_rows_kernel<NS, 33, PM, MAXT, false, RS>), grid, block, 0, stream, a, M);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// 16-row subtiles with two 16-token operands (TH = 2): 5-group waves, one
// group in flight, its successor issued early (as for 32-row subtiles).
template <int NS>
hipError_t launch_rows_halves(GemvArgs a, int M, const GemvPlan& pl, hipStream_t stream) {
  if (pl.nw != 8 || pl.gmax != 5 || !pl.rows_early || pl.rows_p != 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemv_rows_kernel<NS, 5, 1, 512, false, 16, true, 2>), dim3(static_cast<unsigned>(pl.rows_wgs)),
                     dim3(512), 0, stream, a, M);
  return hipGetLastError();
}

template <bool ROT>
hipError_t launch_rows(GemvArgs a, int M, const GemvPlan& pl, hipStream_t stream) {
  if constexpr (!ROT) {
    if (pl.rows_rs == 16 && pl.rows_th == 2) {
      switch (pl.rows_ns) {
        case 1: return launch_rows_halves<1>(a, M, pl, stream);
        case 2: return launch_rows_halves<2>(a, M, pl, stream);
        case 3: return launch_rows_halves<3>(a, M, pl, stream);
        case 4: return launch_rows_halves<4>(a, M, pl, stream);
        case 5: return launch_rows_halves<5>(a, M, pl, stream);
        case 6: return launch_rows_halves<6>(a, M, pl, stream);
        default: return hipErrorInvalidValue;
      }
    }
  }
  if (pl.rows_rs == 16) {
    switch (pl.rows_ns) {
      case 1: return launch_rows_ns<1, 512, ROT, 16>(a, M, pl, stream);
      case 2: return launch_rows_ns<2, 512, ROT, 16>(a, M, pl, stream);
      case 3: return launch_rows_ns<3, 512, ROT, 16>(a, M, pl, stream);
      case 4: return launch_rows_ns<4, 512, ROT, 16>(a, M, pl, stream);
      case 5: return launch_rows_ns<5, 512, ROT, 16>(a, M, pl, stream);
      case 6: return launch_rows_ns<6, 512, ROT, 16>(a, M, pl, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if constexpr (ROT) {
    return hipErrorInvalidValue;  // the fused kernels use 16-row subtiles
  } else {
    switch (pl.rows_ns) {
      case 1: return launch_rows_ns<1, 512, false>(a, M, pl, stream);
      case 2: return launch_rows_ns<2, 512, false>(a, M, pl, stream);
      case 3: return launch_rows_ns<3, 512, false>(a, M, pl, stream);
      default: return hipErrorInvalidValue;
    }
  }
}

hipError_t launch_mfma(GemvArgs a, int M, const GemvPlan& pl, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(pl.n_rb * pl.slices));
  const dim3 block(64 * pl.nw);
  switch (pl.gmax) {
    case 2: hipLaunchKernelGGL((gemv_mfma_kernel<2, 1024>), grid, block, 0, stream, a, M); break;
    case 3: hipLaunchKernelGGL((gemv_mfma_kernel<3, 1024>), grid, block, 0, stream, a, M); break;
    default: hipLaunchKernelGGL((gemv_mfma_kernel<5, 512>), grid, block, 0, stream, a, M); break;
  }
  return hipGetLastError();
}

template <int MT>
hipError_t launch_mt(GemvArgs a, const GemvPlan& pl, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(pl.n_rb * pl.slices));
  const dim3 block(64 * pl.nw);
  switch (pl.gmax) {
    case 2: hipLaunchKernelGGL((gemv_kernel<MT, 2>), grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((gemv_kernel<MT, 3>), grid, block, 0, stream, a); break;
    case 5: hipLaunchKernelGGL((gemv_kernel<MT, 5>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((gemv_kernel<MT, 9>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace

void gemv_plan_info(int64_t M, int64_t N, int64_t K, GemvKind kind, const DeviceInfo& dev, int64_t* info) {
  const GemvPlan pl = make_plan(M, N, K, kind, dev);
  const bool rows = pl.rows_ns > 0;
  info[0] = rows ? 2 : (pl.mfma ? 4 : 3);
  info[1] = rows ? (N + pl.rows_wgs - 1) / pl.rows_wgs : 64;
  info[2] = 0;
  info[3] = pl.slices;
  info[4] = rows ? pl.rows_wgs : static_cast<int64_t>(pl.n_rb) * pl.slices;
  info[5] = pl.nw;
  info[6] = pl.slices > 1 ? 1 : 0;
  info[7] = pl.slices > 1 ? static_cast<int64_t>(pl.slices) * M * N * 4 : 0;
}

size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, GemvKind kind, const DeviceInfo& dev) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  const GemvPlan pl = make_plan(M, N, K, kind, dev);
  if (pl.slices <= 1) return 0;
  return static_cast<size_t>(pl.slices) * static_cast<size_t>(M) * static_cast<size_t>(N) * 4;
}

hipError_t launch_gemv(const int8_t* x_i8, const float* a_scale, const uint8_t* packed,
                       const int8_t* q, const float* smax, int64_t M, int64_t N, int64_t K,
                       void* out, OutKind out_kind, void* part, size_t part_bytes, GemvKind kind,
                       const DeviceInfo& dev, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const GemvPlan pl = make_plan(M, N, K, kind, dev);
  if (pl.slices <= 0 || (kind == kGemvMfma && !pl.mfma)) return hipErrorInvalidValue;
  if (pl.slices > 1 && (part == nullptr || part_bytes < gemv_workspace_bytes(M, N, K, kind, dev)))
    return hipErrorInvalidValue;
  if (std::getenv("TWL_LOG")) {
    // the row kernel's form: subtiles, token operands, groups of loads in
    // flight per wave (as launch_rows_ns dispatches them) and early issue
    char form[96] = "";
    if (pl.rows_ns > 0) {
      const int depth = pl.gmax == 3 ? 3 : (pl.gmax == 5 || (pl.gmax == 17 && pl.rows_early)) ? pl.rows_p : 5;
      std::snprintf(form, sizeof(form), ", %d-row subtiles x%d%s, %d in flight%s", pl.rows_rs, pl.rows_ns,
                    pl.rows_th == 2 ? " (two 16-token operands)" : "", depth, pl.rows_early ? ", early" : "");
    }
    std::fprintf(stderr, "[twl] gemv%s M=%lld N=%lld K=%lld -> <= %d groups/wave, %d waves/WG, %d slices, grid=%d%s\n",
                 pl.rows_ns > 0 ? "-rows" : (pl.mfma ? "-mfma" : ""), static_cast<long long>(M),
                 static_cast<long long>(N), static_cast<long long>(K), pl.gmax, pl.nw, pl.slices,
                 pl.rows_ns > 0 ? pl.rows_wgs : pl.n_rb * pl.slices, form);
  }
  GemvArgs a = {};
  a.x = x_i8;
  a.a_scale = a_scale;
  a.packed = packed;
  a.q = q;
  a.smax = smax;
  a.out = out;
  a.part = static_cast<int32_t*>(part);
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  a.G = static_cast<int>(K >> 7);
  a.n_rb = pl.n_rb;
  a.slices = pl.slices;
  a.out_kind = out_kind;
  hipError_t e = hipErrorInvalidValue;
  if (pl.rows_ns > 0) {
    if (M > kXRows || pl.nw * 64 > 512) return hipErrorInvalidValue;  // x slots hold kXRows tokens
    e = launch_rows<false>(a, static_cast<int>(M), pl, stream);
  } else if (pl.mfma) {
    if (M > 32 || pl.nw * 64 > (pl.gmax <= 3 ? 1024 : 512)) return hipErrorInvalidValue;
    e = launch_mfma(a, static_cast<int>(M), pl, stream);
  } else switch (static_cast<int>(M)) {
    case 1: e = launch_mt<1>(a, pl, stream); break;
    case 2: e = launch_mt<2>(a, pl, stream); break;
    case 3: e = launch_mt<3>(a, pl, stream); break;
    case 4: e = launch_mt<4>(a, pl, stream); break;
    case 5: e = launch_mt<5>(a, pl, stream); break;
    case 6: e = launch_mt<6>(a, pl, stream); break;
    case 7: e = launch_mt<7>(a, pl, stream); break;
    case 8: e = launch_mt<8>(a, pl, stream); break;
    case 9: e = launch_mt<9>(a, pl, stream); break;
    case 10: e = launch_mt<10>(a, pl, stream); break;
    case 11: e = launch_mt<11>(a, pl, stream); break;
    case 12: e = launch_mt<12>(a, pl, stream); break;
    case 13: e = launch_mt<13>(a, pl, stream); break;
    case 14: e = launch_mt<14>(a, pl, stream); break;
    case 15: e = launch_mt<15>(a, pl, stream); break;
    case 16: e = launch_mt<16>(a, pl, stream); break;
    case 17: e = launch_mt<17>(a, pl, stream); break;
    case 18: e = launch_mt<18>(a, pl, stream); break;
    case 19: e = launch_mt<19>(a, pl, stream); break;
    case 20: e = launch_mt<20>(a, pl, stream); break;
    case 21: e = launch_mt<21>(a, pl, stream); break;
    case 22: e = launch_mt<22>(a, pl, stream); break;
    case 23: e = launch_mt<23>(a, pl, stream); break;
    case 24: e = launch_mt<24>(a, pl, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || pl.slices <= 1) return e;
  const size_t total = static_cast<size_t>(M) * static_cast<size_t>(N);
  const unsigned blocks = static_cast<unsigned>(std::min<size_t>((total + 255) / 256, 4096));
  hipLaunchKernelGGL(gemv_reduce_kernel, dim3(blocks), dim3(256), 0, stream, a.part, pl.slices,
                     static_cast<int>(M), a.N, a_scale, smax, out, a.out_kind);
  return hipGetLastError();
}


// The fused decode kernel applies when the row-balanced plan does with one
// round of workgroups and the whole rotation fits the workgroup: at most
// kRotMaxM tokens of at most kRotMaxK, and at most 2 1024-blocks per wave
// (kRotBlocksPerWave = 3 for a single token).  Measured against the two
// launches (µs): 5120 -> 17408 9.7 / 12.0 at M = 1, 10.5 / 11.6 at M = 2,
// but 11.8 / 11.5 at M = 3 and 12.3 / 12.0 at M = 4 (three rounds of
// rotation per wave); 5120 -> 5120 7.4 / 8.5 at M = 1, 9.3 / 8.4 at M = 3;
// 5120 -> 34816 (two rounds of workgroups, each rotating again) 18.0 / 14.5
// at M = 1.
bool gemv_rot_applies(int64_t M, int64_t N, int64_t K, const DeviceInfo& dev) {
  if (M < 1 || M > kRotMaxM || K > kRotMaxK || N < 1) return false;
  const GemvPlan pl = make_rows_plan(N, K, dev);
  if (pl.slices <= 0 || pl.rows_ns <= 0 || pl.gmax > 17 || pl.nw * 64 > 512 || pl.nw > (K >> 7))
    return false;
  if (pl.rows_wgs > dev.cu_count) return false;
  const int64_t rounds = M == 1 ? kRotBlocksPerWave : 2;
  return M * (K >> 10) <= rounds * pl.nw;
}

hipError_t launch_gemv_rot(const uint16_t* x, const int8_t* sign, bool silu, const uint8_t* packed,
                           const int8_t* q, const float* smax, int64_t M, int64_t N, int64_t K,
                           void* out, OutKind out_kind, int8_t* x_i8, float* a_scale,
                           const DeviceInfo& dev, hipStream_t stream) {
  if (!gemv_rot_applies(M, N, K, dev)) return hipErrorNotSupported;
  // 16-row subtiles and v_mfma_i32_16x16x64_i8, tokens padded to 16, as the
  // two-step path uses at these batch sizes
  GemvPlan pl = make_rows_plan(N, K, dev);
  pl.rows_rs = 16;
  pl.rows_ns = static_cast<int>((N + pl.rows_wgs - 1) / pl.rows_wgs + 15) / 16;
  if (std::getenv("TWL_LOG"))
    std::fprintf(stderr, "[twl] gemv-rows+rotation M=%lld N=%lld K=%lld silu=%d -> <= %d groups/wave, %d waves/WG, grid=%d\n",
                 static_cast<long long>(M), static_cast<long long>(N), static_cast<long long>(K),
                 silu ? 1 : 0, pl.gmax, pl.nw, pl.rows_wgs);
  GemvArgs a = {};
  a.a_scale = a_scale;
  a.packed = packed;
  a.q = q;
  a.smax = smax;
  a.out = out;
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  a.G = static_cast<int>(K >> 7);
  a.n_rb = pl.n_rb;
  a.slices = 1;
  a.out_kind = out_kind;
  a.xb = x;
  a.sign = sign;
  a.x_i8_out = x_i8;
  a.a_scale_out = a_scale;
  a.silu = silu ? 1 : 0;
  return launch_rows<true>(a, static_cast<int>(M), pl, stream);
}

}  // namespace twl
