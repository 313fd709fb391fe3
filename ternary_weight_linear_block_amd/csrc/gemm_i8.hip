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
// bytes of its MFMA B operand with 3 shifts, 4 ANDs and 4 byte-permutes
// against the table {-q, 0, +q}.
//
// gfx950 mapping
//   * v_mfma_i32_32x32x32_i8: a 32x32 output tile, K = 32 per instruction;
//     each lane supplies 16 bytes of A (one row) and 16 bytes of B (one
//     column).  Integer accumulation is exact, so the assignment of k values
//     to (lane half, byte) only has to be the same for A and B: lane half h
//     at k-step s of a 128-group covers k = 16 (4h + s) .. +15, which makes a
//     lane's B data for a whole group one 16-byte load of packed words.
//   * Workgroup: 4 waves in a 2x2 grid, wave tile (32 RM) x (32 RN), block
//     tile (64 RM) x (64 RN).  The x_i8 tile of a group (BM x 128 bytes) is
//     staged in LDS, double buffered, with a 16-byte-chunk XOR swizzle so the
//     column-wise ds_read_b128 of the A operand hits distinct banks.
//   * Packed weights go from global memory straight to registers (prefetched
//     one group ahead); they are 1/4 of an int8 operand, so a second LDS
//     round trip would cost more than it saves.
//   * Epilogue: acc -> fp32 with a_scale[row] and smax[col]/127, stored row
//     major (32 consecutive floats per half-wave).
#include "twl_internal.h"

#include <algorithm>

namespace twl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// 16-byte chunk swizzle inside a 128-byte LDS row: distinct chunks for any 8
// consecutive rows (32-bank view) and for the even / odd rows of any 16
// consecutive rows (64-bank view).
__device__ __forceinline__ int chunk_swizzle(int row) { return (row ^ (row >> 3)) & 7; }

// Four int8 bytes {code * q} for the 2-bit fields at bit offset `shift` of
// each byte of `word` (u = 0, 1, 2 selects byte 0, 1, 2 of `table`).
__device__ __forceinline__ int unpack4(uint32_t word, int shift, uint32_t table) {
  const uint32_t sel = (word >> shift) & 0x03030303u;
  return static_cast<int>(__builtin_amdgcn_perm(0u, table, sel));
}

template <int RM, int RN, bool OUT_ACC>
__global__ __launch_bounds__(256, 1) void gemm_kernel(
    const int8_t* __restrict__ x, const float* __restrict__ a_scale,
    const uint8_t* __restrict__ packed, const int8_t* __restrict__ q,
    const float* __restrict__ smax, int M, int N, int K, void* __restrict__ out) {
  constexpr int BM = 64 * RM;
  constexpr int BN = 64 * RN;
  constexpr int A_LOADS = BM * 8 / 256;  // 16-byte chunks per thread per group
  __shared__ __attribute__((aligned(16))) int8_t As[2][BM * 128];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int G = K >> 7;
  const size_t KB = static_cast<size_t>(K) >> 2;

  // Global -> LDS assignment for the A tile: chunk c = tid + 256 p covers row
  // c / 8, 16-byte chunk c % 8 (8 lanes read one 128-byte row segment).
  const int8_t* a_src[A_LOADS];
  int a_dst[A_LOADS];
#pragma unroll
  for (int p = 0; p < A_LOADS; ++p) {
    const int c = tid + 256 * p;
    const int row = c >> 3;
    const int ch = c & 7;
    const int grow = min(m0 + row, M - 1);  // rows past M are computed, never stored
    a_src[p] = x + static_cast<size_t>(grow) * K + ch * 16;
    a_dst[p] = row * 128 + ((ch ^ chunk_swizzle(row)) << 4);
  }

  // B operand rows (weight rows = output columns) of this lane.
  const uint8_t* b_src[RN];
  const int8_t* q_src[RN];
#pragma unroll
  for (int j = 0; j < RN; ++j) {
    const int n = min(n0 + wn * 32 * RN + 32 * j + l32, N - 1);
    b_src[j] = packed + static_cast<size_t>(n) * KB + half * 16;
    q_src[j] = q + static_cast<size_t>(n) * G;
  }

  v16i acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j) acc[i][j] = v16i{0};

  uint4 bcur[RN];
  int qcur[RN];
  uint4 astage[A_LOADS];
#pragma unroll
  for (int p = 0; p < A_LOADS; ++p) astage[p] = *reinterpret_cast<const uint4*>(a_src[p]);
#pragma unroll
  for (int j = 0; j < RN; ++j) {
    bcur[j] = *reinterpret_cast<const uint4*>(b_src[j]);
    qcur[j] = q_src[j][0];
  }
#pragma unroll
  for (int p = 0; p < A_LOADS; ++p) *reinterpret_cast<uint4*>(&As[0][a_dst[p]]) = astage[p];
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    // Prefetch the next group (the last iteration re-reads the last group; its
    // LDS copy lands in the idle buffer and is never read).
    const int gn = min(g + 1, G - 1);
    uint4 bnext[RN];
    int qnext[RN];
#pragma unroll
    for (int p = 0; p < A_LOADS; ++p)
      astage[p] = *reinterpret_cast<const uint4*>(a_src[p] + static_cast<size_t>(gn) * 128);
#pragma unroll
    for (int j = 0; j < RN; ++j) {
      bnext[j] = *reinterpret_cast<const uint4*>(b_src[j] + static_cast<size_t>(gn) * 32);
      qnext[j] = q_src[j][gn];
    }

    uint32_t table[RN];  // bytes {-q, 0, +q, 0}
#pragma unroll
    for (int j = 0; j < RN; ++j)
      table[j] = (static_cast<uint32_t>(-qcur[j]) & 0xFFu) | ((static_cast<uint32_t>(qcur[j]) & 0xFFu) << 16);

#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v4i a[RM];
#pragma unroll
      for (int i = 0; i < RM; ++i) {
        const int row = wm * 32 * RM + 32 * i + l32;
        const int ch = 4 * half + s;
        a[i] = *reinterpret_cast<const v4i*>(&As[buf][row * 128 + ((ch ^ chunk_swizzle(row)) << 4)]);
      }
#pragma unroll
      for (int j = 0; j < RN; ++j) {
        const uint32_t w = (s == 0) ? bcur[j].x : (s == 1) ? bcur[j].y : (s == 2) ? bcur[j].z : bcur[j].w;
        v4i b;
        b.x = unpack4(w, 0, table[j]);
        b.y = unpack4(w, 2, table[j]);
        b.z = unpack4(w, 4, table[j]);
        b.w = unpack4(w, 6, table[j]);
#pragma unroll
        for (int i = 0; i < RM; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b, acc[i][j], 0, 0, 0);
      }
    }

#pragma unroll
    for (int p = 0; p < A_LOADS; ++p) *reinterpret_cast<uint4*>(&As[buf ^ 1][a_dst[p]]) = astage[p];
#pragma unroll
    for (int j = 0; j < RN; ++j) {
      bcur[j] = bnext[j];
      qcur[j] = qnext[j];
    }
    __syncthreads();
  }

  // Epilogue.  32x32 accumulator layout: lane holds column l32; register r
  // holds row 8 (r / 4) + 4 half + (r % 4).
#pragma unroll
  for (int j = 0; j < RN; ++j) {
    const int col = n0 + wn * 32 * RN + 32 * j + l32;
    if (col >= N) continue;
    float cscale = 0.0f;
    if (!OUT_ACC) cscale = smax[col] * (1.0f / 127.0f);
#pragma unroll
    for (int i = 0; i < RM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 32 * RM + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row < M) {
          const size_t o = static_cast<size_t>(row) * N + col;
          if (OUT_ACC) {
            static_cast<int32_t*>(out)[o] = acc[i][j][r];
          } else {
            static_cast<float*>(out)[o] = static_cast<float>(acc[i][j][r]) * a_scale[row] * cscale;
          }
        }
      }
    }
  }
}

struct TileChoice {
  int rm, rn;
};

template <int RM, int RN>
hipError_t launch_tile(const int8_t* x, const float* a_scale, const uint8_t* packed,
                       const int8_t* q, const float* smax, int M, int N, int K, void* out,
                       bool out_acc, hipStream_t stream) {
  const dim3 grid((N + 64 * RN - 1) / (64 * RN), (M + 64 * RM - 1) / (64 * RM));
  if (out_acc)
    hipLaunchKernelGGL((gemm_kernel<RM, RN, true>), grid, dim3(256), 0, stream, x, a_scale, packed,
                       q, smax, M, N, K, out);
  else
    hipLaunchKernelGGL((gemm_kernel<RM, RN, false>), grid, dim3(256), 0, stream, x, a_scale,
                       packed, q, smax, M, N, K, out);
  return hipGetLastError();
}

// Pick the block tile that minimises the estimated makespan: work per tile
// over a per-CU rate that grows with the tile (operand reuse), times the
// number of tiles the busiest CU gets.
TileChoice choose_tile(int64_t M, int64_t N, const DeviceInfo& dev) {
  struct Cand {
    int rm, rn;
    double rate;
  };
  static const Cand cands[] = {{4, 4, 1.00}, {4, 2, 0.85}, {2, 4, 0.85},
                               {2, 2, 0.70}, {1, 4, 0.55}, {1, 2, 0.45}};
  const int64_t cus = std::max(1, dev.cu_count);
  double best = 1e300;
  TileChoice pick{1, 2};
  for (const Cand& c : cands) {
    const int64_t bm = 64 * c.rm, bn = 64 * c.rn;
    const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    const int64_t per_cu = (tiles + cus - 1) / cus;
    const double t = static_cast<double>(per_cu) * static_cast<double>(bm * bn) / c.rate;
    if (t < best * 0.999) {
      best = t;
      pick = {c.rm, c.rn};
    }
  }
  return pick;
}

}  // namespace

size_t gemm_workspace_bytes(int64_t, int64_t, int64_t, const DeviceInfo&) { return 0; }

hipError_t launch_gemm(const int8_t* x_i8, const float* a_scale, const uint8_t* packed,
                       const int8_t* q, const float* smax, int64_t M, int64_t N, int64_t K,
                       void* out, bool out_acc, void*, size_t, const DeviceInfo& dev,
                       hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const TileChoice t = choose_tile(M, N, dev);
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
#define TWL_TILE(RM_, RN_)                                                                   \
  if (t.rm == RM_ && t.rn == RN_)                                                            \
    return launch_tile<RM_, RN_>(x_i8, a_scale, packed, q, smax, m, n, k, out, out_acc, stream);
  TWL_TILE(4, 4)
  TWL_TILE(4, 2)
  TWL_TILE(2, 4)
  TWL_TILE(2, 2)
  TWL_TILE(1, 4)
  TWL_TILE(1, 2)
#undef TWL_TILE
  return hipErrorInvalidValue;
}

}  // namespace twl
