// Decode ternary linear (M <= 24 tokens): an HBM-streaming GEMV over the
// packed 2-bit weights using the VALU int8 dot product (v_dot4), no MFMA.
//
// Method ([P1] "Ternary-Bonsai-2-27B on 2x RTX 5070 with vLLM TP=2", section 4
// for the arithmetic, section 5 for the prior art): the same exact int32
// accumulator as the prefill GEMM,
//   acc[t,n] = sum_k x_i8[t,k] * code[n,k] * q[n, k/128],
//   y[t,n]   = acc[t,n] * a_scale[t] * smax[n] / 127.
// The pages tried a dp4a decode GEMV on their GPU (section 5 table: 2.1x as a
// kernel, +2% end to end, rejected because its error grew); here the GEMV is
// bit-exact with the GEMM because both compute the same integer sum.
//
// gfx950 mapping
//   * One workgroup owns 64 weight rows (lane l <-> row n0 + l) and splits the
//     K groups across its waves, so each lane keeps only M int32 accumulators
//     and the activations of a step are the same for the whole wave (uniform
//     addresses -> scalar loads, shared by the 64 rows).
//   * A wave stages 64 rows x 32 bytes (one 128-group) through LDS with
//     coalesced 16-byte loads, then each lane reads its own row's 8 words.
//   * Per word: 1 shift, 4 ANDs, 4 byte-permutes against tables built from
//     {-q, +q, 0}, then 4 v_dot4 per token.  The waves' partial sums are added with LDS integer
//     atomics (exact, order independent) before the rescale.
#include "twl_internal.h"

#include <algorithm>

namespace twl {
namespace {

constexpr int kRowStrideWords = 9;  // 8 words per row + 1 pad: conflict-free column reads

// Activations are read at wave-uniform addresses; reading them through the
// constant address space makes them scalar loads (one copy in SGPRs for the
// whole wave) instead of 64 identical vector loads.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(4))) const u32x4 const_u32x4;

typedef int v4i __attribute__((ext_vector_type(4)));

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

// MT is the exact number of tokens (1 .. 24).
template <int MT, bool OUT_ACC>
__global__ __launch_bounds__(1024) void gemv_kernel(const int8_t* __restrict__ x,
                                                    const float* __restrict__ a_scale,
                                                    const uint8_t* __restrict__ packed,
                                                    const int8_t* __restrict__ q,
                                                    const float* __restrict__ smax, int N, int K,
                                                    void* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  // wave index as a scalar: everything derived from it (the K range, the
  // activation addresses) is then known to be wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int n0 = blockIdx.x * 64;
  const int G = K >> 7;
  const size_t KB = static_cast<size_t>(K) >> 2;

  __shared__ uint32_t stage[16][64 * kRowStrideWords];
  __shared__ int red[MT][64];
  for (int i = threadIdx.x; i < MT * 64; i += blockDim.x) (&red[0][0])[i] = 0;
  __syncthreads();

  // contiguous range of 128-groups for this wave
  const int g_begin = (G * wave) / nw;
  const int g_end = (G * (wave + 1)) / nw;

  // coalesced staging: 16-byte piece p (0..127) of the wave's 64x32-byte tile
  // is row p / 2, half p % 2; each lane moves pieces lane and lane + 64.
  const int r0 = lane >> 1, r1 = (lane + 64) >> 1;
  const int hp = lane & 1;
  const uint8_t* src0 = packed + static_cast<size_t>(min(n0 + r0, N - 1)) * KB + hp * 16;
  const uint8_t* src1 = packed + static_cast<size_t>(min(n0 + r1, N - 1)) * KB + hp * 16;
  uint32_t* st = stage[wave];
  const int my_row = min(n0 + lane, N - 1);
  const int8_t* qrow = q + static_cast<size_t>(my_row) * G;

  int acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = 0;

  for (int g = g_begin; g < g_end; ++g) {
    const uint4 p0 = *reinterpret_cast<const uint4*>(src0 + static_cast<size_t>(g) * 32);
    const uint4 p1 = *reinterpret_cast<const uint4*>(src1 + static_cast<size_t>(g) * 32);
    const int qv = qrow[g];
    st[r0 * kRowStrideWords + hp * 4 + 0] = p0.x;
    st[r0 * kRowStrideWords + hp * 4 + 1] = p0.y;
    st[r0 * kRowStrideWords + hp * 4 + 2] = p0.z;
    st[r0 * kRowStrideWords + hp * 4 + 3] = p0.w;
    st[r1 * kRowStrideWords + hp * 4 + 0] = p1.x;
    st[r1 * kRowStrideWords + hp * 4 + 1] = p1.y;
    st[r1 * kRowStrideWords + hp * 4 + 2] = p1.z;
    st[r1 * kRowStrideWords + hp * 4 + 3] = p1.w;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint32_t words[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) words[w] = st[lane * kRowStrideWords + w];
    __builtin_amdgcn_wave_barrier();

    const QTables tab = make_tables(qv);
    const int8_t* xg = x + static_cast<size_t>(g) * 128;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const v4i wq = unpack16(words[w], tab);
      const int wq0 = wq.x, wq1 = wq.y, wq2 = wq.z, wq3 = wq.w;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const u32x4 xv = *(const const_u32x4*)(xg + static_cast<size_t>(t) * K + 16 * w);
        int a = acc[t];
        a = __builtin_amdgcn_sdot4(wq0, static_cast<int>(xv.x), a, false);
        a = __builtin_amdgcn_sdot4(wq1, static_cast<int>(xv.y), a, false);
        a = __builtin_amdgcn_sdot4(wq2, static_cast<int>(xv.z), a, false);
        a = __builtin_amdgcn_sdot4(wq3, static_cast<int>(xv.w), a, false);
        acc[t] = a;
      }
    }
  }

  // exact cross-wave reduction (integer LDS atomics), then the rescale
#pragma unroll
  for (int t = 0; t < MT; ++t) atomicAdd(&red[t][lane], acc[t]);
  __syncthreads();
  const int n = n0 + lane;
  for (int t = wave; t < MT; t += nw) {
    const int s = red[t][lane];
    if (n < N) {
      const size_t o = static_cast<size_t>(t) * N + n;
      if (OUT_ACC)
        static_cast<int32_t*>(out)[o] = s;
      else
        static_cast<float*>(out)[o] = static_cast<float>(s) * a_scale[t] * (smax[n] * (1.0f / 127.0f));
    }
  }
}

template <int MT>
hipError_t launch_mt(const int8_t* x, const float* a_scale, const uint8_t* packed, const int8_t* q,
                     const float* smax, int N, int K, void* out, bool out_acc,
                     hipStream_t stream) {
  const int G = K >> 7;
  const int nw = std::max(1, std::min(16, G / 4));
  const dim3 grid((N + 63) / 64);
  if (out_acc)
    hipLaunchKernelGGL((gemv_kernel<MT, true>), grid, dim3(64 * nw), 0, stream, x, a_scale, packed,
                       q, smax, N, K, out);
  else
    hipLaunchKernelGGL((gemv_kernel<MT, false>), grid, dim3(64 * nw), 0, stream, x, a_scale,
                       packed, q, smax, N, K, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const int8_t* x_i8, const float* a_scale, const uint8_t* packed,
                       const int8_t* q, const float* smax, int64_t M, int64_t N, int64_t K,
                       void* out, bool out_acc, const DeviceInfo&, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int n = static_cast<int>(N), k = static_cast<int>(K);
  switch (static_cast<int>(M)) {
    case 1: return launch_mt<1>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 2: return launch_mt<2>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 3: return launch_mt<3>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 4: return launch_mt<4>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 5: return launch_mt<5>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 6: return launch_mt<6>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 7: return launch_mt<7>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 8: return launch_mt<8>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 9: return launch_mt<9>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 10: return launch_mt<10>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 11: return launch_mt<11>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 12: return launch_mt<12>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 13: return launch_mt<13>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 14: return launch_mt<14>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 15: return launch_mt<15>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 16: return launch_mt<16>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 17: return launch_mt<17>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 18: return launch_mt<18>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 19: return launch_mt<19>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 20: return launch_mt<20>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 21: return launch_mt<21>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 22: return launch_mt<22>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 23: return launch_mt<23>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    case 24: return launch_mt<24>(x_i8, a_scale, packed, q, smax, n, k, out, out_acc, stream);
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace twl
