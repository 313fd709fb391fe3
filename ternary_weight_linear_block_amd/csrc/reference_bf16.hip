// Exact-dequant bf16 reference linear: the layer as the pages computed it
// before their int8 path, kept as an accuracy reference and an A/B point.
//
// Method ([P1] "Ternary-Bonsai-2-27B on 2x RTX 5070 with vLLM TP=2", section 4:
// the bf16 path the int8 GEMM replaced, with its lower error; Prerequisites:
// weight = code * s per 128-group):
//   W[n,k]  = code[n,k] * bf16(s[n, k/128])       (the scale rounded to bf16)
//   y[t,n]  = sum_k r_bf16[t,k] * W[n,k]           (fp32 accumulation)
// with r_bf16 the rotated activation rounded to bf16 (twl_rotate_act_bf16).
// The pages expand W into memory and call a library GEMM; here the 2-bit
// codes are expanded to bf16 in registers right before the matrix cores, so
// the weights stay packed in HBM as on the int8 path.
//
// gfx950 mapping: v_mfma_f32_32x32x16_bf16.  A workgroup of 4 waves owns a
// 128 x 64 output tile; wave w owns tokens 32 w .. 32 w + 31 and both 32-row
// weight fragments.  Per 128-group a lane (i, h) loads 16 packed bytes (words
// 4h .. 4h+3 of its weight row) and, per 16-k step t, 16 bytes of its token
// row; lane half h at step t covers k = 64 h + 8 t .. +7 of the group, the same
// k on both operands.  Operands come straight from global memory (L2): this
// is a reference kernel, not tuned like the int8 path.
#include "twl_internal.h"

namespace twl {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// The 8 bf16 weights of codes k = 8 half .. 8 half + 7 of a packed word (the
// fields i = 2 half, 2 half + 1 of every byte) against the table
// [neg_lo neg_hi pos_lo pos_hi] (src1) and zeros (src0): a code u selects the
// byte pair (2u, 2u + 1), so u = 2 (code 0) lands on the zeros.
__device__ __forceinline__ u32x4 dequant8(uint32_t word, int half, uint32_t table) {
  u32x4 out;
#pragma unroll
  for (int ip = 0; ip < 2; ++ip) {
    // fields i = 2 half + ip of bytes b = 0..3: codes k = 8 half + 4 ip + b
    const uint32_t f = (word >> (2 * (2 * half + ip))) & 0x03030303u;
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      // codes of bytes 2 pr and 2 pr + 1 -> selector bytes (2u, 2u+1, 2v, 2v+1)
      const uint32_t spread = __builtin_amdgcn_perm(0u, f, pr == 0 ? 0x01010000u : 0x03030202u);
      const uint32_t sel = (spread << 1) + 0x01000100u;
      out[2 * ip + pr] = __builtin_amdgcn_perm(0u, table, sel);
    }
  }
  return out;
}

__device__ __forceinline__ uint32_t f16_bits_to_bf16_bits(uint16_t h) {
  const float f = static_cast<float>(__builtin_bit_cast(_Float16, h));  // exact
  return f32_to_bf16_rne(f);
}

__global__ __launch_bounds__(256) void reference_bf16_kernel(
    const uint16_t* __restrict__ r, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ s, int M, int N, int K, int tiles_m, float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i = lane & 31, h = lane >> 5;
  const int m0 = (blockIdx.x % tiles_m) * 128, n0 = (blockIdx.x / tiles_m) * 64;
  const int G = K >> 7;
  const int m = min(m0 + 32 * wave + i, M - 1);   // token row of the A operand
  const uint16_t* arow = r + static_cast<size_t>(m) * K + 64 * h;
  int nrow[2];
  size_t wbase[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    nrow[f] = min(n0 + 32 * f + i, N - 1);     // weight row of the B operand
    wbase[f] = static_cast<size_t>(nrow[f] >> 6) * G * 2048 + (nrow[f] & 63) * 32 + 16 * h;
  }
  v16f acc[2] = {v16f{0}, v16f{0}};
  for (int g = 0; g < G; ++g) {
    uint4 wv[2];
    uint32_t table[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      wv[f] = *reinterpret_cast<const uint4*>(packed + wbase[f] + static_cast<size_t>(g) * 2048);
      const uint32_t pos = f16_bits_to_bf16_bits(s[static_cast<size_t>(nrow[f]) * G + g]);
      table[f] = (pos ^ 0x8000u) | (pos << 16);  // [-s, +s] as bf16
    }
    v8bf a[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
      a[t] = *reinterpret_cast<const v8bf*>(arow + static_cast<size_t>(g) * 128 + 8 * t);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const uint32_t words[4] = {wv[f].x, wv[f].y, wv[f].z, wv[f].w};
        const u32x4 b = dequant8(words[t >> 1], t & 1, table[f]);
        acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t], __builtin_bit_cast(v8bf, b), acc[f], 0, 0, 0);
      }
    }
  }
  // lane (i, h) holds weight row n0 + 32 f + i and, in register q, token row
  // 8 (q / 4) + 4 h + (q % 4) of the wave's 32
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int n = n0 + 32 * f + i;
    if (n >= N) continue;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int t = m0 + 32 * wave + 8 * (q >> 2) + 4 * h + (q & 3);
      if (t < M) y[static_cast<size_t>(t) * N + n] = acc[f][q];
    }
  }
}

}  // namespace

hipError_t launch_reference_bf16(const uint16_t* r, const uint8_t* packed, const uint16_t* s,
                                 int64_t M, int64_t N, int64_t K, float* y, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int tiles_m = static_cast<int>((M + 127) / 128);
  const int64_t tiles = static_cast<int64_t>(tiles_m) * ((N + 63) / 64);
  hipLaunchKernelGGL(reference_bf16_kernel, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, stream,
                     r, packed, s, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K),
                     tiles_m, y);
  return hipGetLastError();
}

}  // namespace twl
