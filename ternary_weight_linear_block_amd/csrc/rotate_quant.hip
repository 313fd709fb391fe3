// rotate_quant_act: signed block-1024 Sylvester Hadamard rotation of bf16
// activations, per-token absmax and int8 quantisation, in one pass.
//
// Method ([P1] "Ternary-Bonsai-2-27B on 2x RTX 5070 with vLLM TP=2",
// Prerequisites, section 1 and section 4): the input side of every ternary
// linear carries a block-wise Hadamard rotation whose sign table is keyed by
// the full input width; after rotating, activations are quantised to int8 with
// one scale per token.  Section 1 fixes the recursion
// H1024 [a; b] = [H512 a + H512 b ; H512 a - H512 b], i.e. the last butterfly
// stage combines the two 512-halves, so stages run h = 1, 2, ..., 512.
//
// Layout on the GPU: one workgroup per token.  Wave w owns the 1024-blocks
// w, w + nw, ... of the row; lane l holds the 16 contiguous elements
// 16l .. 16l+15 of each block in registers.  Stages h = 1..8 are in-lane,
// stages h = 16..512 pair lane l with lane l ^ (h/16) through cross-lane
// shuffles.  The per-token absmax is reduced across lanes and waves, then each
// lane quantises its registers and writes 16 bytes.  The input is read once
// and the output written once: the kernel is bound by HBM traffic
// (2 B in + 1 B out per element).
//
// Every butterfly is (lo, hi) -> (lo + hi, lo - hi) in fp32 with the same
// operands as a textbook in-place FWHT, so the result is bit-identical to any
// implementation that follows the same stage order; the build uses
// -ffp-contract=off so no add is fused with anything.
#include "twl_internal.h"

namespace twl {
namespace {

constexpr int kBlock = 1024;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Stages h = 1, 2, 4, 8 inside one lane's 16 consecutive elements.
__device__ __forceinline__ void fwht16_in_lane(float (&v)[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if ((j & h) == 0) {
        const float lo = v[j];
        const float hi = v[j + h];
        v[j] = lo + hi;
        v[j + h] = lo - hi;
      }
    }
  }
}

// One cross-lane stage: the partner lane is lane ^ mask.  The lane whose mask
// bit is clear holds the lower position (lo), its partner the upper one (hi).
__device__ __forceinline__ void fwht_cross_stage(float (&v)[16], int mask, bool upper) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float p = __shfl_xor(v[j], mask);
    v[j] = upper ? (p - v[j]) : (v[j] + p);
  }
}

template <int BPW>
__global__ __launch_bounds__(1024) void rotate_quant_kernel(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ sign, int K, int nblocks,
    int8_t* __restrict__ x_i8, float* __restrict__ a_scale) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const uint16_t* xr = x + static_cast<size_t>(t) * K;

  float v[BPW][16];
  float amax = 0.0f;

#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int b = wave + i * nw;
    if (b < nblocks) {
      const int k0 = b * kBlock + lane * 16;
      const uint4 p0 = *reinterpret_cast<const uint4*>(xr + k0);
      const uint4 p1 = *reinterpret_cast<const uint4*>(xr + k0 + 8);
      const uint4 sg = *reinterpret_cast<const uint4*>(sign + k0);
      const uint32_t pw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
      const uint32_t sw[4] = {sg.x, sg.y, sg.z, sg.w};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t bits = (pw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        // multiply by the +-1 sign: flip the fp32 sign bit when the int8 sign is negative
        const uint32_t flip = ((sw[e >> 2] >> (8 * (e & 3) + 7)) & 1u) << 31;
        v[i][e] = __uint_as_float(__float_as_uint(bf16_bits_to_float(bits)) ^ flip);
      }
      fwht16_in_lane(v[i]);
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) fwht_cross_stage(v[i], m, (lane & m) != 0);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        v[i][e] *= 0.03125f;  // orthonormal 1/sqrt(1024): exact power of two
        amax = fmaxf(amax, fabsf(v[i][e]));
      }
    }
  }

  // per-token absmax over the whole row: lanes, then waves
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  __shared__ float wave_max[16];
  if (lane == 0) wave_max[wave] = amax;
  __syncthreads();
  float tmax = wave_max[0];
  for (int w = 1; w < nw; ++w) tmax = fmaxf(tmax, wave_max[w]);
  const float scale = tmax / 127.0f;  // IEEE division
  if (threadIdx.x == 0) a_scale[t] = scale;

  int8_t* yr = x_i8 + static_cast<size_t>(t) * K;
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int b = wave + i * nw;
    if (b < nblocks) {
      uint32_t packedq[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        int qv = 0;
        if (scale > 0.0f) {
          float r = rintf(v[i][e] / scale);  // IEEE division, ties to even
          r = fminf(fmaxf(r, -127.0f), 127.0f);
          qv = static_cast<int>(r);
        }
        packedq[e >> 2] |= (static_cast<uint32_t>(qv) & 0xFFu) << (8 * (e & 3));
      }
      *reinterpret_cast<uint4*>(yr + b * kBlock + lane * 16) =
          make_uint4(packedq[0], packedq[1], packedq[2], packedq[3]);
    }
  }
}

template <int BPW>
hipError_t launch_bpw(const uint16_t* x, const int8_t* sign, int64_t M, int64_t K,
                      int8_t* x_i8, float* a_scale, hipStream_t stream) {
  const int nblocks = static_cast<int>(K / kBlock);
  const int nw = (nblocks + BPW - 1) / BPW;
  hipLaunchKernelGGL(rotate_quant_kernel<BPW>, dim3(static_cast<unsigned>(M)), dim3(64 * nw), 0,
                     stream, x, sign, static_cast<int>(K), nblocks, x_i8, a_scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rotate_quant(const uint16_t* x, const int8_t* sign, int64_t M, int64_t K,
                               int8_t* x_i8, float* a_scale, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int64_t nblocks = K / kBlock;  // 1 .. 64 (validated by the caller)
  if (nblocks <= 16) return launch_bpw<1>(x, sign, M, K, x_i8, a_scale, stream);
  if (nblocks <= 32) return launch_bpw<2>(x, sign, M, K, x_i8, a_scale, stream);
  return launch_bpw<4>(x, sign, M, K, x_i8, a_scale, stream);
}

}  // namespace twl
