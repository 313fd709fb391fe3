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
// Layout on the GPU: one workgroup per token; wave w owns the 1024-blocks
// w, w + nw, ... of the row and rotates each in registers (rotate_block.h: 16
// elements per lane, butterflies inside lanes, two LDS transposes).  In the
// final layout a lane holds four runs of 4 consecutive elements, which it
// quantises and stores as four dwords (each store instruction writes 256
// contiguous bytes).  The per-token absmax is reduced across lanes and waves.
// The input is read once and the output written once: 2 B in + 1 B out per
// element.
#include "rotate_block.h"

namespace twl {
namespace {

using rot::kBlock;
using rot::kWaveBufWords;

// SILU: x is the gate/up output [M, 2K] (gate = columns 0..K-1) and the
// rotated input is bf16(SiLU(gate) * up), computed as the block is loaded.
// RAW: no quantisation; r itself is written as bf16 (nearest even) to
// `x_i8`, which then points to uint16 [M, K], and a_scale is not touched.
template <int BPW, bool SILU, bool RAW>
__global__ __launch_bounds__(1024) void rotate_quant_kernel(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ sign, int K, int nblocks,
    int8_t* __restrict__ x_i8, float* __restrict__ a_scale) {
  extern __shared__ float wbuf_all[];  // nw x kWaveBufWords
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const uint16_t* xr = x + static_cast<size_t>(t) * (SILU ? 2 * K : K);
  float* wb = wbuf_all + wave * kWaveBufWords;
  float v[BPW][16];
  float amax = 0.0f;

#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int b = wave + i * nw;
    if (b < nblocks) {
      float(&w)[16] = v[i];
      rot::rotate_block<SILU>(xr, sign, K, b, lane, wb, w);
#pragma unroll
      for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(w[e]));
      if (RAW) {
        uint16_t* rr = reinterpret_cast<uint16_t*>(x_i8) + static_cast<size_t>(t) * K + b * kBlock;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t lo = f32_to_bf16_rne(w[4 * c]) | (static_cast<uint32_t>(f32_to_bf16_rne(w[4 * c + 1])) << 16);
          const uint32_t hi = f32_to_bf16_rne(w[4 * c + 2]) | (static_cast<uint32_t>(f32_to_bf16_rne(w[4 * c + 3])) << 16);
          *reinterpret_cast<uint2*>(rr + 256 * c + 4 * lane) = make_uint2(lo, hi);
        }
      }
    }
  }
  if (RAW) return;

  // per-token absmax over the whole row: lanes, then waves
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  __shared__ float wave_max[16];
  if (lane == 0) wave_max[wave] = amax;
  __syncthreads();
  float tmax = wave_max[0];
  for (int w = 1; w < nw; ++w) tmax = fmaxf(tmax, wave_max[w]);
  // a_scale and the quotient (the quantiser of rotate_block.h)
  const rot::TokenQuant tq = rot::token_quant(tmax);
  if (threadIdx.x == 0) a_scale[t] = tq.scale;
  int8_t* yr = x_i8 + static_cast<size_t>(t) * K;
  const auto store_all = [&](auto quotient) {
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int b = wave + i * nw;
      if (b < nblocks) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint32_t word = 0;
#pragma unroll
          for (int d = 0; d < 4; ++d) word |= rot::quant_byte(quotient(v[i][4 * c + d])) << (8 * d);
          *reinterpret_cast<uint32_t*>(yr + b * kBlock + 256 * c + 4 * lane) = word;
        }
      }
    }
  };
  // the test is hoisted out of the element loop (one branch per token)
  if (tq.markstein)
    store_all([&](float w) { return rot::quotient_markstein(w, tq); });
  else
    store_all([&](float w) { return w / tq.div; });
}

template <int BPW, bool SILU, bool RAW>
hipError_t launch_bpw(const uint16_t* x, const int8_t* sign, int64_t M, int64_t K,
                      int8_t* x_i8, float* a_scale, hipStream_t stream) {
  const int nblocks = static_cast<int>(K / kBlock);
  const int nw = (nblocks + BPW - 1) / BPW;
  const size_t lds = static_cast<size_t>(nw) * kWaveBufWords * sizeof(float);
  if (lds > 65536) {
    // more than the default dynamic LDS limit: the part has 160 KiB per CU
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(rotate_quant_kernel<BPW, SILU, RAW>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((rotate_quant_kernel<BPW, SILU, RAW>), dim3(static_cast<unsigned>(M)), dim3(64 * nw),
                     lds, stream, x, sign,
                     static_cast<int>(K), nblocks, x_i8, a_scale);
  return hipGetLastError();
}

template <bool SILU, bool RAW>
hipError_t launch_rotate(const uint16_t* x, const int8_t* sign, int64_t M, int64_t K,
                         int8_t* x_i8, float* a_scale, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int64_t nblocks = K / kBlock;  // 1 .. 64 (validated by the caller)
  if (nblocks <= 16) return launch_bpw<1, SILU, RAW>(x, sign, M, K, x_i8, a_scale, stream);
  if (nblocks <= 32) return launch_bpw<2, SILU, RAW>(x, sign, M, K, x_i8, a_scale, stream);
  return launch_bpw<4, SILU, RAW>(x, sign, M, K, x_i8, a_scale, stream);
}

}  // namespace

hipError_t launch_rotate_quant(const uint16_t* x, const int8_t* sign, int64_t M, int64_t K,
                               int8_t* x_i8, float* a_scale, hipStream_t stream) {
  return launch_rotate<false, false>(x, sign, M, K, x_i8, a_scale, stream);
}

hipError_t launch_silu_mul_rotate_quant(const uint16_t* gate_up, const int8_t* sign, int64_t M,
                                        int64_t K, int8_t* x_i8, float* a_scale,
                                        hipStream_t stream) {
  return launch_rotate<true, false>(gate_up, sign, M, K, x_i8, a_scale, stream);
}

hipError_t launch_rotate_bf16(const uint16_t* x, const int8_t* sign, int64_t M, int64_t K,
                              uint16_t* r, hipStream_t stream) {
  return launch_rotate<false, true>(x, sign, M, K, reinterpret_cast<int8_t*>(r), nullptr, stream);
}

}  // namespace twl
