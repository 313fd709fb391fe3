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
// w, w + nw, ... of the row.  A block lives in registers, 16 elements per
// lane, and every butterfly runs inside a lane: the element index e (10 bits)
// is split between lane and register slot three times, with two LDS
// transposes in between (per-wave buffer, padded to be bank-conflict free):
//   layout 0: lane = e[9:4],            slot = e[3:0]  -> stages h = 1 .. 8
//   layout 1: lane = e[9:8] e[3:0],     slot = e[7:4]  -> stages h = 16 .. 128
//   layout 2: lane = e[7:2],            slot = e[9:8] e[1:0] -> stages h = 256, 512
// so the pass has no cross-lane arithmetic at all.  In layout 2 a lane holds
// four runs of 4 consecutive elements, which it quantises and stores as four
// dwords (each store instruction writes 256 contiguous bytes).  The
// per-token absmax is reduced across lanes and waves.  The input is read once
// and the output written once: 2 B in + 1 B out per element.
//
// Every butterfly is (lo, hi) -> (lo + hi, lo - hi) in fp32 with the same
// operands as a textbook in-place FWHT and in the same stage order, so the
// result is bit-identical to any implementation that follows that order; the
// build uses -ffp-contract=off so no add is fused with anything.
#include "twl_internal.h"

namespace twl {
namespace {

constexpr int kBlock = 1024;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// exp(x) in fp32 by a fixed sequence of operations, so that any two
// implementations of the fused activation agree bit for bit: clamp to
// [-87, 88] (e^x stays a normal float and 1 + e^-x is then exact or finite),
// n = rint(x log2 e), Cody-Waite reduction r = (x - n ln2_hi) - n ln2_lo with
// ln2_hi = 0x1.62e4p-1 (15 significant bits, so n ln2_hi is exact), the
// Taylor polynomial of degree 7 (coefficients 1/k! rounded to fp32) in Horner
// form, and exact scaling by 2^n.  Within 1.2 ulp of exp over the range.
// No operation may be fused (the library is built with -ffp-contract=off).
__device__ __forceinline__ float exp_fixed(float x) {
  x = fminf(fmaxf(x, -87.0f), 88.0f);
  const float n = rintf(x * 0x1.715476p+0f);
  const float r = (x - n * 0x1.62e4p-1f) - n * 0x1.7f7d1cp-20f;
  float p = 0x1.a01a02p-13f;  // 1/7!
  p = p * r + 0x1.6c16c2p-10f;  // 1/6!
  p = p * r + 0x1.111112p-7f;   // 1/5!
  p = p * r + 0x1.555556p-5f;   // 1/4!
  p = p * r + 0x1.555556p-3f;   // 1/3!
  p = p * r + 0.5f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  return ldexpf(p, static_cast<int>(n));
}

// bf16 bits of SiLU(g) * u for bf16 inputs g and u: s = g / (1 + exp(-g)) and
// s * u in fp32, rounded to bf16 (nearest even) as an unfused activation step
// would store it.
__device__ __forceinline__ uint32_t silu_mul_bits(uint32_t g_bits, uint32_t u_bits) {
  const float g = bf16_bits_to_float(g_bits);
  const float u = bf16_bits_to_float(u_bits);
  const float s = g / (1.0f + exp_fixed(-g));  // IEEE division
  return f32_to_bf16_rne(s * u);
}

// The butterflies of stage h = 2^b on register slot bit `sb` of a 16-slot
// lane: slot j (bit sb clear) holds the lower position, j | (1 << sb) the
// upper one.
__device__ __forceinline__ void stage_in_lane(float (&v)[16], int sb) {
  const int m = 1 << sb;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if ((j & m) == 0) {
      const float lo = v[j];
      const float hi = v[j + m];
      v[j] = lo + hi;
      v[j + m] = lo - hi;
    }
  }
}

// LDS word addresses of element e in the two transposes (padded so that both
// the writes and the reads of each transpose hit 64 distinct banks).
__device__ __forceinline__ int addr_a(int e) { return (e >> 4) * 20 + (e & 15) + 16 * (e >> 8); }
__device__ __forceinline__ int addr_b(int e) { return e + 16 * (e >> 8); }
constexpr int kWaveBufWords = 1344;  // > max addr_a (1323) and addr_b (1071)

__device__ __forceinline__ void lds_wave_sync() {
  // LDS operations of one wave execute in order; the fences only keep the
  // compiler from moving reads above the writes they depend on (or the next
  // writes above these reads)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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
  // layout-1 lane bits: e[9:8] = lane >> 4, e[3:0] = lane & 15;
  // layout-2 lane bits: e[7:2] = lane
  const int l1_hi = lane >> 4, l1_lo = lane & 15;

  float v[BPW][16];
  float amax = 0.0f;

#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int b = wave + i * nw;
    if (b < nblocks) {
      // layout 0: element e = 16 lane + slot
      const int k0 = b * kBlock + lane * 16;
      const uint4 p0 = *reinterpret_cast<const uint4*>(xr + k0);
      const uint4 p1 = *reinterpret_cast<const uint4*>(xr + k0 + 8);
      const uint4 sg = *reinterpret_cast<const uint4*>(sign + k0);
      uint32_t pw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
      if (SILU) {
        const uint4 u0 = *reinterpret_cast<const uint4*>(xr + K + k0);
        const uint4 u1 = *reinterpret_cast<const uint4*>(xr + K + k0 + 8);
        const uint32_t uw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pw[e] = silu_mul_bits(pw[e] & 0xFFFFu, uw[e] & 0xFFFFu) |
                  (silu_mul_bits(pw[e] >> 16, uw[e] >> 16) << 16);
      }
      const uint32_t sw[4] = {sg.x, sg.y, sg.z, sg.w};
      float(&w)[16] = v[i];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t bits = (pw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        // multiply by the +-1 sign: flip the fp32 sign bit when the int8 sign is negative
        const uint32_t flip = ((sw[e >> 2] >> (8 * (e & 3) + 7)) & 1u) << 31;
        w[e] = __uint_as_float(__float_as_uint(bf16_bits_to_float(bits)) ^ flip);
      }
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) stage_in_lane(w, sb);  // h = 1, 2, 4, 8

      // transpose to layout 1: slot s holds e = 256 l1_hi + 16 s + l1_lo
      lds_wave_sync();
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(wb + addr_a(16 * lane + 4 * q)) =
            make_float4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
      lds_wave_sync();
#pragma unroll
      for (int sl = 0; sl < 16; ++sl) w[sl] = wb[addr_a(256 * l1_hi + 16 * sl + l1_lo)];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) stage_in_lane(w, sb);  // h = 16, 32, 64, 128

      // transpose to layout 2: slot 4 c + d holds e = 256 c + 4 lane + d
      lds_wave_sync();
#pragma unroll
      for (int sl = 0; sl < 16; ++sl) wb[addr_b(256 * l1_hi + 16 * sl + l1_lo)] = w[sl];
      lds_wave_sync();
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 f = *reinterpret_cast<const float4*>(wb + addr_b(256 * c + 4 * lane));
        w[4 * c] = f.x;
        w[4 * c + 1] = f.y;
        w[4 * c + 2] = f.z;
        w[4 * c + 3] = f.w;
      }
#pragma unroll
      for (int sb = 2; sb < 4; ++sb) stage_in_lane(w, sb);  // h = 256, 512

#pragma unroll
      for (int e = 0; e < 16; ++e) {
        w[e] *= 0.03125f;  // orthonormal 1/sqrt(1024): exact power of two
        amax = fmaxf(amax, fabsf(w[e]));
      }
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
  const float scale = tmax / 127.0f;  // IEEE division
  if (threadIdx.x == 0) a_scale[t] = scale;

  // a zero scale (all-zero row, or an absmax so small that absmax / 127
  // underflows) quantises every element to 0: dividing by 1 instead gives
  // rint(|v| <= tiny) = 0 without a branch per element
  const float div = scale > 0.0f ? scale : 1.0f;
  int8_t* yr = x_i8 + static_cast<size_t>(t) * K;
  // The quotient v / div must be the IEEE-rounded one (the quantiser rounds
  // it to the nearest integer, ties to even).  With inv = RN(1 / div), one
  // IEEE division per token, q0 = RN(v inv) is within one ulp of v / div, the
  // residual v - q0 div is exact in one fma, and RN(q0 + residual * inv) is
  // the correctly rounded quotient (Markstein's theorem), as long as nothing
  // overflows or underflows: 3 operations per element instead of the ~11 of a
  // full division.  Quotients that underflow are far below 1/2 and round to 0
  // either way; a scale below 2^-64 (inv near overflow) keeps the division.
  const bool markstein = div >= 0x1p-64f;  // uniform across the workgroup
  const float inv = 1.0f / div;            // IEEE division
  const auto quant = [&](float q) {
    const float r = fminf(fmaxf(rintf(q), -127.0f), 127.0f);  // ties to even
    return static_cast<uint32_t>(static_cast<int>(r)) & 0xFFu;
  };
  const auto store_all = [&](auto quotient) {
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int b = wave + i * nw;
      if (b < nblocks) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint32_t word = 0;
#pragma unroll
          for (int d = 0; d < 4; ++d) word |= quant(quotient(v[i][4 * c + d])) << (8 * d);
          *reinterpret_cast<uint32_t*>(yr + b * kBlock + 256 * c + 4 * lane) = word;
        }
      }
    }
  };
  // the test is hoisted out of the element loop (one branch per token)
  if (markstein)
    store_all([&](float w) {
      const float q0 = w * inv;
      return __builtin_fmaf(__builtin_fmaf(-q0, div, w), inv, q0);
    });
  else
    store_all([&](float w) { return w / div; });
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
