// Building blocks of rotate_quant_act: the signed block-1024 Sylvester
// Hadamard rotation of one block held by one wave, and the per-token int8
// quantiser.  Shared by rotate_quant_kernel (one workgroup per token) and the
// fused decode kernel that rotates its few tokens itself, so that both compute
// the same operations in the same order and agree bit for bit.
//
// Method ([P1] "Ternary-Bonsai-2-27B on 2x RTX 5070 with vLLM TP=2",
// Prerequisites, section 1 and section 4): the input side of every ternary
// linear carries a block-wise Hadamard rotation whose sign table is keyed by
// the full input width; after rotating, activations are quantised to int8 with
// one scale per token.  Section 1 fixes the recursion
// H1024 [a; b] = [H512 a + H512 b ; H512 a - H512 b], i.e. the last butterfly
// stage combines the two 512-halves, so stages run h = 1, 2, ..., 512.
//
// A block lives in registers, 16 elements per lane, and every butterfly runs
// inside a lane: the element index e (10 bits) is split between lane and
// register slot three times, with two LDS transposes in between (per-wave
// buffer of kWaveBufWords floats, padded to be bank-conflict free):
//   layout 0: lane = e[9:4],            slot = e[3:0]  -> stages h = 1 .. 8
//   layout 1: lane = e[9:8] e[3:0],     slot = e[7:4]  -> stages h = 16 .. 128
//   layout 2: lane = e[7:2],            slot = e[9:8] e[1:0] -> stages h = 256, 512
// so the pass has no cross-lane arithmetic at all.  In layout 2 a lane holds
// four runs of 4 consecutive elements (slot 4 c + d = element 256 c + 4 lane + d).
//
// Every butterfly is (lo, hi) -> (lo + hi, lo - hi) in fp32 with the same
// operands as a textbook in-place FWHT and in the same stage order, so the
// result is bit-identical to any implementation that follows that order; the
// build uses -ffp-contract=off so no add is fused with anything.
#pragma once

#include "twl_internal.h"

namespace twl {
namespace rot {

constexpr int kBlock = 1024;
constexpr int kWaveBufWords = 1344;  // > max addr_a (1323) and addr_b (1071)

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

__device__ __forceinline__ void wave_lds_sync() {
  // LDS operations of one wave execute in order; the fences only keep the
  // compiler from moving reads above the writes they depend on (or the next
  // writes above these reads)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The raw input of one block for one lane (layout 0: elements 16 lane ..
// 16 lane + 15 of the block): 16 bf16 values of x (with SILU the gate, and up
// in `u`) and their 16 signs.
struct BlockIn {
  uint32_t x[8];
  uint32_t u[8];
  uint32_t s[4];
};

// Loads block b (elements 1024 b .. 1024 b + 1023) of one token: xr is the
// token's row (bf16 bits; with SILU the row of [gate | up], gate = elements
// 0..K-1), sign the int8 +-1 table of the full width.
template <bool SILU>
__device__ __forceinline__ BlockIn load_block(const uint16_t* __restrict__ xr, const int8_t* __restrict__ sign,
                                              int K, int b, int lane) {
  const int k0 = b * kBlock + lane * 16;
  const uint4 p0 = *reinterpret_cast<const uint4*>(xr + k0);
  const uint4 p1 = *reinterpret_cast<const uint4*>(xr + k0 + 8);
  const uint4 sg = *reinterpret_cast<const uint4*>(sign + k0);
  BlockIn in = {{p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w}, {}, {sg.x, sg.y, sg.z, sg.w}};
  if (SILU) {
    const uint4 u0 = *reinterpret_cast<const uint4*>(xr + K + k0);
    const uint4 u1 = *reinterpret_cast<const uint4*>(xr + K + k0 + 8);
    const uint32_t uw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) in.u[e] = uw[e];
  }
  return in;
}

// load_block with the SiLU form chosen at run time and no branch: `up` is
// the offset of the up half in the row (K), or 0 without it (`u` then holds a
// second copy of x, which rotate_loaded<false> does not read).
__device__ __forceinline__ BlockIn load_block_rt(const uint16_t* __restrict__ xr, const int8_t* __restrict__ sign,
                                                 int up, int b, int lane) {
  const int k0 = b * kBlock + lane * 16;
  const uint4 p0 = *reinterpret_cast<const uint4*>(xr + k0);
  const uint4 p1 = *reinterpret_cast<const uint4*>(xr + k0 + 8);
  const uint4 u0 = *reinterpret_cast<const uint4*>(xr + up + k0);
  const uint4 u1 = *reinterpret_cast<const uint4*>(xr + up + k0 + 8);
  const uint4 sg = *reinterpret_cast<const uint4*>(sign + k0);
  return BlockIn{{p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w},
                 {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w},
                 {sg.x, sg.y, sg.z, sg.w}};
}

// The rotation of one loaded block by one wave (with SILU the rotated input
// is bf16(SiLU(gate) * up)); wb is this wave's transpose buffer
// (kWaveBufWords floats).  On return w holds (1/32) H1024 (sign . x) of the
// block in layout 2.
template <bool SILU>
__device__ __forceinline__ void rotate_loaded(const BlockIn& in, int lane, float* wb, float (&w)[16]) {
  // layout-1 lane bits: e[9:8] = lane >> 4, e[3:0] = lane & 15
  const int l1_hi = lane >> 4, l1_lo = lane & 15;
  uint32_t pw[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    pw[e] = SILU ? silu_mul_bits(in.x[e] & 0xFFFFu, in.u[e] & 0xFFFFu) |
                       (silu_mul_bits(in.x[e] >> 16, in.u[e] >> 16) << 16)
                 : in.x[e];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t bits = (pw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
    // multiply by the +-1 sign: flip the fp32 sign bit when the int8 sign is negative
    const uint32_t flip = ((in.s[e >> 2] >> (8 * (e & 3) + 7)) & 1u) << 31;
    w[e] = __uint_as_float(__float_as_uint(bf16_bits_to_float(bits)) ^ flip);
  }
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) stage_in_lane(w, sb);  // h = 1, 2, 4, 8

  // transpose to layout 1: slot s holds e = 256 l1_hi + 16 s + l1_lo
  wave_lds_sync();
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<float4*>(wb + addr_a(16 * lane + 4 * q)) =
        make_float4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
  wave_lds_sync();
#pragma unroll
  for (int sl = 0; sl < 16; ++sl) w[sl] = wb[addr_a(256 * l1_hi + 16 * sl + l1_lo)];
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) stage_in_lane(w, sb);  // h = 16, 32, 64, 128

  // transpose to layout 2: slot 4 c + d holds e = 256 c + 4 lane + d
  wave_lds_sync();
#pragma unroll
  for (int sl = 0; sl < 16; ++sl) wb[addr_b(256 * l1_hi + 16 * sl + l1_lo)] = w[sl];
  wave_lds_sync();
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
  for (int e = 0; e < 16; ++e) w[e] *= 0.03125f;  // orthonormal 1/sqrt(1024): exact power of two
}

// Block b of one token, loaded and rotated by one wave (see load_block and
// rotate_loaded).
template <bool SILU>
__device__ __forceinline__ void rotate_block(const uint16_t* __restrict__ xr, const int8_t* __restrict__ sign,
                                             int K, int b, int lane, float* wb, float (&w)[16]) {
  rotate_loaded<SILU>(load_block<SILU>(xr, sign, K, b, lane), lane, wb, w);
}

// The int8 quantiser of one token, given its absmax over the whole row:
// a_scale = absmax / 127 (IEEE division), x_i8 = clamp(rint(r / a_scale), +-127)
// with ties to even.  A zero scale (all-zero row, or an absmax so small that
// absmax / 127 underflows) quantises every element to 0: dividing by 1
// instead gives rint(|v| <= tiny) = 0 without a branch per element.
//
// The quotient v / div must be the IEEE-rounded one.  With inv = RN(1 / div),
// one IEEE division per token, q0 = RN(v inv) is within one ulp of v / div, the
// residual v - q0 div is exact in one fma, and RN(q0 + residual * inv) is the
// correctly rounded quotient (Markstein's theorem), as long as nothing
// overflows or underflows: 3 operations per element instead of the ~11 of a
// full division.  Quotients that underflow are far below 1/2 and round to 0
// either way; a scale below 2^-64 (inv near overflow) keeps the division.
struct TokenQuant {
  float scale;     // a_scale of the token
  float div, inv;
  bool markstein;  // uniform for the token
};

__device__ __forceinline__ TokenQuant token_quant(float absmax) {
  TokenQuant t;
  t.scale = absmax / 127.0f;  // IEEE division
  t.div = t.scale > 0.0f ? t.scale : 1.0f;
  t.markstein = t.div >= 0x1p-64f;
  t.inv = 1.0f / t.div;  // IEEE division
  return t;
}

// rint and clamp of a quotient, as the int8 byte
__device__ __forceinline__ uint32_t quant_byte(float q) {
  const float r = fminf(fmaxf(rintf(q), -127.0f), 127.0f);  // ties to even
  return static_cast<uint32_t>(static_cast<int>(r)) & 0xFFu;
}

__device__ __forceinline__ float quotient_markstein(float w, const TokenQuant& t) {
  const float q0 = w * t.inv;
  return __builtin_fmaf(__builtin_fmaf(-q0, t.div, w), t.inv, q0);
}

// Layout-2 run c of a lane (elements 256 c + 4 lane .. + 3) as one dword of
// four int8 values, low element first.
__device__ __forceinline__ uint32_t quant_run(const float (&w)[16], int c, const TokenQuant& t) {
  uint32_t word = 0;
  if (t.markstein) {
#pragma unroll
    for (int d = 0; d < 4; ++d) word |= quant_byte(quotient_markstein(w[4 * c + d], t)) << (8 * d);
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) word |= quant_byte(w[4 * c + d] / t.div) << (8 * d);
  }
  return word;
}

}  // namespace rot
}  // namespace twl
