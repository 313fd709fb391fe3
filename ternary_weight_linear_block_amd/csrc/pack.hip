// pack_ternary: load-time conversion of {-1,0,+1} codes and fp16 group scales
// into the library's weight format.
//
// Method ([P1] "Ternary-Bonsai-2-27B on 2x RTX 5070 with vLLM TP=2",
// Prerequisites and section 4): each row n has an fp16 scale s[n,g] per
// 128-element group; it is split into the row maximum smax[n] and an 8-bit
// ratio q[n,g] = round(127 s[n,g] / smax[n]) so that code * q fits int8.
// Here smax = max_g |s| kept exactly in fp32, 127*s is exact in fp32 (an
// 11-bit significand times a 7-bit integer), one correctly rounded fp32
// division follows and rintf rounds ties to even.
//
// 2-bit format (this library's choice; the pages fix only "2 bits per code"):
// field u = 0 for -1, 1 for +1, 2 for 0; within a row, code k = 16w + 4i + b
// sits in bits [8b + 2i, 8b + 2i + 1] of little-endian 32-bit word w.  With
// this interleave an AND (and one shared shift) turns a word into four bytes
// holding the fields of four consecutive k, and the field values double as
// byte-permute selectors: fields at bits 0-1 select bytes {0,1,2} of a
// {-q, +q, 0} table, fields at bits 2-3 (selectors {0,4,8}) pick -q, +q or the
// permute's sign-fill byte, which is 0 -- so the GEMM and GEMV expand 16 codes
// into 16 bytes of code*q with 9 ALU operations.
//
// Tiled layout: the 32 bytes (8 words) of each row and 128-group are stored in
// 2048-byte tiles of 64 rows x one group; tile (r, g) starts at byte
// (r * K/128 + g) * 2048 and holds rows 64r .. 64r + 63 in order.  A decode
// wave that owns 64 rows then reads one contiguous 2 KB tile per group, and a
// GEMM stage's weight slice is a few contiguous tiles.  The buffer has
// ceil(N/64) row blocks; rows past N are padding with code 0 (byte 0xAA).
//
// One workgroup per row (padding rows included): the scale reduction, the q
// row and the packed row are produced together.  The pass is HBM bound
// (K + K/4 + K/64 bytes per row).
#include "twl_internal.h"

namespace twl {
namespace {

__device__ __forceinline__ float fp16_bits_to_float(uint16_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, bits));
}

__global__ __launch_bounds__(256) void pack_kernel(const int8_t* __restrict__ code,
                                                   const uint16_t* __restrict__ s, int N, int K,
                                                   uint8_t* __restrict__ packed,
                                                   int8_t* __restrict__ q,
                                                   float* __restrict__ smax,
                                                   int32_t* __restrict__ bad_codes) {
  const int n = blockIdx.x;  // 0 .. ceil(N/64) * 64 - 1
  const int tid = threadIdx.x;
  const int G = K >> 7;
  uint8_t* tile_row = packed + static_cast<size_t>(n >> 6) * G * 2048 + (n & 63) * 32;

  if (n >= N) {  // padding row of the last row block: code 0 everywhere
    for (int w = tid; w < (K >> 4); w += 256)
      *reinterpret_cast<uint32_t*>(tile_row + static_cast<size_t>(w >> 3) * 2048 + (w & 7) * 4) =
          0xAAAAAAAAu;
    return;
  }

  const uint16_t* sr = s + static_cast<size_t>(n) * G;
  // smax[n] = max_g |s[n,g]|
  float m = 0.0f;
  for (int g = tid; g < G; g += 256) m = fmaxf(m, fabsf(fp16_bits_to_float(sr[g])));
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) m = fmaxf(m, __shfl_xor(m, sh));
  __shared__ float wmax[4];
  __shared__ int wbad[4];
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  const float rmax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  if (tid == 0) smax[n] = rmax;

  // q[n,g] = rint(fl32(127 s) / smax), 0 for an all-zero row
  int8_t* qr = q + static_cast<size_t>(n) * G;
  for (int g = tid; g < G; g += 256) {
    float r = 0.0f;
    if (rmax > 0.0f) r = rintf((127.0f * fp16_bits_to_float(sr[g])) / rmax);
    qr[g] = static_cast<int8_t>(static_cast<int>(r));
  }

  // 2-bit packing, one 16-code word per thread iteration; word w of the row is
  // word w % 8 of its row slot in tile (n / 64, w / 8)
  const int8_t* cr = code + static_cast<size_t>(n) * K;
  int nbad = 0;
  for (int w = tid; w < (K >> 4); w += 256) {
    const uint4 c = *reinterpret_cast<const uint4*>(cr + 16 * w);
    const uint32_t d[4] = {c.x, c.y, c.z, c.w};
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t di = d[i];  // bytes: codes k = 16w + 4i + b, b = 0..3
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t byte = (di >> (8 * b)) & 0xFFu;
        if (!(byte == 0x00u || byte == 0x01u || byte == 0xFFu)) {
          ++nbad;
          di &= ~(0xFFu << (8 * b));  // an invalid code packs as 0
        }
      }
      // per byte: code + 1 (0xFF -> 0, 0x00 -> 1, 0x01 -> 2) without carries
      // between bytes, then swap the two bits: field 0 = -1, 1 = +1, 2 = 0
      const uint32_t c1 = ((di & 0x7F7F7F7Fu) + 0x01010101u) & 0x03030303u;
      const uint32_t u = ((c1 & 0x01010101u) << 1) | ((c1 >> 1) & 0x01010101u);
      word |= u << (2 * i);
    }
    *reinterpret_cast<uint32_t*>(tile_row + static_cast<size_t>(w >> 3) * 2048 + (w & 7) * 4) = word;
  }

  if (bad_codes != nullptr) {
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) nbad += __shfl_xor(nbad, sh);
    if ((tid & 63) == 0) wbad[tid >> 6] = nbad;
    __syncthreads();
    if (tid == 0) {
      const int total = wbad[0] + wbad[1] + wbad[2] + wbad[3];
      if (total) atomicAdd(bad_codes, total);
    }
  }
}

}  // namespace

hipError_t launch_pack(const int8_t* code, const uint16_t* s, int64_t N, int64_t K,
                       uint8_t* packed, int8_t* q, float* smax, int32_t* bad_codes,
                       hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int64_t rows = (N + 63) / 64 * 64;
  hipLaunchKernelGGL(pack_kernel, dim3(static_cast<unsigned>(rows)), dim3(256), 0, stream, code, s,
                     static_cast<int>(N), static_cast<int>(K), packed, q, smax, bad_codes);
  return hipGetLastError();
}

}  // namespace twl
