// Microbenchmark kernels for the measured peaks the benchmark reports beside
// the MI355X spec peaks (libtwl_peaks.so; not part of the ternary-linear C ABI
// and not used by it).
//
//   twl_peak_mfma_i8   back-to-back v_mfma_i32_32x32x32_i8 on ten independent
//                      accumulators per wave (the GEMM's instruction, no
//                      memory traffic): the int8 matrix-core rate this part
//                      sustains.
//   twl_peak_read      a nontemporal 16-byte-per-lane read of a buffer, each
//                      workgroup streaming one contiguous chunk: the HBM read
//                      rate, and at the decode weight size (22.3 MB) the time
//                      floor of one streaming call.
//   twl_peak_mix_i8    the prefill GEMM's MFMA + 2-bit unpack instruction mix
//                      without memory traffic, each unpacked operand feeding
//                      2 or 4 MFMAs: the rate that mix sustains.
//   twl_peak_dot4      chains of v_dot4_i32_iu8 on eight independent
//                      accumulators per lane: the VALU int8 dot-product rate.
//
// Every kernel folds its results into one value and stores it only if it
// equals a constant that it cannot take, so nothing is optimised away and
// nothing is written in practice.  Launch errors are returned as hipError_t.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfmaAcc = 10;  // independent accumulators per wave

__global__ __launch_bounds__(256) void peak_mfma_kernel(int iters, int* sink) {
  const int lane = threadIdx.x & 63;
  v16i acc[kMfmaAcc];
#pragma unroll
  for (int i = 0; i < kMfmaAcc; ++i) acc[i] = v16i{0};
  const v4i a0 = {lane, lane + 1, lane + 2, lane + 3};
  const v4i a1 = {lane ^ 5, lane ^ 9, lane ^ 3, lane ^ 7};
  const v4i b0 = {lane * 3, lane * 5, lane * 7, lane * 9};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kMfmaAcc; ++i)
      acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(i & 1 ? a1 : a0, b0, acc[i], 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int i = 0; i < kMfmaAcc; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s ^= acc[i][r];
  if (s == 0x7FFFFFF1) sink[0] = s;
}

template <int U>
__global__ __launch_bounds__(256) void peak_read_kernel(const u32x4* __restrict__ p, size_t per_wg16,
                                                        size_t total16, unsigned* sink) {
  const size_t base = static_cast<size_t>(blockIdx.x) * per_wg16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t i = threadIdx.x; i < per_wg16; i += static_cast<size_t>(blockDim.x) * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t j = i + static_cast<size_t>(u) * blockDim.x;
      const size_t g = base + j;
      v[u] = (j < per_wg16 && g < total16) ? __builtin_nontemporal_load(p + g) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  const unsigned s = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (s == 0x7FFFFFF1u) sink[0] = s;
}

__global__ __launch_bounds__(256) void peak_dot4_kernel(int iters, int* sink) {
  const int lane = threadIdx.x & 63;
  int acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = lane + i;
  const int a = 0x01020304 * (lane + 1), b = 0x05060708 ^ lane;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_sdot4(a ^ i, b, acc[i], false);
  }
  int s = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) s ^= acc[i];
  if (s == 0x7FFFFFF1) sink[0] = s;
}

// The GEMM's inner instruction mix without memory traffic: per column
// fragment one packed word unpacked to 16 int8 weights by the 9-operation
// permute sequence (1 shift, 4 ANDs, 4 v_perm_b32 against {-q, +q, 0}
// tables), feeding RM MFMAs (one per row fragment), RN column fragments per
// wave, WPS waves per SIMD.  The word rotates every iteration so the unpack
// is not hoisted.  Gives the int8 rate this part sustains when each unpacked
// operand is reused RM times, with the clock the mix runs at.
__device__ __forceinline__ v4i mix_unpack(uint32_t w, uint32_t ta, uint32_t tb0, uint32_t tb1) {
  const uint32_t w4 = w >> 4;
  v4i b;
  b.x = static_cast<int>(__builtin_amdgcn_perm(0u, ta, w & 0x03030303u));
  b.y = static_cast<int>(__builtin_amdgcn_perm(tb0, tb1, w & 0x0C0C0C0Cu));
  b.z = static_cast<int>(__builtin_amdgcn_perm(0u, ta, w4 & 0x03030303u));
  b.w = static_cast<int>(__builtin_amdgcn_perm(tb0, tb1, w4 & 0x0C0C0C0Cu));
  return b;
}

template <int RM, int RN, int WPS>
__global__ __launch_bounds__(256 * WPS, 1) void peak_mix_kernel(int iters, int* sink) {
  const int lane = threadIdx.x & 63;
  v16i acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j) acc[i][j] = v16i{0};
  v4i a[RM];
#pragma unroll
  for (int i = 0; i < RM; ++i) a[i] = v4i{lane + i, lane * 3 + i, lane ^ (5 + i), lane + 11 * i};
  uint32_t w[RN], ta[RN], tb0[RN], tb1[RN];
#pragma unroll
  for (int j = 0; j < RN; ++j) {
    w[j] = 0x9E3779B9u * static_cast<uint32_t>(lane + 7 * j + 1);
    const uint32_t q = static_cast<uint32_t>(17 + 9 * j), neg = 0u - q;
    ta[j] = __builtin_amdgcn_perm(q, neg, 0x0C0C0400u);
    tb0[j] = q;
    tb1[j] = __builtin_amdgcn_perm(0u, neg, 0x0C0C0C00u);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < RN; ++j) {
      const v4i b = mix_unpack(w[j], ta[j], tb0[j], tb1[j]);
      w[j] = __builtin_amdgcn_alignbit(w[j], w[j], 3);
#pragma unroll
      for (int i = 0; i < RM; ++i) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b, acc[i][j], 0, 0, 0);
    }
  }
  int s = 0;
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s ^= acc[i][j][r];
  if (s == 0x7FFFFFF1) sink[0] = s;
}

}  // namespace

extern "C" {

// The GEMM's MFMA + unpack mix (no memory traffic).  reuse 2: 2 row
// fragments x 3 column fragments per wave, 3 waves per SIMD (the 12-wave
// prefill tile); reuse 4: 4 x 2, 2 waves per SIMD.  One workgroup per CU.
// Operations of one call: 2 * 32^3 * (row x column fragments) * iters per
// wave, 4 * WPS waves per workgroup.
int twl_peak_mix_i8(int reuse, int workgroups, int iters, int* sink, hipStream_t stream) {
  if (workgroups <= 0 || iters <= 0 || sink == nullptr || (reuse != 2 && reuse != 4))
    return static_cast<int>(hipErrorInvalidValue);
  if (reuse == 2)
    hipLaunchKernelGGL((peak_mix_kernel<2, 3, 3>), dim3(static_cast<unsigned>(workgroups)), dim3(768), 0,
                       stream, iters, sink);
  else
    hipLaunchKernelGGL((peak_mix_kernel<4, 2, 2>), dim3(static_cast<unsigned>(workgroups)), dim3(512), 0,
                       stream, iters, sink);
  return static_cast<int>(hipGetLastError());
}

// Operations of one call: 2 * 32 * 32 * 32 * 10 * iters per wave, 4 waves per
// workgroup (one per SIMD).
int twl_peak_mfma_i8(int workgroups, int iters, int* sink, hipStream_t stream) {
  if (workgroups <= 0 || iters <= 0 || sink == nullptr) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(peak_mfma_kernel, dim3(static_cast<unsigned>(workgroups)), dim3(256), 0, stream,
                     iters, sink);
  return static_cast<int>(hipGetLastError());
}

// Reads `bytes` (a multiple of 16) from `buf` with `workgroups` workgroups of
// 256 threads, each streaming one contiguous chunk.
int twl_peak_read(const void* buf, size_t bytes, int workgroups, unsigned* sink, hipStream_t stream) {
  if (buf == nullptr || bytes == 0 || bytes % 16 != 0 || workgroups <= 0 || sink == nullptr)
    return static_cast<int>(hipErrorInvalidValue);
  const size_t total16 = bytes / 16;
  const size_t per = (total16 + workgroups - 1) / workgroups;
  hipLaunchKernelGGL(peak_read_kernel<4>, dim3(static_cast<unsigned>(workgroups)), dim3(256), 0, stream,
                     static_cast<const u32x4*>(buf), per, total16, sink);
  return static_cast<int>(hipGetLastError());
}

// Operations of one call: 8 (4 multiply-adds) * 8 * iters per lane.
int twl_peak_dot4(int workgroups, int iters, int* sink, hipStream_t stream) {
  if (workgroups <= 0 || iters <= 0 || sink == nullptr) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(peak_dot4_kernel, dim3(static_cast<unsigned>(workgroups)), dim3(256), 0, stream,
                     iters, sink);
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
