// Internal launchers of the ternary linear library (not part of the C ABI).
// Every launcher assumes the host wrapper in api.cpp has already validated
// pointers, alignment and shapes; they only pick a configuration and launch.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace twl {

// Per-device facts the launchers need (cached by api.cpp).
struct DeviceInfo {
  int cu_count = 0;
};

hipError_t launch_rotate_quant(const uint16_t* x, const int8_t* sign, int64_t M, int64_t K,
                               int8_t* x_i8, float* a_scale, hipStream_t stream);
// The rotation alone: r [M, K] as bf16 bit patterns.
hipError_t launch_rotate_bf16(const uint16_t* x, const int8_t* sign, int64_t M, int64_t K,
                              uint16_t* r, hipStream_t stream);
// Exact-dequant bf16 reference linear: y = r_bf16 . (code * bf16(s))^T in fp32.
hipError_t launch_reference_bf16(const uint16_t* r, const uint8_t* packed, const uint16_t* s,
                                 int64_t M, int64_t N, int64_t K, float* y, hipStream_t stream);
// gate_up: bf16 [M, 2K]; rotates bf16(SiLU(gate) * up).
hipError_t launch_silu_mul_rotate_quant(const uint16_t* gate_up, const int8_t* sign, int64_t M,
                                        int64_t K, int8_t* x_i8, float* a_scale,
                                        hipStream_t stream);

hipError_t launch_pack(const int8_t* code, const uint16_t* s, int64_t N, int64_t K,
                       uint8_t* packed, int8_t* q, float* smax, int32_t* bad_codes,
                       hipStream_t stream);

// What the linear layer writes: fp32 y, the raw int32 accumulators, or y
// rounded to bf16 (round to nearest even).
enum OutKind { kOutF32 = 0, kOutAcc = 1, kOutBf16 = 2 };

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Stores one epilogue value v (y before rounding) or the accumulator s at
// element o of `out`, whose type follows `kind`.
__device__ __forceinline__ void store_out(void* out, size_t o, int kind, int32_t s, float v) {
  if (kind == kOutAcc)
    static_cast<int32_t*>(out)[o] = s;
  else if (kind == kOutBf16)
    static_cast<uint16_t*>(out)[o] = f32_to_bf16_rne(v);
  else
    static_cast<float*>(out)[o] = v;
}

hipError_t launch_gemm(const int8_t* x_i8, const float* a_scale, const uint8_t* packed,
                       const int8_t* q, const float* smax, int64_t M, int64_t N, int64_t K,
                       void* out, OutKind out_kind, void* workspace, size_t workspace_bytes,
                       const DeviceInfo& dev, hipStream_t stream);
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, const DeviceInfo& dev);
// The GEMM plan for this shape, as twl_plan_info reports it (info[0..7]).
void gemm_plan_info(int64_t M, int64_t N, int64_t K, const DeviceInfo& dev, int64_t* info);

// Decode kernels (M <= 24): kGemvAuto picks by M, kGemvDot4 / kGemvMfma force
// one.  When K is split across workgroups (gemv_workspace_bytes > 0) the
// kernel writes int32 partial sums to `part` (at least that many bytes).
enum GemvKind { kGemvAuto = 0, kGemvDot4 = 1, kGemvMfma = 2 };
hipError_t launch_gemv(const int8_t* x_i8, const float* a_scale, const uint8_t* packed,
                       const int8_t* q, const float* smax, int64_t M, int64_t N, int64_t K,
                       void* out, OutKind out_kind, void* part, size_t part_bytes, GemvKind kind,
                       const DeviceInfo& dev, hipStream_t stream);
size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, GemvKind kind, const DeviceInfo& dev);
// The decode plan for this shape, as twl_plan_info reports it (info[0..7]).
void gemv_plan_info(int64_t M, int64_t N, int64_t K, GemvKind kind, const DeviceInfo& dev, int64_t* info);

// Fused decode: rotate_quant_act (silu: of bf16(SiLU(gate) * up), x being
// [gate | up] [M, 2K]) and the row-balanced decode kernel in one launch, which
// also writes x_i8 [M, K] and a_scale [M].  gemv_rot_applies tells whether the
// shape fits it; launch_gemv_rot returns hipErrorNotSupported otherwise.
bool gemv_rot_applies(int64_t M, int64_t N, int64_t K, const DeviceInfo& dev);
hipError_t launch_gemv_rot(const uint16_t* x, const int8_t* sign, bool silu, const uint8_t* packed,
                           const int8_t* q, const float* smax, int64_t M, int64_t N, int64_t K,
                           void* out, OutKind out_kind, int8_t* x_i8, float* a_scale,
                           const DeviceInfo& dev, hipStream_t stream);

}  // namespace twl
