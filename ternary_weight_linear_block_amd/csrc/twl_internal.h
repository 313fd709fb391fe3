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

hipError_t launch_pack(const int8_t* code, const uint16_t* s, int64_t N, int64_t K,
                       uint8_t* packed, int8_t* q, float* smax, int32_t* bad_codes,
                       hipStream_t stream);

// out is float* (y) when out_acc is false, int32_t* (acc) otherwise.
hipError_t launch_gemm(const int8_t* x_i8, const float* a_scale, const uint8_t* packed,
                       const int8_t* q, const float* smax, int64_t M, int64_t N, int64_t K,
                       void* out, bool out_acc, void* workspace, size_t workspace_bytes,
                       const DeviceInfo& dev, hipStream_t stream);
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, const DeviceInfo& dev);

// Decode kernels (M <= 24): kGemvAuto picks by M, kGemvDot4 / kGemvMfma force
// one.  When K is split across workgroups (gemv_workspace_bytes > 0) the
// kernel writes int32 partial sums to `part` (at least that many bytes).
enum GemvKind { kGemvAuto = 0, kGemvDot4 = 1, kGemvMfma = 2 };
hipError_t launch_gemv(const int8_t* x_i8, const float* a_scale, const uint8_t* packed,
                       const int8_t* q, const float* smax, int64_t M, int64_t N, int64_t K,
                       void* out, bool out_acc, void* part, size_t part_bytes, GemvKind kind,
                       const DeviceInfo& dev, hipStream_t stream);
size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, GemvKind kind, const DeviceInfo& dev);

}  // namespace twl
