// Host-only driver for the C ABI's validation and status mapping (api.cpp),
// built with AddressSanitizer and UndefinedBehaviorSanitizer and run on the
// CPU.  Nothing here touches a GPU: the few HIP runtime calls api.cpp makes
// (hipGetDevice, hipGetDeviceProperties, hipGetErrorString,
// hipGetSymbolAddress) and the kernel launchers it dispatches to are replaced
// by the stubs below, so a launch failure, a wrong device or a failing
// runtime call can be forced from the host and the returned status checked.
//
// Exit status 0 when every check passes; each failure prints one line.
#include "twl.h"
#include "twl_internal.h"

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

namespace {

int g_failures = 0;

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::printf("FAIL %s:%d: %s (last error: %s)\n", __FILE__, __LINE__, #cond, twl_last_error()); \
      ++g_failures;                                                   \
    }                                                                 \
  } while (0)

// stub state: which device hipGetDevice reports, whether it fails, which
// architecture each device reports, what the launchers return
int g_device = 0;
hipError_t g_get_device_status = hipSuccess;
const char* g_arch[4] = {"gfx950", "gfx942:sramecc+:xnack-", "gfx950", "gfx950"};
hipError_t g_launch_status = hipSuccess;
int g_launches = 0;
size_t g_gemm_ws = 0;   // what the stubbed planners report as workspace need
size_t g_gemv_ws = 0;
// arguments the last stubbed launcher received
int64_t g_last_m = -1, g_last_n = -1, g_last_k = -1;
int g_last_kind = -1;
const void* g_last_ws = nullptr;
// the no-allocation entry point's scratch lookup
hipError_t g_symbol_status = hipSuccess;
int g_symbol_lookups = 0;
alignas(256) unsigned char g_fake_scratch_mem[256];
void* g_fake_scratch = g_fake_scratch_mem;
// whether the fused rotation + decode kernel applies (stubbed planner)
bool g_rot_applies = false;

}  // namespace

// ---- stubbed HIP runtime (the only runtime symbols api.cpp uses)
extern "C" {
hipError_t hipGetDevice(int* dev) {
  if (g_get_device_status != hipSuccess) return g_get_device_status;
  *dev = g_device;
  return hipSuccess;
}
hipError_t hipGetDeviceProperties(hipDeviceProp_t* prop, int dev) {
  std::memset(prop, 0, sizeof *prop);
  if (dev < 0 || dev >= 4) return hipErrorInvalidDevice;
  std::snprintf(prop->gcnArchName, sizeof prop->gcnArchName, "%s", g_arch[dev]);
  prop->multiProcessorCount = 256;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t e) {
  return e == hipSuccess ? "hipSuccess" : "stubbed HIP error";
}
hipError_t hipGetSymbolAddress(void** p, const void*) {
  ++g_symbol_lookups;
  if (g_symbol_status != hipSuccess) return g_symbol_status;
  *p = g_fake_scratch;
  return hipSuccess;
}
}

// ---- stubbed launchers and planners (the kernels are not built here)
namespace twl {
static hipError_t record(int64_t M, int64_t N, int64_t K, int kind, const void* ws) {
  ++g_launches;
  g_last_m = M;
  g_last_n = N;
  g_last_k = K;
  g_last_kind = kind;
  g_last_ws = ws;
  return g_launch_status;
}
hipError_t launch_rotate_quant(const uint16_t*, const int8_t*, int64_t M, int64_t K, int8_t*, float*,
                               hipStream_t) {
  return record(M, 0, K, -1, nullptr);
}
hipError_t launch_rotate_bf16(const uint16_t*, const int8_t*, int64_t M, int64_t K, uint16_t*, hipStream_t) {
  return record(M, 0, K, -1, nullptr);
}
hipError_t launch_reference_bf16(const uint16_t*, const uint8_t*, const uint16_t*, int64_t M, int64_t N,
                                 int64_t K, float*, hipStream_t) {
  return record(M, N, K, -1, nullptr);
}
hipError_t launch_silu_mul_rotate_quant(const uint16_t*, const int8_t*, int64_t M, int64_t K, int8_t*, float*,
                                        hipStream_t) {
  return record(M, 0, K, -2, nullptr);
}
hipError_t launch_pack(const int8_t*, const uint16_t*, int64_t N, int64_t K, uint8_t*, int8_t*, float*,
                       int32_t*, hipStream_t) {
  return record(0, N, K, -1, nullptr);
}
hipError_t launch_gemm(const int8_t*, const float*, const uint8_t*, const int8_t*, const float*, int64_t M,
                       int64_t N, int64_t K, void*, OutKind out_kind, void* ws, size_t, const DeviceInfo& dev,
                       hipStream_t) {
  if (dev.cu_count != 256) return hipErrorInvalidValue;
  return record(M, N, K, 100 + out_kind, ws);
}
size_t gemm_workspace_bytes(int64_t, int64_t, int64_t, const DeviceInfo&) { return g_gemm_ws; }
void gemm_plan_info(int64_t, int64_t, int64_t, const DeviceInfo& dev, int64_t* info) {
  for (int i = 0; i < 8; ++i) info[i] = 1000 + i;
  info[0] = 1;
  info[4] = dev.cu_count;
}
hipError_t launch_gemv(const int8_t*, const float*, const uint8_t*, const int8_t*, const float*, int64_t M,
                       int64_t N, int64_t K, void*, OutKind out_kind, void* ws, size_t, GemvKind kind,
                       const DeviceInfo&, hipStream_t) {
  return record(M, N, K, 200 + 10 * kind + out_kind, ws);
}
size_t gemv_workspace_bytes(int64_t, int64_t, int64_t, GemvKind, const DeviceInfo&) { return g_gemv_ws; }
void gemv_plan_info(int64_t, int64_t, int64_t, GemvKind kind, const DeviceInfo&, int64_t* info) {
  for (int i = 0; i < 8; ++i) info[i] = 2000 + i;
  info[0] = 2 + kind;
}
bool gemv_rot_applies(int64_t, int64_t, int64_t, const DeviceInfo&) { return g_rot_applies; }
hipError_t launch_gemv_rot(const uint16_t*, const int8_t*, bool silu, const uint8_t*, const int8_t*,
                           const float*, int64_t M, int64_t N, int64_t K, void*, OutKind out_kind, int8_t*,
                           float*, const DeviceInfo&, hipStream_t) {
  return record(M, N, K, 300 + 10 * (silu ? 1 : 0) + out_kind, nullptr);
}
}  // namespace twl

namespace {

alignas(16) unsigned char g_buf[4096];
void* P = g_buf;                 // 16-byte aligned, never dereferenced by the stubs
void* P2 = g_buf + 2;            // misaligned

bool msg_has(const char* s) { return std::strstr(twl_last_error(), s) != nullptr; }

void test_validation() {
  auto* x = static_cast<const uint16_t*>(P);
  auto* s8 = static_cast<const int8_t*>(P);
  // shape errors, before any device query or launch
  g_launches = 0;
  CHECK(twl_rotate_quant_act(x, s8, 4, 1000, (int8_t*)P, (float*)P, nullptr) == TWL_ESHAPE);
  CHECK(twl_rotate_quant_act(x, s8, 4, TWL_MAX_K + 1024, (int8_t*)P, (float*)P, nullptr) == TWL_ESHAPE);
  CHECK(twl_rotate_quant_act(x, s8, -1, 1024, (int8_t*)P, (float*)P, nullptr) == TWL_EINVAL);
  CHECK(twl_rotate_quant_act(x, s8, (int64_t{1} << 30) + 1, 1024, (int8_t*)P, (float*)P, nullptr) == TWL_ESHAPE);
  CHECK(twl_rotate_quant_act(nullptr, s8, 4, 1024, (int8_t*)P, (float*)P, nullptr) == TWL_EINVAL);
  CHECK(msg_has("x is NULL"));
  CHECK(twl_rotate_quant_act((const uint16_t*)P2, s8, 4, 1024, (int8_t*)P, (float*)P, nullptr) == TWL_EALIGN);
  CHECK(twl_pack_ternary(s8, x, 8, 1024, (uint8_t*)P, (int8_t*)P, (float*)P, (int32_t*)(g_buf + 1), nullptr) ==
        TWL_EALIGN);
  CHECK(twl_ternary_linear_ex(s8, (float*)P, (uint8_t*)P, s8, (float*)P, 4, 4, 1024, P, 7, 0, nullptr, 0,
                              nullptr) == TWL_EINVAL);
  CHECK(twl_ternary_linear_ex(s8, (float*)P, (uint8_t*)P, s8, (float*)P, 4, 4, 1024, P, 0, 9, nullptr, 0,
                              nullptr) == TWL_EINVAL);
  CHECK(twl_ternary_linear_ex(s8, (float*)P, (uint8_t*)P, s8, (float*)P, 25, 4, 1024, P, 0, TWL_PATH_GEMV,
                              nullptr, 0, nullptr) == TWL_ESHAPE);
  CHECK(g_launches == 0);
  // empty shapes: OK, nothing launched, no device query
  g_get_device_status = hipErrorNoDevice;
  CHECK(twl_rotate_quant_act(nullptr, nullptr, 0, 1024, nullptr, nullptr, nullptr) == TWL_OK);
  CHECK(twl_ternary_linear(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 7, 1024, nullptr, nullptr, 0,
                           nullptr) == TWL_OK);
  CHECK(std::strcmp(twl_last_error(), "") == 0);
  CHECK(g_launches == 0);
  // packed size arithmetic at the limits (no overflow)
  CHECK(twl_packed_bytes(1, 1024) == 64 * 256);
  CHECK(twl_packed_bytes(int64_t{1} << 30, TWL_MAX_K) == (size_t{1} << 30) * (TWL_MAX_K / 4));
  CHECK(twl_packed_bytes((int64_t{1} << 30) + 1, 1024) == 0);
  CHECK(twl_packed_bytes(5, 1000) == 0);
  CHECK(twl_packed_bytes(-5, 1024) == 0);
  g_get_device_status = hipSuccess;
}

void test_status_mapping() {
  auto* x = static_cast<const uint16_t*>(P);
  auto* s8 = static_cast<const int8_t*>(P);
  // a failing runtime query maps to TWL_EHIP
  g_get_device_status = hipErrorNoDevice;
  CHECK(twl_rotate_quant_act(x, s8, 4, 1024, (int8_t*)P, (float*)P, nullptr) == TWL_EHIP);
  CHECK(msg_has("hipGetDevice failed"));
  g_get_device_status = hipSuccess;
  // a device that is not gfx950 maps to TWL_EDEVICE, on first and later calls
  g_device = 1;
  CHECK(twl_rotate_quant_act(x, s8, 4, 1024, (int8_t*)P, (float*)P, nullptr) == TWL_EDEVICE);
  CHECK(msg_has("gfx942"));
  CHECK(twl_pack_ternary(s8, x, 8, 1024, (uint8_t*)P, (int8_t*)P, (float*)P, nullptr, nullptr) == TWL_EDEVICE);
  g_device = 0;
  // a launch failure maps to TWL_EHIP with the call named, for every entry point
  g_launch_status = hipErrorLaunchFailure;
  CHECK(twl_rotate_quant_act(x, s8, 4, 1024, (int8_t*)P, (float*)P, nullptr) == TWL_EHIP);
  CHECK(msg_has("rotate_quant_act launch failed"));
  CHECK(twl_silu_mul_rotate_quant_act(x, s8, 4, 1024, (int8_t*)P, (float*)P, nullptr) == TWL_EHIP);
  CHECK(twl_rotate_act_bf16(x, s8, 4, 1024, (uint16_t*)P, nullptr) == TWL_EHIP);
  CHECK(twl_reference_linear_bf16(x, (uint8_t*)P, x, 4, 8, 1024, (float*)P, nullptr) == TWL_EHIP);
  CHECK(twl_pack_ternary(s8, x, 8, 1024, (uint8_t*)P, (int8_t*)P, (float*)P, nullptr, nullptr) == TWL_EHIP);
  CHECK(twl_ternary_linear(s8, (float*)P, (uint8_t*)P, s8, (float*)P, 64, 8, 1024, (float*)P, nullptr, 0,
                           nullptr) == TWL_EHIP);
  CHECK(msg_has("(GEMM)"));
  CHECK(twl_ternary_linear(s8, (float*)P, (uint8_t*)P, s8, (float*)P, 4, 8, 1024, (float*)P, nullptr, 0,
                           nullptr) == TWL_EHIP);
  CHECK(msg_has("(GEMV)"));
  g_launch_status = hipSuccess;
  // a successful call clears the message
  CHECK(twl_rotate_quant_act(x, s8, 4, 1024, (int8_t*)P, (float*)P, nullptr) == TWL_OK);
  CHECK(std::strcmp(twl_last_error(), "") == 0);
}

void test_dispatch_and_workspace() {
  auto* s8 = static_cast<const int8_t*>(P);
  // M <= 24 goes to the decode kernels, larger M to the GEMM; path overrides
  CHECK(twl_ternary_linear(s8, (float*)P, (uint8_t*)P, s8, (float*)P, 24, 8, 2048, (float*)P, nullptr, 0,
                           nullptr) == TWL_OK);
  CHECK(g_last_kind == 200 + 10 * twl::kGemvAuto + twl::kOutF32 && g_last_m == 24 && g_last_k == 2048);
  CHECK(twl_ternary_linear(s8, (float*)P, (uint8_t*)P, s8, (float*)P, 25, 8, 2048, (float*)P, nullptr, 0,
                           nullptr) == TWL_OK);
  CHECK(g_last_kind == 100 + twl::kOutF32 && g_last_m == 25);
  CHECK(twl_ternary_linear_ex(s8, nullptr, (uint8_t*)P, s8, nullptr, 3, 8, 1024, P, TWL_OUT_ACC_I32,
                              TWL_PATH_GEMV_DOT4, nullptr, 0, nullptr) == TWL_OK);
  CHECK(g_last_kind == 200 + 10 * twl::kGemvDot4 + twl::kOutAcc);
  CHECK(twl_ternary_linear_ex(s8, (float*)P, (uint8_t*)P, s8, (float*)P, 3, 8, 1024, P, TWL_OUT_BF16,
                              TWL_PATH_GEMM, nullptr, 0, nullptr) == TWL_OK);
  CHECK(g_last_kind == 100 + twl::kOutBf16);
  // a needed workspace: missing, too small, misaligned, then given
  g_gemm_ws = 4096;
  CHECK(twl_ternary_linear(s8, (float*)P, (uint8_t*)P, s8, (float*)P, 64, 8, 1024, (float*)P, nullptr, 0,
                           nullptr) == TWL_EINVAL);
  CHECK(msg_has("workspace of 4096 bytes required"));
  CHECK(twl_ternary_linear(s8, (float*)P, (uint8_t*)P, s8, (float*)P, 64, 8, 1024, (float*)P, P, 4095,
                           nullptr) == TWL_EINVAL);
  CHECK(twl_ternary_linear(s8, (float*)P, (uint8_t*)P, s8, (float*)P, 64, 8, 1024, (float*)P, P2, 4096,
                           nullptr) == TWL_EALIGN);
  CHECK(twl_ternary_linear(s8, (float*)P, (uint8_t*)P, s8, (float*)P, 64, 8, 1024, (float*)P, P, 4096,
                           nullptr) == TWL_OK);
  CHECK(g_last_ws == P);
  CHECK(twl_workspace_bytes(64, 8, 1024) == 4096);
  g_gemv_ws = 8192;
  CHECK(twl_workspace_bytes(24, 8, 1024) == 8192);   // the larger of the GEMM's and the decode paths'
  CHECK(twl_workspace_bytes(25, 8, 1024) == 4096);   // no decode path above 24 tokens
  g_gemm_ws = g_gemv_ws = 0;
  // plan queries
  int64_t info[8];
  CHECK(twl_plan_info(512, 17408, 5120, TWL_PATH_AUTO, info) == TWL_OK && info[0] == 1 && info[4] == 256);
  CHECK(twl_plan_info(4, 17408, 5120, TWL_PATH_AUTO, info) == TWL_OK && info[0] == 2 + twl::kGemvAuto);
  CHECK(twl_plan_info(4, 17408, 5120, TWL_PATH_GEMV_DOT4, info) == TWL_OK && info[0] == 2 + twl::kGemvDot4);
  CHECK(twl_plan_info(4, 17408, 5120, TWL_PATH_GEMM, info) == TWL_OK && info[0] == 1);
  CHECK(twl_plan_info(0, 17408, 5120, TWL_PATH_AUTO, info) == TWL_OK && info[0] == 0 && info[7] == 0);
  CHECK(twl_plan_info(4, 8, 5120, TWL_PATH_AUTO, nullptr) == TWL_EINVAL);
  CHECK(twl_plan_info(30, 8, 5120, TWL_PATH_GEMV, info) == TWL_ESHAPE);
  CHECK(twl_plan_info(4, 8, 5000, TWL_PATH_AUTO, info) == TWL_ESHAPE);
}

void test_noalloc() {
  auto* s8 = static_cast<const int8_t*>(P);
  // no scratch needed: no lookup, no workspace passed
  g_device = 2;
  g_gemm_ws = g_gemv_ws = 0;
  g_symbol_lookups = 0;
  CHECK(twl_ternary_linear_noalloc(s8, (float*)P, (uint8_t*)P, s8, (float*)P, 64, 8, 1024, P, TWL_OUT_F32,
                                   TWL_PATH_AUTO, nullptr) == TWL_OK);
  CHECK(g_symbol_lookups == 0 && g_last_ws == nullptr && g_last_kind == 100 + twl::kOutF32);
  // a failing symbol lookup maps to TWL_EHIP and launches nothing
  g_gemm_ws = 4096;
  g_symbol_status = hipErrorInvalidSymbol;
  g_launches = 0;
  CHECK(twl_ternary_linear_noalloc(s8, (float*)P, (uint8_t*)P, s8, (float*)P, 64, 8, 1024, P, TWL_OUT_F32,
                                   TWL_PATH_AUTO, nullptr) == TWL_EHIP);
  CHECK(msg_has("hipGetSymbolAddress") && g_launches == 0);
  // then the scratch's device address is passed as the workspace; looked up
  // once per device
  g_symbol_status = hipSuccess;
  g_symbol_lookups = 0;
  for (int i = 0; i < 3; ++i) {
    CHECK(twl_ternary_linear_noalloc(s8, (float*)P, (uint8_t*)P, s8, (float*)P, 64, 8, 1024, P,
                                     TWL_OUT_ACC_I32, TWL_PATH_GEMM, nullptr) == TWL_OK);
    CHECK(g_last_ws == g_fake_scratch && g_last_kind == 100 + twl::kOutAcc);
  }
  CHECK(g_symbol_lookups == 1);
  g_gemv_ws = 4096;
  CHECK(twl_ternary_linear_noalloc(s8, (float*)P, (uint8_t*)P, s8, (float*)P, 5, 8, 1024, P, TWL_OUT_BF16,
                                   TWL_PATH_GEMV_MFMA, nullptr) == TWL_OK);
  CHECK(g_last_ws == g_fake_scratch && g_last_kind == 200 + 10 * twl::kGemvMfma + twl::kOutBf16);
  // beyond the scratch size: a clear error, nothing launched
  g_launches = 0;
  g_gemm_ws = size_t{TWL_NOALLOC_SCRATCH_BYTES} + 1;
  CHECK(twl_ternary_linear_noalloc(s8, (float*)P, (uint8_t*)P, s8, (float*)P, 64, 8, 1024, P, TWL_OUT_F32,
                                   TWL_PATH_AUTO, nullptr) == TWL_ESHAPE);
  CHECK(msg_has("no-allocation scratch") && g_launches == 0);
  g_gemm_ws = size_t{TWL_NOALLOC_SCRATCH_BYTES};
  CHECK(twl_ternary_linear_noalloc(s8, (float*)P, (uint8_t*)P, s8, (float*)P, 64, 8, 1024, P, TWL_OUT_F32,
                                   TWL_PATH_AUTO, nullptr) == TWL_OK);
  // the same argument checks as twl_ternary_linear_ex
  CHECK(twl_ternary_linear_noalloc(s8, (float*)P, (uint8_t*)P, s8, (float*)P, 64, 8, 1000, P, TWL_OUT_F32,
                                   TWL_PATH_AUTO, nullptr) == TWL_ESHAPE);
  CHECK(twl_ternary_linear_noalloc(s8, nullptr, (uint8_t*)P, s8, (float*)P, 64, 8, 1024, P, TWL_OUT_F32,
                                   TWL_PATH_AUTO, nullptr) == TWL_EINVAL);
  CHECK(twl_ternary_linear_noalloc(s8, (float*)P, (uint8_t*)P, s8, (float*)P, 64, 8, 1024, P2, TWL_OUT_F32,
                                   TWL_PATH_AUTO, nullptr) == TWL_EALIGN);
  g_gemm_ws = g_gemv_ws = 0;
  g_device = 0;
}

// twl_rotate_quant_linear: one fused launch when the (stubbed) planner allows
// it, else the rotation and then the linear layer; every argument and the
// workspace checked before anything is launched
void test_rotate_quant_linear() {
  auto* x = static_cast<const uint16_t*>(P);
  auto* s8 = static_cast<const int8_t*>(P);
  auto* u8 = static_cast<const uint8_t*>(P);
  auto* f = static_cast<float*>(P);
  auto* i8 = static_cast<int8_t*>(P);
  const auto call = [&](int64_t M, int64_t N, int silu, int kind, void* ws, size_t ws_bytes) {
    return twl_rotate_quant_linear(x, s8, u8, s8, f, M, N, 5120, silu, i8, f, P, kind, ws, ws_bytes, nullptr);
  };
  g_device = 0;
  g_launch_status = hipSuccess;
  g_gemm_ws = g_gemv_ws = 0;

  // fused: one launch, with the silu flag and the output kind
  g_rot_applies = true;
  int before = g_launches;
  CHECK(call(1, 17408, 0, TWL_OUT_F32, nullptr, 0) == TWL_OK);
  CHECK(g_launches == before + 1 && g_last_kind == 300 + TWL_OUT_F32 && g_last_m == 1 && g_last_n == 17408);
  CHECK(call(2, 17408, 1, TWL_OUT_BF16, nullptr, 0) == TWL_OK);
  CHECK(g_launches == before + 2 && g_last_kind == 310 + TWL_OUT_BF16);
  CHECK(twl_rotate_quant_linear_fused(1, 17408, 5120) == 1);
  CHECK(twl_rotate_quant_linear_fused(0, 17408, 5120) == 0);
  CHECK(twl_rotate_quant_linear_fused(1, 17408, 1000) == -TWL_ESHAPE);

  // two steps: the rotation (plain or SiLU form), then the decode or GEMM path
  g_rot_applies = false;
  before = g_launches;
  CHECK(call(4, 17408, 0, TWL_OUT_F32, nullptr, 0) == TWL_OK);
  CHECK(g_launches == before + 2 && g_last_kind == 200 + 10 * twl::kGemvAuto + TWL_OUT_F32);
  CHECK(call(100, 17408, 1, TWL_OUT_ACC_I32, nullptr, 0) == TWL_OK);
  CHECK(g_launches == before + 4 && g_last_kind == 100 + TWL_OUT_ACC_I32);
  CHECK(twl_rotate_quant_linear_fused(4, 17408, 5120) == 0);
  // N = 0: the rotation alone
  CHECK(call(4, 0, 1, TWL_OUT_F32, nullptr, 0) == TWL_OK);
  CHECK(g_launches == before + 5 && g_last_kind == -2);

  // a missing workspace is refused before the rotation is enqueued
  g_gemm_ws = 4096;
  before = g_launches;
  CHECK(call(100, 17408, 0, TWL_OUT_F32, nullptr, 0) == TWL_EINVAL && msg_has("workspace"));
  CHECK(call(100, 17408, 0, TWL_OUT_F32, P2, 4096) == TWL_EALIGN);
  CHECK(g_launches == before);
  CHECK(call(100, 17408, 0, TWL_OUT_F32, P, 4096) == TWL_OK);
  CHECK(g_launches == before + 2 && g_last_ws == P);
  g_gemm_ws = 0;

  // a failing launch maps to TWL_EHIP, naming the step; after a failed
  // rotation nothing else is launched
  g_launch_status = hipErrorLaunchFailure;
  g_rot_applies = true;
  CHECK(call(1, 17408, 0, TWL_OUT_F32, nullptr, 0) == TWL_EHIP && msg_has("fused decode"));
  g_rot_applies = false;
  before = g_launches;
  CHECK(call(4, 17408, 0, TWL_OUT_F32, nullptr, 0) == TWL_EHIP && msg_has("rotation"));
  CHECK(g_launches == before + 1);
  g_launch_status = hipSuccess;

  // a device that is not gfx950
  g_device = 1;
  CHECK(call(1, 17408, 0, TWL_OUT_F32, nullptr, 0) == TWL_EDEVICE);
  CHECK(twl_rotate_quant_linear_fused(1, 17408, 5120) == -TWL_EDEVICE);
  g_device = 0;
}

}  // namespace

int main() {
  test_validation();
  test_status_mapping();
  test_dispatch_and_workspace();
  test_noalloc();
  test_rotate_quant_linear();
  if (g_failures == 0) std::printf("abi_driver: all checks passed\n");
  return g_failures == 0 ? 0 : 1;
}
