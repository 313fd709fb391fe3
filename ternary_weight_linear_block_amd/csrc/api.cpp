// C ABI of the ternary linear library: argument validation, device checks,
// GEMM/GEMV dispatch and thread-local error messages.  No allocation, no
// synchronisation; every kernel is enqueued on the caller's stream.
#include "twl.h"
#include "twl_internal.h"

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

namespace {

thread_local std::string g_last_error;

twl_status fail(twl_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

twl_status ok() {
  g_last_error.clear();
  return TWL_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
bool g_dev_known[kMaxDevices];
bool g_dev_ok[kMaxDevices];
twl::DeviceInfo g_dev_info[kMaxDevices];

// Checks the current device is gfx950 and returns its cached facts.
twl_status current_device(twl::DeviceInfo* out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TWL_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(TWL_EDEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_dev_mu);
  if (!g_dev_known[dev]) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(TWL_EHIP, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
    g_dev_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_dev_info[dev].cu_count = prop.multiProcessorCount;
    g_dev_known[dev] = true;
    if (!g_dev_ok[dev])
      return fail(TWL_EDEVICE, "device %d is %s; this library is built for gfx950 only", dev,
                  prop.gcnArchName);
  }
  if (!g_dev_ok[dev]) return fail(TWL_EDEVICE, "device %d is not gfx950", dev);
  *out = g_dev_info[dev];
  return TWL_OK;
}

twl_status check_k(int64_t K) {
  if (K <= 0 || K % TWL_HBLOCK != 0)
    return fail(TWL_ESHAPE, "K=%lld must be a positive multiple of %d", static_cast<long long>(K),
                TWL_HBLOCK);
  if (K > TWL_MAX_K)
    return fail(TWL_ESHAPE, "K=%lld exceeds the maximum %d", static_cast<long long>(K), TWL_MAX_K);
  return TWL_OK;
}

twl_status check_rows(const char* name, int64_t v) {
  if (v < 0) return fail(TWL_EINVAL, "%s=%lld is negative", name, static_cast<long long>(v));
  if (v > (int64_t{1} << 30))
    return fail(TWL_ESHAPE, "%s=%lld is too large", name, static_cast<long long>(v));
  return TWL_OK;
}

#define TWL_REQUIRE_PTR(p)                                                 \
  do {                                                                     \
    if ((p) == nullptr) return fail(TWL_EINVAL, "%s is NULL", #p);          \
    if (!aligned16(p)) return fail(TWL_EALIGN, "%s is not 16-byte aligned", #p); \
  } while (0)

#define TWL_TRY(expr)                    \
  do {                                   \
    twl_status st_ = (expr);             \
    if (st_ != TWL_OK) return st_;       \
  } while (0)

twl_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(TWL_EHIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

// Library-owned K-split scratch for twl_ternary_linear_noalloc: one copy per
// GPU, held until the process ends.  In host code `scratch` is only a stand-in
// for the symbol; the device address of each GPU's copy comes from
// hipGetSymbolAddress (called once per device, with that device current) and
// is the only form ever passed to a kernel.
static __device__ __attribute__((aligned(256))) unsigned char scratch[TWL_NOALLOC_SCRATCH_BYTES];
void* g_scratch_ptr[kMaxDevices];  // guarded by g_dev_mu

// Device address of the current device's scratch (looked up on first use).
twl_status current_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TWL_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(TWL_EDEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_dev_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(TWL_EHIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TWL_OK;
}

twl::GemvKind gemv_kind(int path) {
  return path == TWL_PATH_GEMV_DOT4   ? twl::kGemvDot4
         : path == TWL_PATH_GEMV_MFMA ? twl::kGemvMfma
                                      : twl::kGemvAuto;
}

// Bytes of K-split partial sums the linear layer needs for this shape and
// path (0 when it does not split K).
size_t workspace_need(int64_t M, int64_t N, int64_t K, int path, const twl::DeviceInfo& dev) {
  const bool use_gemv = path >= TWL_PATH_GEMV || (path == TWL_PATH_AUTO && M <= TWL_GEMV_MAX_M);
  return use_gemv ? twl::gemv_workspace_bytes(M, N, K, gemv_kind(path), dev)
                  : twl::gemm_workspace_bytes(M, N, K, dev);
}

twl_status check_workspace(size_t need, const void* workspace, size_t workspace_bytes) {
  if (need == 0) return TWL_OK;
  if (workspace == nullptr || workspace_bytes < need)
    return fail(TWL_EINVAL, "workspace of %zu bytes required (got %zu)", need,
                workspace == nullptr ? size_t{0} : workspace_bytes);
  if (!aligned16(workspace)) return fail(TWL_EALIGN, "workspace is not 16-byte aligned");
  return TWL_OK;
}

// The linear layer with the K-split partial sums either in the caller's
// workspace or (use_scratch) in the library's per-device scratch.
twl_status linear_impl(const int8_t* x_i8, const float* a_scale, const uint8_t* packed,
                       const int8_t* q, const float* smax, int64_t M, int64_t N, int64_t K,
                       void* out, int out_kind, int path, void* workspace, size_t workspace_bytes,
                       bool use_scratch, hipStream_t stream) {
  TWL_TRY(check_rows("M", M));
  TWL_TRY(check_rows("N", N));
  TWL_TRY(check_k(K));
  if (path < TWL_PATH_AUTO || path > TWL_PATH_GEMV_MFMA)
    return fail(TWL_EINVAL, "unknown path %d", path);
  if (out_kind < TWL_OUT_F32 || out_kind > TWL_OUT_BF16)
    return fail(TWL_EINVAL, "unknown output kind %d", out_kind);
  const bool decode_path = path >= TWL_PATH_GEMV;
  if (decode_path && M > TWL_GEMV_MAX_M)
    return fail(TWL_ESHAPE, "the decode paths take M <= %d (got %lld)", TWL_GEMV_MAX_M,
                static_cast<long long>(M));
  if (M == 0 || N == 0) return ok();
  TWL_REQUIRE_PTR(x_i8);
  TWL_REQUIRE_PTR(packed);
  TWL_REQUIRE_PTR(q);
  TWL_REQUIRE_PTR(out);
  if (out_kind != TWL_OUT_ACC_I32) {
    TWL_REQUIRE_PTR(a_scale);
    TWL_REQUIRE_PTR(smax);
  }
  twl::DeviceInfo dev;
  TWL_TRY(current_device(&dev));
  const bool use_gemv = decode_path || (path == TWL_PATH_AUTO && M <= TWL_GEMV_MAX_M);
  const twl::GemvKind kind = gemv_kind(path);
  const size_t part = workspace_need(M, N, K, path, dev);
  if (use_scratch) {
    if (part > TWL_NOALLOC_SCRATCH_BYTES)
      return fail(TWL_ESHAPE,
                  "M=%lld N=%lld K=%lld needs %zu bytes of K-split scratch; the library's "
                  "no-allocation scratch holds %zu (use twl_ternary_linear_ex with a workspace)",
                  static_cast<long long>(M), static_cast<long long>(N), static_cast<long long>(K),
                  part, static_cast<size_t>(TWL_NOALLOC_SCRATCH_BYTES));
    workspace = nullptr;
    workspace_bytes = 0;
    if (part > 0) {
      TWL_TRY(current_scratch(&workspace));
      workspace_bytes = TWL_NOALLOC_SCRATCH_BYTES;
    }
  } else {
    TWL_TRY(check_workspace(part, workspace, workspace_bytes));
  }
  if (use_gemv)
    return launched(twl::launch_gemv(x_i8, a_scale, packed, q, smax, M, N, K, out,
                                     static_cast<twl::OutKind>(out_kind), workspace,
                                     workspace_bytes, kind, dev, stream),
                    "ternary_linear (GEMV)");
  return launched(twl::launch_gemm(x_i8, a_scale, packed, q, smax, M, N, K, out,
                                   static_cast<twl::OutKind>(out_kind), workspace,
                                   workspace_bytes, dev, stream),
                  "ternary_linear (GEMM)");
}

}  // namespace

extern "C" {

const char* twl_last_error(void) { return g_last_error.c_str(); }

int twl_abi_version(void) { return 3; }

size_t twl_packed_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || K % TWL_HBLOCK != 0 || K > TWL_MAX_K || N > (int64_t{1} << 30)) return 0;
  return static_cast<size_t>((N + 63) / 64 * 64) * static_cast<size_t>(K / 4);
}

twl_status twl_rotate_quant_act(const uint16_t* x, const int8_t* sign, int64_t M, int64_t K,
                                int8_t* x_i8, float* a_scale, hipStream_t stream) {
  TWL_TRY(check_rows("M", M));
  TWL_TRY(check_k(K));
  if (M == 0) return ok();
  TWL_REQUIRE_PTR(x);
  TWL_REQUIRE_PTR(sign);
  TWL_REQUIRE_PTR(x_i8);
  TWL_REQUIRE_PTR(a_scale);
  twl::DeviceInfo dev;
  TWL_TRY(current_device(&dev));
  return launched(twl::launch_rotate_quant(x, sign, M, K, x_i8, a_scale, stream),
                  "rotate_quant_act");
}

twl_status twl_silu_mul_rotate_quant_act(const uint16_t* gate_up, const int8_t* sign, int64_t M,
                                         int64_t K, int8_t* x_i8, float* a_scale,
                                         hipStream_t stream) {
  TWL_TRY(check_rows("M", M));
  TWL_TRY(check_k(K));
  if (M == 0) return ok();
  TWL_REQUIRE_PTR(gate_up);
  TWL_REQUIRE_PTR(sign);
  TWL_REQUIRE_PTR(x_i8);
  TWL_REQUIRE_PTR(a_scale);
  twl::DeviceInfo dev;
  TWL_TRY(current_device(&dev));
  return launched(twl::launch_silu_mul_rotate_quant(gate_up, sign, M, K, x_i8, a_scale, stream),
                  "silu_mul_rotate_quant_act");
}

twl_status twl_rotate_act_bf16(const uint16_t* x, const int8_t* sign, int64_t M, int64_t K,
                               uint16_t* r, hipStream_t stream) {
  TWL_TRY(check_rows("M", M));
  TWL_TRY(check_k(K));
  if (M == 0) return ok();
  TWL_REQUIRE_PTR(x);
  TWL_REQUIRE_PTR(sign);
  TWL_REQUIRE_PTR(r);
  twl::DeviceInfo dev;
  TWL_TRY(current_device(&dev));
  return launched(twl::launch_rotate_bf16(x, sign, M, K, r, stream), "rotate_act_bf16");
}

twl_status twl_reference_linear_bf16(const uint16_t* r, const uint8_t* packed, const uint16_t* s,
                                     int64_t M, int64_t N, int64_t K, float* y,
                                     hipStream_t stream) {
  TWL_TRY(check_rows("M", M));
  TWL_TRY(check_rows("N", N));
  TWL_TRY(check_k(K));
  if (M == 0 || N == 0) return ok();
  TWL_REQUIRE_PTR(r);
  TWL_REQUIRE_PTR(packed);
  TWL_REQUIRE_PTR(s);
  TWL_REQUIRE_PTR(y);
  twl::DeviceInfo dev;
  TWL_TRY(current_device(&dev));
  return launched(twl::launch_reference_bf16(r, packed, s, M, N, K, y, stream),
                  "reference_linear_bf16");
}

twl_status twl_pack_ternary(const int8_t* code, const uint16_t* s, int64_t N, int64_t K,
                            uint8_t* packed, int8_t* q, float* smax, int32_t* bad_codes,
                            hipStream_t stream) {
  TWL_TRY(check_rows("N", N));
  TWL_TRY(check_k(K));
  if (N == 0) return ok();
  TWL_REQUIRE_PTR(code);
  TWL_REQUIRE_PTR(s);
  TWL_REQUIRE_PTR(packed);
  TWL_REQUIRE_PTR(q);
  TWL_REQUIRE_PTR(smax);
  if (bad_codes != nullptr && (reinterpret_cast<uintptr_t>(bad_codes) & 3u))
    return fail(TWL_EALIGN, "bad_codes is not 4-byte aligned");
  twl::DeviceInfo dev;
  TWL_TRY(current_device(&dev));
  return launched(twl::launch_pack(code, s, N, K, packed, q, smax, bad_codes, stream),
                  "pack_ternary");
}

size_t twl_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  twl::DeviceInfo dev;
  if (current_device(&dev) != TWL_OK) return 0;
  // the GEMM's need, also for M <= TWL_GEMV_MAX_M (TWL_PATH_GEMM may be forced),
  // and the GEMV's where that path may run
  size_t need = twl::gemm_workspace_bytes(M, N, K, dev);
  if (M <= TWL_GEMV_MAX_M)
    for (twl::GemvKind kind : {twl::kGemvAuto, twl::kGemvDot4, twl::kGemvMfma})
      need = std::max(need, twl::gemv_workspace_bytes(M, N, K, kind, dev));
  return need;
}

twl_status twl_ternary_linear_ex(const int8_t* x_i8, const float* a_scale, const uint8_t* packed,
                                 const int8_t* q, const float* smax, int64_t M, int64_t N,
                                 int64_t K, void* out, int out_kind, int path, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  return linear_impl(x_i8, a_scale, packed, q, smax, M, N, K, out, out_kind, path, workspace,
                     workspace_bytes, false, stream);
}

twl_status twl_ternary_linear_noalloc(const int8_t* x_i8, const float* a_scale,
                                      const uint8_t* packed, const int8_t* q, const float* smax,
                                      int64_t M, int64_t N, int64_t K, void* out, int out_kind,
                                      int path, hipStream_t stream) {
  return linear_impl(x_i8, a_scale, packed, q, smax, M, N, K, out, out_kind, path, nullptr, 0,
                     true, stream);
}

twl_status twl_rotate_quant_linear(const uint16_t* x, const int8_t* sign, const uint8_t* packed,
                                   const int8_t* q, const float* smax, int64_t M, int64_t N,
                                   int64_t K, int silu, int8_t* x_i8, float* a_scale, void* out,
                                   int out_kind, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  TWL_TRY(check_rows("M", M));
  TWL_TRY(check_rows("N", N));
  TWL_TRY(check_k(K));
  if (silu != 0 && silu != 1) return fail(TWL_EINVAL, "silu must be 0 or 1 (got %d)", silu);
  if (out_kind < TWL_OUT_F32 || out_kind > TWL_OUT_BF16)
    return fail(TWL_EINVAL, "unknown output kind %d", out_kind);
  if (M == 0) return ok();
  TWL_REQUIRE_PTR(x);
  TWL_REQUIRE_PTR(sign);
  TWL_REQUIRE_PTR(x_i8);
  TWL_REQUIRE_PTR(a_scale);
  if (N > 0) {
    TWL_REQUIRE_PTR(packed);
    TWL_REQUIRE_PTR(q);
    TWL_REQUIRE_PTR(out);
    if (out_kind != TWL_OUT_ACC_I32) TWL_REQUIRE_PTR(smax);
  }
  twl::DeviceInfo dev;
  TWL_TRY(current_device(&dev));
  if (N > 0 && twl::gemv_rot_applies(M, N, K, dev))
    return launched(twl::launch_gemv_rot(x, sign, silu != 0, packed, q, smax, M, N, K, out,
                                         static_cast<twl::OutKind>(out_kind), x_i8, a_scale, dev,
                                         stream),
                    "rotate_quant_linear (fused decode)");
  // two steps; the linear step's workspace is checked before anything is enqueued
  if (N > 0) TWL_TRY(check_workspace(workspace_need(M, N, K, TWL_PATH_AUTO, dev), workspace, workspace_bytes));
  TWL_TRY(launched(silu ? twl::launch_silu_mul_rotate_quant(x, sign, M, K, x_i8, a_scale, stream)
                        : twl::launch_rotate_quant(x, sign, M, K, x_i8, a_scale, stream),
                   "rotate_quant_linear (rotation)"));
  if (N == 0) return ok();
  return linear_impl(x_i8, a_scale, packed, q, smax, M, N, K, out, out_kind, TWL_PATH_AUTO, workspace,
                     workspace_bytes, false, stream);
}

int twl_rotate_quant_linear_fused(int64_t M, int64_t N, int64_t K) {
  twl_status st = check_rows("M", M);
  if (st == TWL_OK) st = check_rows("N", N);
  if (st == TWL_OK) st = check_k(K);
  twl::DeviceInfo dev;
  if (st == TWL_OK) st = current_device(&dev);
  if (st != TWL_OK) return -static_cast<int>(st);
  ok();
  return M > 0 && N > 0 && twl::gemv_rot_applies(M, N, K, dev) ? 1 : 0;
}

twl_status twl_plan_info(int64_t M, int64_t N, int64_t K, int path, int64_t* info) {
  TWL_TRY(check_rows("M", M));
  TWL_TRY(check_rows("N", N));
  TWL_TRY(check_k(K));
  if (path < TWL_PATH_AUTO || path > TWL_PATH_GEMV_MFMA)
    return fail(TWL_EINVAL, "unknown path %d", path);
  const bool decode_path = path >= TWL_PATH_GEMV;
  if (decode_path && M > TWL_GEMV_MAX_M)
    return fail(TWL_ESHAPE, "the decode paths take M <= %d (got %lld)", TWL_GEMV_MAX_M,
                static_cast<long long>(M));
  if (info == nullptr) return fail(TWL_EINVAL, "info is NULL");
  for (int i = 0; i < 8; ++i) info[i] = 0;
  if (M == 0 || N == 0) return ok();
  twl::DeviceInfo dev;
  TWL_TRY(current_device(&dev));
  const bool use_gemv = decode_path || (path == TWL_PATH_AUTO && M <= TWL_GEMV_MAX_M);
  if (use_gemv) {
    twl::gemv_plan_info(M, N, K, gemv_kind(path), dev, info);
  } else {
    twl::gemm_plan_info(M, N, K, dev, info);
  }
  return ok();
}

twl_status twl_ternary_linear(const int8_t* x_i8, const float* a_scale, const uint8_t* packed,
                              const int8_t* q, const float* smax, int64_t M, int64_t N, int64_t K,
                              float* y, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  return twl_ternary_linear_ex(x_i8, a_scale, packed, q, smax, M, N, K, y, TWL_OUT_F32, TWL_PATH_AUTO,
                               workspace, workspace_bytes, stream);
}

twl_status twl_ternary_linear_acc(const int8_t* x_i8, const uint8_t* packed, const int8_t* q,
                                  int64_t M, int64_t N, int64_t K, int32_t* acc, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  return twl_ternary_linear_ex(x_i8, nullptr, packed, q, nullptr, M, N, K, acc, TWL_OUT_ACC_I32, TWL_PATH_AUTO,
                               workspace, workspace_bytes, stream);
}

}  // extern "C"
