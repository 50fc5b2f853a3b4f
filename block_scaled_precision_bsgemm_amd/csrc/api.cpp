// C ABI of bsgemm: argument validation, device check, dispatch to launchers.
//
// Validation happens before anything is launched, in this order:
//   1. invalid arguments;
//   2. unsupported shapes and formats;
//   3. alignment;
//   4. size limits of the kernels;
//   5. device.
// A failing call therefore launches nothing.  A passing call always launches
// its work (except the documented empty-output cases), and never silently
// does nothing: the planner-hazard lesson of "Add sm121 (GB10) tier to the
// 4-bit GEMM dispatch heuristic", tile-selection follow-up, where a config
// chain with no final else launched nothing.  No C++ exception crosses the
// ABI.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "bsgemm.h"
#include "internal.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return BSGEMM_OK;
}

// Kernels address one tile of an operand with 32-bit offsets; these limits
// keep every such offset below 2^31.
constexpr int64_t MAX_K = int64_t(1) << 21;
constexpr int64_t MAX_ROWS = (int64_t(1) << 31) - 1;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Null is allowed only for a buffer of zero bytes.
#define REQUIRE_PTR(p, nbytes)                                                          \
  do {                                                                                  \
    if ((p) == nullptr && (nbytes) > 0)                                                 \
      return fail(BSGEMM_ERR_INVALID_ARG, "%s: %s is NULL", fn, #p);                    \
  } while (0)
#define REQUIRE_ALIGNED(p)                                                              \
  do {                                                                                  \
    if ((p) != nullptr && !aligned16(p))                                                \
      return fail(BSGEMM_ERR_BAD_ALIGNMENT, "%s: %s is not 16-byte aligned", fn, #p);   \
  } while (0)

struct DeviceInfo {
  std::atomic<int> state{0};   // 0 unknown, 1 gfx950, 2 other
  int num_cus = 0;
  char arch[64] = {0};
};
constexpr int MAX_DEVICES = 64;
DeviceInfo g_devices[MAX_DEVICES];
std::mutex g_device_mutex;

// Checks that the current HIP device is a gfx950 and returns its CU count.
int check_device(const char* fn, int* num_cus) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
    (void)hipGetLastError();
    return fail(BSGEMM_ERR_DEVICE, "%s: no HIP device is available", fn);
  }
  DeviceInfo& d = g_devices[dev];
  if (d.state.load(std::memory_order_acquire) == 0) {
    std::lock_guard<std::mutex> lock(g_device_mutex);
    if (d.state.load(std::memory_order_relaxed) == 0) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(BSGEMM_ERR_DEVICE, "%s: cannot query device %d", fn, dev);
      }
      std::snprintf(d.arch, sizeof d.arch, "%s", prop.gcnArchName);
      d.num_cus = prop.multiProcessorCount;
      d.state.store(std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2,
                    std::memory_order_release);
    }
  }
  if (d.state.load(std::memory_order_acquire) != 1)
    return fail(BSGEMM_ERR_DEVICE, "%s: device %d is %s, this library needs gfx950", fn, dev,
                d.arch);
  *num_cus = d.num_cus;
  return BSGEMM_OK;
}

int finish_launch(const char* fn, hipError_t err, hipStream_t stream) {
  if (err == hipSuccess) {
    static const bool sync_check = [] {
      const char* e = std::getenv("BSGEMM_SYNC_CHECK");
      return e != nullptr && e[0] == '1';
    }();
    if (sync_check) {
      err = hipStreamSynchronize(stream);
      if (err == hipSuccess) err = hipGetLastError();
    }
  }
  if (err != hipSuccess)
    return fail(BSGEMM_ERR_LAUNCH, "%s: HIP error %s", fn, hipGetErrorString(err));
  return ok();
}

int check_k(const char* fn, int64_t k) {
  if (k % 32 != 0)
    return fail(BSGEMM_ERR_UNSUPPORTED, "%s: k = %lld is not a multiple of 32", fn, (long long)k);
  return BSGEMM_OK;
}

int check_limits(const char* fn, int64_t rows_a, int64_t rows_b, int64_t k) {
  if (k > MAX_K || rows_a > MAX_ROWS || rows_b > MAX_ROWS)
    return fail(BSGEMM_ERR_RESOURCE,
                "%s: sizes (%lld, %lld, k = %lld) exceed the kernels' limits (rows < 2^31, k <= 2^21)",
                fn, (long long)rows_a, (long long)rows_b, (long long)k);
  return BSGEMM_OK;
}

}  // namespace

extern "C" {

int bsgemm_version(void) { return 600; }   // 0.6.0: exact-product MXFP8 GEMM (BSGEMM_MXFP8_EXACT)

const char* bsgemm_status_string(int status) {
  switch (status) {
    case BSGEMM_OK: return "BSGEMM_OK";
    case BSGEMM_ERR_INVALID_ARG: return "BSGEMM_ERR_INVALID_ARG";
    case BSGEMM_ERR_UNSUPPORTED: return "BSGEMM_ERR_UNSUPPORTED";
    case BSGEMM_ERR_BAD_ALIGNMENT: return "BSGEMM_ERR_BAD_ALIGNMENT";
    case BSGEMM_ERR_DEVICE: return "BSGEMM_ERR_DEVICE";
    case BSGEMM_ERR_RESOURCE: return "BSGEMM_ERR_RESOURCE";
    case BSGEMM_ERR_LAUNCH: return "BSGEMM_ERR_LAUNCH";
    default: return "unknown status";
  }
}

const char* bsgemm_last_error(void) { return g_last_error.c_str(); }

int bsgemm_quantize_nvfp4(int64_t rows, int64_t k, const float* x, uint8_t* codes,
                          uint8_t* scales, float* tensor_scale, void* stream) {
  static const char* fn = "bsgemm_quantize_nvfp4";
  try {
    if (rows < 0 || k < 0) return fail(BSGEMM_ERR_INVALID_ARG, "%s: negative size", fn);
    const int64_t n = rows * k;
    REQUIRE_PTR(x, n);
    REQUIRE_PTR(codes, n);
    REQUIRE_PTR(scales, n);
    if (tensor_scale == nullptr) return fail(BSGEMM_ERR_INVALID_ARG, "%s: tensor_scale is NULL", fn);
    if (int s = check_k(fn, k)) return s;
    REQUIRE_ALIGNED(x);
    REQUIRE_ALIGNED(codes);
    REQUIRE_ALIGNED(scales);
    if (int s = check_limits(fn, rows, 0, 0)) return s;
    int num_cus = 0;
    if (int s = check_device(fn, &num_cus)) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    return finish_launch(fn, bsg::launch_quantize_nvfp4(rows, k, x, codes, scales, tensor_scale, st, num_cus), st);
  } catch (...) {
    return fail(BSGEMM_ERR_LAUNCH, "%s: internal exception", fn);
  }
}

int bsgemm_quantize_mxfp8(int64_t rows, int64_t k, const float* x, uint8_t* codes,
                          uint8_t* scales, void* stream) {
  static const char* fn = "bsgemm_quantize_mxfp8";
  try {
    if (rows < 0 || k < 0) return fail(BSGEMM_ERR_INVALID_ARG, "%s: negative size", fn);
    const int64_t n = rows * k;
    REQUIRE_PTR(x, n);
    REQUIRE_PTR(codes, n);
    REQUIRE_PTR(scales, n);
    if (int s = check_k(fn, k)) return s;
    REQUIRE_ALIGNED(x);
    REQUIRE_ALIGNED(codes);
    REQUIRE_ALIGNED(scales);
    if (int s = check_limits(fn, rows, 0, 0)) return s;
    int num_cus = 0;
    if (int s = check_device(fn, &num_cus)) return s;
    if (n == 0) return ok();
    hipStream_t st = static_cast<hipStream_t>(stream);
    return finish_launch(fn, bsg::launch_quantize_mxfp8(rows, k, x, codes, scales, st, num_cus), st);
  } catch (...) {
    return fail(BSGEMM_ERR_LAUNCH, "%s: internal exception", fn);
  }
}

int bsgemm_quantize_mxfp4(int64_t rows, int64_t k, const float* x, uint8_t* codes,
                          uint8_t* scales, void* stream) {
  static const char* fn = "bsgemm_quantize_mxfp4";
  try {
    if (rows < 0 || k < 0) return fail(BSGEMM_ERR_INVALID_ARG, "%s: negative size", fn);
    const int64_t n = rows * k;
    REQUIRE_PTR(x, n);
    REQUIRE_PTR(codes, n);
    REQUIRE_PTR(scales, n);
    if (int s = check_k(fn, k)) return s;
    REQUIRE_ALIGNED(x);
    REQUIRE_ALIGNED(codes);
    REQUIRE_ALIGNED(scales);
    if (int s = check_limits(fn, rows, 0, 0)) return s;
    int num_cus = 0;
    if (int s = check_device(fn, &num_cus)) return s;
    if (n == 0) return ok();
    hipStream_t st = static_cast<hipStream_t>(stream);
    return finish_launch(fn, bsg::launch_quantize_mxfp4(rows, k, x, codes, scales, st, num_cus), st);
  } catch (...) {
    return fail(BSGEMM_ERR_LAUNCH, "%s: internal exception", fn);
  }
}

int bsgemm_run(int fmt, int64_t m, int64_t n, int64_t k, const uint8_t* a,
               const uint8_t* a_scales, const float* a_tscale, const uint8_t* b,
               const uint8_t* b_scales, const float* b_tscale, uint16_t* c_bf16, void* stream) {
  static const char* fn = "bsgemm_run";
  try {
    if (m < 0 || n < 0 || k < 0) return fail(BSGEMM_ERR_INVALID_ARG, "%s: negative size", fn);
    REQUIRE_PTR(a, m * k);
    REQUIRE_PTR(a_scales, m * k);
    REQUIRE_PTR(b, n * k);
    REQUIRE_PTR(b_scales, n * k);
    REQUIRE_PTR(c_bf16, m * n);
    if (fmt == BSGEMM_NVFP4) {
      if (a_tscale == nullptr || b_tscale == nullptr)
        return fail(BSGEMM_ERR_INVALID_ARG, "%s: NVFP4 needs a_tscale and b_tscale", fn);
    } else if (fmt == BSGEMM_MXFP8 || fmt == BSGEMM_MXFP4 || fmt == BSGEMM_MXFP8_EXACT) {
      if (a_tscale != nullptr || b_tscale != nullptr)
        return fail(BSGEMM_ERR_UNSUPPORTED, "%s: %s takes no tensor scales (pass NULL)", fn,
                    fmt == BSGEMM_MXFP4 ? "MXFP4" : "MXFP8");
    } else {
      return fail(BSGEMM_ERR_UNSUPPORTED, "%s: unknown format %d", fn, fmt);
    }
    if (int s = check_k(fn, k)) return s;
    REQUIRE_ALIGNED(a);
    REQUIRE_ALIGNED(a_scales);
    REQUIRE_ALIGNED(b);
    REQUIRE_ALIGNED(b_scales);
    REQUIRE_ALIGNED(c_bf16);
    if (int s = check_limits(fn, m, n, k)) return s;
    int num_cus = 0;
    if (int s = check_device(fn, &num_cus)) return s;
    if (m == 0 || n == 0) return ok();
    hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t e =
        fmt == BSGEMM_NVFP4   ? bsg::launch_gemm_nvfp4(m, n, k, a, a_scales, a_tscale, b, b_scales, b_tscale, c_bf16, st)
        : fmt == BSGEMM_MXFP8 ? bsg::launch_gemm_mxfp8(m, n, k, a, a_scales, b, b_scales, c_bf16, st)
        : fmt == BSGEMM_MXFP8_EXACT
            ? bsg::launch_gemm_mxfp8_exact(m, n, k, a, a_scales, b, b_scales, c_bf16, st)
            : bsg::launch_gemm_mxfp4(m, n, k, a, a_scales, b, b_scales, c_bf16, st);
    return finish_launch(fn, e, st);
  } catch (...) {
    return fail(BSGEMM_ERR_LAUNCH, "%s: internal exception", fn);
  }
}

int bsgemm_grouped_run(int num_groups, int64_t m_total, int64_t n, int64_t k, const uint8_t* a,
                       const uint8_t* a_scales, const float* a_tscale,
                       const int32_t* group_offsets, const uint16_t* w_bf16, uint16_t* c_bf16,
                       void* stream) {
  static const char* fn = "bsgemm_grouped_run";
  try {
    if (num_groups < 1) return fail(BSGEMM_ERR_INVALID_ARG, "%s: num_groups must be >= 1", fn);
    if (m_total < 0 || n < 0 || k < 0) return fail(BSGEMM_ERR_INVALID_ARG, "%s: negative size", fn);
    REQUIRE_PTR(a, m_total * k);
    REQUIRE_PTR(a_scales, m_total * k);
    REQUIRE_PTR(w_bf16, n * k);
    REQUIRE_PTR(c_bf16, m_total * n);
    if (a_tscale == nullptr) return fail(BSGEMM_ERR_INVALID_ARG, "%s: a_tscale is NULL", fn);
    if (group_offsets == nullptr) return fail(BSGEMM_ERR_INVALID_ARG, "%s: group_offsets is NULL", fn);
    if (int s = check_k(fn, k)) return s;
    REQUIRE_ALIGNED(a);
    REQUIRE_ALIGNED(a_scales);
    REQUIRE_ALIGNED(w_bf16);
    REQUIRE_ALIGNED(c_bf16);
    if (int s = check_limits(fn, m_total, n, k)) return s;
    if (bsg::grouped_grid_blocks(num_groups, m_total, n, k) > MAX_ROWS)
      return fail(BSGEMM_ERR_RESOURCE, "%s: too many tiles", fn);
    int num_cus = 0;
    if (int s = check_device(fn, &num_cus)) return s;
    if (m_total == 0 || n == 0) return ok();
    hipStream_t st = static_cast<hipStream_t>(stream);
    bsg::GroupedCall call{num_groups, m_total, m_total, n, k, a, a_scales, a_tscale, group_offsets,
                          w_bf16, false, nullptr, nullptr, nullptr, nullptr, c_bf16};
    return finish_launch(fn, bsg::launch_grouped(call, st), st);
  } catch (...) {
    return fail(BSGEMM_ERR_LAUNCH, "%s: internal exception", fn);
  }
}

int bsgemm_grouped_run_ex(int num_groups, int64_t m_total, int64_t n, int64_t k, int64_t a_rows,
                          const uint8_t* a, const uint8_t* a_scales, const float* a_tscale,
                          const int32_t* group_offsets, int w_dtype, const uint16_t* w,
                          const float* bias, const float* gamma, const int32_t* gather_idx,
                          const int32_t* scatter_idx, uint16_t* c_bf16, void* stream) {
  static const char* fn = "bsgemm_grouped_run_ex";
  try {
    if (num_groups < 1) return fail(BSGEMM_ERR_INVALID_ARG, "%s: num_groups must be >= 1", fn);
    if (m_total < 0 || n < 0 || k < 0 || a_rows < 0)
      return fail(BSGEMM_ERR_INVALID_ARG, "%s: negative size", fn);
    if (gather_idx == nullptr && a_rows != m_total)
      return fail(BSGEMM_ERR_INVALID_ARG, "%s: without gather_idx, a_rows must equal m_total", fn);
    REQUIRE_PTR(a, a_rows * k);
    REQUIRE_PTR(a_scales, a_rows * k);
    REQUIRE_PTR(w, n * k);
    REQUIRE_PTR(c_bf16, m_total * n);
    if (a_tscale == nullptr) return fail(BSGEMM_ERR_INVALID_ARG, "%s: a_tscale is NULL", fn);
    if (group_offsets == nullptr) return fail(BSGEMM_ERR_INVALID_ARG, "%s: group_offsets is NULL", fn);
    if (w_dtype != BSGEMM_W_BF16 && w_dtype != BSGEMM_W_F16)
      return fail(BSGEMM_ERR_UNSUPPORTED, "%s: unknown w_dtype %d", fn, w_dtype);
    if (int s = check_k(fn, k)) return s;
    REQUIRE_ALIGNED(a);
    REQUIRE_ALIGNED(a_scales);
    REQUIRE_ALIGNED(w);
    REQUIRE_ALIGNED(c_bf16);
    for (const void* q : {static_cast<const void*>(bias), static_cast<const void*>(gamma),
                          static_cast<const void*>(gather_idx), static_cast<const void*>(scatter_idx)})
      if ((reinterpret_cast<uintptr_t>(q) & 3u) != 0)
        return fail(BSGEMM_ERR_BAD_ALIGNMENT, "%s: bias, gamma and index arrays must be 4-byte aligned", fn);
    if (int s = check_limits(fn, m_total, n, k)) return s;
    if (a_rows > MAX_ROWS || a_rows * (k / 2) > MAX_ROWS)
      return fail(BSGEMM_ERR_RESOURCE, "%s: A (%lld rows of %lld code bytes) exceeds 2^31 bytes", fn,
                  (long long)a_rows, (long long)(k / 2));
    if (bsg::grouped_grid_blocks(num_groups, m_total, n, k) > MAX_ROWS)
      return fail(BSGEMM_ERR_RESOURCE, "%s: too many tiles", fn);
    int num_cus = 0;
    if (int s = check_device(fn, &num_cus)) return s;
    if (m_total == 0 || n == 0) return ok();
    hipStream_t st = static_cast<hipStream_t>(stream);
    bsg::GroupedCall call{num_groups, m_total, a_rows, n, k, a, a_scales, a_tscale, group_offsets,
                          w, w_dtype == BSGEMM_W_F16, bias, gamma, gather_idx, scatter_idx, c_bf16};
    return finish_launch(fn, bsg::launch_grouped(call, st), st);
  } catch (...) {
    return fail(BSGEMM_ERR_LAUNCH, "%s: internal exception", fn);
  }
}

int bsgemm_grouped_kragged_run(int num_groups, int64_t m, int64_t n, int64_t k, const uint8_t* a,
                               const uint8_t* a_scales, const float* a_tscale, const int32_t* k_offsets,
                               int w_dtype, const uint16_t* w, uint16_t* c_bf16, void* stream) {
  static const char* fn = "bsgemm_grouped_kragged_run";
  try {
    if (num_groups < 1) return fail(BSGEMM_ERR_INVALID_ARG, "%s: num_groups must be >= 1", fn);
    if (m < 0 || n < 0 || k < 0) return fail(BSGEMM_ERR_INVALID_ARG, "%s: negative size", fn);
    REQUIRE_PTR(a, m * k);
    REQUIRE_PTR(a_scales, m * k);
    REQUIRE_PTR(w, n * k);
    REQUIRE_PTR(c_bf16, m * n);
    if (a_tscale == nullptr) return fail(BSGEMM_ERR_INVALID_ARG, "%s: a_tscale is NULL", fn);
    if (k_offsets == nullptr) return fail(BSGEMM_ERR_INVALID_ARG, "%s: k_offsets is NULL", fn);
    if (w_dtype != BSGEMM_W_BF16 && w_dtype != BSGEMM_W_F16)
      return fail(BSGEMM_ERR_UNSUPPORTED, "%s: unknown w_dtype %d", fn, w_dtype);
    if (k % 256 != 0)
      return fail(BSGEMM_ERR_UNSUPPORTED, "%s: k = %lld is not a multiple of 256 (the K-slice padding)", fn,
                  (long long)k);
    REQUIRE_ALIGNED(a);
    REQUIRE_ALIGNED(a_scales);
    REQUIRE_ALIGNED(w);
    REQUIRE_ALIGNED(c_bf16);
    if ((reinterpret_cast<uintptr_t>(k_offsets) & 3u) != 0)
      return fail(BSGEMM_ERR_BAD_ALIGNMENT, "%s: k_offsets is not 4-byte aligned", fn);
    if (int s = check_limits(fn, m, n, k)) return s;
    // the launch pads the (group, n tile) units to a multiple of 8
    if (((int64_t)num_groups * ((n + 255) / 256) + 7) / 8 * 8 * ((m + 255) / 256) > MAX_ROWS)
      return fail(BSGEMM_ERR_RESOURCE, "%s: too many tiles", fn);
    int num_cus = 0;
    if (int s = check_device(fn, &num_cus)) return s;
    if (m == 0 || n == 0) return ok();
    hipStream_t st = static_cast<hipStream_t>(stream);
    bsg::KRaggedCall call{num_groups, m, n, k, a, a_scales, a_tscale, k_offsets, w, w_dtype == BSGEMM_W_F16, c_bf16};
    return finish_launch(fn, bsg::launch_grouped_kragged(call, st), st);
  } catch (...) {
    return fail(BSGEMM_ERR_LAUNCH, "%s: internal exception", fn);
  }
}

}  // extern "C"

namespace {

// Configuration forced through the environment for bsgemm_w4a16_run
// (BSGEMM_W4A16_FORCE_CONFIG = an id or a name): -1 when unset, -2 when set
// to something that names no configuration.
int forced_w4a16_config() {
  const char* e = std::getenv("BSGEMM_W4A16_FORCE_CONFIG");
  if (e == nullptr || e[0] == '\0') return -1;
  const int n = bsg::w4a16_num_configs();
  for (int i = 0; i < n; ++i)
    if (std::strcmp(e, bsg::w4a16_config_name(i)) == 0) return i;
  char* end = nullptr;
  const long v = std::strtol(e, &end, 10);
  if (end != e && *end == '\0' && v >= 0 && v < n) return (int)v;
  return -2;
}

// Shared body of the W4A16 entry points; config -1 = the selector's choice.
int w4a16_call(const char* fn, int config, int64_t m, int64_t n, int64_t k, const uint16_t* x_bf16,
               const uint8_t* w, const uint8_t* w_scales, const float* w_tscale, uint16_t* c_bf16,
               void* stream) {
  if (m < 0 || n < 0 || k < 0) return fail(BSGEMM_ERR_INVALID_ARG, "%s: negative size", fn);
  REQUIRE_PTR(x_bf16, m * k);
  REQUIRE_PTR(w, n * k);
  REQUIRE_PTR(w_scales, n * k);
  REQUIRE_PTR(c_bf16, m * n);
  if (w_tscale == nullptr) return fail(BSGEMM_ERR_INVALID_ARG, "%s: w_tscale is NULL", fn);
  if (config >= bsg::w4a16_num_configs() || config < -1)
    return fail(BSGEMM_ERR_UNSUPPORTED, "%s: unknown configuration %d", fn, config);
  if (int s = check_k(fn, k)) return s;
  REQUIRE_ALIGNED(x_bf16);
  REQUIRE_ALIGNED(w);
  REQUIRE_ALIGNED(w_scales);
  REQUIRE_ALIGNED(c_bf16);
  if (int s = check_limits(fn, m, n, k)) return s;
  const int cfg = config >= 0 ? config : bsg::w4a16_select(m, n, k);
  if (k % bsg::w4a16_config_k_multiple(cfg) != 0)
    return fail(BSGEMM_ERR_UNSUPPORTED, "%s: configuration %s needs k %% %d == 0", fn, bsg::w4a16_config_name(cfg),
                bsg::w4a16_config_k_multiple(cfg));
  if (m > bsg::w4a16_config_max_m(cfg))
    return fail(BSGEMM_ERR_RESOURCE, "%s: configuration %s takes m <= %d", fn, bsg::w4a16_config_name(cfg),
                bsg::w4a16_config_max_m(cfg));
  int num_cus = 0;
  if (int s = check_device(fn, &num_cus)) return s;
  if (m == 0 || n == 0) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  return finish_launch(fn, bsg::launch_w4a16(cfg, m, n, k, x_bf16, w, w_scales, w_tscale, c_bf16, st), st);
}

}  // namespace

extern "C" {

int bsgemm_w4a16_run(int64_t m, int64_t n, int64_t k, const uint16_t* x_bf16, const uint8_t* w,
                     const uint8_t* w_scales, const float* w_tscale, uint16_t* c_bf16,
                     void* stream) {
  static const char* fn = "bsgemm_w4a16_run";
  try {
    const int forced = forced_w4a16_config();
    if (forced == -2)
      return fail(BSGEMM_ERR_UNSUPPORTED, "%s: BSGEMM_W4A16_FORCE_CONFIG names no configuration", fn);
    return w4a16_call(fn, forced, m, n, k, x_bf16, w, w_scales, w_tscale, c_bf16, stream);
  } catch (...) {
    return fail(BSGEMM_ERR_LAUNCH, "%s: internal exception", fn);
  }
}

int bsgemm_w4a16_run_config(int config, int64_t m, int64_t n, int64_t k, const uint16_t* x_bf16,
                            const uint8_t* w, const uint8_t* w_scales, const float* w_tscale,
                            uint16_t* c_bf16, void* stream) {
  static const char* fn = "bsgemm_w4a16_run_config";
  try {
    if (config < 0) return fail(BSGEMM_ERR_UNSUPPORTED, "%s: unknown configuration %d", fn, config);
    return w4a16_call(fn, config, m, n, k, x_bf16, w, w_scales, w_tscale, c_bf16, stream);
  } catch (...) {
    return fail(BSGEMM_ERR_LAUNCH, "%s: internal exception", fn);
  }
}

int bsgemm_w4a16_num_configs(void) { return bsg::w4a16_num_configs(); }

const char* bsgemm_w4a16_config_name(int config) { return bsg::w4a16_config_name(config); }

int bsgemm_w4a16_select(int64_t m, int64_t n, int64_t k) {
  if (m < 0 || n < 0 || k < 0 || k % 32 != 0) return -1;
  return bsg::w4a16_select(m, n, k);
}

}  // extern "C"
