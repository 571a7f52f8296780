// capi.hip -- the extern "C" entry points of libnvfp4.so (declared and
// documented in include/nvfp4.h): host-side validation, the error
// convention, the one-time architecture check, and dispatch to the kernels.
//
// Validation follows the pages' op layer ("mlx 0.30.7.2 -> 0.30.7.6" diff
// page 8: validate_global_scale, validate_qqmm_inputs, fp_quantize's group
// size / bits check, quantize / dequantize shape checks; page 7: float64
// rejected in the dispatch).  Messages use the pages' "[op] message" form.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/nvfp4.h"
#include "nvfp4_internal.h"

namespace {

thread_local std::string g_last_error;
std::mutex g_arch_mu;
std::string g_arch_override;
bool g_has_override = false;
int g_arch_ok[64];  // 0 unknown, 1 gfx950, 2 other

nvfp4_status fail(nvfp4_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

nvfp4_status ok() {
  g_last_error.clear();
  return NVFP4_OK;
}

bool dtype_ok(int dt) { return dt == NVFP4_F32 || dt == NVFP4_F16 || dt == NVFP4_BF16; }

size_t dtype_size(int dt) { return dt == NVFP4_F32 ? 4 : 2; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// operands the matrix-core kernels address with 32-bit buffer offsets
constexpr int64_t kOffsetLimit = (int64_t)1 << 31;

#define CHECK_PTR(op, p)                                                          \
  do {                                                                            \
    if ((p) == nullptr)                                                           \
      return fail(NVFP4_ERR_INVALID_ARGUMENT, "[" op "] " #p " must not be NULL."); \
  } while (0)

#define CHECK_DTYPE(op, dt)                                                               \
  do {                                                                                    \
    if (!dtype_ok(dt))                                                                    \
      return fail(NVFP4_ERR_INVALID_ARGUMENT,                                             \
                  "[" op "] Unsupported dtype code %d (float32, float16 and bfloat16 only).", \
                  (int)(dt));                                                             \
  } while (0)

// Group size 16 along the last axis (the pages' nvfp4 mode: group 16, bits 4).
nvfp4_status check_k(const char* op, int64_t k) {
  if (k <= 0 || k % 16 != 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[%s] The last dimension (%lld) must be a positive multiple of the group size 16.",
                op, (long long)k);
  return NVFP4_OK;
}

// The device behind `stream` (the current device for the null stream) must be
// gfx950 (the analogue of the pages' compute-capability gate in
// QQMatmul::eval_gpu).  Checked once per device.
nvfp4_status check_device(const char* op, hipStream_t stream) {
  {
    std::lock_guard<std::mutex> lk(g_arch_mu);
    if (g_has_override) {
      if (g_arch_override.rfind("gfx950", 0) != 0)
        return fail(NVFP4_ERR_UNSUPPORTED, "[%s] Device architecture %s is not gfx950.", op,
                    g_arch_override.c_str());
      return NVFP4_OK;
    }
  }
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(NVFP4_ERR_DEVICE, "[%s] No HIP device behind the stream: %s", op, hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_arch_mu);
  if (dev < 0 || dev >= 64) return fail(NVFP4_ERR_DEVICE, "[%s] Device id %d out of range.", op, dev);
  if (g_arch_ok[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(NVFP4_ERR_DEVICE, "[%s] hipGetDeviceProperties: %s", op, hipGetErrorString(e));
    g_arch_ok[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    if (g_arch_ok[dev] == 2) {
      std::string name = prop.gcnArchName;
      return fail(NVFP4_ERR_UNSUPPORTED, "[%s] Device architecture %s is not gfx950.", op,
                  name.c_str());
    }
  }
  if (g_arch_ok[dev] == 2)
    return fail(NVFP4_ERR_UNSUPPORTED, "[%s] Device architecture is not gfx950.", op);
  return NVFP4_OK;
}

nvfp4_status launched(const char* op, hipError_t e) {
  if (e != hipSuccess) return fail(NVFP4_ERR_DEVICE, "[%s] Kernel launch failed: %s", op, hipGetErrorString(e));
  return ok();
}

// Device scratch of nvfp4_gather_qmm_noalloc: the routing tables live here
// instead of in a caller workspace.  Each GPU holds its own copy for the life
// of the process; host code uses only the per-device address from
// hipGetSymbolAddress, never the array's name (a host-side stand-in).
constexpr size_t kNoAllocScratchBytes = (size_t)5 << 20;
static __device__ __align__(256) uint8_t noalloc_scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

// the address of `dev`'s copy, looked up once per device with `dev` current
nvfp4_status noalloc_scratch_of(const char* op, int dev, void** out) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (dev < 0 || dev >= 64) return fail(NVFP4_ERR_DEVICE, "[%s] Device id %d out of range.", op, dev);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch));
    if (cur != dev) {
      hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess || p == nullptr)
      return fail(NVFP4_ERR_DEVICE, "[%s] hipGetSymbolAddress of the scratch array: %s", op,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return NVFP4_OK;
}

}  // namespace

extern "C" {

const char* nvfp4_last_error(void) { return g_last_error.c_str(); }

int nvfp4_version(void) { return 100; }

void nvfp4_debug_set_arch_override(const char* arch) {
  std::lock_guard<std::mutex> lk(g_arch_mu);
  if (arch) {
    g_arch_override = arch;
    g_has_override = true;
  } else {
    g_arch_override.clear();
    g_has_override = false;
  }
}

nvfp4_status nvfp4_tensor_amax(const void* x, nvfp4_dtype dt, int64_t n, float* amax_out,
                               hipStream_t stream) {
  const char* op = "tensor_amax";
  CHECK_DTYPE("tensor_amax", dt);
  CHECK_PTR("tensor_amax", amax_out);
  if (n < 0) return fail(NVFP4_ERR_INVALID_ARGUMENT, "[tensor_amax] n (%lld) must be >= 0.", (long long)n);
  if (n > 0) CHECK_PTR("tensor_amax", x);
  if (n > 0 && !aligned(x, 16))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[tensor_amax] x must be 16-byte aligned.");
  if (nvfp4_status st = check_device(op, stream)) return st;
  return launched(op, nvfp4::launch_tensor_amax(x, dt, n, amax_out, stream));
}

static nvfp4_status check_codec(const char* op, const void* x, nvfp4_dtype dt, int64_t rows,
                                int64_t k) {
  if (!dtype_ok(dt))
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[%s] Unsupported dtype code %d (float32, float16 and bfloat16 only).", op, (int)dt);
  if (rows < 0) return fail(NVFP4_ERR_INVALID_ARGUMENT, "[%s] rows (%lld) must be >= 0.", op, (long long)rows);
  if (nvfp4_status st = check_k(op, k)) return st;
  if (rows > 0 && x == nullptr) return fail(NVFP4_ERR_INVALID_ARGUMENT, "[%s] input must not be NULL.", op);
  if (rows > 0 && !aligned(x, 16))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[%s] input must be 16-byte aligned.", op);
  return NVFP4_OK;
}

nvfp4_status nvfp4_quantize(const void* x, nvfp4_dtype dt, int64_t rows, int64_t k,
                            const float* global_scale, uint8_t* codes, uint8_t* scales,
                            hipStream_t stream) {
  const char* op = "quantize";
  if (nvfp4_status st = check_codec(op, x, dt, rows, k)) return st;
  if (rows > 0) {
    CHECK_PTR("quantize", codes);
    CHECK_PTR("quantize", scales);
    if (!aligned(codes, 4))
      return fail(NVFP4_ERR_INVALID_ARGUMENT, "[quantize] codes must be 4-byte aligned.");
  }
  if (nvfp4_status st = check_device(op, stream)) return st;
  if (rows == 0) return ok();
  return launched(op, nvfp4::launch_quantize(x, dt, rows, k, global_scale, codes, scales, stream));
}

nvfp4_status nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                              int64_t k, const float* global_scale, void* out,
                              nvfp4_dtype out_dt, hipStream_t stream) {
  const char* op = "dequantize";
  if (nvfp4_status st = check_codec(op, out, out_dt, rows, k)) return st;
  if (rows > 0) {
    CHECK_PTR("dequantize", codes);
    CHECK_PTR("dequantize", scales);
    if (!aligned(codes, 4))
      return fail(NVFP4_ERR_INVALID_ARGUMENT, "[dequantize] codes must be 4-byte aligned.");
  }
  if (nvfp4_status st = check_device(op, stream)) return st;
  if (rows == 0) return ok();
  return launched(op, nvfp4::launch_dequantize(codes, scales, rows, k, global_scale, out, out_dt, stream));
}

nvfp4_status nvfp4_quant_dequant(const void* x, nvfp4_dtype dt, int64_t rows, int64_t k,
                                 const float* global_scale, void* x_hat, hipStream_t stream) {
  const char* op = "quant_dequant";
  if (nvfp4_status st = check_codec(op, x, dt, rows, k)) return st;
  if (rows > 0) {
    CHECK_PTR("quant_dequant", x_hat);
    if (!aligned(x_hat, 16))
      return fail(NVFP4_ERR_INVALID_ARGUMENT, "[quant_dequant] x_hat must be 16-byte aligned.");
  }
  if (nvfp4_status st = check_device(op, stream)) return st;
  if (rows == 0) return ok();
  return launched(op, nvfp4::launch_quant_dequant(x, dt, rows, k, global_scale, x_hat, stream));
}

static nvfp4_status check_matmul(const char* op, const void* x, nvfp4_dtype dt, const float* gx,
                                 const uint8_t* wc, const uint8_t* ws, const float* gw, int64_t m,
                                 int64_t n, int64_t k, const void* out) {
  if (!dtype_ok(dt))
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[%s] Unsupported dtype code %d (float32, float16 and bfloat16 only).", op, (int)dt);
  if (m <= 0 || n <= 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[%s] m (%lld) and n (%lld) must be positive.", op,
                (long long)m, (long long)n);
  if (nvfp4_status st = check_k(op, k)) return st;
  if (!x || !wc || !ws || !out)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[%s] x, w_codes, w_scales and out must not be NULL.", op);
  if ((gx == nullptr) != (gw == nullptr))
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[%s] For nvfp4 mode, either both global_scale_x and global_scale_w must be "
                "provided, or neither.", op);
  if (!aligned(x, 16) || !aligned(wc, 16))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[%s] x and w_codes must be 16-byte aligned.", op);
  if (m * n > (int64_t)1 << 46 || n > INT32_MAX || m > INT32_MAX || k > INT32_MAX)
    return fail(NVFP4_ERR_UNSUPPORTED, "[%s] Sizes too large.", op);
  // the contraction kernels for m > 1 address x (or x_hat) and the weight's
  // codes with 32-bit buffer offsets
  if (m > 1 && (m * k * (int64_t)dtype_size(dt) >= kOffsetLimit || n * (k / 2) >= kOffsetLimit))
    return fail(NVFP4_ERR_UNSUPPORTED,
                "[%s] x (%lld x %lld) and the weight's codes (%lld x %lld bytes) must each stay "
                "below 2 GB for m > 1.", op, (long long)m, (long long)k, (long long)n,
                (long long)(k / 2));
  return NVFP4_OK;
}

nvfp4_status nvfp4_qmv(const void* x, nvfp4_dtype dt, const float* global_scale_x,
                       const uint8_t* w_codes, const uint8_t* w_scales,
                       const float* global_scale_w, int64_t n, int64_t k, void* out,
                       hipStream_t stream) {
  const char* op = "qmv";
  if (nvfp4_status st = check_matmul(op, x, dt, global_scale_x, w_codes, w_scales, global_scale_w,
                                     1, n, k, out))
    return st;
  if (k > nvfp4::kQmvMaxK)
    return fail(NVFP4_ERR_UNSUPPORTED, "[qmv] k (%lld) above the supported maximum %lld.",
                (long long)k, (long long)nvfp4::kQmvMaxK);
  if (nvfp4_status st = check_device(op, stream)) return st;
  return launched(op, nvfp4::launch_qmv(x, dt, global_scale_x, w_codes, w_scales, global_scale_w,
                                        n, k, out, stream));
}

size_t nvfp4_qqmm_workspace_size(int64_t m, int64_t n, int64_t k, nvfp4_dtype dt) {
  (void)n;
  if (m <= 1 || k <= 0 || !dtype_ok(dt)) return 0;
  size_t bytes = (size_t)m * (size_t)k * dtype_size(dt);
  return (bytes + 255) & ~(size_t)255;
}

nvfp4_status nvfp4_qqmm(const void* x, nvfp4_dtype dt, const float* global_scale_x,
                        const uint8_t* w_codes, const uint8_t* w_scales,
                        const float* global_scale_w, int64_t m, int64_t n, int64_t k, void* out,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* op = "qqmm";
  if (nvfp4_status st = check_matmul(op, x, dt, global_scale_x, w_codes, w_scales, global_scale_w,
                                     m, n, k, out))
    return st;
  if (m == 1 && k <= nvfp4::kQmvMaxK) {
    if (nvfp4_status st = check_device(op, stream)) return st;
    return launched(op, nvfp4::launch_qmv(x, dt, global_scale_x, w_codes, w_scales,
                                          global_scale_w, n, k, out, stream));
  }
  size_t need = (size_t)m * (size_t)k * dtype_size(dt);
  if (workspace_bytes < need || workspace == nullptr)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[qqmm] workspace of %zu bytes is smaller than %zu.",
                workspace_bytes, need);
  if (!aligned(workspace, 256))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[qqmm] workspace must be 256-byte aligned.");
  if (nvfp4_status st = check_device(op, stream)) return st;
  if (nvfp4::small_m_ok(dt, false, m, n, k))  // x's round trip happens inside the kernel
    return launched(op, nvfp4::launch_small_m(x, dt, true, global_scale_x, w_codes, w_scales,
                                              false, global_scale_w, m, n, k, out, stream));
  hipError_t e = nvfp4::launch_quant_dequant(x, dt, m, k, global_scale_x, workspace, stream);
  if (e != hipSuccess) return launched(op, e);
  return launched(op, nvfp4::launch_qqmm_gemm(workspace, dt, w_codes, w_scales, global_scale_w, m,
                                               n, k, out, stream));
}

nvfp4_status nvfp4_qmm(const void* x, nvfp4_dtype dt, const uint8_t* w_codes,
                       const uint8_t* w_scales, const float* global_scale_w, int64_t m, int64_t n,
                       int64_t k, void* out, hipStream_t stream) {
  const char* op = "qmm";
  if (nvfp4_status st = check_matmul(op, x, dt, global_scale_w, w_codes, w_scales, global_scale_w,
                                     m, n, k, out))
    return st;
  if (nvfp4_status st = check_device(op, stream)) return st;
  if (nvfp4::small_m_ok(dt, false, m, n, k))
    return launched(op, nvfp4::launch_small_m(x, dt, false, nullptr, w_codes, w_scales, false,
                                              global_scale_w, m, n, k, out, stream));
  return launched(op, nvfp4::launch_qqmm_gemm(x, dt, w_codes, w_scales, global_scale_w, m, n, k,
                                               out, stream));
}

// ------------------------------------------------------------------ backward

static nvfp4_status check_colwise(const char* op, const void* x, nvfp4_dtype dt, int64_t rows,
                                  int64_t cols) {
  if (!dtype_ok(dt))
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[%s] Unsupported dtype code %d (float32, float16 and bfloat16 only).", op, (int)dt);
  if (rows < 0 || rows % 16 != 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[%s] The quantized dimension (rows, %lld) must be a non-negative multiple of the "
                "group size 16.", op, (long long)rows);
  const int64_t cq = dt == NVFP4_F32 ? 4 : 8;
  if (cols < 0 || cols % cq != 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[%s] cols (%lld) must be a non-negative multiple of %lld.",
                op, (long long)cols, (long long)cq);
  if (rows > INT32_MAX || cols > INT32_MAX)
    return fail(NVFP4_ERR_UNSUPPORTED, "[%s] Sizes too large.", op);
  if (rows > 0 && cols > 0 && (x == nullptr || !aligned(x, 16)))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[%s] input must be non-NULL and 16-byte aligned.", op);
  return NVFP4_OK;
}

nvfp4_status nvfp4_quantize_columnwise(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols,
                                       const float* global_scale, uint8_t* codes, uint8_t* scales,
                                       hipStream_t stream) {
  const char* op = "quantize_columnwise";
  if (nvfp4_status st = check_colwise(op, x, dt, rows, cols)) return st;
  if (rows > 0 && cols > 0) {
    CHECK_PTR("quantize_columnwise", codes);
    CHECK_PTR("quantize_columnwise", scales);
    if (!aligned(codes, 8))
      return fail(NVFP4_ERR_INVALID_ARGUMENT, "[quantize_columnwise] codes must be 8-byte aligned.");
  }
  if (nvfp4_status st = check_device(op, stream)) return st;
  if (rows == 0 || cols == 0) return ok();
  return launched(op, nvfp4::launch_quantize_colwise(x, dt, rows, cols, global_scale, codes, scales,
                                                     stream));
}

nvfp4_status nvfp4_quant_dequant_columnwise(const void* x, nvfp4_dtype dt, int64_t rows,
                                            int64_t cols, const float* global_scale, void* xhat_t,
                                            hipStream_t stream) {
  const char* op = "quant_dequant_columnwise";
  if (nvfp4_status st = check_colwise(op, x, dt, rows, cols)) return st;
  if (rows > 0 && cols > 0 && (xhat_t == nullptr || !aligned(xhat_t, 16)))
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[quant_dequant_columnwise] xhat_t must be non-NULL and 16-byte aligned.");
  if (nvfp4_status st = check_device(op, stream)) return st;
  if (rows == 0 || cols == 0) return ok();
  return launched(op, nvfp4::launch_quant_dequant_colwise(x, dt, rows, cols, global_scale, xhat_t,
                                                          stream));
}

// Workspace of the vjp, each region 256-byte aligned: the cotangent's amax,
// w^T's codes and scales, dy_hat [m, n] (for dx), dy^T_hat [n, m] (for dw),
// x^T's codes and scales.
namespace {
struct VjpLayout {
  size_t g, wc, ws, dyh, dyth, xc, xs, total;
};
size_t up256(size_t b) { return (b + 255) & ~(size_t)255; }
VjpLayout vjp_layout(int64_t m, int64_t n, int64_t k, nvfp4_dtype dt) {
  VjpLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += up256(bytes); return o; };
  L.g = take(sizeof(float));
  L.wc = take((size_t)k * (size_t)n / 2);
  L.ws = take((size_t)k * (size_t)n / 16);
  L.dyh = take((size_t)m * (size_t)n * dtype_size(dt));
  L.dyth = take((size_t)n * (size_t)m * dtype_size(dt));
  L.xc = take((size_t)k * (size_t)m / 2);
  L.xs = take((size_t)k * (size_t)m / 16);
  L.total = off;
  return L;
}

// out [rows, cols] = x_hat @ w^T over kc, x_hat the round trip of x under gx
// (quantize_x) or x itself; w given as codes [cols, kc/2] and scales.
hipError_t contract(const void* x, nvfp4_dtype dt, bool quantize_x, const float* gx,
                    const uint8_t* wc, const uint8_t* ws, const float* gw, int64_t rows,
                    int64_t cols, int64_t kc, void* out, void* xhat_ws, hipStream_t s) {
  if (nvfp4::small_m_ok(dt, false, rows, cols, kc))
    return nvfp4::launch_small_m(x, dt, quantize_x, gx, wc, ws, false, gw, rows, cols, kc, out, s);
  const void* a = x;
  if (quantize_x) {
    hipError_t e = nvfp4::launch_quant_dequant(x, dt, rows, kc, gx, xhat_ws, s);
    if (e != hipSuccess) return e;
    a = xhat_ws;
  }
  return nvfp4::launch_qqmm_gemm(a, dt, wc, ws, gw, rows, cols, kc, out, s);
}
}  // namespace

size_t nvfp4_qqmm_vjp_workspace_size(int64_t m, int64_t n, int64_t k, nvfp4_dtype dt) {
  if (m <= 0 || n <= 0 || k <= 0 || !dtype_ok(dt)) return 0;
  return vjp_layout(m, n, k, dt).total;
}

nvfp4_status nvfp4_qqmm_vjp(const void* x, const void* w, const void* dy, nvfp4_dtype dt,
                            const float* global_scale_x, const float* global_scale_w, int64_t m,
                            int64_t n, int64_t k, void* dx, void* dw, float* dy_amax,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* op = "qqmm_vjp";
  if (!dtype_ok(dt))
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[qqmm_vjp] Unsupported dtype code %d (float32, float16 and bfloat16 only).", (int)dt);
  if (m <= 0 || n <= 0 || k <= 0 || m % 16 != 0 || n % 16 != 0 || k % 16 != 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[qqmm_vjp] m (%lld), n (%lld) and k (%lld) must be positive multiples of 16: each is "
                "the quantized dimension of one operand.", (long long)m, (long long)n, (long long)k);
  if (m > INT32_MAX || n > INT32_MAX || k > INT32_MAX || m * n > (int64_t)1 << 46 ||
      n * k > (int64_t)1 << 46 || m * k > (int64_t)1 << 46)
    return fail(NVFP4_ERR_UNSUPPORTED, "[qqmm_vjp] Sizes too large.");
  if ((global_scale_x == nullptr) != (global_scale_w == nullptr))
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[qqmm_vjp] For nvfp4 mode, either both global_scale_x and global_scale_w must be "
                "provided, or neither.");
  CHECK_PTR("qqmm_vjp", dy);
  if (!dx && !dw) return fail(NVFP4_ERR_INVALID_ARGUMENT, "[qqmm_vjp] dx and dw are both NULL.");
  if (dw) CHECK_PTR("qqmm_vjp", x);
  if (dx) CHECK_PTR("qqmm_vjp", w);
  if ((x && !aligned(x, 16)) || (w && !aligned(w, 16)) || !aligned(dy, 16))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[qqmm_vjp] x, w and dy must be 16-byte aligned.");
  const VjpLayout L = vjp_layout(m, n, k, dt);
  if (workspace == nullptr || workspace_bytes < L.total || !aligned(workspace, 256))
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[qqmm_vjp] workspace of %zu bytes is smaller than %zu or not 256-byte aligned.",
                workspace_bytes, L.total);
  if (nvfp4_status st = check_device(op, stream)) return st;
  char* base = reinterpret_cast<char*>(workspace);
  const bool has_g = global_scale_x != nullptr;
  // the cotangent's global scale: its amax as float32 (none without global scales)
  float* gdy = nullptr;
  if (has_g) {
    gdy = dy_amax ? dy_amax : reinterpret_cast<float*>(base + L.g);
    if (hipError_t e = nvfp4::launch_tensor_amax(dy, dt, m * n, gdy, stream)) return launched(op, e);
  }
  uint8_t* wc = reinterpret_cast<uint8_t*>(base + L.wc);
  uint8_t* ws = reinterpret_cast<uint8_t*>(base + L.ws);
  uint8_t* xc = reinterpret_cast<uint8_t*>(base + L.xc);
  uint8_t* xs = reinterpret_cast<uint8_t*>(base + L.xs);
  if (dx) {
    // dx = qqmm(dy, w^T): w^T [k, n] quantized along n under g_w
    if (hipError_t e = nvfp4::launch_quantize_colwise(w, dt, n, k, global_scale_w, wc, ws, stream))
      return launched(op, e);
    if (hipError_t e = contract(dy, dt, true, gdy, wc, ws, global_scale_w, m, k, n, dx,
                                base + L.dyh, stream))
      return launched(op, e);
  }
  if (dw) {
    // dw = qqmm(dy^T, x^T): dy^T round-tripped along m under g_dy, x^T [k, m]
    // quantized along m under g_x
    void* dyth = base + L.dyth;
    if (hipError_t e = nvfp4::launch_quant_dequant_colwise(dy, dt, m, n, gdy, dyth, stream))
      return launched(op, e);
    if (hipError_t e = nvfp4::launch_quantize_colwise(x, dt, m, k, global_scale_x, xc, xs, stream))
      return launched(op, e);
    if (hipError_t e = contract(dyth, dt, false, nullptr, xc, xs, global_scale_x, n, k, m, dw,
                                nullptr, stream))
      return launched(op, e);
  }
  return ok();
}

namespace {
// the routing tables of a gather: offsets [e + 1], perm [rows] and the
// routing's per-chunk counts, each 256-byte aligned
struct RouteLayout {
  size_t offsets, perm, scratch, total;
};
RouteLayout route_layout(int64_t rows, int64_t e) {
  RouteLayout l;
  l.offsets = 0;
  l.perm = up256((size_t)(e + 1) * sizeof(int32_t));
  l.scratch = l.perm + up256((size_t)rows * sizeof(int32_t));
  l.total = l.scratch + up256(nvfp4::route_scratch_bytes(rows, e));
  return l;
}
}  // namespace

size_t nvfp4_gather_qmm_workspace_size(int64_t t, int64_t top_k, int64_t e, int64_t n,
                                       int64_t k) {
  (void)n;
  (void)k;
  if (t <= 0 || top_k <= 0 || e <= 0 || t * top_k >= ((int64_t)1 << 31)) return 0;
  return route_layout(t * top_k, e).total;
}

size_t nvfp4_moe_route_workspace_size(int64_t t, int64_t top_k, int64_t e) {
  if (t <= 0 || top_k <= 0 || e <= 0 || t * top_k >= ((int64_t)1 << 31)) return 0;
  return up256(nvfp4::route_scratch_bytes(t * top_k, e));
}

nvfp4_status nvfp4_moe_route(const int32_t* expert_idx, int64_t t, int64_t top_k, int64_t e,
                             int32_t* offsets, int32_t* perm, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  const char* op = "moe_route";
  if (t <= 0 || top_k <= 0 || e <= 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[moe_route] t, top_k and e must be positive.");
  if (t * top_k >= ((int64_t)1 << 31))
    return fail(NVFP4_ERR_UNSUPPORTED, "[moe_route] t * top_k must be below 2^31.");
  if (e > 1024)
    return fail(NVFP4_ERR_UNSUPPORTED, "[moe_route] at most 1024 experts are supported.");
  CHECK_PTR("moe_route", expert_idx);
  CHECK_PTR("moe_route", offsets);
  CHECK_PTR("moe_route", perm);
  const size_t need = nvfp4_moe_route_workspace_size(t, top_k, e);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256))
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[moe_route] workspace of %zu bytes is smaller than %zu or not 256-byte aligned.",
                workspace_bytes, need);
  if (nvfp4_status st = check_device(op, stream)) return st;
  return launched(op, nvfp4::launch_moe_route(expert_idx, t * top_k, 1, e, offsets, perm,
                                              reinterpret_cast<int32_t*>(workspace), nullptr, 0,
                                              stream));
}

nvfp4_status nvfp4_gather_qmm(const void* x, nvfp4_dtype dt, const uint8_t* w_codes,
                              const uint8_t* w_scales, const float* global_scale_w,
                              const int32_t* expert_idx, int64_t t, int64_t top_k, int64_t e,
                              int64_t n, int64_t k, void* out, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  const char* op = "gather_qmm";
  if (!dtype_ok(dt))
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[gather_qmm] Unsupported dtype code %d (float32, float16 and bfloat16 only).", (int)dt);
  if (t <= 0 || top_k <= 0 || e <= 0 || n <= 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[gather_qmm] t, top_k, e and n must be positive.");
  if (nvfp4_status st = check_k(op, k)) return st;
  if (!x || !w_codes || !w_scales || !expert_idx || !out)
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[gather_qmm] x, w_codes, w_scales, expert_idx and out must not be NULL.");
  if (!aligned(x, 16) || !aligned(w_codes, 16))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[gather_qmm] x and w_codes must be 16-byte aligned.");
  if (t * top_k >= ((int64_t)1 << 31) || n > INT32_MAX || k > INT32_MAX)
    return fail(NVFP4_ERR_UNSUPPORTED, "[gather_qmm] Sizes too large.");
  if (t * k * (int64_t)dtype_size(dt) >= kOffsetLimit || n * (k / 2) >= kOffsetLimit)
    return fail(NVFP4_ERR_UNSUPPORTED,
                "[gather_qmm] x and one expert's codes must each stay below 2 GB.");
  if (e > 1024)
    return fail(NVFP4_ERR_UNSUPPORTED, "[gather_qmm] at most 1024 experts are supported.");
  size_t need = nvfp4_gather_qmm_workspace_size(t, top_k, e, n, k);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[gather_qmm] workspace of %zu bytes is smaller than %zu.",
                workspace_bytes, need);
  if (!aligned(workspace, 256))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[gather_qmm] workspace must be 256-byte aligned.");
  if (nvfp4_status st = check_device(op, stream)) return st;
  const RouteLayout rl = route_layout(t * top_k, e);
  char* wsb = reinterpret_cast<char*>(workspace);
  int32_t* offsets = reinterpret_cast<int32_t*>(wsb + rl.offsets);
  int32_t* perm = reinterpret_cast<int32_t*>(wsb + rl.perm);
  hipError_t he = nvfp4::launch_moe_route(expert_idx, t * top_k, 1, e, offsets, perm,
                                          reinterpret_cast<int32_t*>(wsb + rl.scratch), out,
                                          n * (int64_t)dtype_size(dt), stream);
  if (he != hipSuccess) return launched(op, he);
  return launched(op, nvfp4::launch_gather_gemm(x, dt, w_codes, w_scales, global_scale_w, offsets,
                                                 perm, t, t * top_k, top_k, nullptr, e, n, k, out,
                                                 stream));
}

nvfp4_status nvfp4_gather_qmm_noalloc(const void* x, nvfp4_dtype dt, const uint8_t* w_codes,
                                      const uint8_t* w_scales, const float* global_scale_w,
                                      const int32_t* expert_idx, int64_t t, int64_t top_k,
                                      int64_t e, int64_t n, int64_t k, void* out,
                                      hipStream_t stream) {
  const char* op = "gather_qmm_noalloc";
  if (!dtype_ok(dt))
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[gather_qmm_noalloc] Unsupported dtype code %d (float32, float16 and bfloat16 only).",
                (int)dt);
  if (t <= 0 || top_k <= 0 || e <= 0 || n <= 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[gather_qmm_noalloc] t, top_k, e and n must be positive.");
  if (nvfp4_status st = check_k(op, k)) return st;
  if (!x || !w_codes || !w_scales || !expert_idx || !out)
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[gather_qmm_noalloc] x, w_codes, w_scales, expert_idx and out must not be NULL.");
  if (!aligned(x, 16) || !aligned(w_codes, 16))
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[gather_qmm_noalloc] x and w_codes must be 16-byte aligned.");
  if (t * top_k >= ((int64_t)1 << 31) || n > INT32_MAX || k > INT32_MAX)
    return fail(NVFP4_ERR_UNSUPPORTED, "[gather_qmm_noalloc] Sizes too large.");
  if (t * k * (int64_t)dtype_size(dt) >= kOffsetLimit || n * (k / 2) >= kOffsetLimit)
    return fail(NVFP4_ERR_UNSUPPORTED,
                "[gather_qmm_noalloc] x and one expert's codes must each stay below 2 GB.");
  if (e > 1024)
    return fail(NVFP4_ERR_UNSUPPORTED, "[gather_qmm_noalloc] at most 1024 experts are supported.");
  const RouteLayout rl = route_layout(t * top_k, e);
  if (rl.total > kNoAllocScratchBytes)
    return fail(NVFP4_ERR_UNSUPPORTED,
                "[gather_qmm_noalloc] the routing tables of %lld pairs and %lld experts need %zu bytes, "
                "above the library's fixed scratch of %zu bytes (use nvfp4_gather_qmm with a workspace).",
                (long long)(t * top_k), (long long)e, rl.total, kNoAllocScratchBytes);
  if (nvfp4_status st = check_device(op, stream)) return st;
  int dev = 0;
  hipError_t he = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (he != hipSuccess)
    return fail(NVFP4_ERR_DEVICE, "[%s] No HIP device behind the stream: %s", op, hipGetErrorString(he));
  void* scratch = nullptr;
  if (nvfp4_status st = noalloc_scratch_of(op, dev, &scratch)) return st;
  char* base = reinterpret_cast<char*>(scratch);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + rl.offsets);
  int32_t* perm = reinterpret_cast<int32_t*>(base + rl.perm);
  he = nvfp4::launch_moe_route(expert_idx, t * top_k, 1, e, offsets, perm,
                               reinterpret_cast<int32_t*>(base + rl.scratch), out,
                               n * (int64_t)dtype_size(dt), stream);
  if (he != hipSuccess) return launched(op, he);
  return launched(op, nvfp4::launch_gather_gemm(x, dt, w_codes, w_scales, global_scale_w, offsets,
                                                 perm, t, t * top_k, top_k, nullptr, e, n, k, out,
                                                 stream));
}

// ------------------------------------------------------------------ packed weights

nvfp4_status nvfp4_mfma_pack_size(int64_t rows, int64_t k, size_t* codes_bytes,
                                  size_t* scales_bytes) {
  CHECK_PTR("mfma_pack_size", codes_bytes);
  CHECK_PTR("mfma_pack_size", scales_bytes);
  *codes_bytes = 0;
  *scales_bytes = 0;
  if (rows <= 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[mfma_pack_size] rows (%lld) must be positive.",
                (long long)rows);
  if (k <= 0 || k % nvfp4::kPackK != 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[mfma_pack_size] k (%lld) must be a positive multiple of 64.", (long long)k);
  const size_t blocks = (size_t)((rows + 31) / 32) * (size_t)(k / nvfp4::kPackK);
  *codes_bytes = blocks * (size_t)nvfp4::kPackCodeBytes;
  *scales_bytes = blocks * (size_t)nvfp4::kPackScaleBytes;
  return ok();
}

nvfp4_status nvfp4_mfma_pack(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                             uint8_t* packed_codes, uint8_t* packed_scales, hipStream_t stream) {
  const char* op = "mfma_pack";
  size_t cb = 0, sb = 0;
  if (nvfp4_status st = nvfp4_mfma_pack_size(rows, k, &cb, &sb)) {
    g_last_error.replace(0, std::strlen("[mfma_pack_size]"), "[mfma_pack]");
    return st;
  }
  CHECK_PTR("mfma_pack", codes);
  CHECK_PTR("mfma_pack", scales);
  CHECK_PTR("mfma_pack", packed_codes);
  CHECK_PTR("mfma_pack", packed_scales);
  if (!aligned(codes, 16) || !aligned(packed_codes, 16) || !aligned(scales, 4) ||
      !aligned(packed_scales, 4))
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[mfma_pack] codes must be 16-byte and scales 4-byte aligned.");
  if (rows > INT32_MAX || k > INT32_MAX)
    return fail(NVFP4_ERR_UNSUPPORTED, "[mfma_pack] Sizes too large.");
  if (nvfp4_status st = check_device(op, stream)) return st;
  return launched(op, nvfp4::launch_mfma_pack(codes, scales, rows, k, packed_codes, packed_scales,
                                              stream));
}

// the packed contractions run only the matrix-core path
static nvfp4_status check_packed(const char* op, nvfp4_dtype dt, int64_t n, int64_t k) {
  if (dt != NVFP4_F16 && dt != NVFP4_BF16)
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[%s] packed weights need float16 or bfloat16 activations (dtype code %d).", op,
                (int)dt);
  if (k % nvfp4::kPackK != 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[%s] packed weights need k (%lld) a multiple of 64.",
                op, (long long)k);
  if (n % 4 != 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[%s] packed weights need n (%lld) a multiple of 4.",
                op, (long long)n);
  return NVFP4_OK;
}

nvfp4_status nvfp4_qqmm_packed(const void* x, nvfp4_dtype dt, const float* global_scale_x,
                               const uint8_t* packed_codes, const uint8_t* packed_scales,
                               const float* global_scale_w, int64_t m, int64_t n, int64_t k,
                               void* out, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  const char* op = "qqmm_packed";
  if (nvfp4_status st = check_matmul(op, x, dt, global_scale_x, packed_codes, packed_scales,
                                     global_scale_w, m, n, k, out))
    return st;
  if (nvfp4_status st = check_packed(op, dt, n, k)) return st;
  size_t need = (size_t)m * (size_t)k * dtype_size(dt);
  if (workspace_bytes < need || workspace == nullptr)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[qqmm_packed] workspace of %zu bytes is smaller than %zu.",
                workspace_bytes, need);
  if (!aligned(workspace, 256))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[qqmm_packed] workspace must be 256-byte aligned.");
  if (nvfp4_status st = check_device(op, stream)) return st;
  if (nvfp4::small_m_ok(dt, true, m, n, k))
    return launched(op, nvfp4::launch_small_m(x, dt, true, global_scale_x, packed_codes,
                                              packed_scales, true, global_scale_w, m, n, k, out,
                                              stream));
  hipError_t e = nvfp4::launch_quant_dequant(x, dt, m, k, global_scale_x, workspace, stream);
  if (e != hipSuccess) return launched(op, e);
  return launched(op, nvfp4::launch_qqmm_gemm_packed(workspace, dt, packed_codes, packed_scales,
                                                      global_scale_w, m, n, k, out, stream));
}

nvfp4_status nvfp4_qmm_packed(const void* x, nvfp4_dtype dt, const uint8_t* packed_codes,
                              const uint8_t* packed_scales, const float* global_scale_w, int64_t m,
                              int64_t n, int64_t k, void* out, hipStream_t stream) {
  const char* op = "qmm_packed";
  if (nvfp4_status st = check_matmul(op, x, dt, global_scale_w, packed_codes, packed_scales,
                                     global_scale_w, m, n, k, out))
    return st;
  if (nvfp4_status st = check_packed(op, dt, n, k)) return st;
  if (nvfp4_status st = check_device(op, stream)) return st;
  if (nvfp4::small_m_ok(dt, true, m, n, k))
    return launched(op, nvfp4::launch_small_m(x, dt, false, nullptr, packed_codes, packed_scales,
                                              true, global_scale_w, m, n, k, out, stream));
  return launched(op, nvfp4::launch_qqmm_gemm_packed(x, dt, packed_codes, packed_scales,
                                                      global_scale_w, m, n, k, out, stream));
}

nvfp4_status nvfp4_gather_qmm_packed(const void* x, nvfp4_dtype dt, const uint8_t* packed_codes,
                                     const uint8_t* packed_scales, const float* global_scale_w,
                                     const int32_t* expert_idx, int64_t t, int64_t top_k,
                                     int64_t e, int64_t n, int64_t k, void* out, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  const char* op = "gather_qmm_packed";
  if (t <= 0 || top_k <= 0 || e <= 0 || n <= 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[gather_qmm_packed] t, top_k, e and n must be positive.");
  if (nvfp4_status st = check_k(op, k)) return st;
  if (nvfp4_status st = check_packed(op, dt, n, k)) return st;
  if (n % 32 != 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[gather_qmm_packed] packed experts need n (%lld) a multiple of 32.", (long long)n);
  if (!x || !packed_codes || !packed_scales || !expert_idx || !out)
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[gather_qmm_packed] x, packed_codes, packed_scales, expert_idx and out must not be NULL.");
  if (!aligned(x, 16) || !aligned(packed_codes, 16))
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[gather_qmm_packed] x and packed_codes must be 16-byte aligned.");
  if (t * top_k >= ((int64_t)1 << 31) || n > INT32_MAX || k > INT32_MAX)
    return fail(NVFP4_ERR_UNSUPPORTED, "[gather_qmm_packed] Sizes too large.");
  if (t * k * (int64_t)dtype_size(dt) >= kOffsetLimit || n * (k / 2) >= kOffsetLimit)
    return fail(NVFP4_ERR_UNSUPPORTED,
                "[gather_qmm_packed] x and one expert's codes must each stay below 2 GB.");
  if (e > 1024)
    return fail(NVFP4_ERR_UNSUPPORTED, "[gather_qmm_packed] at most 1024 experts are supported.");
  size_t need = nvfp4_gather_qmm_workspace_size(t, top_k, e, n, k);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[gather_qmm_packed] workspace of %zu bytes is smaller than %zu.", workspace_bytes, need);
  if (!aligned(workspace, 256))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[gather_qmm_packed] workspace must be 256-byte aligned.");
  if (nvfp4_status st = check_device(op, stream)) return st;
  const RouteLayout rl = route_layout(t * top_k, e);
  char* wsb = reinterpret_cast<char*>(workspace);
  int32_t* offsets = reinterpret_cast<int32_t*>(wsb + rl.offsets);
  int32_t* perm = reinterpret_cast<int32_t*>(wsb + rl.perm);
  hipError_t he = nvfp4::launch_moe_route(expert_idx, t * top_k, 1, e, offsets, perm,
                                          reinterpret_cast<int32_t*>(wsb + rl.scratch), out,
                                          n * (int64_t)dtype_size(dt), stream);
  if (he != hipSuccess) return launched(op, he);
  return launched(op, nvfp4::launch_gather_gemm_packed(x, dt, packed_codes, packed_scales,
                                                       global_scale_w, offsets, perm, t, t * top_k,
                                                       top_k, nullptr, e, n, k, out, stream));
}

// ------------------------------------------------------------------ indexed gather_qmm

namespace {
struct GatherIxLayout {
  size_t offsets, perm, amap, scratch, total;
};
GatherIxLayout gather_ix_layout(int64_t pairs, int64_t mr, int64_t e, bool with_lhs) {
  GatherIxLayout l;
  const size_t rows = (size_t)(pairs * mr);
  l.offsets = 0;
  l.perm = ((size_t)(e + 1) * 4 + 255) & ~(size_t)255;
  l.amap = l.perm + ((rows * 4 + 255) & ~(size_t)255);
  l.scratch = with_lhs ? l.amap + ((rows * 4 + 255) & ~(size_t)255) : l.amap;
  l.total = l.scratch + up256(nvfp4::route_scratch_bytes((int64_t)rows, e));
  return l;
}
}  // namespace

size_t nvfp4_gather_qmm_indexed_workspace_size(int64_t pairs, int64_t rows_per_entry, int64_t e,
                                               int with_lhs) {
  if (pairs <= 0 || rows_per_entry <= 0 || e <= 0) return 0;
  return gather_ix_layout(pairs, rows_per_entry, e, with_lhs != 0).total;
}

nvfp4_status nvfp4_gather_qmm_indexed(const void* x, nvfp4_dtype dt, int64_t entries,
                                      int64_t rows_per_entry, const uint8_t* w_codes,
                                      const uint8_t* w_scales, const float* global_scale_w,
                                      const int32_t* lhs_indices, const int32_t* rhs_indices,
                                      int64_t pairs, int64_t e, int64_t n, int64_t k, int transpose,
                                      int sorted_indices, void* out, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  const char* op = "gather_qmm_indexed";
  if (!dtype_ok(dt))
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[gather_qmm_indexed] Unsupported dtype code %d (float32, float16 and bfloat16 only).",
                (int)dt);
  if (entries <= 0 || rows_per_entry <= 0 || pairs <= 0 || e <= 0 || n <= 0 || k <= 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[gather_qmm_indexed] entries, rows_per_entry, pairs, e, n and k must be positive.");
  if (transpose) {
    if (nvfp4_status st = check_k(op, k)) return st;
  } else {
    if (n % 16 != 0)
      return fail(NVFP4_ERR_INVALID_ARGUMENT,
                  "[gather_qmm_indexed] With transpose = 0 the weights are quantized along n, which "
                  "(%lld) must be a multiple of the group size 16.",
                  (long long)n);
    if (k % 8 != 0)
      return fail(NVFP4_ERR_INVALID_ARGUMENT,
                  "[gather_qmm_indexed] With transpose = 0, k (%lld) must be a multiple of 8.",
                  (long long)k);
  }
  if (!lhs_indices && pairs > entries)
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[gather_qmm_indexed] Without lhs_indices pair p uses x entry p: pairs (%lld) must not "
                "exceed entries (%lld).",
                (long long)pairs, (long long)entries);
  if (!x || !w_codes || !w_scales || !rhs_indices || !out)
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[gather_qmm_indexed] x, w_codes, w_scales, rhs_indices and out must not be NULL.");
  if (!aligned(x, 16) || !aligned(w_codes, 16))
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[gather_qmm_indexed] x and w_codes must be 16-byte aligned.");
  if (pairs * rows_per_entry >= ((int64_t)1 << 31) || entries * rows_per_entry >= ((int64_t)1 << 31) ||
      n > INT32_MAX || k > INT32_MAX)
    return fail(NVFP4_ERR_UNSUPPORTED, "[gather_qmm_indexed] Sizes too large.");
  if (transpose && dt != NVFP4_F32 &&
      (entries * rows_per_entry * k * (int64_t)dtype_size(dt) >= kOffsetLimit ||
       n * (k / 2) >= kOffsetLimit))
    return fail(NVFP4_ERR_UNSUPPORTED,
                "[gather_qmm_indexed] x and one expert's codes must each stay below 2 GB.");
  if (e > 1024)
    return fail(NVFP4_ERR_UNSUPPORTED, "[gather_qmm_indexed] at most 1024 experts are supported.");
  const GatherIxLayout l = gather_ix_layout(pairs, rows_per_entry, e, lhs_indices != nullptr);
  if (workspace == nullptr || workspace_bytes < l.total)
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[gather_qmm_indexed] workspace of %zu bytes is smaller than %zu.", workspace_bytes,
                l.total);
  if (!aligned(workspace, 256))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[gather_qmm_indexed] workspace must be 256-byte aligned.");
  if (nvfp4_status st = check_device(op, stream)) return st;
  char* base = reinterpret_cast<char*>(workspace);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + l.offsets);
  int32_t* perm = reinterpret_cast<int32_t*>(base + l.perm);
  int32_t* amap = lhs_indices ? reinterpret_cast<int32_t*>(base + l.amap) : nullptr;
  const int64_t rows = pairs * rows_per_entry;
  const int64_t row_bytes = n * (int64_t)dtype_size(dt);
  hipError_t he = sorted_indices
                      ? nvfp4::launch_sorted_route(rhs_indices, pairs, rows_per_entry, e, offsets, perm,
                                                   out, row_bytes, stream)
                      : nvfp4::launch_moe_route(rhs_indices, pairs, rows_per_entry, e, offsets, perm,
                                                reinterpret_cast<int32_t*>(base + l.scratch), out,
                                                row_bytes, stream);
  if (he == hipSuccess && amap)
    he = nvfp4::launch_amap(perm, lhs_indices, rows, rows_per_entry, amap, stream);
  if (he == hipSuccess) {
    if (transpose)
      he = nvfp4::launch_gather_gemm(x, dt, w_codes, w_scales, global_scale_w, offsets, perm,
                                     entries * rows_per_entry, rows, 1, amap, e, n, k, out, stream);
    else
      he = nvfp4::launch_gather_gemm_t(x, dt, w_codes, w_scales, global_scale_w, offsets, perm,
                                       entries * rows_per_entry, rows, 1, amap, e, n, k, out, stream);
  }
  return launched(op, he);
}

// ------------------------------------------------------------------ mx modes

static bool mx_mode_ok(int mode) { return mode == NVFP4_MXFP4 || mode == NVFP4_MXFP8; }

static nvfp4_status check_mx(const char* op, const void* x, nvfp4_dtype dt, int mode, int64_t rows,
                             int64_t k) {
  if (!dtype_ok(dt))
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[%s] Unsupported dtype code %d (float32, float16 and bfloat16 only).", op, (int)dt);
  if (!mx_mode_ok(mode))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[%s] Unsupported mx mode %d (4: mxfp4, 8: mxfp8).", op,
                mode);
  if (rows < 0) return fail(NVFP4_ERR_INVALID_ARGUMENT, "[%s] rows (%lld) must be >= 0.", op, (long long)rows);
  if (k <= 0 || k % 32 != 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[%s] The last dimension (%lld) must be a positive multiple of the group size 32.",
                op, (long long)k);
  if (rows > 0 && x == nullptr) return fail(NVFP4_ERR_INVALID_ARGUMENT, "[%s] input must not be NULL.", op);
  if (rows > 0 && !aligned(x, 16))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[%s] input must be 16-byte aligned.", op);
  return NVFP4_OK;
}

nvfp4_status nvfp4_mx_quantize(const void* x, nvfp4_dtype dt, nvfp4_mx_mode mode, int64_t rows,
                               int64_t k, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const char* op = "mx_quantize";
  if (nvfp4_status st = check_mx(op, x, dt, mode, rows, k)) return st;
  if (rows > 0) {
    CHECK_PTR("mx_quantize", codes);
    CHECK_PTR("mx_quantize", scales);
    if (!aligned(codes, 16))
      return fail(NVFP4_ERR_INVALID_ARGUMENT, "[mx_quantize] codes must be 16-byte aligned.");
  }
  if (nvfp4_status st = check_device(op, stream)) return st;
  if (rows == 0) return ok();
  return launched(op, nvfp4::launch_mx_quantize(x, dt, mode, rows, k, codes, scales, stream));
}

nvfp4_status nvfp4_mx_dequantize(const uint8_t* codes, const uint8_t* scales, nvfp4_mx_mode mode,
                                 int64_t rows, int64_t k, void* out, nvfp4_dtype out_dt,
                                 hipStream_t stream) {
  const char* op = "mx_dequantize";
  if (nvfp4_status st = check_mx(op, out, out_dt, mode, rows, k)) return st;
  if (rows > 0) {
    CHECK_PTR("mx_dequantize", codes);
    CHECK_PTR("mx_dequantize", scales);
    if (!aligned(codes, 16))
      return fail(NVFP4_ERR_INVALID_ARGUMENT, "[mx_dequantize] codes must be 16-byte aligned.");
  }
  if (nvfp4_status st = check_device(op, stream)) return st;
  if (rows == 0) return ok();
  return launched(op, nvfp4::launch_mx_dequantize(codes, scales, mode, rows, k, out, out_dt, stream));
}

nvfp4_status nvfp4_mx_quant_dequant(const void* x, nvfp4_dtype dt, nvfp4_mx_mode mode,
                                    int64_t rows, int64_t k, void* x_hat, hipStream_t stream) {
  const char* op = "mx_quant_dequant";
  if (nvfp4_status st = check_mx(op, x, dt, mode, rows, k)) return st;
  if (rows > 0) {
    CHECK_PTR("mx_quant_dequant", x_hat);
    if (!aligned(x_hat, 16))
      return fail(NVFP4_ERR_INVALID_ARGUMENT, "[mx_quant_dequant] x_hat must be 16-byte aligned.");
  }
  if (nvfp4_status st = check_device(op, stream)) return st;
  if (rows == 0) return ok();
  return launched(op, nvfp4::launch_mx_quant_dequant(x, dt, mode, rows, k, x_hat, stream));
}

nvfp4_status nvfp4_mx_pack_size(nvfp4_mx_mode mode, int64_t rows, int64_t k, size_t* codes_bytes,
                                size_t* scales_bytes) {
  CHECK_PTR("mx_pack_size", codes_bytes);
  CHECK_PTR("mx_pack_size", scales_bytes);
  *codes_bytes = 0;
  *scales_bytes = 0;
  if (!mx_mode_ok(mode))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[mx_pack_size] Unsupported mx mode %d (4: mxfp4, 8: mxfp8).",
                (int)mode);
  if (rows <= 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[mx_pack_size] rows (%lld) must be positive.", (long long)rows);
  if (k <= 0 || k % 32 != 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[mx_pack_size] k (%lld) must be a positive multiple of 32.", (long long)k);
  *codes_bytes = nvfp4::mx_packed_code_bytes(rows, k, mode);
  *scales_bytes = nvfp4::mx_packed_scale_bytes(rows, k);
  return ok();
}

nvfp4_status nvfp4_mx_pack(const uint8_t* codes, const uint8_t* scales, nvfp4_mx_mode mode,
                           int64_t rows, int64_t k, uint8_t* packed_codes, uint8_t* packed_scales,
                           hipStream_t stream) {
  const char* op = "mx_pack";
  size_t cb = 0, sb = 0;
  if (nvfp4_status st = nvfp4_mx_pack_size(mode, rows, k, &cb, &sb)) {
    g_last_error.replace(0, std::strlen("[mx_pack_size]"), "[mx_pack]");
    return st;
  }
  CHECK_PTR("mx_pack", codes);
  CHECK_PTR("mx_pack", scales);
  CHECK_PTR("mx_pack", packed_codes);
  CHECK_PTR("mx_pack", packed_scales);
  if (!aligned(codes, 16) || !aligned(packed_codes, 16))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[mx_pack] codes and packed_codes must be 16-byte aligned.");
  if (rows > INT32_MAX || k > INT32_MAX)
    return fail(NVFP4_ERR_UNSUPPORTED, "[mx_pack] Sizes too large.");
  if (nvfp4_status st = check_device(op, stream)) return st;
  return launched(op, nvfp4::launch_mx_pack(codes, scales, mode, rows, k, packed_codes, packed_scales,
                                            stream));
}

nvfp4_status nvfp4_mx_quantize_packed(const void* x, nvfp4_dtype dt, nvfp4_mx_mode mode,
                                      int64_t rows, int64_t k, uint8_t* packed_codes,
                                      uint8_t* packed_scales, hipStream_t stream) {
  const char* op = "mx_quantize_packed";
  if (nvfp4_status st = check_mx(op, x, dt, mode, rows, k)) return st;
  if (rows <= 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[mx_quantize_packed] rows (%lld) must be positive.",
                (long long)rows);
  CHECK_PTR("mx_quantize_packed", packed_codes);
  CHECK_PTR("mx_quantize_packed", packed_scales);
  if (!aligned(packed_codes, 16))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[mx_quantize_packed] packed_codes must be 16-byte aligned.");
  if (rows > INT32_MAX || k > INT32_MAX)
    return fail(NVFP4_ERR_UNSUPPORTED, "[mx_quantize_packed] Sizes too large.");
  if (nvfp4_status st = check_device(op, stream)) return st;
  return launched(op, nvfp4::launch_mx_quantize_packed(x, dt, mode, rows, k, packed_codes,
                                                       packed_scales, stream));
}

nvfp4_status nvfp4_mx_mm_packed(const uint8_t* x_packed_codes, const uint8_t* x_packed_scales,
                                const uint8_t* w_packed_codes, const uint8_t* w_packed_scales,
                                nvfp4_mx_mode mode, int64_t m, int64_t n, int64_t k, void* out,
                                nvfp4_dtype out_dt, hipStream_t stream) {
  const char* op = "mx_mm_packed";
  if (nvfp4_status st = check_mx(op, out, out_dt, mode, m, k)) return st;
  if (m <= 0 || n <= 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[mx_mm_packed] m and n must be positive.");
  if (!x_packed_codes || !x_packed_scales || !w_packed_codes || !w_packed_scales)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[mx_mm_packed] the packed operands must not be NULL.");
  if (!aligned(x_packed_codes, 16) || !aligned(w_packed_codes, 16))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[mx_mm_packed] packed codes must be 16-byte aligned.");
  if (m > INT32_MAX || n > INT32_MAX || k > INT32_MAX ||
      nvfp4::mx_packed_code_bytes(m, k, mode) >= nvfp4::kMxMaxPackedBytes ||
      nvfp4::mx_packed_code_bytes(n, k, mode) >= nvfp4::kMxMaxPackedBytes)
    return fail(NVFP4_ERR_UNSUPPORTED, "[mx_mm_packed] Sizes too large (a packed operand of 2 GB or more).");
  if (nvfp4_status st = check_device(op, stream)) return st;
  return launched(op, nvfp4::launch_mx_gemm(x_packed_codes, x_packed_scales, w_packed_codes,
                                            w_packed_scales, mode, m, n, k, out, out_dt, stream));
}

namespace {
// workspace of the mx contractions: x's packed codes and scales, then (for a
// row-major weight) the weight's packed codes and scales, each 256-aligned
struct MxLayout {
  size_t xc, xs, wc, ws, total;
};
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
MxLayout mx_layout(int mode, int64_t m, int64_t n, int64_t k, bool packed_w) {
  MxLayout l;
  l.xc = 0;
  l.xs = align256(nvfp4::mx_packed_code_bytes(m, k, mode));
  l.wc = l.xs + align256(nvfp4::mx_packed_scale_bytes(m, k));
  if (packed_w) {
    l.ws = l.wc;
    l.total = l.wc;
  } else {
    l.ws = l.wc + align256(nvfp4::mx_packed_code_bytes(n, k, mode));
    l.total = l.ws + align256(nvfp4::mx_packed_scale_bytes(n, k));
  }
  return l;
}
}  // namespace

size_t nvfp4_mx_qqmm_workspace_size(nvfp4_mx_mode mode, int64_t m, int64_t n, int64_t k,
                                    int packed_w) {
  if (!mx_mode_ok(mode) || m <= 0 || n <= 0 || k <= 0 || k % 32 != 0) return 0;
  if (!packed_w && nvfp4::mx_qmv_ok(mode, m, n, k)) return 0;  // the matrix-vector kernel needs none
  return mx_layout(mode, m, n, k, packed_w != 0).total;
}

static nvfp4_status mx_qqmm_common(const char* op, const void* x, nvfp4_dtype dt, int mode,
                                   const uint8_t* wc, const uint8_t* ws, int64_t m, int64_t n,
                                   int64_t k, void* out, void* workspace, size_t workspace_bytes) {
  if (nvfp4_status st = check_mx(op, x, dt, mode, m, k)) return st;
  if (m <= 0 || n <= 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[%s] m and n must be positive.", op);
  if (!x || !wc || !ws || !out)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[%s] x, the weight's codes and scales and out must not be NULL.", op);
  if (!aligned(wc, 16) || !aligned(out, 16))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[%s] the weight's codes and out must be 16-byte aligned.", op);
  if (m > INT32_MAX || n > INT32_MAX || k > INT32_MAX ||
      nvfp4::mx_packed_code_bytes(m, k, mode) >= nvfp4::kMxMaxPackedBytes ||
      nvfp4::mx_packed_code_bytes(n, k, mode) >= nvfp4::kMxMaxPackedBytes)
    return fail(NVFP4_ERR_UNSUPPORTED, "[%s] Sizes too large (a packed operand of 2 GB or more).", op);
  return NVFP4_OK;
}

static nvfp4_status mx_workspace_ok(const char* op, void* workspace, size_t workspace_bytes, size_t need) {
  if (need == 0) return NVFP4_OK;
  if (workspace == nullptr || !aligned(workspace, 256))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[%s] workspace must be a 256-byte aligned device buffer.", op);
  if (workspace_bytes < need)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[%s] workspace of %zu bytes is smaller than %zu.", op,
                workspace_bytes, need);
  return NVFP4_OK;
}

nvfp4_status nvfp4_mx_qqmm(const void* x, nvfp4_dtype dt, nvfp4_mx_mode mode,
                           const uint8_t* w_codes, const uint8_t* w_scales, int64_t m, int64_t n,
                           int64_t k, void* out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  const char* op = "mx_qqmm";
  if (nvfp4_status st =
          mx_qqmm_common(op, x, dt, mode, w_codes, w_scales, m, n, k, out, workspace, workspace_bytes))
    return st;
  const bool qmv = nvfp4::mx_qmv_ok(mode, m, n, k);  // one row of x: the streaming matrix-vector kernel
  const MxLayout l = mx_layout(mode, m, n, k, false);
  if (nvfp4_status st = mx_workspace_ok(op, workspace, workspace_bytes, qmv ? 0 : l.total)) return st;
  if (nvfp4_status st = check_device(op, stream)) return st;
  if (qmv) return launched(op, nvfp4::launch_mx_qmv(x, dt, mode, w_codes, w_scales, n, k, out, stream));
  uint8_t* base = reinterpret_cast<uint8_t*>(workspace);
  hipError_t e = nvfp4::launch_mx_pack(w_codes, w_scales, mode, n, k, base + l.wc, base + l.ws, stream);
  if (e == hipSuccess)
    e = nvfp4::launch_mx_quantize_packed(x, dt, mode, m, k, base + l.xc, base + l.xs, stream);
  if (e == hipSuccess)
    e = nvfp4::launch_mx_gemm(base + l.xc, base + l.xs, base + l.wc, base + l.ws, mode, m, n, k, out,
                              dt, stream);
  return launched(op, e);
}

nvfp4_status nvfp4_mx_qqmm_packed(const void* x, nvfp4_dtype dt, nvfp4_mx_mode mode,
                                  const uint8_t* packed_codes, const uint8_t* packed_scales,
                                  int64_t m, int64_t n, int64_t k, void* out, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  const char* op = "mx_qqmm_packed";
  if (nvfp4_status st = mx_qqmm_common(op, x, dt, mode, packed_codes, packed_scales, m, n, k, out,
                                       workspace, workspace_bytes))
    return st;
  const MxLayout l = mx_layout(mode, m, n, k, true);
  if (nvfp4_status st = mx_workspace_ok(op, workspace, workspace_bytes, l.total)) return st;
  if (nvfp4_status st = check_device(op, stream)) return st;
  uint8_t* base = reinterpret_cast<uint8_t*>(workspace);
  hipError_t e = nvfp4::launch_mx_quantize_packed(x, dt, mode, m, k, base + l.xc, base + l.xs, stream);
  if (e == hipSuccess)
    e = nvfp4::launch_mx_gemm(base + l.xc, base + l.xs, packed_codes, packed_scales, mode, m, n, k,
                              out, dt, stream);
  return launched(op, e);
}

nvfp4_status nvfp4_mx_gather_qmm(const void* x, nvfp4_dtype dt, nvfp4_mx_mode mode,
                                 const uint8_t* w_codes, const uint8_t* w_scales,
                                 const int32_t* expert_idx, int64_t t, int64_t top_k, int64_t e,
                                 int64_t n, int64_t k, void* out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  const char* op = "mx_gather_qmm";
  if (t <= 0 || top_k <= 0 || e <= 0 || n <= 0)
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[mx_gather_qmm] t, top_k, e and n must be positive.");
  if (nvfp4_status st = check_mx(op, x, dt, mode, t, k)) return st;
  if (!w_codes || !w_scales || !expert_idx || !out)
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[mx_gather_qmm] w_codes, w_scales, expert_idx and out must not be NULL.");
  if (!aligned(w_codes, 16))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[mx_gather_qmm] w_codes must be 16-byte aligned.");
  if (t * top_k >= ((int64_t)1 << 31) || n > INT32_MAX || k > INT32_MAX)
    return fail(NVFP4_ERR_UNSUPPORTED, "[mx_gather_qmm] Sizes too large.");
  const int64_t row_bytes = mode == NVFP4_MXFP8 ? k : k / 2;
  if (t * k * (int64_t)dtype_size(dt) >= kOffsetLimit || n * row_bytes >= kOffsetLimit)
    return fail(NVFP4_ERR_UNSUPPORTED,
                "[mx_gather_qmm] x and one expert's codes must each stay below 2 GB.");
  if (e > 1024)
    return fail(NVFP4_ERR_UNSUPPORTED, "[mx_gather_qmm] at most 1024 experts are supported.");
  const size_t need = nvfp4_gather_qmm_workspace_size(t, top_k, e, n, k);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(NVFP4_ERR_INVALID_ARGUMENT,
                "[mx_gather_qmm] workspace of %zu bytes is smaller than %zu.", workspace_bytes, need);
  if (!aligned(workspace, 256))
    return fail(NVFP4_ERR_INVALID_ARGUMENT, "[mx_gather_qmm] workspace must be 256-byte aligned.");
  if (nvfp4_status st = check_device(op, stream)) return st;
  const RouteLayout rl = route_layout(t * top_k, e);
  char* wsb = reinterpret_cast<char*>(workspace);
  int32_t* offsets = reinterpret_cast<int32_t*>(wsb + rl.offsets);
  int32_t* perm = reinterpret_cast<int32_t*>(wsb + rl.perm);
  hipError_t he = nvfp4::launch_moe_route(expert_idx, t * top_k, 1, e, offsets, perm,
                                          reinterpret_cast<int32_t*>(wsb + rl.scratch), out,
                                          n * (int64_t)dtype_size(dt), stream);
  if (he != hipSuccess) return launched(op, he);
  return launched(op, nvfp4::launch_mx_gather_gemm(x, dt, mode, w_codes, w_scales, offsets, perm, t,
                                                    t * top_k, top_k, e, n, k, out, stream));
}

}  // extern "C"
