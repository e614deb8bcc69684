// q4k_api.hip -- the extern "C" boundary of libq4k (declared in include/q4k.h).
//
// Validates arguments on the host (before anything touches the device),
// checks the device once per device id, then enqueues the kernels on the
// caller's stream.  Conventions follow the C API described on the
// "xpu-kernels" page, sections "Use from C" and "API": int status codes, a
// last-error string, an init call, int64 sizes, stream-taking entry points.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/q4k.h"
#include "../../include/w8a8.h"
#include "q4k_launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return Q4K_OK;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];  // 0 unknown, 1 gfx950, -1 unusable
char g_device_name[kMaxDevices][64];

int check_device() {
  int dev = -1;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return fail(Q4K_ERR_DEVICE, "no HIP device is visible");
  }
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return fail(Q4K_ERR_DEVICE, "cannot query the current HIP device");
  }
  int st = g_device_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(Q4K_ERR_DEVICE, "cannot read the properties of device %d", dev);
    }
    snprintf(g_device_name[dev], sizeof g_device_name[dev], "%s", p.gcnArchName);
    st = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_device_state[dev].store(st, std::memory_order_release);
  }
  if (st != 1) {
    return fail(Q4K_ERR_DEVICE, "device %d is %s; libq4k is built for gfx950 only", dev,
                g_device_name[dev]);
  }
  return Q4K_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a+na) and [b, b+nb) overlap (byte ranges)?
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

bool valid_k(int64_t k) { return k >= 256 && k % 256 == 0 && k <= INT32_MAX; }

size_t q4k_bytes(int64_t rows, int64_t k, size_t block = 144u) {
  return static_cast<size_t>(rows) * static_cast<size_t>(k / 256) * block;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    return fail(Q4K_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

extern "C" {

int q4k_version(void) { return 100; }  // 0.1.0

int q4k_init(void) {
  const int rc = check_device();
  return rc == Q4K_OK ? ok() : rc;
}

const char* q4k_device_name(void) {
  const std::string saved = g_last_error;  // a query leaves the last error alone
  (void)check_device();
  g_last_error = saved;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices ||
      g_device_name[dev][0] == 0) {
    (void)hipGetLastError();
    return "none";
  }
  return g_device_name[dev];
}

const char* q4k_last_error(void) { return g_last_error.c_str(); }

// Argument checks shared by the GEMVs of every format (block: bytes per
// super-block of the format), before the device check.
static int gemv_args(const char* what, const void* w, const float* x, const float* y,
                       int64_t m, int64_t n, int64_t k, size_t block) {
  if (!w || !x || !y) return fail(Q4K_ERR_INVALID_ARG, "%s: null pointer", what);
  if (m < 1 || m > Q4K_GEMV_MAX_M)
    return fail(Q4K_ERR_INVALID_ARG, "%s: m=%lld outside 1..%d", what, (long long)m,
                Q4K_GEMV_MAX_M);
  if (n < 1 || n > Q4K_MAX_N) return fail(Q4K_ERR_INVALID_ARG, "%s: n=%lld", what, (long long)n);
  if (!valid_k(k))
    return fail(Q4K_ERR_INVALID_ARG, "%s: k=%lld is not a positive multiple of 256", what,
                (long long)k);
  if (!aligned16(w) || !aligned16(x) || !aligned16(y))
    return fail(Q4K_ERR_ALIGN, "%s: w, x and y must be 16-byte aligned", what);
  const size_t ny = static_cast<size_t>(m * n) * 4;
  if (overlap(y, ny, x, static_cast<size_t>(m * k) * 4) ||
      overlap(y, ny, w, q4k_bytes(n, k, block)))
    return fail(Q4K_ERR_INVALID_ARG, "%s: y overlaps an input", what);
  return Q4K_OK;
}

static int gemv_checks(const char* what, const void* w, const float* x, const float* y,
                       int64_t m, int64_t n, int64_t k, size_t block) {
  if (int rc = gemv_args(what, w, x, y, m, n, k, block)) return rc;
  return check_device();
}

int q4k_gemv(const void* w, const float* x, float* y, int64_t m, int64_t n, int64_t k,
             void* stream) {
  if (int rc = gemv_checks("q4k_gemv", w, x, y, m, n, k, 144u)) return rc;
  return launched(q4k::launch_gemv(static_cast<const uint8_t*>(w), x, y, m, n, k,
                                   static_cast<hipStream_t>(stream)),
                  "q4k_gemv");
}

int q4k_gemv_layers(const void* const* w, const float* const* x, float* const* y,
                    int64_t layers, int64_t n, int64_t k, void* stream) {
  const char* what = "q4k_gemv_layers";
  if (!w || !x || !y) return fail(Q4K_ERR_INVALID_ARG, "%s: null pointer array", what);
  if (layers < 1 || layers > Q4K_LAYERS_MAX)
    return fail(Q4K_ERR_INVALID_ARG, "%s: layers=%lld outside 1..%d", what, (long long)layers,
                Q4K_LAYERS_MAX);
  if (k > Q4K_LAYERS_MAX_K)
    return fail(Q4K_ERR_INVALID_ARG, "%s: k=%lld is above Q4K_LAYERS_MAX_K=%d", what,
                (long long)k, Q4K_LAYERS_MAX_K);
  for (int64_t l = 0; l < layers; ++l) {
    // each layer is a batch-1 GEMV with its own checks
    if (int rc = gemv_args(what, w[l], x[l], y[l], 1, n, k, 144u)) return rc;
  }
  // The layers run concurrently: no output may overlap another layer's
  // inputs or output either.
  const size_t ny = static_cast<size_t>(n) * 4, nx = static_cast<size_t>(k) * 4;
  const size_t nw = q4k_bytes(n, k);
  for (int64_t l = 0; l < layers; ++l)
    for (int64_t j = 0; j < layers; ++j) {
      if (overlap(y[l], ny, x[j], nx) || overlap(y[l], ny, w[j], nw) ||
          (j != l && overlap(y[l], ny, y[j], ny)))
        return fail(Q4K_ERR_INVALID_ARG, "%s: y[%lld] overlaps an input or output of layer %lld",
                    what, (long long)l, (long long)j);
    }
  if (int rc = check_device()) return rc;
  return launched(q4k::launch_gemv_layers(reinterpret_cast<const uint8_t* const*>(w), x, y,
                                          layers, n, k, static_cast<hipStream_t>(stream)),
                  what);
}

int q5k_gemv(const void* w, const float* x, float* y, int64_t m, int64_t n, int64_t k,
             void* stream) {
  if (int rc = gemv_checks("q5k_gemv", w, x, y, m, n, k, 176u)) return rc;
  return launched(q4k::launch_q5k_gemv(static_cast<const uint8_t*>(w), x, y, m, n, k,
                                       static_cast<hipStream_t>(stream)),
                  "q5k_gemv");
}

int q6k_gemv(const void* w, const float* x, float* y, int64_t m, int64_t n, int64_t k,
             void* stream) {
  if (int rc = gemv_checks("q6k_gemv", w, x, y, m, n, k, 210u)) return rc;
  return launched(q4k::launch_q6k_gemv(static_cast<const uint8_t*>(w), x, y, m, n, k,
                                       static_cast<hipStream_t>(stream)),
                  "q6k_gemv");
}

int q3k_gemv(const void* w, const float* x, float* y, int64_t m, int64_t n, int64_t k,
             void* stream) {
  if (int rc = gemv_checks("q3k_gemv", w, x, y, m, n, k, 110u)) return rc;
  return launched(q4k::launch_q3k_gemv(static_cast<const uint8_t*>(w), x, y, m, n, k,
                                       static_cast<hipStream_t>(stream)),
                  "q3k_gemv");
}

// Argument checks shared by the Q4_K and Q5_K GEMMs.
static int gemm_checks(const char* what, const void* w, const uint16_t* x_bf16, const float* y,
                       int64_t m, int64_t n, int64_t k, size_t block) {
  if (!w || !x_bf16 || !y) return fail(Q4K_ERR_INVALID_ARG, "%s: null pointer", what);
  if (m < 1 || m > INT32_MAX) return fail(Q4K_ERR_INVALID_ARG, "%s: m=%lld", what, (long long)m);
  if (n < 1 || n > Q4K_MAX_N) return fail(Q4K_ERR_INVALID_ARG, "%s: n=%lld", what, (long long)n);
  if (!valid_k(k))
    return fail(Q4K_ERR_INVALID_ARG, "%s: k=%lld is not a positive multiple of 256", what,
                (long long)k);
  if (k > Q4K_GEMM_MAX_K)
    return fail(Q4K_ERR_INVALID_ARG, "%s: k=%lld is above Q4K_GEMM_MAX_K=%d", what,
                (long long)k, Q4K_GEMM_MAX_K);
  if (!aligned16(w) || !aligned16(x_bf16) || !aligned16(y))
    return fail(Q4K_ERR_ALIGN, "%s: w, x and y must be 16-byte aligned", what);
  const size_t ny = static_cast<size_t>(m) * static_cast<size_t>(n) * 4;
  if (overlap(y, ny, x_bf16, static_cast<size_t>(m) * static_cast<size_t>(k) * 2) ||
      overlap(y, ny, w, q4k_bytes(n, k, block)))
    return fail(Q4K_ERR_INVALID_ARG, "%s: y overlaps an input", what);
  return check_device();
}

int q4k_gemm(const void* w, const uint16_t* x_bf16, float* y, int64_t m, int64_t n, int64_t k,
             void* stream) {
  if (int rc = gemm_checks("q4k_gemm", w, x_bf16, y, m, n, k, 144u)) return rc;
  return launched(q4k::launch_gemm(static_cast<const uint8_t*>(w), x_bf16, y, m, n, k,
                                   static_cast<hipStream_t>(stream)),
                  "q4k_gemm");
}

int q5k_gemm(const void* w, const uint16_t* x_bf16, float* y, int64_t m, int64_t n, int64_t k,
             void* stream) {
  if (int rc = gemm_checks("q5k_gemm", w, x_bf16, y, m, n, k, 176u)) return rc;
  return launched(q4k::launch_q5k_gemm(static_cast<const uint8_t*>(w), x_bf16, y, m, n, k,
                                       static_cast<hipStream_t>(stream)),
                  "q5k_gemm");
}

int q6k_gemm(const void* w, const uint16_t* x_bf16, float* y, int64_t m, int64_t n, int64_t k,
             void* stream) {
  if (int rc = gemm_checks("q6k_gemm", w, x_bf16, y, m, n, k, 210u)) return rc;
  return launched(q4k::launch_q6k_gemm(static_cast<const uint8_t*>(w), x_bf16, y, m, n, k,
                                       static_cast<hipStream_t>(stream)),
                  "q6k_gemm");
}

int q3k_gemm(const void* w, const uint16_t* x_bf16, float* y, int64_t m, int64_t n, int64_t k,
             void* stream) {
  if (int rc = gemm_checks("q3k_gemm", w, x_bf16, y, m, n, k, 110u)) return rc;
  return launched(q4k::launch_q3k_gemm(static_cast<const uint8_t*>(w), x_bf16, y, m, n, k,
                                       static_cast<hipStream_t>(stream)),
                  "q3k_gemm");
}

// Host checks of the SwiGLU MLP's arguments (h may be the library's own
// scratch, in which case the caller passes h_bytes = 0 to skip its overlap
// checks: the device array overlaps no caller buffer).
static int mlp_checks(const char* what, const void* w_gate, const void* w_up, const void* w_down,
                      const float* x, const float* h, size_t h_bytes, const float* out,
                      int64_t d_model, int64_t d_ff) {
  if (!w_gate || !w_up || !w_down || !x || !h || !out)
    return fail(Q4K_ERR_INVALID_ARG, "%s: null pointer", what);
  if (!valid_k(d_model) || !valid_k(d_ff))
    return fail(Q4K_ERR_INVALID_ARG,
                "%s: d_model=%lld and d_ff=%lld must be positive multiples of 256", what,
                (long long)d_model, (long long)d_ff);
  if (!aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) || !aligned16(x) ||
      !aligned16(h) || !aligned16(out))
    return fail(Q4K_ERR_ALIGN, "%s: all pointers must be 16-byte aligned", what);
  const size_t no = static_cast<size_t>(d_model) * 4;
  const size_t nw = q4k_bytes(d_ff, d_model);
  if (overlap(h, h_bytes, x, no) || overlap(h, h_bytes, w_gate, nw) ||
      overlap(h, h_bytes, w_up, nw) || overlap(h, h_bytes, w_down, nw) ||
      overlap(out, no, x, no) || overlap(out, no, h, h_bytes) || overlap(out, no, w_gate, nw) ||
      overlap(out, no, w_up, nw) || overlap(out, no, w_down, nw))
    return fail(Q4K_ERR_INVALID_ARG, "%s: h or out overlaps another buffer", what);
  return Q4K_OK;
}

// Gate/up + SwiGLU into h, then the down projection of h into out.
static int mlp_launch(const char* what, const void* w_gate, const void* w_up, const void* w_down,
                      const float* x, float* h, float* out, int64_t d_model, int64_t d_ff,
                      void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = q4k::launch_gateup_swiglu(static_cast<const uint8_t*>(w_gate),
                                           static_cast<const uint8_t*>(w_up), x, h, d_model,
                                           d_ff, s);
  if (e != hipSuccess) return launched(e, what);
  e = q4k::launch_gemv(static_cast<const uint8_t*>(w_down), h, out, 1, d_model, d_ff, s);
  return launched(e, what);
}

int q4k_swiglu_mlp(const void* w_gate, const void* w_up, const void* w_down, const float* x,
                   float* h, float* out, int64_t d_model, int64_t d_ff, void* stream) {
  const char* what = "q4k_swiglu_mlp";
  if (int rc = mlp_checks(what, w_gate, w_up, w_down, x, h, static_cast<size_t>(d_ff) * 4, out,
                          d_model, d_ff))
    return rc;
  if (int rc = check_device()) return rc;
  return mlp_launch(what, w_gate, w_up, w_down, x, h, out, d_model, d_ff, stream);
}

// ---- the SwiGLU MLP without allocation -------------------------------------
// h lives in `scratch`, a file-scope device array (each device holds its own
// copy for the life of the process).  Host code never passes the array's name
// to a kernel: the name is a host-side stand-in.  The device address is read
// once per device with hipGetSymbolAddress and kept in g_scratch[dev].
}  // extern "C"

namespace {
static __device__ __align__(256) float scratch[Q4K_NOALLOC_MAX_D_FF];
std::atomic<float*> g_scratch[kMaxDevices];

// This device's address of `scratch`, resolved on first use with the device
// current; nullptr (and the last-error string set) if the runtime refuses.
float* scratch_address(int dev) {
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* a = nullptr;
  const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !a) {
    (void)hipGetLastError();
    fail(Q4K_ERR_DEVICE, "q4k_swiglu_mlp_noalloc: hipGetSymbolAddress failed on device %d: %s",
         dev, hipGetErrorString(e));
    return nullptr;
  }
  p = static_cast<float*>(a);
  g_scratch[dev].store(p, std::memory_order_release);  // same value if two threads race
  return p;
}
}  // namespace

extern "C" {

int q4k_swiglu_mlp_noalloc(const void* w_gate, const void* w_up, const void* w_down,
                           const float* x, float* out, int64_t d_model, int64_t d_ff,
                           void* stream) {
  const char* what = "q4k_swiglu_mlp_noalloc";
  if (d_ff > Q4K_NOALLOC_MAX_D_FF)
    return fail(Q4K_ERR_INVALID_ARG, "%s: d_ff=%lld is above Q4K_NOALLOC_MAX_D_FF=%d", what,
                (long long)d_ff, Q4K_NOALLOC_MAX_D_FF);
  // The scratch address stands in for h in the pointer checks (it is aligned
  // and overlaps no caller buffer); resolve it only after the device check.
  static const float kAligned[4] __attribute__((aligned(16))) = {0, 0, 0, 0};
  if (int rc = mlp_checks(what, w_gate, w_up, w_down, x, kAligned, 0, out, d_model, d_ff))
    return rc;
  if (int rc = check_device()) return rc;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return fail(Q4K_ERR_DEVICE, "%s: cannot query the current HIP device", what);
  }
  float* h = scratch_address(dev);
  if (!h) return Q4K_ERR_DEVICE;
  return mlp_launch(what, w_gate, w_up, w_down, x, h, out, d_model, d_ff, stream);
}

static int dequant_checks(const char* what, const void* w, const void* out, int64_t n,
                          int64_t k, size_t elem, size_t block = 144u) {
  if (!w || !out) return fail(Q4K_ERR_INVALID_ARG, "%s: null pointer", what);
  if (n < 1 || n > INT32_MAX) return fail(Q4K_ERR_INVALID_ARG, "%s: n=%lld", what, (long long)n);
  if (!valid_k(k))
    return fail(Q4K_ERR_INVALID_ARG, "%s: k=%lld is not a positive multiple of 256", what,
                (long long)k);
  if (!aligned16(w) || !aligned16(out))
    return fail(Q4K_ERR_ALIGN, "%s: w and out must be 16-byte aligned", what);
  if (overlap(out, static_cast<size_t>(n) * static_cast<size_t>(k) * elem, w,
              q4k_bytes(n, k, block)))
    return fail(Q4K_ERR_INVALID_ARG, "%s: out overlaps w", what);
  return check_device();
}

int q4k_dequantize_f32(const void* w, float* out, int64_t n, int64_t k, void* stream) {
  if (int rc = dequant_checks("q4k_dequantize_f32", w, out, n, k, 4)) return rc;
  return launched(q4k::launch_dequant_f32(static_cast<const uint8_t*>(w), out, n, k,
                                          static_cast<hipStream_t>(stream)),
                  "q4k_dequantize_f32");
}

int q4k_dequantize_bf16(const void* w, uint16_t* out, int64_t n, int64_t k, void* stream) {
  if (int rc = dequant_checks("q4k_dequantize_bf16", w, out, n, k, 2)) return rc;
  return launched(q4k::launch_dequant_bf16(static_cast<const uint8_t*>(w), out, n, k,
                                           static_cast<hipStream_t>(stream)),
                  "q4k_dequantize_bf16");
}

int q5k_dequantize_f32(const void* w, float* out, int64_t n, int64_t k, void* stream) {
  if (int rc = dequant_checks("q5k_dequantize_f32", w, out, n, k, 4, 176u)) return rc;
  return launched(q4k::launch_q5k_dequant_f32(static_cast<const uint8_t*>(w), out, n, k,
                                              static_cast<hipStream_t>(stream)),
                  "q5k_dequantize_f32");
}

int q5k_dequantize_bf16(const void* w, uint16_t* out, int64_t n, int64_t k, void* stream) {
  if (int rc = dequant_checks("q5k_dequantize_bf16", w, out, n, k, 2, 176u)) return rc;
  return launched(q4k::launch_q5k_dequant_bf16(static_cast<const uint8_t*>(w), out, n, k,
                                               static_cast<hipStream_t>(stream)),
                  "q5k_dequantize_bf16");
}

int q6k_dequantize_f32(const void* w, float* out, int64_t n, int64_t k, void* stream) {
  if (int rc = dequant_checks("q6k_dequantize_f32", w, out, n, k, 4, 210u)) return rc;
  return launched(q4k::launch_q6k_dequant_f32(static_cast<const uint8_t*>(w), out, n, k,
                                              static_cast<hipStream_t>(stream)),
                  "q6k_dequantize_f32");
}

int q6k_dequantize_bf16(const void* w, uint16_t* out, int64_t n, int64_t k, void* stream) {
  if (int rc = dequant_checks("q6k_dequantize_bf16", w, out, n, k, 2, 210u)) return rc;
  return launched(q4k::launch_q6k_dequant_bf16(static_cast<const uint8_t*>(w), out, n, k,
                                               static_cast<hipStream_t>(stream)),
                  "q6k_dequantize_bf16");
}

int q3k_dequantize_f32(const void* w, float* out, int64_t n, int64_t k, void* stream) {
  if (int rc = dequant_checks("q3k_dequantize_f32", w, out, n, k, 4, 110u)) return rc;
  return launched(q4k::launch_q3k_dequant_f32(static_cast<const uint8_t*>(w), out, n, k,
                                              static_cast<hipStream_t>(stream)),
                  "q3k_dequantize_f32");
}

int q3k_dequantize_bf16(const void* w, uint16_t* out, int64_t n, int64_t k, void* stream) {
  if (int rc = dequant_checks("q3k_dequantize_bf16", w, out, n, k, 2, 110u)) return rc;
  return launched(q4k::launch_q3k_dequant_bf16(static_cast<const uint8_t*>(w), out, n, k,
                                               static_cast<hipStream_t>(stream)),
                  "q3k_dequantize_bf16");
}

int q4k_read_probe(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return fail(Q4K_ERR_INVALID_ARG, "q4k_read_probe: null pointer");
  if (bytes < 16 || bytes % 16 != 0)
    return fail(Q4K_ERR_INVALID_ARG, "q4k_read_probe: bytes=%lld is not a positive multiple of 16",
                (long long)bytes);
  if (!aligned16(buf) || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return fail(Q4K_ERR_ALIGN, "q4k_read_probe: buf must be 16-byte and sink 4-byte aligned");
  if (overlap(sink, 4, buf, static_cast<size_t>(bytes)))
    return fail(Q4K_ERR_INVALID_ARG, "q4k_read_probe: sink overlaps buf");
  if (int rc = check_device()) return rc;
  return launched(q4k::launch_read_probe(buf, bytes, sink, static_cast<hipStream_t>(stream)),
                  "q4k_read_probe");
}

// ---------------------------------------------------------------- INT8 W8A8

static bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Shared by the two GEMM entry points: sizes, alignment of x and w, and the
// output range [out, out + out_bytes) against the inputs.
static int w8a8_gemm_checks(const char* what, const int8_t* x, const int8_t* w, const void* out,
                            size_t out_elem, int64_t m, int64_t n, int64_t k) {
  if (!x || !w || !out) return fail(Q4K_ERR_INVALID_ARG, "%s: null pointer", what);
  if (m < 1 || m > INT32_MAX) return fail(Q4K_ERR_INVALID_ARG, "%s: m=%lld", what, (long long)m);
  if (n < 1 || n > INT32_MAX) return fail(Q4K_ERR_INVALID_ARG, "%s: n=%lld", what, (long long)n);
  if (k < W8A8_K_STEP || k % W8A8_K_STEP != 0 || k > W8A8_MAX_K)
    return fail(Q4K_ERR_INVALID_ARG, "%s: k=%lld is not a multiple of %d in %d..%d", what,
                (long long)k, W8A8_K_STEP, W8A8_K_STEP, W8A8_MAX_K);
  if (!aligned16(x) || !aligned16(w) || !aligned16(out))
    return fail(Q4K_ERR_ALIGN, "%s: x, w and the output must be 16-byte aligned", what);
  const size_t no = static_cast<size_t>(m) * static_cast<size_t>(n) * out_elem;
  if (overlap(out, no, x, static_cast<size_t>(m) * static_cast<size_t>(k)) ||
      overlap(out, no, w, static_cast<size_t>(n) * static_cast<size_t>(k)))
    return fail(Q4K_ERR_INVALID_ARG, "%s: the output overlaps x or w", what);
  return Q4K_OK;
}

// Scales and bias of an epilogue writing `out` (bf16 [m, n]).
static int w8a8_vector_checks(const char* what, const float* x_scale, const float* w_scale,
                              const float* bias, const void* out, int64_t m, int64_t n) {
  if (!x_scale || !w_scale) return fail(Q4K_ERR_INVALID_ARG, "%s: null scale pointer", what);
  if (!aligned4(x_scale) || !aligned4(w_scale) || (bias && !aligned4(bias)))
    return fail(Q4K_ERR_ALIGN, "%s: x_scale, w_scale and bias must be 4-byte aligned", what);
  const size_t no = static_cast<size_t>(m) * static_cast<size_t>(n) * 2;
  if (overlap(out, no, x_scale, static_cast<size_t>(m) * 4) ||
      overlap(out, no, w_scale, static_cast<size_t>(n) * 4) ||
      (bias && overlap(out, no, bias, static_cast<size_t>(n) * 4)))
    return fail(Q4K_ERR_INVALID_ARG, "%s: out overlaps a scale or the bias", what);
  return Q4K_OK;
}

int w8a8_linear(const int8_t* x, const float* x_scale, const int8_t* w, const float* w_scale,
                const float* bias, uint16_t* out, int64_t m, int64_t n, int64_t k,
                void* stream) {
  const char* what = "w8a8_linear";
  if (int rc = w8a8_gemm_checks(what, x, w, out, 2, m, n, k)) return rc;
  if (int rc = w8a8_vector_checks(what, x_scale, w_scale, bias, out, m, n)) return rc;
  if (int rc = check_device()) return rc;
  return launched(q4k::launch_w8a8_linear(x, x_scale, w, w_scale, bias, out, m, n, k,
                                          static_cast<hipStream_t>(stream)),
                  what);
}

int w8a8_linear_acc(const int8_t* x, const int8_t* w, int32_t* acc, int64_t m, int64_t n,
                    int64_t k, void* stream) {
  const char* what = "w8a8_linear_acc";
  if (int rc = w8a8_gemm_checks(what, x, w, acc, 4, m, n, k)) return rc;
  if (int rc = check_device()) return rc;
  return launched(q4k::launch_w8a8_linear_acc(x, w, acc, m, n, k,
                                              static_cast<hipStream_t>(stream)),
                  what);
}

int w8a8_dequant_epilogue(const int32_t* acc, uint16_t* out, const float* x_scale,
                          const float* w_scale, const float* bias, int64_t m, int64_t n,
                          void* stream) {
  const char* what = "w8a8_dequant_epilogue";
  if (!acc || !out) return fail(Q4K_ERR_INVALID_ARG, "%s: null pointer", what);
  if (m < 1 || m > INT32_MAX) return fail(Q4K_ERR_INVALID_ARG, "%s: m=%lld", what, (long long)m);
  if (n < 1 || n > INT32_MAX) return fail(Q4K_ERR_INVALID_ARG, "%s: n=%lld", what, (long long)n);
  if (!aligned16(acc) || !aligned16(out))
    return fail(Q4K_ERR_ALIGN, "%s: acc and out must be 16-byte aligned", what);
  if (overlap(out, static_cast<size_t>(m) * static_cast<size_t>(n) * 2, acc,
              static_cast<size_t>(m) * static_cast<size_t>(n) * 4))
    return fail(Q4K_ERR_INVALID_ARG, "%s: out overlaps acc", what);
  if (int rc = w8a8_vector_checks(what, x_scale, w_scale, bias, out, m, n)) return rc;
  if (int rc = check_device()) return rc;
  return launched(q4k::launch_w8a8_epilogue(acc, out, x_scale, w_scale, bias, m, n,
                                            static_cast<hipStream_t>(stream)),
                  what);
}

int w8a8_quantize_rows(const uint16_t* x_bf16, int8_t* q, float* scale, int64_t rows, int64_t k,
                       void* stream) {
  const char* what = "w8a8_quantize_rows";
  if (!x_bf16 || !q || !scale) return fail(Q4K_ERR_INVALID_ARG, "%s: null pointer", what);
  if (rows < 1 || rows > INT32_MAX)
    return fail(Q4K_ERR_INVALID_ARG, "%s: rows=%lld", what, (long long)rows);
  if (k < 8 || k % 8 != 0 || k > INT32_MAX)
    return fail(Q4K_ERR_INVALID_ARG, "%s: k=%lld is not a positive multiple of 8", what,
                (long long)k);
  if (!aligned16(x_bf16) || !aligned16(q) || !aligned4(scale))
    return fail(Q4K_ERR_ALIGN, "%s: x and q must be 16-byte and scale 4-byte aligned", what);
  const size_t nx = static_cast<size_t>(rows) * static_cast<size_t>(k);
  if (overlap(q, nx, x_bf16, nx * 2) || overlap(scale, static_cast<size_t>(rows) * 4, x_bf16, nx * 2) ||
      overlap(scale, static_cast<size_t>(rows) * 4, q, nx))
    return fail(Q4K_ERR_INVALID_ARG, "%s: outputs overlap", what);
  if (int rc = check_device()) return rc;
  return launched(q4k::launch_w8a8_quantize_rows(x_bf16, q, scale, rows, k,
                                                 static_cast<hipStream_t>(stream)),
                  what);
}

}  // extern "C"
