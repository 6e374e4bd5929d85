// C-ABI layer: host-side argument validation and kernel launches for the
// entry points declared in include/svdq.h.  Every check happens before any
// HIP call; no exception leaves this file.
#include <atomic>
#include <mutex>

#include "../../include/svdq.h"
#include "kernels.h"

using namespace svdq;

// svdq_linear_noalloc's workspace: a static device array, one per GPU the library runs on (each
// holds its own copy, at its own address, until the process ends).  In host code `scratch` is
// only a stand-in for the symbol: its device address comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[SVDQ_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDim = 1 << 24;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

inline bool fmt_ok(int f) {
  return f == SVDQ_INT4_G64 || f == SVDQ_INT8_G64 || f == SVDQ_FP4_G16 || f == SVDQ_INT4_G64_E2M3 ||
         f == SVDQ_MXFP4_G32;
}

inline size_t code_bytes(int K, int fmt) {
  if (fmt == SVDQ_INT8_G64) return (size_t)K;
  if (fmt == SVDQ_INT4_G64_E2M3) return (size_t)K / 4 * 3;
  return (size_t)K / 2;
}
inline size_t scale_bytes(int K, int fmt) {
  return fmt == SVDQ_FP4_G16 ? (size_t)K / 16 : (fmt == SVDQ_MXFP4_G32 ? (size_t)K / 32 : (size_t)K / 64 * 2);
}

svdq_status check_dims(int M, int N, int K, int r) {
  if (M < 0 || N < 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return SVDQ_ERR_SHAPE;
  if (K % 64 != 0 || N % 16 != 0) return SVDQ_ERR_SHAPE;
  if (r < 0 || r > 64 || r % 16 != 0) return SVDQ_ERR_SHAPE;
  return SVDQ_OK;
}

svdq_status map_launch(hipError_t e) {
  if (e == hipSuccess) return SVDQ_OK;
  if (e == hipErrorNoBinaryForGpu || e == hipErrorInvalidDeviceFunction) return SVDQ_ERR_DEVICE;
  return SVDQ_ERR_LAUNCH;
}

struct Workspace {
  void* xq; void* xs; void* t; void* part; size_t part_bytes; void* y0; size_t total;
};

// Kernel A's partial sums of T (0 bytes when its K is not sliced)
// Kernel A's partial sums (the plain and the smoothing variant slice K alike)
size_t partial_bytes(int M, int K, int r) { return round256(quant_down_plan(M, K, r, true, false).partial_bytes); }

Workspace carve(void* base, int M, int N, int K, int r, int fmt, bool with_y0) {
  Workspace w{};
  size_t off = 0;
  char* b = static_cast<char*>(base);
  w.xq = b ? b + off : nullptr; off += round256((size_t)M * code_bytes(K, fmt));
  w.xs = b ? b + off : nullptr; off += round256((size_t)M * scale_bytes(K, fmt));
  w.t = (r > 0 && b) ? b + off : nullptr; off += round256((size_t)M * r * 2);
  w.part_bytes = partial_bytes(M, K, r);
  w.part = (w.part_bytes && b) ? b + off : nullptr; off += w.part_bytes;
  if (with_y0) { w.y0 = b ? b + off : nullptr; off += round256((size_t)M * N * 2); }
  w.total = off;
  return w;
}

svdq_status check_quant_down(const void* x_hat, const void* l1t, int M, int K, int r, int fmt,
                             const void* xq, const void* xs, const void* t) {
  if (!fmt_ok(fmt)) return SVDQ_ERR_FORMAT;
  svdq_status st = check_dims(M, 16, K, r);
  if (st != SVDQ_OK) return st;
  if (M == 0) return SVDQ_OK;
  if (!x_hat || !xq || !xs) return SVDQ_ERR_NULL;
  if (r > 0 && (!l1t || !t)) return SVDQ_ERR_NULL;
  if (!aligned16(x_hat) || !aligned16(xq) || !aligned16(xs)) return SVDQ_ERR_ALIGN;
  if (r > 0 && (!aligned16(l1t) || !aligned16(t))) return SVDQ_ERR_ALIGN;
  return SVDQ_OK;
}

svdq_status check_gemm(const void* xq, const void* xs, const void* t, const void* wq, const void* ws,
                       const void* l2, const void* bias, int M, int N, int K, int r, int fmt,
                       const void* y) {
  if (!fmt_ok(fmt)) return SVDQ_ERR_FORMAT;
  svdq_status st = check_dims(M, N, K, r);
  if (st != SVDQ_OK) return st;
  // the GEMM kernels address each code operand with 32-bit byte offsets
  if (((size_t)M * code_bytes(K, (svdq_format)fmt) >= (1ull << 32) ||
       (size_t)N * code_bytes(K, (svdq_format)fmt) >= (1ull << 32)))
    return SVDQ_ERR_SHAPE;
  if (M == 0 || N == 0) return SVDQ_OK;
  if (!xq || !xs || !wq || !ws || !y) return SVDQ_ERR_NULL;
  if (r > 0 && (!t || !l2)) return SVDQ_ERR_NULL;
  if (!aligned16(xq) || !aligned16(xs) || !aligned16(wq) || !aligned16(ws) || !aligned16(y)) return SVDQ_ERR_ALIGN;
  if (r > 0 && (!aligned16(t) || !aligned16(l2))) return SVDQ_ERR_ALIGN;
  if (bias && !aligned16(bias)) return SVDQ_ERR_ALIGN;
  return SVDQ_OK;
}

// The device address of `scratch` on the current device, looked up on the first call made on
// that device and kept: lookups are serialized by a mutex, readers take the published value.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

svdq_status static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SVDQ_ERR_DEVICE;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SVDQ_ERR_DEVICE;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SVDQ_OK;
}

// svdq_linear's work once the workspace is known: checks of the carved buffers, Kernel A, Kernel B.
svdq_status run_linear(const void* x_hat, const void* l1t, const void* wq, const void* ws, const void* l2,
                       const void* bias, int M, int N, int K, int r, int fmt, const Workspace& w, void* y,
                       hipStream_t s) {
  svdq_status st = check_quant_down(x_hat, l1t, M, K, r, fmt, w.xq, w.xs, w.t);
  if (st != SVDQ_OK) return st;
  st = check_gemm(w.xq, w.xs, w.t, wq, ws, l2, bias, M, N, K, r, fmt, y);
  if (st != SVDQ_OK) return st;
  QuantDownArgs qa{x_hat, l1t, M, K, r, fmt, w.xq, w.xs, w.t, w.part, w.part_bytes};
  st = map_launch(launch_quant_down(qa, s));
  if (st != SVDQ_OK) return st;
  GemmArgs ga{w.xq, w.xs, w.t, wq, ws, l2, bias, M, N, K, r, fmt, y};
  return map_launch(launch_gemm(ga, s));
}

}  // namespace

extern "C" {

size_t svdq_code_row_bytes(int K, svdq_format fmt) {
  if (!fmt_ok(fmt) || K <= 0 || K % 64) return 0;
  return code_bytes(K, fmt);
}

size_t svdq_scale_row_bytes(int K, svdq_format fmt) {
  if (!fmt_ok(fmt) || K <= 0 || K % 64) return 0;
  return scale_bytes(K, fmt);
}

size_t svdq_quantize_down_workspace_bytes(int M, int K, int r, svdq_format fmt) {
  if (!fmt_ok(fmt) || check_dims(M, 16, K, r) != SVDQ_OK) return 0;
  return partial_bytes(M, K, r);
}

svdq_status svdq_quantize_down(const void* x_hat, const void* l1t, int M, int K, int r, svdq_format fmt,
                               void* xq, void* xs, void* t, void* workspace, size_t workspace_bytes,
                               void* stream) {
  svdq_status st = check_quant_down(x_hat, l1t, M, K, r, fmt, xq, xs, t);
  if (st != SVDQ_OK) return st;
  if (M == 0) return SVDQ_OK;
  // a workspace, when given, must hold the partial sums; without one K is not sliced
  const size_t need = partial_bytes(M, K, r);
  if (workspace && need) {
    if (!aligned16(workspace)) return SVDQ_ERR_ALIGN;
    if (workspace_bytes < need) return SVDQ_ERR_WORKSPACE;
  }
  QuantDownArgs a{x_hat, l1t, M, K, r, (int)fmt, xq, xs, t, need ? workspace : nullptr, need ? workspace_bytes : 0};
  return map_launch(launch_quant_down(a, static_cast<hipStream_t>(stream)));
}

svdq_status svdq_gemm_w4a4_up(const void* xq, const void* xs, const void* t, const void* wq, const void* ws,
                              const void* l2, const void* bias, int M, int N, int K, int r, svdq_format fmt,
                              void* y, void* stream) {
  svdq_status st = check_gemm(xq, xs, t, wq, ws, l2, bias, M, N, K, r, fmt, y);
  if (st != SVDQ_OK) return st;
  if (M == 0 || N == 0) return SVDQ_OK;
  GemmArgs a{xq, xs, t, wq, ws, l2, bias, M, N, K, r, (int)fmt, y};
  return map_launch(launch_gemm(a, static_cast<hipStream_t>(stream)));
}

size_t svdq_linear_workspace_bytes(int M, int K, int r, svdq_format fmt) {
  if (!fmt_ok(fmt) || check_dims(M, 16, K, r) != SVDQ_OK) return 0;
  return carve(nullptr, M, 0, K, r, fmt, false).total;
}

svdq_status svdq_linear(const void* x_hat, const void* l1t, const void* wq, const void* ws, const void* l2,
                        const void* bias, int M, int N, int K, int r, svdq_format fmt, void* workspace,
                        size_t workspace_bytes, void* y, void* stream) {
  if (!fmt_ok(fmt)) return SVDQ_ERR_FORMAT;
  svdq_status st = check_dims(M, N, K, r);
  if (st != SVDQ_OK) return st;
  if (M == 0 || N == 0) return SVDQ_OK;
  if (!x_hat || !wq || !ws || !y || !workspace) return SVDQ_ERR_NULL;
  if (r > 0 && (!l1t || !l2)) return SVDQ_ERR_NULL;
  if (!aligned16(workspace)) return SVDQ_ERR_ALIGN;
  const Workspace w = carve(workspace, M, N, K, r, fmt, false);
  if (workspace_bytes < w.total) return SVDQ_ERR_WORKSPACE;
  return run_linear(x_hat, l1t, wq, ws, l2, bias, M, N, K, r, (int)fmt, w, y, static_cast<hipStream_t>(stream));
}

svdq_status svdq_linear_noalloc(const void* x_hat, const void* l1t, const void* wq, const void* ws, const void* l2,
                                const void* bias, int M, int N, int K, int r, svdq_format fmt, void* y,
                                void* stream) {
  if (!fmt_ok(fmt)) return SVDQ_ERR_FORMAT;
  svdq_status st = check_dims(M, N, K, r);
  if (st != SVDQ_OK) return st;
  if (M == 0 || N == 0) return SVDQ_OK;
  if (!x_hat || !wq || !ws || !y) return SVDQ_ERR_NULL;
  if (r > 0 && (!l1t || !l2)) return SVDQ_ERR_NULL;
  // the whole workspace (codes, scales, T, Kernel A's partial sums) must fit the static array
  if (carve(nullptr, M, N, K, r, fmt, false).total > (size_t)SVDQ_STATIC_SCRATCH_BYTES) return SVDQ_ERR_WORKSPACE;
  void* base = nullptr;
  st = static_scratch(&base);
  if (st != SVDQ_OK) return st;
  const Workspace w = carve(base, M, N, K, r, fmt, false);
  return run_linear(x_hat, l1t, wq, ws, l2, bias, M, N, K, r, (int)fmt, w, y, static_cast<hipStream_t>(stream));
}

svdq_status svdq_quantize_down_smooth(const void* x, const float* lambda, const void* l1t, int M, int K, int r,
                                      svdq_format fmt, void* xq, void* xs, void* t, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  svdq_status st = check_quant_down(x, l1t, M, K, r, fmt, xq, xs, t);
  if (st != SVDQ_OK) return st;
  if (M == 0) return SVDQ_OK;
  if (!lambda) return SVDQ_ERR_NULL;
  if (!aligned16(lambda)) return SVDQ_ERR_ALIGN;
  const size_t need = partial_bytes(M, K, r);
  if (workspace && need) {
    if (!aligned16(workspace)) return SVDQ_ERR_ALIGN;
    if (workspace_bytes < need) return SVDQ_ERR_WORKSPACE;
  }
  QuantDownArgs a{x, l1t, M, K, r, (int)fmt, xq, xs, t, need ? workspace : nullptr, need ? workspace_bytes : 0, lambda};
  return map_launch(launch_quant_down(a, static_cast<hipStream_t>(stream)));
}

svdq_status svdq_gemm_w4a4_up_gelu_smooth(const void* xq, const void* xs, const void* t, const void* wq,
                                          const void* ws, const void* l2, const void* bias,
                                          const float* lambda_next, int M, int N, int K, int r, svdq_format fmt,
                                          void* y, void* stream) {
  svdq_status st = check_gemm(xq, xs, t, wq, ws, l2, bias, M, N, K, r, fmt, y);
  if (st != SVDQ_OK) return st;
  if (M == 0 || N == 0) return SVDQ_OK;
  if (!lambda_next) return SVDQ_ERR_NULL;
  if (!aligned16(lambda_next)) return SVDQ_ERR_ALIGN;
  GemmArgs a{xq, xs, t, wq, ws, l2, bias, M, N, K, r, (int)fmt, y, lambda_next};
  return map_launch(launch_gemm(a, static_cast<hipStream_t>(stream)));
}

svdq_status svdq_linear_folded(const void* x, const float* lambda_in, const void* l1t, const void* wq,
                               const void* ws, const void* l2, const void* bias, const float* lambda_next, int M,
                               int N, int K, int r, svdq_format fmt, void* workspace, size_t workspace_bytes,
                               void* y, void* stream) {
  if (!fmt_ok(fmt)) return SVDQ_ERR_FORMAT;
  svdq_status st = check_dims(M, N, K, r);
  if (st != SVDQ_OK) return st;
  if (M == 0 || N == 0) return SVDQ_OK;
  if (!x || !wq || !ws || !y || !workspace) return SVDQ_ERR_NULL;
  if (r > 0 && (!l1t || !l2)) return SVDQ_ERR_NULL;
  if (!aligned16(workspace)) return SVDQ_ERR_ALIGN;
  if ((lambda_in && !aligned16(lambda_in)) || (lambda_next && !aligned16(lambda_next))) return SVDQ_ERR_ALIGN;
  const Workspace w = carve(workspace, M, N, K, r, fmt, false);
  if (workspace_bytes < w.total) return SVDQ_ERR_WORKSPACE;
  st = check_quant_down(x, l1t, M, K, r, fmt, w.xq, w.xs, w.t);
  if (st != SVDQ_OK) return st;
  st = check_gemm(w.xq, w.xs, w.t, wq, ws, l2, bias, M, N, K, r, fmt, y);
  if (st != SVDQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  QuantDownArgs qa{x, l1t, M, K, r, (int)fmt, w.xq, w.xs, w.t, w.part, w.part_bytes, lambda_in};
  st = map_launch(launch_quant_down(qa, s));
  if (st != SVDQ_OK) return st;
  GemmArgs ga{w.xq, w.xs, w.t, wq, ws, l2, bias, M, N, K, r, (int)fmt, y, lambda_next};
  return map_launch(launch_gemm(ga, s));
}

svdq_status svdq_pack_weight(const int8_t* codes, const void* scales, int N, int K, svdq_format fmt, void* wq,
                             void* ws, void* stream) {
  if (!fmt_ok(fmt)) return SVDQ_ERR_FORMAT;
  if (fmt != SVDQ_INT4_G64 && fmt != SVDQ_INT4_G64_E2M3 && fmt != SVDQ_INT8_G64) return SVDQ_ERR_FORMAT;
  if (N < 0 || K <= 0 || K % 64 != 0 || N % 16 != 0 || N > kMaxDim || K > kMaxDim) return SVDQ_ERR_SHAPE;
  if (N == 0) return SVDQ_OK;
  if (!codes || !scales || !wq || !ws) return SVDQ_ERR_NULL;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(wq) || !aligned16(ws)) return SVDQ_ERR_ALIGN;
  return map_launch(launch_pack_weight(codes, static_cast<const uint16_t*>(scales), N, K, (int)fmt, wq, ws,
                                       static_cast<hipStream_t>(stream)));
}

svdq_status svdq_relayout(const void* codes_in, const void* scales_in, int rows, int K, svdq_format fmt,
                          int to_canonical, void* codes_out, void* scales_out, void* stream) {
  if (!fmt_ok(fmt)) return SVDQ_ERR_FORMAT;
  if (rows < 0 || K <= 0 || K % 64 != 0 || rows > kMaxDim || K > kMaxDim) return SVDQ_ERR_SHAPE;
  if (to_canonical != 0 && to_canonical != 1) return SVDQ_ERR_SHAPE;
  if (rows == 0) return SVDQ_OK;
  if (!codes_in || !scales_in || !codes_out || !scales_out) return SVDQ_ERR_NULL;
  if (!aligned16(codes_in) || !aligned16(scales_in) || !aligned16(codes_out) || !aligned16(scales_out))
    return SVDQ_ERR_ALIGN;
  return map_launch(launch_relayout(codes_in, scales_in, rows, K, (int)fmt, to_canonical != 0, codes_out, scales_out,
                                    static_cast<hipStream_t>(stream)));
}

svdq_status svdq_quantize_weight(const float* r_t, int N, int K, svdq_format fmt, void* wq, void* ws,
                                 void* stream) {
  if (!fmt_ok(fmt)) return SVDQ_ERR_FORMAT;
  svdq_status st = check_dims(0, N, K, 0);
  if (st != SVDQ_OK) return st;
  if (N == 0) return SVDQ_OK;
  if (!r_t || !wq || !ws) return SVDQ_ERR_NULL;
  if (!aligned16(r_t) || !aligned16(wq) || !aligned16(ws)) return SVDQ_ERR_ALIGN;
  if (N == 0) return SVDQ_OK;
  return map_launch(launch_quant_weight(r_t, N, K, (int)fmt, wq, ws, static_cast<hipStream_t>(stream)));
}

size_t svdq_linear_unfused_workspace_bytes(int M, int N, int K, int r, svdq_format fmt) {
  if (!fmt_ok(fmt) || check_dims(M, N, K, r) != SVDQ_OK) return 0;
  return carve(nullptr, M, N, K, r, fmt, true).total;
}

svdq_status svdq_linear_unfused(const void* x_hat, const void* l1t, const void* wq, const void* ws,
                                const void* l2, const void* bias, int M, int N, int K, int r, svdq_format fmt,
                                void* workspace, size_t workspace_bytes, void* y, void* stream) {
  if (!fmt_ok(fmt)) return SVDQ_ERR_FORMAT;
  svdq_status st = check_dims(M, N, K, r);
  if (st != SVDQ_OK) return st;
  if (M == 0 || N == 0) return SVDQ_OK;
  if (!x_hat || !wq || !ws || !y || !workspace) return SVDQ_ERR_NULL;
  if (r > 0 && (!l1t || !l2)) return SVDQ_ERR_NULL;
  if (!aligned16(workspace)) return SVDQ_ERR_ALIGN;
  const Workspace w = carve(workspace, M, N, K, r, fmt, true);
  if (workspace_bytes < w.total) return SVDQ_ERR_WORKSPACE;
  st = check_quant_down(x_hat, l1t, M, K, r, fmt, w.xq, w.xs, w.t);
  if (st != SVDQ_OK) return st;
  st = check_gemm(w.xq, w.xs, w.t, wq, ws, l2, bias, M, N, K, r, fmt, y);
  if (st != SVDQ_OK) return st;
  if (M == 0 || N == 0) return SVDQ_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = map_launch(launch_quant_only(x_hat, M, K, (int)fmt, w.xq, w.xs, s));
  if (st != SVDQ_OK) return st;
  if (r > 0) {
    st = map_launch(launch_down_only(x_hat, l1t, M, K, r, w.t, w.part, w.part_bytes, s));
    if (st != SVDQ_OK) return st;
  }
  GemmArgs ga{w.xq, w.xs, nullptr, wq, ws, nullptr, bias, M, N, K, 0, (int)fmt, r > 0 ? w.y0 : y};
  st = map_launch(launch_gemm(ga, s));
  if (st != SVDQ_OK || r == 0) return st;
  return map_launch(launch_up_add(w.y0, w.t, l2, M, N, r, y, s));
}

svdq_status svdq_gemm_w4a16(const void* x, const void* wq, const void* ws, const void* bias, int M, int N,
                            int K, void* y, void* stream) {
  svdq_status st = check_dims(M, N, K, 0);
  if (st != SVDQ_OK) return st;
  if (M == 0 || N == 0) return SVDQ_OK;
  if (!x || !wq || !ws || !y) return SVDQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(wq) || !aligned16(ws) || !aligned16(y)) return SVDQ_ERR_ALIGN;
  if (bias && !aligned16(bias)) return SVDQ_ERR_ALIGN;
  // the kernel addresses X and the codes with 32-bit byte offsets
  if ((size_t)M * K * 2 >= (1ull << 32) || (size_t)N * K / 2 >= (1ull << 32)) return SVDQ_ERR_SHAPE;
  return map_launch(launch_w4a16(x, wq, ws, bias, M, N, K, y, static_cast<hipStream_t>(stream)));
}

svdq_status svdq_gelu_tanh_smooth(const void* y, const float* lambda, int M, int C, void* out, void* stream) {
  if (M < 0 || C <= 0 || C % 8 != 0 || M > kMaxDim || C > kMaxDim) return SVDQ_ERR_SHAPE;
  if (M == 0) return SVDQ_OK;
  if (!y || !lambda || !out) return SVDQ_ERR_NULL;
  if (!aligned16(y) || !aligned16(lambda) || !aligned16(out)) return SVDQ_ERR_ALIGN;
  return map_launch(launch_gelu_smooth(y, lambda, M, C, out, static_cast<hipStream_t>(stream)));
}

const char* svdq_status_string(svdq_status s) {
  switch (s) {
    case SVDQ_OK: return "ok";
    case SVDQ_ERR_NULL: return "a required pointer is NULL";
    case SVDQ_ERR_SHAPE: return "shape outside the supported constraints (K % 64 == 0, N % 16 == 0, r in {0,16,32,48,64}, dims <= 2^24)";
    case SVDQ_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case SVDQ_ERR_FORMAT: return "unknown or unsupported format";
    case SVDQ_ERR_WORKSPACE: return "workspace too small (for svdq_linear_noalloc: the shape needs more than its static scratch)";
    case SVDQ_ERR_DEVICE: return "no gfx950 code object for the current device";
    case SVDQ_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

const char* svdq_version(void) { return "svdq-mi355x 0.1 (gfx950)"; }

}  // extern "C"
