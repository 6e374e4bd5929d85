// Internal interface between the C-ABI layer (svdq_api.hip) and the kernels.
// Not installed; the public interface is include/svdq.h.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stddef.h>
#include <stdint.h>

namespace svdq {

enum Fmt { FMT_INT4 = 0, FMT_INT8 = 1, FMT_FP4 = 2, FMT_INT4_E2M3 = 3, FMT_MXFP4 = 4 };

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8h as_h8(const uint4& u) {
  v8h h;
  __builtin_memcpy(&h, &u, 16);
  return h;
}

__device__ __forceinline__ v4i as_i4(const uint4& u) {
  v4i h;
  __builtin_memcpy(&h, &u, 16);
  return h;
}

// Buffer resources: loads through them are range-checked against `bytes` (a load past the end
// returns zeros and touches no memory; a resource of 0 bytes makes every load return zeros).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, size_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)n, 0x00020000);
}
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 as_u4(u32x4_t v) { return make_uint4(v[0], v[1], v[2], v[3]); }
__device__ __forceinline__ uint2 as_u2(u32x2_t v) { return make_uint2(v[0], v[1]); }

// Four fp32 values at element index i of a vector behind a buffer resource, without a branch:
// zeros past its end, and everywhere for an absent vector (a 0-byte resource).
__device__ __forceinline__ float4 load_f4(rsrc_t r, int i) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, i * 4, 0, 0);
  return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
}

__device__ __forceinline__ void unpack_h8(const uint4& u, float* f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    f[2 * i] = __half2float(__ushort_as_half((unsigned short)(w[i] & 0xFFFFu)));
    f[2 * i + 1] = __half2float(__ushort_as_half((unsigned short)(w[i] >> 16)));
  }
}

struct QuantDownArgs {
  const void* x; const void* l1t; int M, K, r; int fmt;
  void* xq; void* xs; void* t;
  void* part; size_t part_bytes;             // fp32 partial sums of T when K is sliced (may be null)
  const float* lam = nullptr;                // fp32 [K]: x arrives unsmoothed, X_hat = fp16(x / lam)
};

// Kernel A's launch: row blocks of 16 nrt rows, K in `slices` slices of cpb 64-column chunks;
// partial_bytes of fp32 partial sums of T are needed when r > 0 and slices > 1.  `smooth`:
// the variant that smooths x itself (its own register budget).
struct QuantDownPlan {
  int nrt, cpb, slices, rows_blocks;
  size_t partial_bytes;
};
QuantDownPlan quant_down_plan(int M, int K, int r, bool have_partials, bool smooth);

// Workgroups that stay resident on the current device at two per CU (cached per device).
int resident_workgroups();

struct GemmArgs {
  const void* xq; const void* xs; const void* t; const void* wq; const void* ws;
  const void* l2; const void* bias; int M, N, K, r; int fmt;
  void* y;
  const float* lam = nullptr;                // fp32 [N]: epilogue emits fp16(gelu(y) / lam) instead of y
};

// GELU(tanh) of v divided by a smoothing factor, in fp32.  0.5 (1 + tanh(u)) equals
// 1 / (1 + exp(-2u)), so gelu_tanh(v) / lam = v / ((1 + exp(-2u)) lam): no cancellation for
// negative v, and overflow of the denominator gives the correct limit (a signed zero).
// exp(-2u) = 2^(-2u log2(e)) on v_exp_f32 and the quotient from v_rcp_f32, each within about
// one fp32 ulp, so the value is within a few fp32 ulps of the exact one and its fp16 rounding
// within one fp16 ulp of the exactly rounded result.
__device__ __forceinline__ float gelu_div(float v, float lam) {
  const float u = 0.7978845608028654f * __builtin_fmaf(0.044715f * v, v * v, v);   // sqrt(2/pi) (v + 0.044715 v^3)
  const float e = __builtin_amdgcn_exp2f(-2.8853900817779268f * u);                 // -2 log2(e) u
  return v * __builtin_amdgcn_rcpf((1.0f + e) * lam);
}

// An epilogue's fp16 output y (bits) turned into the next layer's smoothed input,
// fp16(gelu_tanh(float(y)) / lam): the MLP glue folded into the producing GEMM.
__device__ __forceinline__ uint32_t gelu_div_h(uint32_t ybits, float lam) {
  return __half_as_ushort(__float2half_rn(gelu_div(__half2float(__ushort_as_half((unsigned short)ybits)), lam)));
}

hipError_t launch_quant_down(const QuantDownArgs& a, hipStream_t s);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm2(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm3(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_i8(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_f4(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_mx(const GemmArgs& a, hipStream_t s);
hipError_t launch_quant_weight(const float* r_t, int N, int K, int fmt, void* wq, void* ws, hipStream_t s);
hipError_t launch_pack_weight(const int8_t* codes, const uint16_t* scales, int N, int K, int fmt, void* wq,
                              void* ws, hipStream_t s);

// codes and scales between the exchange layout (row-major) and the device layouts
hipError_t launch_relayout(const void* codes_in, const void* scales_in, int rows, int K, int fmt, bool to_canonical,
                           void* codes_out, void* scales_out, hipStream_t s);

// unfused comparison pieces
hipError_t launch_quant_only(const void* x, int M, int K, int fmt, void* xq, void* xs, hipStream_t s);
hipError_t launch_down_only(const void* x, const void* l1t, int M, int K, int r, void* t, void* part,
                            size_t part_bytes, hipStream_t s);
hipError_t launch_up_add(const void* y0, const void* t, const void* l2, int M, int N, int r, void* y,
                         hipStream_t s);

hipError_t launch_w4a16(const void* x, const void* wq, const void* ws, const void* bias, int M, int N,
                        int K, void* y, hipStream_t s);
hipError_t launch_gelu_smooth(const void* y, const float* lam, int M, int C, void* out, hipStream_t s);

}  // namespace svdq
