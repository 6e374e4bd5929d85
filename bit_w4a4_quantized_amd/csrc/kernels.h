// Internal interface between the C-ABI layer (svdq_api.hip) and the kernels.
// Not installed; the public interface is include/svdq.h.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stddef.h>
#include <stdint.h>

namespace svdq {

enum Fmt { FMT_INT4 = 0, FMT_INT8 = 1, FMT_FP4 = 2, FMT_INT4_E2M3 = 3 };
enum Core { CORE_E2M3 = 0, CORE_I4 = 1 };

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
};

// Kernel A's launch: row blocks of 16 nrt rows, K in `slices` slices of cpb 64-column chunks;
// partial_bytes of fp32 partial sums of T are needed when r > 0 and slices > 1.
struct QuantDownPlan {
  int nrt, cpb, slices, rows_blocks;
  size_t partial_bytes;
};
QuantDownPlan quant_down_plan(int M, int K, int r, bool have_partials);

// Workgroups that stay resident on the current device at two per CU (cached per device).
int resident_workgroups();

struct GemmArgs {
  const void* xq; const void* xs; const void* t; const void* wq; const void* ws;
  const void* l2; const void* bias; int M, N, K, r; int fmt;
  void* y;
};

hipError_t launch_quant_down(const QuantDownArgs& a, hipStream_t s);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm2(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm3(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_i8(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_f4(const GemmArgs& a, hipStream_t s);
hipError_t launch_quant_weight(const float* r_t, int N, int K, int fmt, void* wq, void* ws, hipStream_t s);

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
