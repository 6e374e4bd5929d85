// Control and glue kernels around the fused layer:
//   * up projection as a separate kernel, for the unfused comparison
//     ("sota-314", "Do this", latency table);
//   * GELU(tanh) + smoothing glue between an MLP's two linears.
#include <atomic>

#include "kernels.h"
#include "quant_core.h"

namespace svdq {

// Workgroups that stay resident on the current device at two per CU.  The CU count is read once
// per device and cached (atomically: concurrent first calls store the same value).
int resident_workgroups() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    v = 2 * cus;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// ---------------------------------------------------------------- up projection (unfused)
// Y = fp16( float(Y0) + T L2 ): reads the fp16 output of the bare GEMM back.
template <int RB>
__global__ void __launch_bounds__(256)
k_up_add(const __half* __restrict__ y0, const __half* __restrict__ t, const __half* __restrict__ l2,
         int M, int N, __half* __restrict__ y) {
  constexpr int R = RB * 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int m_base = blockIdx.y * 128 + (wave >> 1) * 64;
  const int n_base = blockIdx.x * 128 + (wave & 1) * 64;
  int arow[2], bcol[2];
  bool aok[2], bok[2];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    arow[i] = m_base + i * 32 + l32; aok[i] = arow[i] < M;
    bcol[i] = n_base + i * 32 + l32; bok[i] = bcol[i] < N;
  }
  v16f acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; a++)
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int mrow = m_base + a * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        acc[a][b][i] = (mrow < M && bok[b]) ? __half2float(y0[(size_t)mrow * N + bcol[b]]) : 0.f;
      }
#pragma unroll
  for (int kb = 0; kb < RB; kb++) {
    uint4 ta[2], lb[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
      ta[i] = aok[i] ? *reinterpret_cast<const uint4*>(t + (size_t)arow[i] * R + kb * 16 + 8 * h) : make_uint4(0, 0, 0, 0);
      uint16_t hv[8];
#pragma unroll
      for (int e = 0; e < 8; e++)
        hv[e] = bok[i] ? __half_as_ushort(l2[(size_t)(kb * 16 + 8 * h + e) * N + bcol[i]]) : (uint16_t)0;
      lb[i] = make_uint4(hv[0] | ((uint32_t)hv[1] << 16), hv[2] | ((uint32_t)hv[3] << 16),
                         hv[4] | ((uint32_t)hv[5] << 16), hv[6] | ((uint32_t)hv[7] << 16));
    }
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
      for (int b = 0; b < 2; b++)
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(ta[a]), as_h8(lb[b]), acc[a][b], 0, 0, 0);
  }
#pragma unroll
  for (int b = 0; b < 2; b++) {
    if (!bok[b]) continue;
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int mrow = m_base + a * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        if (mrow < M) y[(size_t)mrow * N + bcol[b]] = __float2half_rn(acc[a][b][i]);
      }
  }
}

hipError_t launch_up_add(const void* y0, const void* t, const void* l2, int M, int N, int r, void* y,
                         hipStream_t s) {
  dim3 grid((N + 127) / 128, (M + 127) / 128);
#define UPADD(RB_) hipLaunchKernelGGL(k_up_add<RB_>, grid, dim3(256), 0, s, (const __half*)y0, (const __half*)t, \
                                      (const __half*)l2, M, N, (__half*)y)
  switch (r) {
    case 16: UPADD(1); break;
    case 32: UPADD(2); break;
    case 48: UPADD(3); break;
    case 64: UPADD(4); break;
    default: return hipErrorInvalidValue;
  }
#undef UPADD
  return hipGetLastError();
}

// ---------------------------------------------------------------- GELU + smoothing glue
// out = fp16( gelu_tanh(float(y)) / lambda[c] ) (gelu_div), 8 values per thread: the same
// arithmetic as a GEMM epilogue with the glue folded in, so the two agree bit for bit.
__global__ void __launch_bounds__(256)
k_gelu_smooth(const __half* __restrict__ y, const float* __restrict__ lam, int M, int C,
              __half* __restrict__ out) {
  const size_t idx8 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total8 = (size_t)M * C / 8;
  if (idx8 >= total8) return;
  const int c0 = (int)((idx8 * 8) % (size_t)C);
  const uint4 u = reinterpret_cast<const uint4*>(y)[idx8];
  float v[8];
  unpack_h8(u, v);
  const float4 l0 = *reinterpret_cast<const float4*>(lam + c0);
  const float4 l1 = *reinterpret_cast<const float4*>(lam + c0 + 4);
  const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t a = __half_as_ushort(__float2half_rn(gelu_div(v[2 * i], lv[2 * i])));
    const uint32_t b = __half_as_ushort(__float2half_rn(gelu_div(v[2 * i + 1], lv[2 * i + 1])));
    w[i] = a | (b << 16);
  }
  reinterpret_cast<uint4*>(out)[idx8] = make_uint4(w[0], w[1], w[2], w[3]);
}

hipError_t launch_gelu_smooth(const void* y, const float* lam, int M, int C, void* out, hipStream_t s) {
  const size_t total8 = (size_t)M * C / 8;
  dim3 grid((unsigned)((total8 + 255) / 256));
  hipLaunchKernelGGL(k_gelu_smooth, grid, dim3(256), 0, s, (const __half*)y, lam, M, C, (__half*)out);
  return hipGetLastError();
}

}  // namespace svdq
