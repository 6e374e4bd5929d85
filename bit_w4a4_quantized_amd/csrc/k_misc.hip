// Control and glue kernels around the fused layer:
//   * W4A16 control: fp16 activations times int4 group-64 weights (practice
//     page "sota-314", sections "Do this" and "What it buys": the W4A16
//     baseline and the layers that stay W4A16);
//   * up projection as a separate kernel, for the unfused comparison
//     ("sota-314", "Do this", latency table);
//   * GELU(tanh) + smoothing glue between an MLP's two linears.
#include "kernels.h"
#include "quant_core.h"

namespace svdq {

// ---------------------------------------------------------------- W4A16
// Tile 128 x 128, four waves of 64 x 64, v_mfma_f32_32x32x16_f16.  The int4
// codes become exact fp16 integers (fp16 1024 + (q + 8), minus 1032, packed
// fp16 arithmetic); per group of 64 the fp32 partial X q is scaled by the
// column's fp16 scale, so the product is that of the exact dequantized weight.
__device__ __forceinline__ uint32_t nib2_to_h2(uint32_t w, int j) {
  const uint32_t u = ((w >> (8 * j)) & 0xFu) | (((w >> (8 * j + 4)) & 0xFu) << 16);
  __half2 hv = __halves2half2(__ushort_as_half((unsigned short)((u ^ 0x6408u) & 0xFFFFu)),
                              __ushort_as_half((unsigned short)(((u >> 16) ^ 0x6408u) & 0xFFFFu)));
  hv = __hsub2(hv, __half2half2(__float2half(1032.0f)));
  uint32_t r;
  __builtin_memcpy(&r, &hv, 4);
  return r;
}

template <bool BIAS>
__global__ void __launch_bounds__(256)
k_w4a16(const __half* __restrict__ x, const uint8_t* __restrict__ wq, const __half* __restrict__ ws,
        const __half* __restrict__ bias, int M, int N, int K, __half* __restrict__ y) {
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
      for (int i = 0; i < 16; i++) acc[a][b][i] = 0.f;
  const int ngroups = K >> 6;
  for (int g = 0; g < ngroups; g++) {
    v16f p[2][2];
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
      for (int b = 0; b < 2; b++)
#pragma unroll
        for (int i = 0; i < 16; i++) p[a][b][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      const int k0 = g * 64 + ks * 16 + 8 * h;
      uint4 av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; i++) {
        av[i] = aok[i] ? *reinterpret_cast<const uint4*>(x + (size_t)arow[i] * K + k0) : make_uint4(0, 0, 0, 0);
        const uint32_t w = bok[i] ? *reinterpret_cast<const uint32_t*>(wq + (size_t)bcol[i] * (K >> 1) + (k0 >> 1)) : 0u;
        bv[i] = make_uint4(nib2_to_h2(w, 0), nib2_to_h2(w, 1), nib2_to_h2(w, 2), nib2_to_h2(w, 3));
      }
#pragma unroll
      for (int a = 0; a < 2; a++)
#pragma unroll
        for (int b = 0; b < 2; b++)
          p[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(av[a]), as_h8(bv[b]), p[a][b], 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < 2; b++) {
      const float s = bok[b] ? __half2float(ws[(size_t)bcol[b] * ngroups + g]) : 0.f;
#pragma unroll
      for (int a = 0; a < 2; a++)
#pragma unroll
        for (int i = 0; i < 16; i++) acc[a][b][i] = __builtin_fmaf(p[a][b][i], s, acc[a][b][i]);
    }
  }
#pragma unroll
  for (int b = 0; b < 2; b++) {
    if (!bok[b]) continue;
    const float bv = BIAS ? __half2float(bias[bcol[b]]) : 0.f;
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int mrow = m_base + a * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        if (mrow < M) y[(size_t)mrow * N + bcol[b]] = __float2half_rn(acc[a][b][i] + bv);
      }
  }
}

hipError_t launch_w4a16(const void* x, const void* wq, const void* ws, const void* bias, int M, int N,
                        int K, void* y, hipStream_t s) {
  dim3 grid((N + 127) / 128, (M + 127) / 128);
  if (bias)
    hipLaunchKernelGGL(k_w4a16<true>, grid, dim3(256), 0, s, (const __half*)x, (const uint8_t*)wq,
                       (const __half*)ws, (const __half*)bias, M, N, K, (__half*)y);
  else
    hipLaunchKernelGGL(k_w4a16<false>, grid, dim3(256), 0, s, (const __half*)x, (const uint8_t*)wq,
                       (const __half*)ws, (const __half*)nullptr, M, N, K, (__half*)y);
  return hipGetLastError();
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
// out = fp16( gelu_tanh(float(y)) / lambda[c] ), fp32 arithmetic, 8 values per thread.
// 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)) exactly, so gelu_tanh(v) = v / (1 + exp(-2u));
// this form has no cancellation for negative v, where 1 + tanh(u) would lose
// most of its bits in fp32.
__device__ __forceinline__ float gelu_tanh(float v) {
  const float k0 = 0.7978845608028654f;   // sqrt(2/pi)
  const float u = k0 * (v + 0.044715f * v * v * v);
  return v / (1.0f + expf(-2.0f * u));
}

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
    const uint32_t a = __half_as_ushort(__float2half_rn(gelu_tanh(v[2 * i]) / lv[2 * i]));
    const uint32_t b = __half_as_ushort(__float2half_rn(gelu_tanh(v[2 * i + 1]) / lv[2 * i + 1]));
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
