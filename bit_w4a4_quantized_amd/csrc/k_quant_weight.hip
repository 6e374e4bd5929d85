// Offline weight quantizer: the residual R = W_hat - L1 L2 (given as R^T fp32
// [N, K], K contiguous per output column) to the codes and scales Kernel B
// reads.  Practice page "sota-314", section "Do this": only the residual is
// quantized, per group along K with a symmetric absmax scale.  One thread
// per group; not on the timed path.
#include "kernels.h"
#include "quant_core.h"

namespace svdq {

// One INT group's codes (64 values, code e of group g of output column n) and fp16 scale bits
// into the layouts Kernel B reads, all group-major: packed nibbles [K/64][N][32] (INT4), int8
// [K/64][N][64] (INT8), or the 6-bit container [K/64][N][48] (INT4_E2M3); the scales
// [K/64, N].
template <int FMT>
__device__ __forceinline__ void store_int_group(const int* q, uint16_t sbits, int n, int g, int N,
                                                uint8_t* __restrict__ wq, uint8_t* __restrict__ ws) {
  constexpr int G = 64;
  reinterpret_cast<uint16_t*>(ws)[(size_t)g * N + n] = sbits;
  if (FMT == FMT_INT4_E2M3) {
    // 48 bytes per (group, column): two halves of 32 six-bit fields
    uint32_t wv[12];
#pragma unroll
    for (int hh = 0; hh < 2; hh++) {
      uint64_t f[4];
#pragma unroll
      for (int j = 0; j < 4; j++) f[j] = pack6x8(q + 32 * hh + 8 * j);
      // 4 x 48 bits -> 6 dwords
      wv[6 * hh + 0] = (uint32_t)f[0];
      wv[6 * hh + 1] = (uint32_t)(f[0] >> 32) | (uint32_t)(f[1] << 16);
      wv[6 * hh + 2] = (uint32_t)(f[1] >> 16);
      wv[6 * hh + 3] = (uint32_t)f[2];
      wv[6 * hh + 4] = (uint32_t)(f[2] >> 32) | (uint32_t)(f[3] << 16);
      wv[6 * hh + 5] = (uint32_t)(f[3] >> 16);
    }
    // within the 48 bytes: half 0 bytes 0..15, half 1 bytes 0..15, half 0 bytes 16..23,
    // half 1 bytes 16..23
    uint4* dst = reinterpret_cast<uint4*>(wq + ((size_t)g * N + n) * 48);
    dst[0] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    dst[1] = make_uint4(wv[6], wv[7], wv[8], wv[9]);
    dst[2] = make_uint4(wv[4], wv[5], wv[10], wv[11]);
  } else if (FMT == FMT_INT4) {
    uint32_t* dst = reinterpret_cast<uint32_t*>(wq + ((size_t)g * N + n) * (G >> 1));
#pragma unroll
    for (int e = 0; e < G; e += 8) dst[e >> 3] = pack8(q + e);
  } else {
    uint32_t* dst = reinterpret_cast<uint32_t*>(wq + ((size_t)g * N + n) * 64);
#pragma unroll
    for (int e = 0; e < G; e += 4) dst[e >> 2] = pack4_i8(q + e);
  }
}

template <int FMT>
__global__ void __launch_bounds__(256)
k_quant_weight(const float* __restrict__ r_t, int N, int K, uint8_t* __restrict__ wq,
               uint8_t* __restrict__ ws) {
  constexpr int G = FMT == FMT_FP4 ? 16 : (FMT == FMT_MXFP4 ? 32 : 64);
  const int gpr = K / G;
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (size_t)N * gpr) return;
  const int n = (int)(gid / gpr), g = (int)(gid % gpr);
  const float* src = r_t + (size_t)n * K + (size_t)g * G;
  float v[G];
#pragma unroll
  for (int e = 0; e < G; e += 4) {
    const float4 f = *reinterpret_cast<const float4*>(src + e);
    v[e] = f.x; v[e + 1] = f.y; v[e + 2] = f.z; v[e + 3] = f.w;
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < G; e++) amax = fmaxf(amax, fabsf(v[e]));
  if constexpr (FMT == FMT_INT4 || FMT == FMT_INT8 || FMT == FMT_INT4_E2M3) {
    const float qmax = FMT == FMT_INT8 ? 127.0f : 7.0f;
    uint16_t sbits;
    const float s = int_scale(amax, qmax, &sbits);
    int q[G];
#pragma unroll
    for (int e = 0; e < G; e++) q[e] = int_code(v[e], s, qmax);
    store_int_group<FMT>(q, sbits, n, g, N, wq, ws);
  } else if constexpr (FMT == FMT_MXFP4) {
    // chunk-major: group g is half g % 2 of 64-K chunk g / 2; codes [K/64][N][32 bytes],
    // E8M0 bytes [K/64][N][2]
    const int ex = mx_exponent(amax);
    const size_t cn = (size_t)(g >> 1) * N + n;
    ws[cn * 2 + (g & 1)] = (uint8_t)(ex + 127);
    int q[G];
#pragma unroll
    for (int e = 0; e < G; e++) q[e] = (int)fp4_code_q(ldexpf(v[e], -ex));   // v / 2^ex, exact
    uint32_t* dst = reinterpret_cast<uint32_t*>(wq + cn * 32 + (g & 1) * 16);
#pragma unroll
    for (int e = 0; e < G; e += 8) dst[e >> 3] = pack8(q + e);
  } else {
    // chunk-major: group g of 16 is piece g % 4 of 64-K chunk g / 4; codes [K/64][N][32 bytes],
    // E4M3 bytes [K/64][N][4]
    uint32_t b;
    const float s = fp4_scale(amax, &b);
    const size_t cn = (size_t)(g >> 2) * N + n;
    ws[cn * 4 + (g & 3)] = (uint8_t)b;
    int q[G];
#pragma unroll
    for (int e = 0; e < G; e++) q[e] = (int)fp4_code(v[e], s);
    uint32_t* dst = reinterpret_cast<uint32_t*>(wq + cn * 32 + (g & 3) * 8);
#pragma unroll
    for (int e = 0; e < G; e += 8) dst[e >> 3] = pack8(q + e);
  }
}

// Codes and scales computed elsewhere (e.g. GPTQ on the host: int8 codes [N, K], fp16 scales
// [N, K/64]) into the same layouts, one thread per group.
template <int FMT>
__global__ void __launch_bounds__(256)
k_pack_weight(const int8_t* __restrict__ codes, const uint16_t* __restrict__ scales, int N, int K,
              uint8_t* __restrict__ wq, uint8_t* __restrict__ ws) {
  const int gpr = K / 64;
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (size_t)N * gpr) return;
  const int n = (int)(gid / gpr), g = (int)(gid % gpr);
  const int8_t* src = codes + (size_t)n * K + (size_t)g * 64;
  int q[64];
#pragma unroll
  for (int e = 0; e < 64; e += 16) {
    const int4 c = *reinterpret_cast<const int4*>(src + e);
    const uint32_t w[4] = {(uint32_t)c.x, (uint32_t)c.y, (uint32_t)c.z, (uint32_t)c.w};
#pragma unroll
    for (int i = 0; i < 16; i++) q[e + i] = (int)(int8_t)(w[i >> 2] >> (8 * (i & 3)));
  }
  store_int_group<FMT>(q, scales[(size_t)n * gpr + g], n, g, N, wq, ws);
}

hipError_t launch_pack_weight(const int8_t* codes, const uint16_t* scales, int N, int K, int fmt, void* wq,
                              void* ws, hipStream_t s) {
  const size_t groups = (size_t)N * (K / 64);
  dim3 grid((unsigned)((groups + 255) / 256));
  switch (fmt) {
    case FMT_INT4:
      hipLaunchKernelGGL(k_pack_weight<FMT_INT4>, grid, dim3(256), 0, s, codes, scales, N, K, (uint8_t*)wq, (uint8_t*)ws);
      break;
    case FMT_INT4_E2M3:
      hipLaunchKernelGGL(k_pack_weight<FMT_INT4_E2M3>, grid, dim3(256), 0, s, codes, scales, N, K, (uint8_t*)wq,
                         (uint8_t*)ws);
      break;
    case FMT_INT8:
      hipLaunchKernelGGL(k_pack_weight<FMT_INT8>, grid, dim3(256), 0, s, codes, scales, N, K, (uint8_t*)wq, (uint8_t*)ws);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quant_weight(const float* r_t, int N, int K, int fmt, void* wq, void* ws, hipStream_t s) {
  const int G = fmt == FMT_FP4 ? 16 : (fmt == FMT_MXFP4 ? 32 : 64);
  const size_t groups = (size_t)N * (K / G);
  dim3 grid((unsigned)((groups + 255) / 256));
  switch (fmt) {
    case FMT_INT4:
      hipLaunchKernelGGL(k_quant_weight<FMT_INT4>, grid, dim3(256), 0, s, r_t, N, K, (uint8_t*)wq, (uint8_t*)ws);
      break;
    case FMT_INT4_E2M3:
      hipLaunchKernelGGL(k_quant_weight<FMT_INT4_E2M3>, grid, dim3(256), 0, s, r_t, N, K, (uint8_t*)wq, (uint8_t*)ws);
      break;
    case FMT_INT8:
      hipLaunchKernelGGL(k_quant_weight<FMT_INT8>, grid, dim3(256), 0, s, r_t, N, K, (uint8_t*)wq, (uint8_t*)ws);
      break;
    case FMT_FP4:
      hipLaunchKernelGGL(k_quant_weight<FMT_FP4>, grid, dim3(256), 0, s, r_t, N, K, (uint8_t*)wq, (uint8_t*)ws);
      break;
    case FMT_MXFP4:
      hipLaunchKernelGGL(k_quant_weight<FMT_MXFP4>, grid, dim3(256), 0, s, r_t, N, K, (uint8_t*)wq, (uint8_t*)ws);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace svdq
