// Kernel B: low-bit GEMM on the matrix cores with the up projection and the
// bias in the epilogue.
//
// Practice page "sota-314", section "Do this": the up projection is fused
// with the 4-bit compute because both write the same output; reading note
// "note-257", section "Key results": unfused, the branch pays an extra 16-bit
// write of the output.
//
//   Y[m,n] = fp16_rne( sum_g sx[m,g] sw[n,g] P_g[m,n] + (T L2)[m,n] + b[n] )
//   P_g    = sum_{k in group g} q_x[m,k] q_w[n,k]   (exact, int32 on the MFMA)
//
// gfx950 mapping:
//   workgroup tile 128 x 128, four waves in 2 x 2, each wave 64 x 64 = 2 x 2
//   tiles of 32 x 32 held as fp32 accumulators (v_mfma 32x32 layout: lane l
//   holds column l % 32 and rows 8 (i/4) + 4 (l/32) + i%4).
//   INT4 (group 64): each lane loads 16 bytes = 32 codes of its row / column;
//     nibbles become int8 16q with two masks and a shift ((w<<4) & 0xF0F0F0F0
//     and w & 0xF0F0F0F0), giving two v_mfma_i32_32x32x32_i8 per 32 x 32 tile
//     per group; the factor 256 is folded into the weight scale.  A and B use
//     the same permutation of K inside the group, so the dot product is
//     unchanged.
//   INT8 (group 64): the codes feed the same MFMA directly.
//   FP4 (group 16, E4M3 scales): an E2M1 code times 2 is an integer in
//     [-12, 12]; one v_mfma_i32_32x32x16_i8 per group, factor 4 folded into
//     the scale.
//   Per group the int32 partial is converted to fp32 and accumulated with the
//   product of the two scales.
//   Epilogue: acc += T L2 on v_mfma_f32_32x32x16_f16 (fp16 in, fp32 out),
//   + bias, RNE to fp16, store.
#include "kernels.h"
#include "quant_core.h"

namespace svdq {

__device__ __forceinline__ uint32_t nib_lo16(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t nib_hi16(uint32_t w) { return w & 0xF0F0F0F0u; }

// 4 packed E2M1 nibbles in the low nibbles of each byte of `n` -> bytes 2*value.
__device__ __forceinline__ uint32_t e2m1x2_bytes(uint32_t n) {
  // magnitude table {0,1,2,3,4,6,8,12} and its negation, selected by the sign bit (bit 3)
  const uint32_t pos_lo = 0x03020100u, pos_hi = 0x0C080604u;
  const uint32_t neg_lo = 0xFDFEFF00u, neg_hi = 0xF4F8FAFCu;
  const uint32_t sel = n & 0x07070707u;
  const uint32_t p = __builtin_amdgcn_perm(pos_hi, pos_lo, sel);
  const uint32_t q = __builtin_amdgcn_perm(neg_hi, neg_lo, sel);
  const uint32_t sgn = ((n >> 3) & 0x01010101u) * 0xFFu;
  return (p & ~sgn) | (q & sgn);
}

template <int FMT>
__device__ __forceinline__ float load_scale(const void* s, size_t idx) {
  if (FMT == FMT_FP4) return e4m3_decode(reinterpret_cast<const uint8_t*>(s)[idx]);
  return __half2float(reinterpret_cast<const __half*>(s)[idx]);
}

template <int FMT, int RB, bool BIAS>
__global__ void __launch_bounds__(256)
k_gemm(const uint8_t* __restrict__ xq, const void* __restrict__ xs, const __half* __restrict__ t,
       const uint8_t* __restrict__ wq, const void* __restrict__ ws, const __half* __restrict__ l2,
       const __half* __restrict__ bias, int M, int N, int K, __half* __restrict__ y) {
  constexpr int R = RB * 16;
  constexpr int G = FMT == FMT_FP4 ? 16 : 64;
  constexpr float PSCALE = FMT == FMT_INT4 ? (1.0f / 256.0f) : (FMT == FMT_FP4 ? 0.25f : 1.0f);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int m_base = blockIdx.y * 128 + (wave >> 1) * 64;
  const int n_base = blockIdx.x * 128 + (wave & 1) * 64;
  const int row_bytes = FMT == FMT_INT8 ? K : (K >> 1);
  const int gpr = K / G;

  int arow[2], bcol[2];
  bool aok[2], bok[2];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    arow[i] = m_base + i * 32 + l32; aok[i] = arow[i] < M;
    bcol[i] = n_base + i * 32 + l32; bok[i] = bcol[i] < N;
  }
  // row of accumulator entry i of row tile ti held by this lane
  auto orow = [&](int ti, int i) { return m_base + ti * 32 + 8 * (i >> 2) + 4 * h + (i & 3); };

  v16f acc[2][2];
#pragma unroll
  for (int ti = 0; ti < 2; ti++)
#pragma unroll
    for (int tj = 0; tj < 2; tj++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[ti][tj][i] = 0.f;

  const int nchunks = K >> 6;
  for (int c = 0; c < nchunks; c++) {
    if (FMT == FMT_INT4 || FMT == FMT_INT8) {
      v4i a[2][2], b[2][2];   // [tile][k-step]
#pragma unroll
      for (int i = 0; i < 2; i++) {
        if (FMT == FMT_INT4) {
          uint4 ua = aok[i] ? *reinterpret_cast<const uint4*>(xq + (size_t)arow[i] * row_bytes + c * 32 + 16 * h) : make_uint4(0, 0, 0, 0);
          uint4 ub = bok[i] ? *reinterpret_cast<const uint4*>(wq + (size_t)bcol[i] * row_bytes + c * 32 + 16 * h) : make_uint4(0, 0, 0, 0);
          a[i][0] = v4i{(int)nib_lo16(ua.x), (int)nib_hi16(ua.x), (int)nib_lo16(ua.y), (int)nib_hi16(ua.y)};
          a[i][1] = v4i{(int)nib_lo16(ua.z), (int)nib_hi16(ua.z), (int)nib_lo16(ua.w), (int)nib_hi16(ua.w)};
          b[i][0] = v4i{(int)nib_lo16(ub.x), (int)nib_hi16(ub.x), (int)nib_lo16(ub.y), (int)nib_hi16(ub.y)};
          b[i][1] = v4i{(int)nib_lo16(ub.z), (int)nib_hi16(ub.z), (int)nib_lo16(ub.w), (int)nib_hi16(ub.w)};
        } else {
          const uint4 z = make_uint4(0, 0, 0, 0);
          const uint8_t* pa = xq + (size_t)arow[i] * row_bytes + c * 64 + 32 * h;
          const uint8_t* pb = wq + (size_t)bcol[i] * row_bytes + c * 64 + 32 * h;
          a[i][0] = as_i4(aok[i] ? *reinterpret_cast<const uint4*>(pa) : z);
          a[i][1] = as_i4(aok[i] ? *reinterpret_cast<const uint4*>(pa + 16) : z);
          b[i][0] = as_i4(bok[i] ? *reinterpret_cast<const uint4*>(pb) : z);
          b[i][1] = as_i4(bok[i] ? *reinterpret_cast<const uint4*>(pb + 16) : z);
        }
      }
      float sx[2][16], sw[2];
#pragma unroll
      for (int ti = 0; ti < 2; ti++)
#pragma unroll
        for (int i = 0; i < 16; i++) sx[ti][i] = orow(ti, i) < M ? load_scale<FMT>(xs, (size_t)orow(ti, i) * gpr + c) : 0.f;
#pragma unroll
      for (int tj = 0; tj < 2; tj++) sw[tj] = bok[tj] ? load_scale<FMT>(ws, (size_t)bcol[tj] * gpr + c) * PSCALE : 0.f;
#pragma unroll
      for (int ti = 0; ti < 2; ti++)
#pragma unroll
        for (int tj = 0; tj < 2; tj++) {
          v16i p = {};
          p = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[ti][0], b[tj][0], p, 0, 0, 0);
          p = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[ti][1], b[tj][1], p, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 16; i++) acc[ti][tj][i] = __builtin_fmaf((float)p[i], sx[ti][i] * sw[tj], acc[ti][tj][i]);
        }
    } else {  // FP4: four groups of 16 per 64-column chunk
      uint4 ua[2][2], ub[2][2];
#pragma unroll
      for (int i = 0; i < 2; i++) {
        const uint4 z = make_uint4(0, 0, 0, 0);
        const uint8_t* pa = xq + (size_t)arow[i] * row_bytes + c * 32;
        const uint8_t* pb = wq + (size_t)bcol[i] * row_bytes + c * 32;
        ua[i][0] = aok[i] ? *reinterpret_cast<const uint4*>(pa) : z;
        ua[i][1] = aok[i] ? *reinterpret_cast<const uint4*>(pa + 16) : z;
        ub[i][0] = bok[i] ? *reinterpret_cast<const uint4*>(pb) : z;
        ub[i][1] = bok[i] ? *reinterpret_cast<const uint4*>(pb + 16) : z;
      }
#pragma unroll 1
      for (int gg = 0; gg < 4; gg++) {
        // group gg occupies bytes [8 gg, 8 gg + 8) of the chunk row; lane half h takes 4 of them
        long a8[2], b8[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
          // dword 2 gg + h of the 32-byte chunk row
          const uint4 va = (gg >> 1) ? ua[i][1] : ua[i][0];
          const uint4 vb = (gg >> 1) ? ub[i][1] : ub[i][0];
          const uint32_t na = (gg & 1) ? (h ? va.w : va.z) : (h ? va.y : va.x);
          const uint32_t nb = (gg & 1) ? (h ? vb.w : vb.z) : (h ? vb.y : vb.x);
          const uint64_t qa = (uint64_t)e2m1x2_bytes(na & 0x0F0F0F0Fu) | ((uint64_t)e2m1x2_bytes((na >> 4) & 0x0F0F0F0Fu) << 32);
          const uint64_t qb = (uint64_t)e2m1x2_bytes(nb & 0x0F0F0F0Fu) | ((uint64_t)e2m1x2_bytes((nb >> 4) & 0x0F0F0F0Fu) << 32);
          a8[i] = (long)qa;
          b8[i] = (long)qb;
        }
        const int g = c * 4 + gg;
        float sx[2][16], sw[2];
#pragma unroll
        for (int ti = 0; ti < 2; ti++)
#pragma unroll
          for (int i = 0; i < 16; i++) sx[ti][i] = orow(ti, i) < M ? load_scale<FMT>(xs, (size_t)orow(ti, i) * gpr + g) : 0.f;
#pragma unroll
        for (int tj = 0; tj < 2; tj++) sw[tj] = bok[tj] ? load_scale<FMT>(ws, (size_t)bcol[tj] * gpr + g) * PSCALE : 0.f;
#pragma unroll
        for (int ti = 0; ti < 2; ti++)
#pragma unroll
          for (int tj = 0; tj < 2; tj++) {
            v16i p = {};
            p = __builtin_amdgcn_mfma_i32_32x32x16_i8(a8[ti], b8[tj], p, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 16; i++) acc[ti][tj][i] = __builtin_fmaf((float)p[i], sx[ti][i] * sw[tj], acc[ti][tj][i]);
          }
      }
    }
  }

  // ---- epilogue: up projection T L2 on the matrix core, bias, fp16 store
  if (RB > 0) {
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
      for (int ti = 0; ti < 2; ti++)
#pragma unroll
        for (int tj = 0; tj < 2; tj++)
          acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(ta[ti]), as_h8(lb[tj]), acc[ti][tj], 0, 0, 0);
    }
  }
#pragma unroll
  for (int tj = 0; tj < 2; tj++) {
    if (!bok[tj]) continue;
    const float bv = BIAS ? __half2float(bias[bcol[tj]]) : 0.f;
#pragma unroll
    for (int ti = 0; ti < 2; ti++)
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int mrow = orow(ti, i);
        if (mrow < M) y[(size_t)mrow * N + bcol[tj]] = __float2half_rn(acc[ti][tj][i] + bv);
      }
  }
}

template <int FMT, int RB, bool BIAS>
static hipError_t launch_g(const GemmArgs& a, hipStream_t s) {
  dim3 grid((a.N + 127) / 128, (a.M + 127) / 128);
  hipLaunchKernelGGL((k_gemm<FMT, RB, BIAS>), grid, dim3(256), 0, s, (const uint8_t*)a.xq, a.xs,
                     (const __half*)a.t, (const uint8_t*)a.wq, a.ws, (const __half*)a.l2,
                     (const __half*)a.bias, a.M, a.N, a.K, (__half*)a.y);
  return hipGetLastError();
}

template <int FMT, bool BIAS>
static hipError_t launch_g_r(const GemmArgs& a, hipStream_t s) {
  switch (a.r) {
    case 0: return launch_g<FMT, 0, BIAS>(a, s);
    case 16: return launch_g<FMT, 1, BIAS>(a, s);
    case 32: return launch_g<FMT, 2, BIAS>(a, s);
    case 48: return launch_g<FMT, 3, BIAS>(a, s);
    case 64: return launch_g<FMT, 4, BIAS>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int FMT>
static hipError_t launch_g_b(const GemmArgs& a, hipStream_t s) {
  return a.bias ? launch_g_r<FMT, true>(a, s) : launch_g_r<FMT, false>(a, s);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  switch (a.fmt) {
    case FMT_INT4: return launch_gemm2(a, s);
    case FMT_INT4_E2M3: return launch_gemm3(a, s);
    case FMT_INT8: return launch_g_b<FMT_INT8>(a, s);
    case FMT_FP4: return launch_g_b<FMT_FP4>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace svdq
