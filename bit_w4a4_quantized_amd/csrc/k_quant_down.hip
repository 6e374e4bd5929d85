// Kernel A: quantize the smoothed activations and compute the down projection
// T = X_hat L1 in one pass over X_hat.
//
// Practice page "sota-314", section "Do this": the down projection is fused
// with quantization because the two read the same input; reading note
// "note-257", section "Key results": unfused, the branch pays an extra 16-bit
// read of the activations.
//
// Work decomposition (gfx950, wave64):
//   one workgroup = NW waves = 16 token rows; the waves split K into 64-column
//   chunks round-robin and each keeps its 16 x r partial of T in MFMA
//   accumulators; the partials are summed through LDS at the end (fixed order,
//   deterministic, no atomics).  Eight waves per workgroup and at most 128
//   VGPRs let two workgroups share a CU, so the last partial round of
//   workgroups does not leave most CUs idle.
//   Lane l of a wave owns row (l % 16) and the 8-column slices
//   [8 (l/16), +8) and [32 + 8 (l/16), +8) of each chunk: one 16-byte load
//   each.  That is exactly the operand layout of v_mfma_f32_16x16x32_f16 for
//   the chunk's two 32-column halves, so the fp16 values feed the matrix core
//   straight from the registers they were quantized from.
//   Group absmax: within the lane, then across the 4 lanes of the row with two
//   cross-lane xor shuffles (INT, group 64) or one (FP4, group 16).
//   INT codes use the division-free rule of int_code_f16 (exact for fp16
//   inputs); NB chunks are loaded before any is processed, to keep HBM reads in
//   flight.
#include "kernels.h"
#include "quant_core.h"

namespace svdq {

constexpr int QD_WAVES = 8;

template <int FMT, int RB, bool QUANT>
__global__ void __launch_bounds__(64 * QD_WAVES, 2)
k_quant_down(const __half* __restrict__ x, const __half* __restrict__ l1t, int M, int K,
             uint8_t* __restrict__ xq, uint8_t* __restrict__ xs, __half* __restrict__ t) {
  constexpr int NB = 2;                     // chunks in flight per wave
  constexpr int NW = QD_WAVES;
  constexpr int R = RB * 16;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = lane & 15;
  const int sub = lane >> 4;
  const int m = blockIdx.x * 16 + row;
  const bool valid = m < M;
  const int nchunks = K >> 6;
  const __half* xrow = x + (size_t)(valid ? m : 0) * K;

  v4f acc[RB > 0 ? RB : 1];
#pragma unroll
  for (int j = 0; j < (RB > 0 ? RB : 1); j++) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Codes of one chunk (16 rows x CB bytes) are assembled in this wave's LDS slot and
  // written back with whole 16-byte stores per lane: the per-lane pieces (2 to 6 bytes,
  // odd offsets for the 6-bit container) would otherwise be many small scattered stores.
  constexpr int CB = FMT == FMT_INT4_E2M3 ? 48 : (FMT == FMT_INT8 ? 64 : 32);   // code bytes per row per chunk
  __shared__ __attribute__((aligned(16))) uint8_t cstage[NW][16 * CB];
  uint8_t* slot = cstage[wave];
  // row-major codes [M, K * bits / 8]; the 6-bit container is group-major [K/64][M][48]
  const size_t code_row = FMT == FMT_INT4_E2M3 ? (size_t)48 : (FMT == FMT_INT8 ? (size_t)K : (size_t)(K >> 1));
  const size_t code_chunk = FMT == FMT_INT4_E2M3 ? (size_t)M * 48 : (size_t)CB;   // bytes between chunks

  for (int c0 = wave; c0 < nchunks; c0 += NW * NB) {
    uint4 xv[NB][2];
    uint4 bv[NB][RB > 0 ? RB : 1][2];
#pragma unroll
    for (int i = 0; i < NB; i++) {
      const int c = min(c0 + NW * i, nchunks - 1);   // a chunk past the end re-reads the last (unused)
      const int col = c * 64 + sub * 8;
      xv[i][0] = *reinterpret_cast<const uint4*>(xrow + col);
      xv[i][1] = *reinterpret_cast<const uint4*>(xrow + col + 32);
#pragma unroll
      for (int j = 0; j < RB; j++) {
        const __half* lrow = l1t + (size_t)(j * 16 + row) * K + col;
        bv[i][j][0] = *reinterpret_cast<const uint4*>(lrow);
        bv[i][j][1] = *reinterpret_cast<const uint4*>(lrow + 32);
      }
    }
#pragma unroll
    for (int i = 0; i < NB; i++) {
      const int c = c0 + NW * i;
      if (c >= nchunks) break;
      if (!valid) {                          // rows past M contribute zeros to the MFMA
        xv[i][0] = make_uint4(0, 0, 0, 0);
        xv[i][1] = make_uint4(0, 0, 0, 0);
      }
      // ---- down projection on the matrix core (fp16 in, fp32 accumulate)
#pragma unroll
      for (int j = 0; j < RB; j++) {
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(xv[i][0]), as_h8(bv[i][j][0]), acc[j], 0, 0, 0);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(xv[i][1]), as_h8(bv[i][j][1]), acc[j], 0, 0, 0);
      }
      if (!QUANT) continue;
      // ---- quantize
      float v[16];
      unpack_h8(xv[i][0], v);
      unpack_h8(xv[i][1], v + 8);
      const int col = c * 64 + sub * 8;
      if (FMT == FMT_INT4 || FMT == FMT_INT8 || FMT == FMT_INT4_E2M3) {
        const float qmax = FMT == FMT_INT8 ? 127.0f : 7.0f;
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < 16; e++) amax = fmaxf(amax, fabsf(v[e]));
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        uint16_t sbits;
        const float s = int_scale(amax, qmax, &sbits);
        const float rs = s == 0.0f ? 0.0f : 1.0f / s;
        float q[16];
#pragma unroll
        for (int e = 0; e < 16; e++) q[e] = int_code_f16(v[e], rs, qmax);
        {
          uint8_t* srow = slot + row * CB;   // this row's bytes of the chunk, in LDS
          if (FMT == FMT_INT4) {
            uint32_t w0 = 0, w1 = 0;
#pragma unroll
            for (int e = 0; e < 8; e++) {
              w0 |= ((uint32_t)(int)q[e] & 0xFu) << (4 * e);
              w1 |= ((uint32_t)(int)q[8 + e] & 0xFu) << (4 * e);
            }
            *reinterpret_cast<uint32_t*>(srow + 4 * sub) = w0;
            *reinterpret_cast<uint32_t*>(srow + 16 + 4 * sub) = w1;
          } else if (FMT == FMT_INT4_E2M3) {
            // 6-bit container: a (row, group) has 48 bytes; half h (codes 32h..32h+31) is 24
            // bytes of 6-bit fields whose bytes 0..15 sit at 16h and bytes 16..23 at 32 + 8h.
            // This lane's 8 codes of each half are fields 8 sub .. 8 sub + 7: the 6 bytes at
            // offset 6 sub of the half, written as three 16-bit pieces (none crosses byte 16).
#pragma unroll
            for (int hh = 0; hh < 2; hh++) {
              uint32_t lo = 0;                   // bits 0..31 of the 48-bit run
#pragma unroll
              for (int e = 0; e < 5; e++) lo |= e2m3_field(q[8 * hh + e]) << (6 * e);
              const uint32_t f5 = e2m3_field(q[8 * hh + 5]);
              lo |= f5 << 30;
              // bits 32..47
              const uint32_t hi = (f5 >> 2) | (e2m3_field(q[8 * hh + 6]) << 4) | (e2m3_field(q[8 * hh + 7]) << 10);
              const uint32_t piece[3] = {lo & 0xFFFFu, lo >> 16, hi & 0xFFFFu};
#pragma unroll
              for (int j = 0; j < 3; j++) {
                const int o = 6 * sub + 2 * j;   // byte offset within the half (even)
                const int pos = o < 16 ? 16 * hh + o : 32 + 8 * hh + (o - 16);
                *reinterpret_cast<uint16_t*>(srow + pos) = (uint16_t)piece[j];
              }
            }
          } else {
            uint32_t w[4];
#pragma unroll
            for (int k4 = 0; k4 < 4; k4++) {
              w[k4] = 0;
#pragma unroll
              for (int e = 0; e < 4; e++) w[k4] |= ((uint32_t)(int)q[4 * k4 + e] & 0xFFu) << (8 * e);
            }
            *reinterpret_cast<uint2*>(srow + 8 * sub) = make_uint2(w[0], w[1]);
            *reinterpret_cast<uint2*>(srow + 32 + 8 * sub) = make_uint2(w[2], w[3]);
          }
        }
        // the wave's 16 x CB bytes go out as CB/16 16-byte pieces per row
        __builtin_amdgcn_wave_barrier();
        if (lane < CB) {
          const int rr = lane / (CB / 16), part = lane % (CB / 16);
          const int mm = blockIdx.x * 16 + rr;
          const uint4 v16 = *reinterpret_cast<const uint4*>(slot + rr * CB + part * 16);
          if (mm < M) *reinterpret_cast<uint4*>(xq + (size_t)mm * code_row + (size_t)c * code_chunk + part * 16) = v16;
        }
        __builtin_amdgcn_wave_barrier();
        if (valid) {
          if (sub == 0) {
            // row-major scales [M, K/64]; the 6-bit container format keeps them group-major [K/64, M]
            const size_t si = FMT == FMT_INT4_E2M3 ? (size_t)c * M + m : (size_t)m * (K >> 6) + c;
            reinterpret_cast<uint16_t*>(xs)[si] = sbits;
          }
        }
      } else {  // FP4: groups of 16 = two lanes (sub, sub^1) x 8 values
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e++) { a0 = fmaxf(a0, fabsf(v[e])); a1 = fmaxf(a1, fabsf(v[8 + e])); }
        a0 = fmaxf(a0, __shfl_xor(a0, 16));
        a1 = fmaxf(a1, __shfl_xor(a1, 16));
        uint32_t b0, b1;
        const float s0 = fp4_scale(a0, &b0);
        const float s1 = fp4_scale(a1, &b1);
        int q[16];
#pragma unroll
        for (int e = 0; e < 8; e++) { q[e] = (int)fp4_code(v[e], s0); q[8 + e] = (int)fp4_code(v[8 + e], s1); }
        if (valid) {
          uint8_t* dst = xq + (size_t)m * (K >> 1);
          *reinterpret_cast<uint32_t*>(dst + (col >> 1)) = pack8(q);
          *reinterpret_cast<uint32_t*>(dst + ((col + 32) >> 1)) = pack8(q + 8);
          if ((sub & 1) == 0) {
            uint8_t* sd = xs + (size_t)m * (K >> 4) + c * 4 + (sub >> 1);
            sd[0] = (uint8_t)b0;
            sd[2] = (uint8_t)b1;
          }
        }
      }
    }
  }

  if (RB > 0) {
    // ---- reduce the waves' partials of T (fixed order) and store fp16
    __shared__ float part[NW][16][R > 0 ? R : 1];
#pragma unroll
    for (int j = 0; j < RB; j++)
#pragma unroll
      for (int i = 0; i < 4; i++) part[wave][4 * sub + i][j * 16 + row] = acc[j][i];
    __syncthreads();
    for (int idx = threadIdx.x; idx < 16 * R; idx += 64 * NW) {
      const int rr = idx / R, cc = idx % R;
      const int mm = blockIdx.x * 16 + rr;
      if (mm < M) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < NW; w++) s += part[w][rr][cc];
        t[(size_t)mm * R + cc] = __float2half_rn(s);
      }
    }
  }
}

template <int FMT, int RB, bool QUANT = true>
static hipError_t launch_qd(const QuantDownArgs& a, hipStream_t s) {
  dim3 grid((a.M + 15) / 16);
  hipLaunchKernelGGL((k_quant_down<FMT, RB, QUANT>), grid, dim3(64 * QD_WAVES), 0, s, (const __half*)a.x,
                     (const __half*)a.l1t, a.M, a.K, (uint8_t*)a.xq, (uint8_t*)a.xs, (__half*)a.t);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_qd_r(const QuantDownArgs& a, hipStream_t s) {
  switch (a.r) {
    case 0: return launch_qd<FMT, 0>(a, s);
    case 16: return launch_qd<FMT, 1>(a, s);
    case 32: return launch_qd<FMT, 2>(a, s);
    case 48: return launch_qd<FMT, 3>(a, s);
    case 64: return launch_qd<FMT, 4>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_quant_down(const QuantDownArgs& a, hipStream_t s) {
  switch (a.fmt) {
    case FMT_INT4: return launch_qd_r<FMT_INT4>(a, s);
    case FMT_INT4_E2M3: return launch_qd_r<FMT_INT4_E2M3>(a, s);
    case FMT_INT8: return launch_qd_r<FMT_INT8>(a, s);
    case FMT_FP4: return launch_qd_r<FMT_FP4>(a, s);
  }
  return hipErrorInvalidValue;
}

// Unfused comparison: quantization alone (no branch) ...
hipError_t launch_quant_only(const void* x, int M, int K, int fmt, void* xq, void* xs, hipStream_t s) {
  QuantDownArgs a{x, nullptr, M, K, 0, fmt, xq, xs, nullptr};
  return launch_quant_down(a, s);
}

// ... and the down projection alone, a second full read of X_hat.
hipError_t launch_down_only(const void* x, const void* l1t, int M, int K, int r, void* t, hipStream_t s) {
  QuantDownArgs a{x, l1t, M, K, r, FMT_INT4, nullptr, nullptr, t};
  switch (r) {
    case 16: return launch_qd<FMT_INT4, 1, false>(a, s);
    case 32: return launch_qd<FMT_INT4, 2, false>(a, s);
    case 48: return launch_qd<FMT_INT4, 3, false>(a, s);
    case 64: return launch_qd<FMT_INT4, 4, false>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace svdq
