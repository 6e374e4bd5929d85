// Kernel A: quantize the smoothed activations and compute the down projection
// T = X_hat L1 in one pass over X_hat.
//
// Practice page "sota-314", section "Do this": the down projection is fused
// with quantization since both consume X_hat; reading note
// "note-257", section "Key results": unfused, the branch pays an extra 16-bit
// read of the activations.
//
// Work decomposition (gfx950, wave64):
//   a workgroup (four waves) takes a block of 16 NRT token rows and a slice of
//   K (cpb 64-column chunks); its waves take the slice's chunks round-robin,
//   one chunk in flight per wave (the chunk is loaded, then processed).  Slicing K
//   gives enough workgroups to cover the chip whatever K is, and keeps each
//   wave's chain of dependent loads short.  Each wave keeps its NRT x r/16 tiles of 16 x 16 partial sums of T
//   in MFMA accumulators; the four waves' partials are added through LDS in a
//   fixed order; with one slice the workgroup rounds T to fp16, otherwise it
//   writes its fp32 partial to the caller's workspace and k_t_finalize adds
//   the slices in slice order and rounds (deterministic, no atomics).
//   Lane l of a wave owns row (l % 16) of each 16-row tile and the 8-column
//   slices [8 (l/16), +8) and [32 + 8 (l/16), +8) of each chunk: one 16-byte
//   load each, which is exactly the operand layout of v_mfma_f32_16x16x32_f16
//   for the chunk's two 32-column halves, so the fp16 values feed the matrix
//   core straight from the registers they are quantized from, and one L1^T
//   fragment serves all NRT row tiles.
//   Group absmax: within the lane, then across the 4 lanes of the row with two
//   cross-lane xor shuffles (INT, group 64) or one (FP4, group 16).
//   Codes are computed without divisions: the scale from amax times RN(1/qmax)
//   and the quotient x/s from v_rcp_f32 and one fma refinement, both provably
//   equal to the divisions' correctly rounded results for fp16 inputs
//   (quant_core.h); the 6-bit container's fields are packed by the FP6 convert
//   instruction.  A chunk's codes are assembled in the wave's LDS slot and
//   written with whole 16-byte stores.
// With SMOOTH the input is the unsmoothed x and lam [K] the layer's smoothing factors: each
// lane fetches one lam value per chunk with the chunk's loads (the chunk's 64 values across
// the wave), takes its 16 columns' values from the other lanes with cross-lane shuffles, and
// replaces each fp16 x by X_hat = fp16_rne(x / lam) (IEEE fp32 division, one rounding to
// fp16) before anything else reads it: codes, scales and T are those of X_hat.
#include "kernels.h"
#include "quant_core.h"

namespace svdq {

namespace {

constexpr int QD_NT = 256;                  // four waves
constexpr int QD_NRT = 4;                   // 16-row tiles per block for r <= 32 (2 above)
constexpr int QD_TARGET_BLOCKS = 512;       // workgroups that cover the chip once
constexpr int QD_FEW_ROWS = 256;            // up to this many token rows: 16-row blocks

template <int FMT>
__host__ __device__ constexpr int chunk_code_bytes() {   // code bytes per row and 64-column chunk
  return FMT == FMT_INT4_E2M3 ? 48 : (FMT == FMT_INT8 ? 64 : 32);
}

__host__ __device__ constexpr int cmax(int a, int b) { return a > b ? a : b; }

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef int v6i_t __attribute__((ext_vector_type(6)));
__device__ __forceinline__ h2_t as_h2(uint32_t w) { return __builtin_bit_cast(h2_t, w); }

}  // namespace

// waves per SIMD that the register budget allows at NRT row tiles and r = 16 RB (no spills);
// the smoothing variant holds the chunk's factors and division temporaries as well
__host__ __device__ constexpr int qd_waves_per_simd(int nrt, int rb, bool smooth) {
  return cmax(2, (nrt >= 4 ? 2 : (nrt == 2 ? (rb <= 2 ? 3 : 2) : (rb <= 2 ? 4 : (rb == 3 ? 3 : 2)))) - (smooth ? 1 : 0));
}

template <int FMT, int NRT, int RB, bool QUANT, bool SMOOTH>
__global__ void __launch_bounds__(QD_NT, qd_waves_per_simd(NRT, RB, SMOOTH))
k_quant_down(const __half* __restrict__ x, const __half* __restrict__ l1t, int M, int K, int cpb,
             uint8_t* __restrict__ xq, uint8_t* __restrict__ xs, __half* __restrict__ t,
             float* __restrict__ part, const float* __restrict__ lam) {
  constexpr int R = RB * 16;
  constexpr int RBX = RB > 0 ? RB : 1;
  constexpr int ROWS = 16 * NRT;
  constexpr int CB = chunk_code_bytes<FMT>();
  constexpr bool STAGE = QUANT;                            // codes go out through LDS
  constexpr int RP = R + 4;                                 // padded row of the partial sums
  constexpr int SMEM = cmax(cmax(STAGE ? 4 * ROWS * CB : 0, RB > 0 ? 4 * ROWS * RP * 4 : 0), 16);
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = lane & 15, sub = lane >> 4;
  const int m0 = blockIdx.y * ROWS;
  const int nch = K >> 6;
  const int cbeg = blockIdx.x * cpb;
  const int cend = min(nch, cbeg + cpb);

  // rows past M re-read row M - 1: T rows are independent, and nothing of theirs is stored
  const __half* xr[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; rt++) xr[rt] = x + (size_t)min(m0 + rt * 16 + row, M - 1) * K + sub * 8;
  const __half* lr[RBX];
#pragma unroll
  for (int j = 0; j < RBX; j++) lr[j] = RB > 0 ? l1t + (size_t)(j * 16 + row) * K + sub * 8 : nullptr;

  v4f acc[NRT][RBX];
#pragma unroll
  for (int rt = 0; rt < NRT; rt++)
#pragma unroll
    for (int j = 0; j < RBX; j++) acc[rt][j] = v4f{0.f, 0.f, 0.f, 0.f};

  struct Buf {
    uint4 x[NRT][2];
    uint4 b[RBX][2];
    float l;                                 // SMOOTH: lam of the chunk's column `lane`
  };
  auto load = [&](int c, Buf& B) {
    const int col = c * 64;
    B.l = SMOOTH ? lam[col + lane] : 0.0f;
#pragma unroll
    for (int rt = 0; rt < NRT; rt++) {
      B.x[rt][0] = *reinterpret_cast<const uint4*>(xr[rt] + col);
      B.x[rt][1] = *reinterpret_cast<const uint4*>(xr[rt] + col + 32);
    }
#pragma unroll
    for (int j = 0; j < RB; j++) {
      B.b[j][0] = *reinterpret_cast<const uint4*>(lr[j] + col);
      B.b[j][1] = *reinterpret_cast<const uint4*>(lr[j] + col + 32);
    }
  };

  uint8_t* slot = smem + wave * ROWS * CB;   // this wave's code staging (STAGE)

  auto process = [&](int c, Buf& B) {
    if constexpr (SMOOTH) {
      // this lane's columns: 8 sub + e (first 16-byte piece) and 32 + 8 sub + e (second)
      float lv[16];
#pragma unroll
      for (int e = 0; e < 8; e++) {
        lv[e] = __shfl(B.l, sub * 8 + e);
        lv[8 + e] = __shfl(B.l, 32 + sub * 8 + e);
      }
#pragma unroll
      for (int rt = 0; rt < NRT; rt++)
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
          float v[8];
          unpack_h8(B.x[rt][hh], v);
          uint32_t w[4];
#pragma unroll
          for (int i = 0; i < 4; i++)
            w[i] = (uint32_t)__half_as_ushort(__float2half_rn(v[2 * i] / lv[8 * hh + 2 * i])) |
                   ((uint32_t)__half_as_ushort(__float2half_rn(v[2 * i + 1] / lv[8 * hh + 2 * i + 1])) << 16);
          B.x[rt][hh] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
    // ---- down projection on the matrix core (fp16 in, fp32 accumulate)
#pragma unroll
    for (int rt = 0; rt < NRT; rt++)
#pragma unroll
      for (int j = 0; j < RB; j++) {
        acc[rt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(B.x[rt][0]), as_h8(B.b[j][0]), acc[rt][j], 0, 0, 0);
        acc[rt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(B.x[rt][1]), as_h8(B.b[j][1]), acc[rt][j], 0, 0, 0);
      }
    if (!QUANT) return;
    // ---- quantize
    if (FMT == FMT_INT4 || FMT == FMT_INT8 || FMT == FMT_INT4_E2M3) {
      const float qmax = FMT == FMT_INT8 ? 127.0f : 7.0f;
      const float inv_qmax = FMT == FMT_INT8 ? 1.0f / 127.0f : 1.0f / 7.0f;   // RN(1 / qmax)
      // row tiles in pairs (one FP6 convert packs two tiles' fields); NRT == 1: a lone tile
#pragma unroll
      for (int rp = 0; rp < NRT; rp += 2) {
        constexpr int NP = NRT > 1 ? 2 : 1;
        float qv[NP][16];                    // the codes, as floats (+0 for code 0)
#pragma unroll
        for (int k = 0; k < NP; k++) {
          const int rt = rp + k;
          // group absmax: the lane's 16 fp16 values (packed max), then across the row's 4 lanes
          h2_t mx = h2_t{(_Float16)0, (_Float16)0};
#pragma unroll
          for (int hh = 0; hh < 2; hh++) {
            const uint32_t w[4] = {B.x[rt][hh].x, B.x[rt][hh].y, B.x[rt][hh].z, B.x[rt][hh].w};
#pragma unroll
            for (int i = 0; i < 4; i++) mx = __builtin_elementwise_max(mx, __builtin_elementwise_abs(as_h2(w[i])));
          }
          float amax = fmaxf((float)mx.x, (float)mx.y);
          amax = fmaxf(amax, __shfl_xor(amax, 16));
          amax = fmaxf(amax, __shfl_xor(amax, 32));
          uint16_t sbits;
          const float s = int_scale_f16in(amax, inv_qmax, &sbits);
          const float r = s == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(s);
          const _Float16* hv0 = reinterpret_cast<const _Float16*>(&B.x[rt][0]);
          const _Float16* hv1 = reinterpret_cast<const _Float16*>(&B.x[rt][1]);
          // code = rint_half_even(clamp(RN(x / s), +-qmax)); + 0.0f turns -0 into +0.  The fp16
          // values go into the mixed-precision fmas as they are (quot_rn_h).
#pragma unroll
          for (int e = 0; e < 16; e++)
            qv[k][e] = rintf(__builtin_amdgcn_fmed3f(quot_rn_h(e < 8 ? hv0[e] : hv1[e - 8], s, r), -qmax, qmax)) + 0.0f;
          const int m = m0 + rt * 16 + row;
          if (sub == 0 && m < M) {
            // group-major scales [K/64, M]
            reinterpret_cast<uint16_t*>(xs)[(size_t)c * M + m] = sbits;
          }
          uint8_t* srow = slot + (rt * 16 + row) * CB;   // this row's bytes of the chunk, in LDS
          if (FMT == FMT_INT4) {
            uint32_t w0 = 0, w1 = 0;
#pragma unroll
            for (int e = 0; e < 8; e++) {
              w0 |= ((uint32_t)(int)qv[k][e] & 0xFu) << (4 * e);
              w1 |= ((uint32_t)(int)qv[k][8 + e] & 0xFu) << (4 * e);
            }
            *reinterpret_cast<uint32_t*>(srow + 4 * sub) = w0;
            *reinterpret_cast<uint32_t*>(srow + 16 + 4 * sub) = w1;
          } else if (FMT == FMT_INT8) {
            uint32_t w[4];
#pragma unroll
            for (int k4 = 0; k4 < 4; k4++) {
              w[k4] = 0;
#pragma unroll
              for (int e = 0; e < 4; e++) w[k4] |= ((uint32_t)(int)qv[k][4 * k4 + e] & 0xFFu) << (8 * e);
            }
            *reinterpret_cast<uint2*>(srow + 8 * sub) = make_uint2(w[0], w[1]);
            *reinterpret_cast<uint2*>(srow + 32 + 8 * sub) = make_uint2(w[2], w[3]);
          }
        }
        if (FMT == FMT_INT4_E2M3) {
          // 6-bit container: a (row, group) has 48 bytes; half h (codes 32h..32h+31) is 24
          // bytes of 6-bit fields (the E2M3 encoding of code/8) whose bytes 0..15 sit at 16h
          // and bytes 16..23 at 32 + 8h.  This lane's 8 codes of each half are fields
          // 8 sub .. 8 sub + 7: the 6 bytes at offset 6 sub of the half.  One
          // v_cvt_scalef32_2xpk16_fp6_f32 (scale 8: exact division by 8; field 2j from the
          // first source, 2j + 1 from the second) packs the pair's 4 runs of 8 fields.
          v16f ev, od;
#pragma unroll
          for (int run = 0; run < 4; run++) {      // run = 2 (tile in the pair) + half
            const int k = run >> 1, hh = run & 1;
#pragma unroll
            for (int i = 0; i < 4; i++) {
              ev[4 * run + i] = k < NP ? qv[k < NP ? k : 0][8 * hh + 2 * i] : 0.0f;
              od[4 * run + i] = k < NP ? qv[k < NP ? k : 0][8 * hh + 2 * i + 1] : 0.0f;
            }
          }
          const v6i_t f = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 8.0f);
          const uint32_t d[6] = {(uint32_t)f[0], (uint32_t)f[1], (uint32_t)f[2], (uint32_t)f[3], (uint32_t)f[4], (uint32_t)f[5]};
#pragma unroll
          for (int run = 0; run < 2 * NP; run++) {
            const int rt = rp + (run >> 1), hh = run & 1;
            uint8_t* srow = slot + (rt * 16 + row) * CB;
#pragma unroll
            for (int j = 0; j < 3; j++) {
              const int p16 = 3 * run + j;           // 16-bit piece of the 192-bit result
              const uint16_t piece = (uint16_t)(d[p16 >> 1] >> (16 * (p16 & 1)));
              const int o = 6 * sub + 2 * j;         // byte offset within the half (even)
              const int pos = o < 16 ? 16 * hh + o : 32 + 8 * hh + (o - 16);
              *reinterpret_cast<uint16_t*>(srow + pos) = piece;
            }
          }
        }
      }
    } else if (FMT == FMT_MXFP4) {  // MXFP4: groups of 32 = the row's four lanes x 8 values, per half
#pragma unroll
      for (int rt = 0; rt < NRT; rt++) {
        float v[16];
        unpack_h8(B.x[rt][0], v);
        unpack_h8(B.x[rt][1], v + 8);
        const int m = m0 + rt * 16 + row;
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e++) { a0 = fmaxf(a0, fabsf(v[e])); a1 = fmaxf(a1, fabsf(v[8 + e])); }
        a0 = fmaxf(a0, __shfl_xor(a0, 16));
        a0 = fmaxf(a0, __shfl_xor(a0, 32));
        a1 = fmaxf(a1, __shfl_xor(a1, 16));
        a1 = fmaxf(a1, __shfl_xor(a1, 32));
        const int e0 = mx_exponent(a0), e1 = mx_exponent(a1);
        // codes from the hardware convert: v_cvt_scalef32_pk_fp4_f32 divides by the power-of-two
        // scale (exact) and rounds to the nearest E2M1 value, ties to the even mantissa,
        // saturating at 6, two values per instruction -- the quantizer's rule, checked against
        // it on tie points, saturation and signed zeros; a negative value that rounds to zero
        // comes out as -0 and is made +0.  (fp16 inputs keep e >= -26, a normal scale.)
        // the row's 32 code bytes of this chunk, in LDS (written out chunk-major below)
        uint8_t* srow = slot + (rt * 16 + row) * CB;
        *reinterpret_cast<uint32_t*>(srow + 4 * sub) = fp4_codes8(v, ldexpf(1.0f, e0));
        *reinterpret_cast<uint32_t*>(srow + 16 + 4 * sub) = fp4_codes8(v + 8, ldexpf(1.0f, e1));
        if (sub == 0 && m < M)                   // the row's two E8M0 bytes of this chunk
          *reinterpret_cast<uint16_t*>(xs + ((size_t)c * M + m) * 2) = (uint16_t)((e0 + 127) | ((e1 + 127) << 8));
      }
    } else {  // FP4: groups of 16 = two lanes (sub, sub^1) x 8 values
#pragma unroll
      for (int rt = 0; rt < NRT; rt++) {
        float v[16];
        unpack_h8(B.x[rt][0], v);
        unpack_h8(B.x[rt][1], v + 8);
        const int m = m0 + rt * 16 + row;
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e++) { a0 = fmaxf(a0, fabsf(v[e])); a1 = fmaxf(a1, fabsf(v[8 + e])); }
        a0 = fmaxf(a0, __shfl_xor(a0, 16));
        a1 = fmaxf(a1, __shfl_xor(a1, 16));
        uint32_t b0, b1;
        const float s0 = fp4_scale(a0, &b0);
        const float s1 = fp4_scale(a1, &b1);
        const float r0 = s0 == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(s0);
        const float r1 = s1 == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(s1);
        // codes of the exact quotients t = RN(v / s) from the hardware convert at scale 1
        float t[16];
#pragma unroll
        for (int e = 0; e < 8; e++) {
          t[e] = s0 == 0.0f ? 0.0f : quot_rn(v[e], s0, r0);
          t[8 + e] = s1 == 0.0f ? 0.0f : quot_rn(v[8 + e], s1, r1);
        }
        // the row's 32 code bytes of this chunk, in LDS (written out chunk-major below)
        uint8_t* srow = slot + (rt * 16 + row) * CB;
        *reinterpret_cast<uint32_t*>(srow + 4 * sub) = fp4_codes8(t, 1.0f);
        *reinterpret_cast<uint32_t*>(srow + 16 + 4 * sub) = fp4_codes8(t + 8, 1.0f);
        if (m < M && (sub & 1) == 0) {           // E4M3 bytes chunk-major [K/64][M][4]
          uint8_t* sd = xs + ((size_t)c * M + m) * 4 + (sub >> 1);
          sd[0] = (uint8_t)b0;
          sd[2] = (uint8_t)b1;
        }
      }
    }
    if (STAGE) {
      // the wave's ROWS x CB bytes go out as 16-byte pieces: the rows of one 64-K chunk are
      // contiguous ([K/64][M][CB]) in every format
      __builtin_amdgcn_wave_barrier();
      constexpr int PR = CB / 16;            // pieces per row
#pragma unroll
      for (int p0 = 0; p0 < ROWS * PR; p0 += 64) {
        const int p = p0 + lane;
        const int rr = p / PR, pc = p % PR;
        const int mm = m0 + rr;
        if (p < ROWS * PR && mm < M) {
          const uint4 v16 = *reinterpret_cast<const uint4*>(slot + rr * CB + pc * 16);
          uint8_t* dst = xq + ((size_t)c * M + mm) * CB + pc * 16;
          *reinterpret_cast<uint4*>(dst) = v16;
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  };

  // ---- this wave's chunks: cbeg + wave, + 4, ... up to clast, one at a time.  (With each wave
  // issuing its next chunk's loads before processing the current one, the whole input was
  // requested at once, every wave's data arrived near the end of the load phase and all the
  // quantization ran after it: 18.8 against 16.4 us at K = 3072, M = 4608; and the second buffer
  // held the kernel to two waves per SIMD instead of four.)
  int c = cbeg + wave;
  if (c < cend) {
    const int clast = c + ((cend - 1 - c) / 4) * 4;
    Buf B0;
    while (true) {
      load(c, B0);
      process(c, B0);
      c += 4;
      if (c > clast) break;
    }
  }

  if (RB > 0) {
    // ---- the four waves' partials of T, added in wave order through LDS
    __syncthreads();                         // the code staging shares these bytes
    float* red = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int rt = 0; rt < NRT; rt++)
#pragma unroll
      for (int j = 0; j < RB; j++)
#pragma unroll
        for (int i = 0; i < 4; i++) red[(wave * ROWS + rt * 16 + 4 * sub + i) * RP + j * 16 + row] = acc[rt][j][i];
    __syncthreads();
    for (int idx = tid; idx < ROWS * (R / 4); idx += QD_NT) {
      const int rr = idx / (R / 4), c4 = (idx % (R / 4)) * 4;
      const int mm = m0 + rr;
      if (mm >= M) continue;
      float sum[4];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        float s = red[rr * RP + c4 + e];
#pragma unroll
        for (int w = 1; w < 4; w++) s += red[(w * ROWS + rr) * RP + c4 + e];
        sum[e] = s;
      }
      if (part) {
        *reinterpret_cast<float4*>(part + ((size_t)blockIdx.x * M + mm) * R + c4) = make_float4(sum[0], sum[1], sum[2], sum[3]);
      } else {
        const uint32_t h0 = __half_as_ushort(__float2half_rn(sum[0])) | ((uint32_t)__half_as_ushort(__float2half_rn(sum[1])) << 16);
        const uint32_t h1 = __half_as_ushort(__float2half_rn(sum[2])) | ((uint32_t)__half_as_ushort(__float2half_rn(sum[3])) << 16);
        *reinterpret_cast<uint2*>(t + (size_t)mm * R + c4) = make_uint2(h0, h1);
      }
    }
  }
}

// T = fp16_rne( sum over slices s = 0, 1, ... of part[s] ), slices added in order; each
// thread issues up to 16 slices' loads before adding them (few token rows slice K into 12:
// one round of loads instead of two).
__global__ void __launch_bounds__(64)
k_t_finalize(const float* __restrict__ part, int S, size_t MR, __half* __restrict__ t) {
  constexpr int SR = 16;
  const size_t i = ((size_t)blockIdx.x * 64 + threadIdx.x) * 4;
  if (i >= MR) return;
  float4 a = *reinterpret_cast<const float4*>(part + i);
  for (int s0 = 1; s0 < S; s0 += SR) {
    float4 b[SR];
#pragma unroll
    for (int k = 0; k < SR; k++)
      if (s0 + k < S) b[k] = *reinterpret_cast<const float4*>(part + (size_t)(s0 + k) * MR + i);
#pragma unroll
    for (int k = 0; k < SR; k++)
      if (s0 + k < S) { a.x += b[k].x; a.y += b[k].y; a.z += b[k].z; a.w += b[k].w; }
  }
  const uint32_t h0 = __half_as_ushort(__float2half_rn(a.x)) | ((uint32_t)__half_as_ushort(__float2half_rn(a.y)) << 16);
  const uint32_t h1 = __half_as_ushort(__float2half_rn(a.z)) | ((uint32_t)__half_as_ushort(__float2half_rn(a.w)) << 16);
  *reinterpret_cast<uint2*>(t + i) = make_uint2(h0, h1);
}

// ---- launch plan: row blocks of 64 (32 for r > 32, and for r = 32 with smoothing; 16 when K
// cannot be sliced for want of a workspace), K sliced into chunks-per-block multiples of 4 so
// that about QD_TARGET_BLOCKS workgroups cover the chip.  The slicing is that of the plain
// variant's row blocks in both variants: T's partial sums are then added in the same groups
// and order, and the smoothing variant's T equals the plain one's on the smoothed input.
QuantDownPlan quant_down_plan(int M, int K, int r, bool have_partials, bool smooth) {
  QuantDownPlan p{};
  const int nch = K >> 6;
  const bool can_slice = r == 0 || have_partials;
  // rows per block within the register budget; few token rows (M <= 256) take 16-row blocks so
  // that more workgroups share the rows (M = 64, fc1 shape: 8.5 -> 6.2 us, graph-timed; the
  // slices, and so T's summation order, stay the same)
  const int nrt_plain = can_slice ? (M <= QD_FEW_ROWS ? 1 : (r <= 32 ? QD_NRT : 2)) : 1;
  p.nrt = smooth && can_slice && r == 32 ? 2 : nrt_plain;
  const long rows_blocks = (M + 16 * nrt_plain - 1) / (16 * nrt_plain);
  if (!can_slice) {
    p.cpb = nch;
  } else {
    long q = (long)nch * rows_blocks;                        // wave-chunks
    long per_wave = (q + 4L * QD_TARGET_BLOCKS / 2) / (4L * QD_TARGET_BLOCKS);
    if (per_wave < 1) per_wave = 1;
    p.cpb = (int)(4 * per_wave);
    if (p.cpb > nch) p.cpb = ((nch + 3) / 4) * 4;
  }
  p.slices = (nch + p.cpb - 1) / p.cpb;
  p.rows_blocks = (M + 16 * p.nrt - 1) / (16 * p.nrt);
  p.partial_bytes = (r > 0 && p.slices > 1) ? (size_t)p.slices * M * r * 4 : 0;
  return p;
}

template <int FMT, int NRT, int RB, bool QUANT, bool SMOOTH>
static hipError_t launch_qd(const QuantDownArgs& a, const QuantDownPlan& p, hipStream_t s) {
  float* part = (RB > 0 && p.slices > 1) ? static_cast<float*>(a.part) : nullptr;
  hipLaunchKernelGGL((k_quant_down<FMT, NRT, RB, QUANT, SMOOTH>), dim3(p.slices, p.rows_blocks), dim3(QD_NT), 0, s,
                     (const __half*)a.x, (const __half*)a.l1t, a.M, a.K, p.cpb, (uint8_t*)a.xq, (uint8_t*)a.xs,
                     (__half*)a.t, part, a.lam);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !part) return e;
  const size_t MR = (size_t)a.M * a.r;
  const unsigned blocks = (unsigned)((MR / 4 + 63) / 64);
  hipLaunchKernelGGL(k_t_finalize, dim3(blocks), dim3(64), 0, s, (const float*)part, p.slices, MR, (__half*)a.t);
  return hipGetLastError();
}

template <int FMT, int RB, bool QUANT, bool SMOOTH>
static hipError_t launch_qd_n(const QuantDownArgs& a, const QuantDownPlan& p, hipStream_t s) {
  switch (p.nrt) {
    case 4:
      if constexpr (RB <= 2 && QD_NRT == 4 && !(SMOOTH && RB == 2)) return launch_qd<FMT, 4, RB, QUANT, SMOOTH>(a, p, s);
      break;
    case 2: return launch_qd<FMT, 2, RB, QUANT, SMOOTH>(a, p, s);
    case 1: return launch_qd<FMT, 1, RB, QUANT, SMOOTH>(a, p, s);
  }
  return hipErrorInvalidValue;
}

template <int FMT, bool QUANT, bool SMOOTH = false>
static hipError_t launch_qd_r(const QuantDownArgs& a, hipStream_t s) {
  QuantDownPlan p = quant_down_plan(a.M, a.K, a.r, true, SMOOTH);
  if (p.partial_bytes > 0 && (!a.part || a.part_bytes < p.partial_bytes)) p = quant_down_plan(a.M, a.K, a.r, false, SMOOTH);
  switch (a.r) {
    case 0: return launch_qd_n<FMT, 0, QUANT, SMOOTH>(a, p, s);
    case 16: return launch_qd_n<FMT, 1, QUANT, SMOOTH>(a, p, s);
    case 32: return launch_qd_n<FMT, 2, QUANT, SMOOTH>(a, p, s);
    case 48: return launch_qd_n<FMT, 3, QUANT, SMOOTH>(a, p, s);
    case 64: return launch_qd_n<FMT, 4, QUANT, SMOOTH>(a, p, s);
  }
  return hipErrorInvalidValue;
}

template <bool SMOOTH>
static hipError_t launch_quant_down_s(const QuantDownArgs& a, hipStream_t s) {
  switch (a.fmt) {
    case FMT_INT4: return launch_qd_r<FMT_INT4, true, SMOOTH>(a, s);
    case FMT_INT4_E2M3: return launch_qd_r<FMT_INT4_E2M3, true, SMOOTH>(a, s);
    case FMT_INT8: return launch_qd_r<FMT_INT8, true, SMOOTH>(a, s);
    case FMT_FP4: return launch_qd_r<FMT_FP4, true, SMOOTH>(a, s);
    case FMT_MXFP4: return launch_qd_r<FMT_MXFP4, true, SMOOTH>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_quant_down(const QuantDownArgs& a, hipStream_t s) {
  return a.lam ? launch_quant_down_s<true>(a, s) : launch_quant_down_s<false>(a, s);
}

// Unfused comparison: quantization alone (no branch) ...
hipError_t launch_quant_only(const void* x, int M, int K, int fmt, void* xq, void* xs, hipStream_t s) {
  QuantDownArgs a{x, nullptr, M, K, 0, fmt, xq, xs, nullptr, nullptr, 0};
  return launch_quant_down(a, s);
}

// ... and the down projection alone, a second full read of X_hat.
hipError_t launch_down_only(const void* x, const void* l1t, int M, int K, int r, void* t, void* part,
                            size_t part_bytes, hipStream_t s) {
  QuantDownArgs a{x, l1t, M, K, r, FMT_INT4, nullptr, nullptr, t, part, part_bytes};
  return launch_qd_r<FMT_INT4, false>(a, s);
}

}  // namespace svdq
