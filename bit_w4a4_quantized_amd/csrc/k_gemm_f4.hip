// Kernel B for the FP4 setting (SVDQ_FP4_G16): E2M1 codes, two per byte, and
// one E4M3FN scale per 16 along K ("sota-314", "Do this": NVFP4 group 16 with
// FP8 scales; "Conditions": the format ranking depends on the GPU).
//
//   Y[m,n] = fp16_rne( sum_k (e2m1(q_x[m,k]) sx[m,k/16]) (e2m1(q_w[n,k]) sw[n,k/16])
//                      + (T L2)[m,n] + b[n] )
//
// gfx950's block-scaled FP4 matrix instruction applies one power-of-two scale
// per 32 values of K, so it cannot apply E4M3 scales per 16.  An E2M1 value
// times an E4M3 scale needs at most 6 significant bits and lies in
// [2^-10, 2688], so it is exact in fp16; the kernel therefore dequantizes both
// operands exactly to fp16 in registers (v_cvt_scalef32_pk_f16_fp4 with scale
// 1, then one packed fp16 multiply by the scale) and runs the fp16 matrix
// cores, v_mfma_f32_32x32x16_f16.  Every product is exact in fp32, so the
// result is the exact sum over all of K (the same value as summing the per-16
// partials P_g times sx sw), up to the order of the fp32 additions.
//
// Stages of two 64-K chunks.  Per chunk and workgroup: each operand's 128 rows
// x 32 code bytes arrive by 16-byte LDS-DMA loads into 16-byte slots swapped by
// row (slot c of row r at c ^ ((r / 8) % 2)), and the rows' 4 scale bytes by
// 4-byte loads.  Lane half h takes the chunk's codes 32 h .. 32 h + 31 (one
// 16-byte read): k-step ks uses codes 32 h + 8 ks .. + 7 (dword ks), whose
// scale is byte 2 h + ks / 2 of the row's scale dword.
#include "gemm_skel.h"

namespace svdq {

namespace {

using namespace skel;

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

// Eight E2M1 codes (dword, code j at bits 4j..4j+3) times the fp16 scale pair s2: the four
// fp16 pairs of the MFMA operand.
__device__ __forceinline__ uint4 dequant_fp4x8(uint32_t d, h2_t s2) {
  uint32_t r[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    h2_t v;
    switch (j) {                             // the byte selector is an immediate
      case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0); break;
      case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1); break;
      case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2); break;
      default: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3); break;
    }
    v = v * s2;                              // exact: the product fits fp16
    __builtin_memcpy(&r[j], &v, 4);
  }
  return make_uint4(r[0], r[1], r[2], r[3]);
}

// fp16 pairs (s, s) of the two E4M3FN scale bytes in bits 0..15 of sd (exact conversions)
__device__ __forceinline__ void scale_pairs(uint32_t sd, h2_t* lo, h2_t* hi) {
  const float a = __builtin_amdgcn_cvt_f32_fp8((int)sd, 0);
  const float b = __builtin_amdgcn_cvt_f32_fp8((int)sd, 1);
  *lo = __builtin_bit_cast(h2_t, __builtin_amdgcn_cvt_pkrtz(a, a));
  *hi = __builtin_bit_cast(h2_t, __builtin_amdgcn_cvt_pkrtz(b, b));
}

struct OpF4 {
  static constexpr int KC = 2;               // 64-K chunks per stage
  static constexpr int SUB_PD = 4;           // sub-tile jobs: units in flight per wave
  static constexpr int L_X = 0, L_W = 4096, L_SX = 8192, L_SW = 8704, CHUNK = 9216;
  static constexpr int BUF = KC * CHUNK;
  int M, N, K, C, NS, NU;
  int lane, h, wave;
  rsrc_t rx, rw, rs;
  rsrc_t gxs, gws;                           // whole scale arrays, for the sub-tile jobs' loads
  int xo[2], wo[2], sxo[2], swo[2];          // per-lane LDS read offsets within a chunk

  struct Src {
    uint32_t vx, vw, vs;
  };
  struct Regs {
    uint4 x[KC][2], w[KC][2];
    uint32_t sx[KC][2], sw[KC][2];
  };

  __device__ OpF4(const uint8_t* xq, const uint8_t* xs, const uint8_t* wq, const uint8_t* ws, int M_, int N_, int K_)
      : M(M_), N(N_), K(K_) {
    C = K >> 6;
    NS = (C + KC - 1) / KC;
    NU = C;
    gxs = make_rsrc(xs, (size_t)M * K / 16);
    gws = make_rsrc(ws, (size_t)N * K / 16);
    lane = threadIdx.x & 63;
    h = lane >> 5;
    wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    rx = make_rsrc(xq, (size_t)M * K / 2);
    rw = make_rsrc(wq, (size_t)N * K / 2);
    rs = wave < 2 ? make_rsrc(xs, (size_t)M * K / 16) : make_rsrc(ws, (size_t)N * K / 16);
    const int wm = wave >> 1, wn = wave & 1, r32 = lane & 31;
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int xr = wm * 64 + i * 32 + r32, wr = wn * 64 + i * 32 + r32;
      xo[i] = L_X + xr * 32 + 16 * (h ^ ((xr >> 3) & 1));
      wo[i] = L_W + wr * 32 + 16 * (h ^ ((wr >> 3) & 1));
      sxo[i] = L_SX + xr * 4;
      swo[i] = L_SW + wr * 4;
    }
  }

  // wave w loads rows 32 w .. 32 w + 31 of both code tiles (lane -> row lane / 2, slot
  // lane % 2 holding the swapped piece) and rows 64 (w % 2) .. + 63 of the X (w < 2) or W
  // scales.  Rows past the edge re-read the last row (their outputs are never stored).
  __device__ Src src(int m0, int n0) const {
    const int row = wave * 32 + (lane >> 1);
    const int c = (lane & 1) ^ ((row >> 3) & 1);
    Src s;
    s.vx = (uint32_t)min(m0 + row, M - 1) * 32u + 16u * c;
    s.vw = (uint32_t)min(n0 + row, N - 1) * 32u + 16u * c;
    const int srow = (wave & 1) * 64 + lane;
    s.vs = wave < 2 ? (uint32_t)min(m0 + srow, M - 1) * 4u : (uint32_t)min(n0 + srow, N - 1) * 4u;
    return s;
  }
  __device__ void load(const Src& s, int st, uint8_t* buf) const {
#pragma unroll
    for (int k = 0; k < KC; k++) {
      const int c = min(st * KC + k, C - 1);  // a chunk past the end re-reads the last one (unused)
      uint8_t* b = buf + k * CHUNK;
      dma16(rx, b + L_X + wave * 1024, s.vx, (uint32_t)c * (uint32_t)M * 32u);
      dma16(rw, b + L_W + wave * 1024, s.vw, (uint32_t)c * (uint32_t)N * 32u);
      dma4(rs, b + (wave < 2 ? L_SX : L_SW) + (wave & 1) * 256, s.vs, (uint32_t)c * (uint32_t)(wave < 2 ? M : N) * 4u);
    }
  }
  __device__ void read(const uint8_t* buf, int st, Regs& r) const {
#pragma unroll
    for (int k = 0; k < KC; k++) {
      if (st * KC + k >= C) break;
      const uint8_t* b = buf + k * CHUNK;
#pragma unroll
      for (int i = 0; i < 2; i++) {
        r.x[k][i] = *reinterpret_cast<const uint4*>(b + xo[i]);
        r.w[k][i] = *reinterpret_cast<const uint4*>(b + wo[i]);
        r.sx[k][i] = *reinterpret_cast<const uint32_t*>(b + sxo[i]);
        r.sw[k][i] = *reinterpret_cast<const uint32_t*>(b + swo[i]);
      }
    }
  }
  // sub-tile jobs: chunk u of the lane's X row m and W row n, codes 32 h .. 32 h + 31 (one
  // 16-byte piece) and their two scale bytes 2 h, 2 h + 1 (the LDS path's mapping)
  struct UR {
    uint4 x, w;
    uint32_t sx, sw;
  };
  __device__ void gload(int u, int m, int n, UR& o) const {
    o.x = as_u4(__builtin_amdgcn_raw_buffer_load_b128(rx, (int)((uint32_t)m * 32u + 16u * h), (int)((uint32_t)u * (uint32_t)M * 32u), 0));
    o.w = as_u4(__builtin_amdgcn_raw_buffer_load_b128(rw, (int)((uint32_t)n * 32u + 16u * h), (int)((uint32_t)u * (uint32_t)N * 32u), 0));
    o.sx = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(gxs, (int)((uint32_t)m * 4u + 2u * h), (int)((uint32_t)u * (uint32_t)M * 4u), 0);
    o.sw = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(gws, (int)((uint32_t)n * 4u + 2u * h), (int)((uint32_t)u * (uint32_t)N * 4u), 0);
  }
  __device__ void gmma(const UR& o, bool zero, v16f& acc) const {
    h2_t xs_lo, xs_hi, ws_lo, ws_hi;         // a zero scale makes every dequantized value 0
    scale_pairs(zero ? 0u : o.sx, &xs_lo, &xs_hi);
    scale_pairs(zero ? 0u : o.sw, &ws_lo, &ws_hi);
    const uint32_t xd[4] = {o.x.x, o.x.y, o.x.z, o.x.w}, wd[4] = {o.w.x, o.w.y, o.w.z, o.w.w};
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      const uint4 xv = dequant_fp4x8(xd[ks], ks < 2 ? xs_lo : xs_hi);
      const uint4 wv = dequant_fp4x8(wd[ks], ks < 2 ? ws_lo : ws_hi);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(wv), as_h8(xv), acc, 0, 0, 0);
    }
  }
  __device__ void finish(v16f (&)[2][2]) const {}
  __device__ void mma(const Regs& r, int st, v16f (&acc)[2][2]) const {
#pragma unroll
    for (int k = 0; k < KC; k++) {
      if (st * KC + k >= C) break;
      h2_t xs_lo[2], xs_hi[2], ws_lo[2], ws_hi[2];
#pragma unroll
      for (int i = 0; i < 2; i++) {
        scale_pairs(r.sx[k][i] >> (16 * h), &xs_lo[i], &xs_hi[i]);
        scale_pairs(r.sw[k][i] >> (16 * h), &ws_lo[i], &ws_hi[i]);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ks++) {
        uint4 xv[2], wv[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
          const uint32_t xd = ks == 0 ? r.x[k][i].x : ks == 1 ? r.x[k][i].y : ks == 2 ? r.x[k][i].z : r.x[k][i].w;
          const uint32_t wd = ks == 0 ? r.w[k][i].x : ks == 1 ? r.w[k][i].y : ks == 2 ? r.w[k][i].z : r.w[k][i].w;
          xv[i] = dequant_fp4x8(xd, ks < 2 ? xs_lo[i] : xs_hi[i]);
          wv[i] = dequant_fp4x8(wd, ks < 2 ? ws_lo[i] : ws_hi[i]);
        }
#pragma unroll
        for (int tj = 0; tj < 2; tj++)
#pragma unroll
          for (int ti = 0; ti < 2; ti++)
            acc[tj][ti] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(wv[tj]), as_h8(xv[ti]), acc[tj][ti], 0, 0, 0);
      }
    }
  }
};

}  // namespace

template <int RB, bool BIAS>
__global__ void __launch_bounds__(NT, 2)
k_gemm_f4(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, const __half* __restrict__ t,
          const uint8_t* __restrict__ wq, const uint8_t* __restrict__ ws, const __half* __restrict__ l2,
          const __half* __restrict__ bias, const float* __restrict__ lam, int M, int N, int K,
          __half* __restrict__ y, int tiles_run) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * OpF4::BUF];
  OpF4 op(xq, xs, wq, ws, M, N, K);
  persistent<OpF4, RB, BIAS>(op, lds, t, l2, bias, lam, M, N, tiles_run, y);
  subtile_jobs<OpF4, RB, BIAS>(op, lds, t, l2, bias, lam, M, N, tiles_run, y);
}

template <int RB, bool BIAS>
static hipError_t launch_f4_t(const GemmArgs& a, hipStream_t s) {
  int nb;
  const int main_tiles = persistent_split(a.M, a.N, &nb);
  hipLaunchKernelGGL((k_gemm_f4<RB, BIAS>), dim3(nb), dim3(NT), 0, s, (const uint8_t*)a.xq, (const uint8_t*)a.xs,
                     (const __half*)a.t, (const uint8_t*)a.wq, (const uint8_t*)a.ws, (const __half*)a.l2,
                     (const __half*)a.bias, a.lam, a.M, a.N, a.K, (__half*)a.y, main_tiles);
  return hipGetLastError();
}

template <bool BIAS>
static hipError_t launch_f4_r(const GemmArgs& a, hipStream_t s) {
  switch (a.r) {
    case 0: return launch_f4_t<0, BIAS>(a, s);
    case 16: return launch_f4_t<1, BIAS>(a, s);
    case 32: return launch_f4_t<2, BIAS>(a, s);
    case 48: return launch_f4_t<3, BIAS>(a, s);
    case 64: return launch_f4_t<4, BIAS>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_f4(const GemmArgs& a, hipStream_t s) {
  return a.bias ? launch_f4_r<true>(a, s) : launch_f4_r<false>(a, s);
}

}  // namespace svdq
