// Kernel B for the 8-bit setting (SVDQ_INT8_G64): codes in [-127, 127], one
// byte each, fp16 scale per 64 along K ("sota-314", "Do this": rank 16 at 8
// bits; same group rule as the 4-bit format with 127 in place of 7).
//
//   Y[m,n] = fp16_rne( sum_g sx[m,g] sw[n,g] P_g[m,n] + (T L2)[m,n] + b[n] )
//   P_g    = sum_{k in group g} q_x[m,k] q_w[n,k]   (exact int32)
//
// Per 32 x 32 tile and group: two v_mfma_i32_32x32x32_i8 give P_g exactly; one
// v_mfma_f32_32x32x8_f16 with the scales in K slot 0 gives sw[n] sx[m]
// exactly; the vector ALU converts P_g to fp32 (exact, |P_g| < 2^20) and does
// one fma per element.  Stages of two groups; per group and workgroup the 128
// rows x 64 bytes of each operand arrive by 16-byte LDS-DMA loads into
// 16-byte slots XOR-swizzled by row (slot c of row r at c ^ ((r / 4) % 4)), so
// the 16-byte reads of 16 consecutive rows hit distinct banks.  Lane half h
// takes bytes 32 h .. 32 h + 31 of each row's group (two k-steps of 16) for
// both operands.  The persistent loop and the epilogue are the shared skeleton.
#include "gemm_skel.h"

namespace svdq {

namespace {

using namespace skel;

struct OpI8 {
  static constexpr int KC = 2;               // groups per stage
  static constexpr int L_X = 0, L_W = 8192, L_SX = 16384, L_SW = 16896, GROUP = 17408;
  static constexpr int BUF = KC * GROUP;
  int M, N, K, G, NS;
  int lane, h, wave;
  bool s_x;                                  // this wave loads X (waves 0, 1) or W (2, 3)
  int rows;                                  // rows of the operand this wave loads (M or N)
  rsrc_t rc, rs;
  int xo[2][2], wo[2][2], sxo[2], swo[2];    // per-lane LDS read offsets within a group

  struct Src {
    uint32_t vc[4], vs;
  };
  struct Regs {
    uint4 x[KC][2][2], w[KC][2][2];
    uint32_t sx[KC][2], sw[KC][2];
  };

  __device__ OpI8(const int8_t* xq, const __half* xs, const int8_t* wq, const __half* ws, int M_, int N_, int K_)
      : M(M_), N(N_), K(K_) {
    G = K >> 6;
    NS = (G + KC - 1) / KC;
    lane = threadIdx.x & 63;
    h = lane >> 5;
    wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    s_x = wave < 2;
    rows = s_x ? M : N;
    rc = s_x ? make_rsrc(xq, (size_t)M * K) : make_rsrc(wq, (size_t)N * K);
    rs = s_x ? make_rsrc(xs, (size_t)M * G * 2) : make_rsrc(ws, (size_t)N * G * 2);
    const int wm = wave >> 1, wn = wave & 1, r32 = lane & 31;
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int xr = wm * 64 + i * 32 + r32, wr = wn * 64 + i * 32 + r32;
#pragma unroll
      for (int ks = 0; ks < 2; ks++) {
        xo[i][ks] = L_X + xr * 64 + 16 * ((2 * h + ks) ^ ((xr >> 2) & 3));
        wo[i][ks] = L_W + wr * 64 + 16 * ((2 * h + ks) ^ ((wr >> 2) & 3));
      }
      sxo[i] = L_SX + xr * 4;
      swo[i] = L_SW + wr * 4;
    }
  }

  // wave w loads rows 64 (w % 2) .. + 63 of its operand: four 16-row DMAs of codes (lane ->
  // row lane / 4, slot lane % 4 holding the swizzled piece) and one of scales.  Codes are
  // group-major ([K/64][rows][64 bytes], scales [K/64][rows]): the group's offset is scalar,
  // and a DMA's 16 rows are one contiguous 1 KB run.  Rows past the edge re-read the last row
  // (their outputs are never stored).
  __device__ Src src(int m0, int n0) const {
    const int r0 = s_x ? m0 : n0;
    Src s;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int row = (wave & 1) * 64 + 16 * i + (lane >> 2);
      const int c = (lane & 3) ^ ((row >> 2) & 3);
      s.vc[i] = (uint32_t)min(r0 + row, rows - 1) * 64u + 16u * c;
    }
    s.vs = (uint32_t)min(r0 + (wave & 1) * 64 + lane, rows - 1) * 2u;
    return s;
  }
  __device__ void load(const Src& s, int st, uint8_t* buf) const {
#pragma unroll
    for (int k = 0; k < KC; k++) {
      const int g = min(st * KC + k, G - 1);  // a group past the end re-reads the last one (unused)
      uint8_t* b = buf + k * GROUP;
#pragma unroll
      for (int i = 0; i < 4; i++)
        dma16(rc, b + (s_x ? L_X : L_W) + ((wave & 1) * 64 + 16 * i) * 64, s.vc[i], (uint32_t)g * (uint32_t)rows * 64u);
      dma2(rs, b + (s_x ? L_SX : L_SW) + (wave & 1) * 256, s.vs, (uint32_t)g * (uint32_t)rows * 2u);
    }
  }
  __device__ void read(const uint8_t* buf, int st, Regs& r) const {
#pragma unroll
    for (int k = 0; k < KC; k++) {
      if (st * KC + k >= G) break;
      const uint8_t* b = buf + k * GROUP;
#pragma unroll
      for (int i = 0; i < 2; i++) {
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
          r.x[k][i][ks] = *reinterpret_cast<const uint4*>(b + xo[i][ks]);
          r.w[k][i][ks] = *reinterpret_cast<const uint4*>(b + wo[i][ks]);
        }
        r.sx[k][i] = *reinterpret_cast<const uint32_t*>(b + sxo[i]);
        r.sw[k][i] = *reinterpret_cast<const uint32_t*>(b + swo[i]);
      }
    }
  }
  __device__ void finish(v16f (&)[2][2]) const {}
  __device__ void mma(const Regs& r, int st, v16f (&acc)[2][2]) const {
#pragma unroll
    for (int k = 0; k < KC; k++) {
      if (st * KC + k >= G) break;
#pragma unroll
      for (int tj = 0; tj < 2; tj++)
#pragma unroll
        for (int ti = 0; ti < 2; ti++) {
          v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(as_i4(r.w[k][tj][0]), as_i4(r.x[k][ti][0]), v16i{}, 0, 0, 0);
          p = __builtin_amdgcn_mfma_i32_32x32x32_i8(as_i4(r.w[k][tj][1]), as_i4(r.x[k][ti][1]), p, 0, 0, 0);
          const v16f sc = __builtin_amdgcn_mfma_f32_32x32x8f16(scale_operand(r.sw[k][tj], h),
                                                                scale_operand(r.sx[k][ti], h), v16f{}, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 16; i++) acc[tj][ti][i] = __builtin_fmaf((float)p[i], sc[i], acc[tj][ti][i]);
        }
    }
  }
};

}  // namespace

template <int RB, bool BIAS>
__global__ void __launch_bounds__(NT, 2)
k_gemm_i8(const int8_t* __restrict__ xq, const __half* __restrict__ xs, const __half* __restrict__ t,
          const int8_t* __restrict__ wq, const __half* __restrict__ ws, const __half* __restrict__ l2,
          const __half* __restrict__ bias, const float* __restrict__ lam, int M, int N, int K,
          __half* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * OpI8::BUF];
  OpI8 op(xq, xs, wq, ws, M, N, K);
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  persistent<OpI8, RB, BIAS>(op, lds, t, l2, bias, lam, M, N, tiles, y);
}

template <int RB, bool BIAS>
static hipError_t launch_i8_t(const GemmArgs& a, int nb, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm_i8<RB, BIAS>), dim3(nb), dim3(NT), 0, s, (const int8_t*)a.xq, (const __half*)a.xs,
                     (const __half*)a.t, (const int8_t*)a.wq, (const __half*)a.ws, (const __half*)a.l2,
                     (const __half*)a.bias, a.lam, a.M, a.N, a.K, (__half*)a.y);
  return hipGetLastError();
}

template <bool BIAS>
static hipError_t launch_i8_r(const GemmArgs& a, int nb, hipStream_t s) {
  switch (a.r) {
    case 0: return launch_i8_t<0, BIAS>(a, nb, s);
    case 16: return launch_i8_t<1, BIAS>(a, nb, s);
    case 32: return launch_i8_t<2, BIAS>(a, nb, s);
    case 48: return launch_i8_t<3, BIAS>(a, nb, s);
    case 64: return launch_i8_t<4, BIAS>(a, nb, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_i8(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const int nb = tiles < resident_workgroups() ? tiles : resident_workgroups();
  return a.bias ? launch_i8_r<true>(a, nb, s) : launch_i8_r<false>(a, nb, s);
}

}  // namespace svdq
