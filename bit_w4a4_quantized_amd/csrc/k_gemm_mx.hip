// Kernel B for MXFP4 (SVDQ_MXFP4_G32): E2M1 codes, two per byte, and one E8M0 scale (a power of
// two) per 32 along K -- the block-scaled format of OCP Microscaling Formats v1.0, which
// gfx950's matrix cores take natively ("sota-314", "Conditions": the format ranking follows
// the hardware's native group support).
//
//   Y[m,n] = fp16_rne( sum_k (e2m1(q_x[m,k]) 2^(ex[m,k/32]-127)) (e2m1(q_w[n,k]) 2^(ew[n,k/32]-127))
//                      + (T L2)[m,n] + b[n] )
//
// In v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands (cbsz = blgp = 4) lane l holds row
// l % 32 and the 32 consecutive K values of half l / 32 of the 64-wide chunk, which is
// exactly one scale group, and takes one E8M0 scale per operand: the matrix core applies both
// groups' scales itself.  One instruction per 32 x 32 tile and chunk, and no vector work:
// no dequantization, no per-group rescale.  Products of E2M1 values times powers of two are
// exact, so the result is the exact sum up to the order of the fp32 additions.
//
// Codes and scales are chunk-major ([K/64][rows][32 bytes], [K/64][rows][2 bytes]), so a
// tile's operand rows for one 64-K chunk are one contiguous 4 KB run (and 256 bytes of scales):
// with rows laid out along K instead, each 16-byte load would touch 32 cache lines 1.5 KB apart
// and the staging ran at half the bandwidth.
//
// Stages of four 64-K chunks on the shared persistent skeleton (two chunks a stage left each
// stage waiting on the next one's loads: 142 -> 129 us at the fc1 shape).  Per chunk and workgroup: each
// operand's 128 rows x 32 code bytes arrive by 16-byte LDS-DMA loads into 16-byte slots
// swapped by row (slot c of row r at c ^ ((r / 8) % 2)), and the rows' 2 scale bytes by 2-byte
// loads into 4-byte slots.  Lane half h reads the chunk's codes 32 h .. 32 h + 31 (one
// 16-byte read) and scale byte h.
#include "gemm_skel.h"

namespace svdq {

namespace {

using namespace skel;

__device__ __forceinline__ v8i fp4_operand(const uint4& c) {
  return v8i{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
}

__device__ __forceinline__ v16f mx_mma(const uint4& w, const uint4& x, uint32_t sw, uint32_t sx, const v16f& acc) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(w), fp4_operand(x), acc, 4, 4, 0, (int)sw, 0,
                                                         (int)sx);
}

struct OpMX {
  static constexpr int KC = 4;               // 64-K chunks per stage: 4 x 9 KB of operands in flight per load
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

  __device__ OpMX(const uint8_t* xq, const uint8_t* xs, const uint8_t* wq, const uint8_t* ws, int M_, int N_, int K_)
      : M(M_), N(N_), K(K_) {
    C = K >> 6;
    NS = (C + KC - 1) / KC;
    NU = C;
    gxs = make_rsrc(xs, (size_t)M * K / 32);
    gws = make_rsrc(ws, (size_t)N * K / 32);
    lane = threadIdx.x & 63;
    h = lane >> 5;
    wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    rx = make_rsrc(xq, (size_t)M * K / 2);
    rw = make_rsrc(wq, (size_t)N * K / 2);
    rs = wave < 2 ? gxs : gws;
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
    s.vs = wave < 2 ? (uint32_t)min(m0 + srow, M - 1) * 2u : (uint32_t)min(n0 + srow, N - 1) * 2u;
    return s;
  }
  __device__ void load(const Src& s, int st, uint8_t* buf) const {
#pragma unroll
    for (int k = 0; k < KC; k++) {
      const int c = min(st * KC + k, C - 1);  // a chunk past the end re-reads the last one (unused)
      uint8_t* b = buf + k * CHUNK;
      dma16(rx, b + L_X + wave * 1024, s.vx, (uint32_t)c * (uint32_t)M * 32u);
      dma16(rw, b + L_W + wave * 1024, s.vw, (uint32_t)c * (uint32_t)N * 32u);
      dma2(rs, b + (wave < 2 ? L_SX : L_SW) + (wave & 1) * 256, s.vs, (uint32_t)c * (uint32_t)(wave < 2 ? M : N) * 2u);
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
        r.sx[k][i] = (*reinterpret_cast<const uint32_t*>(b + sxo[i]) >> (8 * h)) & 0xFFu;
        r.sw[k][i] = (*reinterpret_cast<const uint32_t*>(b + swo[i]) >> (8 * h)) & 0xFFu;
      }
    }
  }
  // sub-tile jobs: chunk u of the lane's X row m and W row n, codes 32 h .. 32 h + 31 (one
  // 16-byte piece) and their scale byte h (the LDS path's mapping)
  struct UR {
    uint4 x, w;
    uint32_t sx, sw;
  };
  __device__ void gload(int u, int m, int n, UR& o) const {
    o.x = as_u4(__builtin_amdgcn_raw_buffer_load_b128(rx, (int)((uint32_t)m * 32u + 16u * h), (int)((uint32_t)u * (uint32_t)M * 32u), 0));
    o.w = as_u4(__builtin_amdgcn_raw_buffer_load_b128(rw, (int)((uint32_t)n * 32u + 16u * h), (int)((uint32_t)u * (uint32_t)N * 32u), 0));
    o.sx = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(gxs, (int)((uint32_t)m * 2u + (uint32_t)h), (int)((uint32_t)u * (uint32_t)M * 2u), 0);
    o.sw = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(gws, (int)((uint32_t)n * 2u + (uint32_t)h), (int)((uint32_t)u * (uint32_t)N * 2u), 0);
  }
  __device__ void gmma(const UR& o, bool zero, v16f& acc) const {
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);   // zero codes: the unit adds exactly +0
    acc = mx_mma(zero ? z : o.w, zero ? z : o.x, o.sw, o.sx, acc);
  }
  __device__ void finish(v16f (&)[2][2]) const {}
  __device__ void mma(const Regs& r, int st, v16f (&acc)[2][2]) const {
#pragma unroll
    for (int k = 0; k < KC; k++) {
      if (st * KC + k >= C) break;
#pragma unroll
      for (int tj = 0; tj < 2; tj++)
#pragma unroll
        for (int ti = 0; ti < 2; ti++)
          acc[tj][ti] = mx_mma(r.w[k][tj], r.x[k][ti], r.sw[k][tj], r.sx[k][ti], acc[tj][ti]);
    }
  }
};

}  // namespace

template <int RB, bool BIAS>
__global__ void __launch_bounds__(NT, 2)
k_gemm_mx(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, const __half* __restrict__ t,
          const uint8_t* __restrict__ wq, const uint8_t* __restrict__ ws, const __half* __restrict__ l2,
          const __half* __restrict__ bias, const float* __restrict__ lam, int M, int N, int K,
          __half* __restrict__ y, int tiles_run) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * OpMX::BUF];
  OpMX op(xq, xs, wq, ws, M, N, K);
  persistent<OpMX, RB, BIAS>(op, lds, t, l2, bias, lam, M, N, tiles_run, y);
  subtile_jobs<OpMX, RB, BIAS>(op, lds, t, l2, bias, lam, M, N, tiles_run, y);
}

template <int RB, bool BIAS>
static hipError_t launch_mx_t(const GemmArgs& a, hipStream_t s) {
  int nb;
  const int main_tiles = persistent_split(a.M, a.N, &nb);
  hipLaunchKernelGGL((k_gemm_mx<RB, BIAS>), dim3(nb), dim3(NT), 0, s, (const uint8_t*)a.xq, (const uint8_t*)a.xs,
                     (const __half*)a.t, (const uint8_t*)a.wq, (const uint8_t*)a.ws, (const __half*)a.l2,
                     (const __half*)a.bias, a.lam, a.M, a.N, a.K, (__half*)a.y, main_tiles);
  return hipGetLastError();
}

template <bool BIAS>
static hipError_t launch_mx_r(const GemmArgs& a, hipStream_t s) {
  switch (a.r) {
    case 0: return launch_mx_t<0, BIAS>(a, s);
    case 16: return launch_mx_t<1, BIAS>(a, s);
    case 32: return launch_mx_t<2, BIAS>(a, s);
    case 48: return launch_mx_t<3, BIAS>(a, s);
    case 64: return launch_mx_t<4, BIAS>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_mx(const GemmArgs& a, hipStream_t s) {
  return a.bias ? launch_mx_r<true>(a, s) : launch_mx_r<false>(a, s);
}

}  // namespace svdq
