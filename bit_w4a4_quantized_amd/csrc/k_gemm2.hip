// Kernel B for the packed-nibble format (SVDQ_INT4_G64): the low-bit GEMM on the INT8 matrix
// cores, the per-group rescale into fp32, the up projection and the bias in the epilogue.
//
// Practice page "sota-314", section "Do this": the up projection is fused with the 4-bit
// compute since both produce Y.
//
//   Y[m,n] = fp16_rne( sum_g sx[m,g] sw[n,g] P_g[m,n] + (T L2)[m,n] + b[n] )
//   P_g    = sum_{k in group g} q_x[m,k] q_w[n,k]   (exact)
//
// Codes and scales are group-major ([K/64][rows][32 bytes], [K/64][rows] fp16), so a GEMM
// tile's rows of one group are one contiguous run.  A lane takes the 16 bytes of codes
// 32 h .. 32 h + 31 of its row's group (h its half of the wave) and turns them into int8 16 q
// with two masks and a shift: the operands of two v_mfma_i32_32x32x32_i8, in the same K order
// for both operands, whose int32 result is 256 P_g exactly.  The scale products S = sw sx of
// a 32 x 32 tile come from one v_mfma_f32_32x32x8_f16 with the scales in K slot 0 (exact);
// the vector ALU converts the partial to fp32 (exact) and does one fma per element and group,
// acc += 256 P_g S; the accumulator is scaled by 1/256 once (exact: a power of two).
//
// Two kernels: the tiled one on the shared persistent LDS-DMA skeleton (gemm_skel.h), and, for
// few token rows, a weight-streaming one.  (The 6-bit container format has its own kernels on
// the FP6 matrix cores.)
#include "gemm_skel.h"
#include "quant_core.h"

namespace svdq {

namespace {

constexpr int NTHREADS = 256;

__device__ __forceinline__ uint32_t nib_lo16(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t nib_hi16(uint32_t w) { return w & 0xF0F0F0F0u; }

}  // namespace

// Few token rows (the weight-streaming regime, M <= 256): one workgroup per 32 output columns
// and a slab of up to 128 rows (MT tiles of 32; blockIdx.y picks the slab), so each weight row
// is read once per slab, in its packed layout (2/3 of the 6-bit container's bytes).  The
// four waves split K (groups w, w + 4, ...), each holding PD groups of loads in flight straight
// into registers: lane (r32, h) loads the 16 bytes of codes 32 h .. 32 h + 31 of its weight row
// and of each of its token rows, which, unpacked to 16 q with two masks and a shift, are its
// operands of the two v_mfma_i32_32x32x32_i8 of a group (the same K order on both sides).  The
// int32 result is 256 P_g exactly; the scale-product MFMA gives S = sw sx, one fma per element
// and group adds 256 P_g S, and the accumulator is scaled by 1/256 once (exact).  The waves'
// partial sums are added in LDS in wave order; wave 0 adds T L2 and the bias and stores.
template <int RB, bool BIAS, int MT, int PD>
__global__ void __launch_bounds__(NTHREADS, 2)
k_gemm2_skinny(const uint8_t* __restrict__ xq, const __half* __restrict__ xs, const __half* __restrict__ t,
               const uint8_t* __restrict__ wq, const __half* __restrict__ ws, const __half* __restrict__ l2,
               const __half* __restrict__ bias, const float* __restrict__ lam, int M, int N, int K,
               __half* __restrict__ y) {
  constexpr int R = RB * 16;
  __shared__ __attribute__((aligned(16))) float red[3][16][64];   // partials of waves 1..3, one row tile
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, r32 = lane & 31;
  const int G = K >> 6;
  const int nb = blockIdx.x * 32;
  const int mb = blockIdx.y * 32 * MT;
  const int n = min(nb + r32, N - 1);                    // this lane's weight row
  int mrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; mt++) mrow[mt] = min(mb + mt * 32 + r32, M - 1);

  typedef _Float16 v4h_t __attribute__((ext_vector_type(4)));
  struct Op { uint4 w; uint32_t sw; uint4 x[MT]; uint32_t sx[MT]; };
  // codes group-major [K/64][rows][32], scales [K/64][rows]: group offsets in the scalar
  // offset, row offsets per lane
  const rsrc_t rxq = make_rsrc(xq, (size_t)M * (K >> 1)), rwq = make_rsrc(wq, (size_t)N * (K >> 1));
  const rsrc_t rxs = make_rsrc(xs, (size_t)M * G * 2), rws = make_rsrc(ws, (size_t)N * G * 2);
  const uint32_t vw = (uint32_t)n * 32u + 16u * h, vsw = (uint32_t)n * 2u;
  auto load = [&](int g, Op& o) {
    const uint32_t gx = (uint32_t)g * (uint32_t)M, gw = (uint32_t)g * (uint32_t)N;
    o.w = as_u4(__builtin_amdgcn_raw_buffer_load_b128(rwq, (int)vw, (int)(gw * 32u), 0));
    // every lane loads (no branch around a load); the upper K half's scale is zeroed at use
    o.sw = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rws, (int)vsw, (int)(gw * 2u), 0);
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      o.x[mt] = as_u4(__builtin_amdgcn_raw_buffer_load_b128(rxq, (int)((uint32_t)mrow[mt] * 32u + 16u * h),
                                                            (int)(gx * 32u), 0));
      o.sx[mt] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rxs, (int)((uint32_t)mrow[mt] * 2u), (int)(gx * 2u), 0);
    }
  };
  // the epilogue's operands (L2 columns, bias, and T rows when MT <= 2), loaded by wave 0, which
  // alone uses them, before the K loop so that their latency overlaps it (from every wave they
  // were 26 more load instructions per wave ahead of the ring's)
  constexpr int MTT = MT <= 2 ? MT : 1;
  uint32_t lv[RB > 0 ? RB : 1][8];
  uint4 tv[MTT][RB > 0 ? RB : 1];
  uint2 braw[4];
  float4 lam4[4];                            // with the MLP glue folded in: the next layer's factors
#pragma unroll
  for (int kb = 0; kb < (RB > 0 ? RB : 1); kb++) {
#pragma unroll
    for (int e = 0; e < 8; e++) lv[kb][e] = 0u;
#pragma unroll
    for (int mt = 0; mt < MTT; mt++) tv[mt][kb] = make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int q = 0; q < 4; q++) {
    braw[q] = make_uint2(0u, 0u);
    lam4[q] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (wave == 0) {
#pragma unroll
    for (int kb = 0; kb < RB; kb++) {
#pragma unroll
      for (int e = 0; e < 8; e++) lv[kb][e] = __half_as_ushort(l2[(size_t)(kb * 16 + 8 * h + e) * N + n]);
      if (MT <= 2) {
#pragma unroll
        for (int mt = 0; mt < MTT; mt++)
          tv[mt][kb] = *reinterpret_cast<const uint4*>(t + (size_t)mrow[mt] * R + kb * 16 + 8 * h);
      }
    }
    const rsrc_t rl = make_rsrc(lam, lam ? (size_t)N * 4 : 0);
#pragma unroll
    for (int q = 0; q < 4; q++) {  // columns past N read the last four (their outputs are not stored)
      if (BIAS) braw[q] = *reinterpret_cast<const uint2*>(bias + min(nb + 8 * q + 4 * h, N - 4));
      if (lam) lam4[q] = load_f4(rl, min(nb + 8 * q + 4 * h, N - 4));
    }
  }
  v16f acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int i = 0; i < 16; i++) acc[mt][i] = 0.f;
  // step s processes slot s % PD (the wave's group s - PD, or, for s < PD and past the wave's
  // last group, a zeroed slot whose scale product is zero: exactly +0) and refills it with the
  // wave's group s (past the last one: the last one again, unused)
  const int ng = wave < G ? (G - 1 - wave) / 4 + 1 : 0;   // this wave's groups
  Op ring[PD];
#pragma unroll
  for (int j = 0; j < PD; j++) ring[j] = Op{};
  for (int s0 = 0; s0 < ng + PD; s0 += PD) {
#pragma unroll
    for (int j = 0; j < PD; j++) {
      const int st = s0 + j;
      // a slot without a group (st < PD, or past the wave's last group) adds nothing: its
      // work is skipped (a wave-uniform branch; the slot's refill below is unconditional)
      const bool empty = st < PD || st - PD >= ng;
      const bool zero = h;                   // the upper K half's lanes carry no scale
      const Op& cur = ring[j];
      if (!empty) {
      const v4i w0 = v4i{(int)nib_lo16(cur.w.x), (int)nib_hi16(cur.w.x), (int)nib_lo16(cur.w.y), (int)nib_hi16(cur.w.y)};
      const v4i w1 = v4i{(int)nib_lo16(cur.w.z), (int)nib_hi16(cur.w.z), (int)nib_lo16(cur.w.w), (int)nib_hi16(cur.w.w)};
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        const uint4 xc = cur.x[mt];
        const v4i x0 = v4i{(int)nib_lo16(xc.x), (int)nib_hi16(xc.x), (int)nib_lo16(xc.y), (int)nib_hi16(xc.y)};
        const v4i x1 = v4i{(int)nib_lo16(xc.z), (int)nib_hi16(xc.z), (int)nib_lo16(xc.w), (int)nib_hi16(xc.w)};
        v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(w0, x0, v16i{}, 0, 0, 0);
        p = __builtin_amdgcn_mfma_i32_32x32x32_i8(w1, x1, p, 0, 0, 0);
        // K slot 0 holds the scale for the lower-K-half lanes; the upper half contributes zeros
        const v16f sc = __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(v4h_t, make_uint2(zero ? 0u : cur.sw, 0u)),
                                                              __builtin_bit_cast(v4h_t, make_uint2(zero ? 0u : cur.sx[mt], 0u)),
                                                              v16f{}, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 16; i++) acc[mt][i] = __builtin_fmaf((float)p[i], sc[i], acc[mt][i]);
      }
      }
      load(ng > 0 ? wave + 4 * min(st, ng - 1) : 0, ring[j]);
      __builtin_amdgcn_sched_barrier(0);     // keep the slots in order: each waits for its own loads only
    }
  }
  // the four waves' partials (256 P_g S), added in wave order, one row tile at a time
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
    if (wave > 0) {
#pragma unroll
      for (int i = 0; i < 16; i++) red[wave - 1][i][lane] = acc[mt][i];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int i = 0; i < 16; i++)
        acc[mt][i] = (((acc[mt][i] + red[0][i][lane]) + red[1][i][lane]) + red[2][i][lane]) * (1.0f / 256.0f);
    }
    if (mt + 1 < MT) __syncthreads();        // red is reused by the next row tile
  }
  if (wave != 0) return;
  // up projection: row operand L2^T (columns n, gathered once), column operand T (rows m)
  uint4 lw[RB > 0 ? RB : 1];
#pragma unroll
  for (int kb = 0; kb < RB; kb++)
    lw[kb] = make_uint4(lv[kb][0] | (lv[kb][1] << 16), lv[kb][2] | (lv[kb][3] << 16),
                        lv[kb][4] | (lv[kb][5] << 16), lv[kb][6] | (lv[kb][7] << 16));
  float bv[4][4];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    bv[q][0] = BIAS ? __half2float(__ushort_as_half((unsigned short)(braw[q].x & 0xFFFFu))) : 0.f;
    bv[q][1] = BIAS ? __half2float(__ushort_as_half((unsigned short)(braw[q].x >> 16))) : 0.f;
    bv[q][2] = BIAS ? __half2float(__ushort_as_half((unsigned short)(braw[q].y & 0xFFFFu))) : 0.f;
    bv[q][3] = BIAS ? __half2float(__ushort_as_half((unsigned short)(braw[q].y >> 16))) : 0.f;
  }
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
#pragma unroll
    for (int kb = 0; kb < RB; kb++) {
      const uint4 tvk = MT <= 2 ? tv[MT <= 2 ? mt : 0][kb]
                                : *reinterpret_cast<const uint4*>(t + (size_t)mrow[mt] * R + kb * 16 + 8 * h);
      acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(lw[kb]), as_h8(tvk), acc[mt], 0, 0, 0);
    }
    // lane owns row mb + mt*32 + r32 and columns nb + 8 q + 4 h + j (reg 4 q + j)
    const int mo = mb + mt * 32 + r32;
    if (mo >= M) continue;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int no = nb + 8 * q + 4 * h;
      if (no >= N) continue;
      uint32_t hv[4];
#pragma unroll
      for (int j = 0; j < 4; j++) hv[j] = __half_as_ushort(__float2half_rn(acc[mt][4 * q + j] + bv[q][j]));
      if (lam) {                             // the MLP glue folded in: fp16(gelu(y) / lam)
        const float lq[4] = {lam4[q].x, lam4[q].y, lam4[q].z, lam4[q].w};
#pragma unroll
        for (int j = 0; j < 4; j++) hv[j] = gelu_div_h(hv[j], lq[j]);
      }
      *reinterpret_cast<uint2*>(y + (size_t)mo * N + no) = make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
    }
  }
}

// The tiled kernel on the shared persistent LDS-DMA skeleton (gemm_skel.h), in stages of three
// groups (fc1 shape: 306 us against 309 with four and 313 with two; the register-staged kernel
// it replaced took 334).  Per group and workgroup each operand's 128 rows x 32 code bytes arrive by 16-byte
// LDS-DMA loads into 16-byte slots swapped by row (slot c of row r at c ^ ((r / 8) % 2)), and
// the rows' fp16 scales by 2-byte loads into 4-byte slots.  Lane half h reads the group's codes
// 32 h .. 32 h + 31 of its rows (one 16-byte read), unpacked to 16 q for the two
// v_mfma_i32_32x32x32_i8 (the same K order for both operands), so each partial is 256 P_g and
// the accumulator is scaled by 1/256 once per tile (exact).
using skel::dma16;
using skel::dma2;
using skel::scale_operand;

struct OpI4 {
  static constexpr int KC = 3;               // groups per stage
  static constexpr int L_X = 0, L_W = 4096, L_SX = 8192, L_SW = 8704, GROUP = 9216;
  static constexpr int BUF = KC * GROUP;
  int M, N, K, G, NS;
  int lane, h, wave;
  rsrc_t rx, rw, rs;
  int xo[2], wo[2], sxo[2], swo[2];          // per-lane LDS read offsets within a group

  struct Src {
    uint32_t vx, vw, vs;
  };
  struct Regs {
    uint4 x[KC][2], w[KC][2];
    uint32_t sx[KC][2], sw[KC][2];
  };

  __device__ OpI4(const uint8_t* xq, const __half* xs, const uint8_t* wq, const __half* ws, int M_, int N_, int K_)
      : M(M_), N(N_), K(K_) {
    G = K >> 6;
    NS = (G + KC - 1) / KC;
    lane = threadIdx.x & 63;
    h = lane >> 5;
    wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    rx = make_rsrc(xq, (size_t)M * K / 2);
    rw = make_rsrc(wq, (size_t)N * K / 2);
    rs = wave < 2 ? make_rsrc(xs, (size_t)M * G * 2) : make_rsrc(ws, (size_t)N * G * 2);
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
      const int g = min(st * KC + k, G - 1);  // a group past the end re-reads the last one (unused)
      uint8_t* b = buf + k * GROUP;
      dma16(rx, b + L_X + wave * 1024, s.vx, (uint32_t)g * (uint32_t)M * 32u);
      dma16(rw, b + L_W + wave * 1024, s.vw, (uint32_t)g * (uint32_t)N * 32u);
      dma2(rs, b + (wave < 2 ? L_SX : L_SW) + (wave & 1) * 256, s.vs, (uint32_t)g * (uint32_t)(wave < 2 ? M : N) * 2u);
    }
  }
  __device__ void read(const uint8_t* buf, int st, Regs& r) const {
#pragma unroll
    for (int k = 0; k < KC; k++) {
      if (st * KC + k >= G) break;
      const uint8_t* b = buf + k * GROUP;
#pragma unroll
      for (int i = 0; i < 2; i++) {
        r.x[k][i] = *reinterpret_cast<const uint4*>(b + xo[i]);
        r.w[k][i] = *reinterpret_cast<const uint4*>(b + wo[i]);
        r.sx[k][i] = *reinterpret_cast<const uint32_t*>(b + sxo[i]);
        r.sw[k][i] = *reinterpret_cast<const uint32_t*>(b + swo[i]);
      }
    }
  }
  __device__ void finish(v16f (&acc)[2][2]) const {
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
      for (int b = 0; b < 2; b++)
#pragma unroll
        for (int i = 0; i < 16; i++) acc[a][b][i] *= 1.0f / 256.0f;
  }
  __device__ void mma(const Regs& r, int st, v16f (&acc)[2][2]) const {
#pragma unroll
    for (int k = 0; k < KC; k++) {
      if (st * KC + k >= G) break;
      v4i w[2][2], x[2][2];
#pragma unroll
      for (int i = 0; i < 2; i++) {
        const uint4 a = r.w[k][i], c = r.x[k][i];
        w[i][0] = v4i{(int)nib_lo16(a.x), (int)nib_hi16(a.x), (int)nib_lo16(a.y), (int)nib_hi16(a.y)};
        w[i][1] = v4i{(int)nib_lo16(a.z), (int)nib_hi16(a.z), (int)nib_lo16(a.w), (int)nib_hi16(a.w)};
        x[i][0] = v4i{(int)nib_lo16(c.x), (int)nib_hi16(c.x), (int)nib_lo16(c.y), (int)nib_hi16(c.y)};
        x[i][1] = v4i{(int)nib_lo16(c.z), (int)nib_hi16(c.z), (int)nib_lo16(c.w), (int)nib_hi16(c.w)};
      }
#pragma unroll
      for (int tj = 0; tj < 2; tj++)
#pragma unroll
        for (int ti = 0; ti < 2; ti++) {
          v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(w[tj][0], x[ti][0], v16i{}, 0, 0, 0);
          p = __builtin_amdgcn_mfma_i32_32x32x32_i8(w[tj][1], x[ti][1], p, 0, 0, 0);
          const v16f sc = __builtin_amdgcn_mfma_f32_32x32x8f16(scale_operand(r.sw[k][tj], h),
                                                                scale_operand(r.sx[k][ti], h), v16f{}, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 16; i++) acc[tj][ti][i] = __builtin_fmaf((float)p[i], sc[i], acc[tj][ti][i]);
        }
    }
  }
};

template <int RB, bool BIAS>
__global__ void __launch_bounds__(skel::NT, 2)
k_gemm2_lds(const uint8_t* __restrict__ xq, const __half* __restrict__ xs, const __half* __restrict__ t,
            const uint8_t* __restrict__ wq, const __half* __restrict__ ws, const __half* __restrict__ l2,
            const __half* __restrict__ bias, const float* __restrict__ lam, int M, int N, int K,
            __half* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * OpI4::BUF];
  OpI4 op(xq, xs, wq, ws, M, N, K);
  const int tiles = ((M + skel::BM - 1) / skel::BM) * ((N + skel::BN - 1) / skel::BN);
  skel::persistent<OpI4, RB, BIAS>(op, lds, t, l2, bias, lam, M, N, tiles, y);
}

template <int RB, bool BIAS>
static hipError_t launch_g2_lds(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.M + skel::BM - 1) / skel::BM) * ((a.N + skel::BN - 1) / skel::BN);
  const int nb = tiles < resident_workgroups() ? tiles : resident_workgroups();
  hipLaunchKernelGGL((k_gemm2_lds<RB, BIAS>), dim3(nb), dim3(skel::NT), 0, s, (const uint8_t*)a.xq,
                     (const __half*)a.xs, (const __half*)a.t, (const uint8_t*)a.wq, (const __half*)a.ws,
                     (const __half*)a.l2, (const __half*)a.bias, a.lam, a.M, a.N, a.K, (__half*)a.y);
  return hipGetLastError();
}

// Up to this many token rows the weight-streaming kernel runs (in 32- or 128-row slabs).
constexpr int kSkinnyRows2 = 256;

template <int RB, bool BIAS, int MT, int PD = (MT <= 2 ? 4 : 2)>
static hipError_t launch_g2_skinny(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm2_skinny<RB, BIAS, MT, PD>), dim3((a.N + 31) / 32, (a.M + 32 * MT - 1) / (32 * MT)),
                     dim3(NTHREADS), 0, s, (const uint8_t*)a.xq, (const __half*)a.xs, (const __half*)a.t,
                     (const uint8_t*)a.wq, (const __half*)a.ws, (const __half*)a.l2, (const __half*)a.bias, a.lam,
                     a.M, a.N, a.K, (__half*)a.y);
  return hipGetLastError();
}

template <int RB, bool BIAS>
static hipError_t launch_g2(const GemmArgs& a, hipStream_t s) {
  // 32-row slabs up to 192 rows: three such workgroups fit a CU, which spreads the column
  // blocks over the CUs more evenly than 64- or 128-row slabs; at 256 rows the 128-row slabs,
  // which unpack each weight fragment once for four row tiles, are faster.  Ring depth: fewer
  // groups in flight per wave get each wave's data sooner once every wave also has work to
  // do with it (4 up to 32 rows, then 2; 1 for the 128-row slabs)
  if (a.M <= 32) return launch_g2_skinny<RB, BIAS, 1, 4>(a, s);
  if (a.M <= 192) return launch_g2_skinny<RB, BIAS, 1, 2>(a, s);
  if (a.M <= kSkinnyRows2) return launch_g2_skinny<RB, BIAS, 4, 1>(a, s);
  return launch_g2_lds<RB, BIAS>(a, s);
}

template <bool BIAS>
static hipError_t launch_g2_r(const GemmArgs& a, hipStream_t s) {
  switch (a.r) {
    case 0: return launch_g2<0, BIAS>(a, s);
    case 16: return launch_g2<1, BIAS>(a, s);
    case 32: return launch_g2<2, BIAS>(a, s);
    case 48: return launch_g2<3, BIAS>(a, s);
    case 64: return launch_g2<4, BIAS>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm2(const GemmArgs& a, hipStream_t s) {
  const bool b = a.bias != nullptr;
  if (a.fmt == FMT_INT4) return b ? launch_g2_r<true>(a, s) : launch_g2_r<false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace svdq
