// Kernel B for the canonical packed-nibble format (SVDQ_INT4_G64), LDS-staged:
// low-bit GEMM on the INT8 matrix cores, per-group rescale into fp32, up
// projection and bias in the epilogue.
//
// Practice page "sota-314", section "Do this": the up projection is fused
// with the 4-bit compute since both produce Y.
//
//   Y[m,n] = fp16_rne( sum_g sx[m,g] sw[n,g] P_g[m,n] + (T L2)[m,n] + b[n] )
//   P_g    = sum_{k in group g} q_x[m,k] q_w[n,k]   (exact)
//
// Each lane reads 16 bytes of packed nibbles and turns them into int8 16q with
// two masks and a shift; two v_mfma_i32_32x32x32_i8 per tile per group; the
// int32 partial is converted to fp32.  Codes and scales are group-major
// ([K/64][rows][32 bytes], [K/64][rows] fp16), so a tile's rows of one group are
// one contiguous run.  (The 6-bit container format has its own kernel on the
// FP6 matrix cores.)
//
// Tiling (gfx950, wave64): workgroup tile 128 x 128, four waves in 2 x 2 of
// 64 x 64 (2 x 2 MFMA tiles of 32 x 32), two workgroups per CU.  K advances in
// stages of KC groups of 64: the workgroup stages both code tiles and the
// 256 fp16 scales per group in LDS, in a ring of two stages, and the
// global loads run two stages ahead of the compute (registers hold stage s+2
// while LDS holds s and s+1), so a stage's HBM/L2 latency is covered by a full
// stage of compute.  LDS row strides (56 and 48 bytes) make the
// per-lane 8- and 16-byte reads of 16 / 8 consecutive rows hit distinct banks.
// The block index is remapped so that each XCD (own L2) works on a
// contiguous range of tiles, rastered in groups of 8 tile rows.
//
// Rescale: the per-group scale products S = sx sw^T of a 32 x 32 tile come from
// one v_mfma_f32_32x32x16_f16 with the scales in a single K slot (exact), so
// the vector ALU does one fma per element and group, acc += P_g * S.
//
// Epilogue: acc += T L2 on v_mfma_f32_32x32x16_f16 (fp16 in, fp32 out),
// + bias, RNE to fp16, store.
#include <type_traits>

#include "kernels.h"
#include "quant_core.h"

namespace svdq {

namespace {

constexpr int BM = 128, BN = 128, NTHREADS = 256;

template <int CORE> struct CoreCfg;
template <> struct CoreCfg<CORE_I4> {
  static constexpr int GB = 32;
  static constexpr int LS = 48;
  static constexpr int CHUNKS = 2;
};

__device__ __forceinline__ uint32_t nib_lo16(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t nib_hi16(uint32_t w) { return w & 0xF0F0F0F0u; }

// Map the launch index to an output tile: contiguous ranges per XCD (blocks are
// dealt round-robin to the 8 XCDs), then 8-tile-row groups within a range.
__device__ __forceinline__ void tile_of(int bid, int nblocks, int tiles_m, int tiles_n, int* tm, int* tn) {
  const int n8 = nblocks & ~7;
  int lid = bid;
  if (bid < n8) lid = (bid & 7) * (n8 >> 3) + (bid >> 3);
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int grp = lid / per_group;
  const int first_m = grp * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int in = lid - grp * per_group;
  *tm = first_m + in % gm;
  *tn = in / gm;
}

}  // namespace

template <int CORE, int RB, bool BIAS>
__global__ void __launch_bounds__(NTHREADS, 2)
k_gemm2(const uint8_t* __restrict__ xq, const __half* __restrict__ xs, const __half* __restrict__ t,
        const uint8_t* __restrict__ wq, const __half* __restrict__ ws, const __half* __restrict__ l2,
        const __half* __restrict__ bias, const float* __restrict__ lam, int M, int N, int K,
        __half* __restrict__ y) {
  using C = CoreCfg<CORE>;
  constexpr int R = RB * 16;
  constexpr int KC = 2;                                  // groups per stage
  constexpr int TILE_BYTES = BM * C::LS;                 // one operand tile of one group in LDS
  constexpr int GROUP_BYTES = 2 * TILE_BYTES + 256 * 2;  // A, B, 128 + 128 fp16 scales
  constexpr int STAGE_BYTES = KC * GROUP_BYTES;
  // The MFMA partial of one group times PFACT is P_g (the operands are 16q).
  // Every rescaled partial carries the same factor, so it is applied once to the
  // accumulator (exact: a power of two) before the branch is added.
  constexpr float PFACT = 1.0f / 256.0f;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, r32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int G = K >> 6;
  const int NS = (G + KC - 1) / KC;                       // stages

  // ---- per-thread staging assignment (global -> registers -> LDS)
  // codes and scales are group-major ([K/64][rows][32], [K/64][rows]): a tile's rows of one
  // group are contiguous
  const uint8_t* src[C::CHUNKS];
  size_t gstep[C::CHUNKS];                                // bytes between consecutive groups
  int dst[C::CHUNKS];
  bool ok[C::CHUNKS];
#pragma unroll
  for (int i = 0; i < C::CHUNKS; i++) {
    const int c = tid + NTHREADS * i;                        // chunk id over both tiles
    const int per_tile = BM * C::CHUNKS;
    const int tile = c / per_tile, rr = c % per_tile;
    const int row = rr / C::CHUNKS, part = rr % C::CHUNKS;
    const int grow = (tile == 0 ? m0 : n0) + row;
    ok[i] = grow < (tile == 0 ? M : N);
    // rows past the edge re-read row 0 of the tile's operand and are never stored
    src[i] = (tile == 0 ? xq : wq) + (size_t)(ok[i] ? grow : 0) * C::GB + part * 16;
    gstep[i] = (size_t)(tile == 0 ? M : N) * C::GB;
    dst[i] = tile * TILE_BYTES + row * C::LS + part * 16;
  }
  // scale staging: thread < 128 -> sx of row m0+tid, else sw of column n0+tid-128 (raw fp16)
  const bool s_is_x = tid < 128;
  const int s_row = (s_is_x ? m0 : n0) + (tid & 127);
  const bool s_ok = s_row < (s_is_x ? M : N);
  const unsigned short* s_base = reinterpret_cast<const unsigned short*>(s_is_x ? xs : ws);
  const unsigned short* s_ptr = s_base + (s_ok ? s_row : 0);
  const size_t s_step = (size_t)(s_is_x ? M : N);   // between consecutive groups

  uint4 stage_reg[KC][C::CHUNKS];
  unsigned short stage_s[KC];
  auto load_stage = [&](int st) {
#pragma unroll
    for (int k = 0; k < KC; k++) {
      const int g = min(st * KC + k, G - 1);   // a group past the end re-reads the last one (unused)
#pragma unroll
      for (int i = 0; i < C::CHUNKS; i++) stage_reg[k][i] = *reinterpret_cast<const uint4*>(src[i] + (size_t)g * gstep[i]);
      stage_s[k] = s_ptr[(size_t)g * s_step];
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int k = 0; k < KC; k++) {
      uint8_t* base = lds + buf * STAGE_BYTES + k * GROUP_BYTES;
#pragma unroll
      for (int i = 0; i < C::CHUNKS; i++) {
        uint4 v = ok[i] ? stage_reg[k][i] : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(base + dst[i]) = v;
      }
      reinterpret_cast<unsigned short*>(base + 2 * TILE_BYTES)[tid] = s_ok ? stage_s[k] : (unsigned short)0;
    }
  };

  v16f acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; a++)
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[a][b][i] = 0.f;

  load_stage(0);
  store_stage(0);
  if (NS > 1) load_stage(1);
  __syncthreads();

  const int arow0 = wm * 64 + r32;          // LDS row of this lane's A operand (tile 0)
  const int brow0 = wn * 64 + r32;
  const int a_off = arow0 * C::LS + h * 16;
  const int b_off = TILE_BYTES + brow0 * C::LS + h * 16;
  const int sx_off = 2 * TILE_BYTES + 2 * arow0;
  const int sw_off = 2 * TILE_BYTES + 2 * (128 + brow0);
  for (int st = 0; st < NS; st++) {
    const int buf = st & 1;
#pragma unroll
    for (int k = 0; k < KC; k++) {
      if (st * KC + k >= G) break;
      const uint8_t* base = lds + buf * STAGE_BYTES + k * GROUP_BYTES;
      // scale operands for the outer product S = sx sw^T on v_mfma_f32_32x32x16_f16: the
      // scale sits in K-slot 0 (element 0 of the lanes of the first half), every other slot
      // is zero, so the MFMA returns sx[m] * sw[n] exactly (fp16 x fp16 in fp32) in the
      // accumulator layout of the partials.
      v8h sa[2], sb[2];
#pragma unroll
      for (int i = 0; i < 2; i++) {
        const unsigned short xa = *reinterpret_cast<const unsigned short*>(base + sx_off + 64 * i);
        const unsigned short xb = *reinterpret_cast<const unsigned short*>(base + sw_off + 64 * i);
        sa[i] = as_h8(make_uint4(h ? 0u : (uint32_t)xa, 0u, 0u, 0u));
        sb[i] = as_h8(make_uint4(h ? 0u : (uint32_t)xb, 0u, 0u, 0u));
      }
      v4i a[2][2], b[2][2];
#pragma unroll
      for (int i = 0; i < 2; i++) {
        const uint4 ua = *reinterpret_cast<const uint4*>(base + a_off + i * 32 * C::LS);
        const uint4 ub = *reinterpret_cast<const uint4*>(base + b_off + i * 32 * C::LS);
        a[i][0] = v4i{(int)nib_lo16(ua.x), (int)nib_hi16(ua.x), (int)nib_lo16(ua.y), (int)nib_hi16(ua.y)};
        a[i][1] = v4i{(int)nib_lo16(ua.z), (int)nib_hi16(ua.z), (int)nib_lo16(ua.w), (int)nib_hi16(ua.w)};
        b[i][0] = v4i{(int)nib_lo16(ub.x), (int)nib_hi16(ub.x), (int)nib_lo16(ub.y), (int)nib_hi16(ub.y)};
        b[i][1] = v4i{(int)nib_lo16(ub.z), (int)nib_hi16(ub.z), (int)nib_lo16(ub.w), (int)nib_hi16(ub.w)};
      }
#pragma unroll
      for (int ti = 0; ti < 2; ti++)
#pragma unroll
        for (int tj = 0; tj < 2; tj++) {
          v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[ti][0], b[tj][0], v16i{}, 0, 0, 0);
          p = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[ti][1], b[tj][1], p, 0, 0, 0);
          const v16f sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(sa[ti], sb[tj], v16f{}, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 16; i++) acc[ti][tj][i] = __builtin_fmaf((float)p[i], sc[i], acc[ti][tj][i]);
        }
    }
    // keep the next stage's LDS writes (and their wait on the global loads) after this compute
    __builtin_amdgcn_sched_barrier(0);
    if (st + 1 < NS) {
      store_stage(buf ^ 1);
      if (st + 2 < NS) load_stage(st + 2);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 2; a++)
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[a][b][i] *= PFACT;

  // ---- epilogue: up projection T L2 on the matrix core, bias, fp16 store
  int arow[2], bcol[2];
  bool aok[2], bok[2];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    arow[i] = m0 + arow0 + i * 32; aok[i] = arow[i] < M;
    bcol[i] = n0 + brow0 + i * 32; bok[i] = bcol[i] < N;
  }
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
    const float lv = lam ? lam[bcol[tj]] : 0.f;   // with the MLP glue folded in: the next layer's factor
#pragma unroll
    for (int ti = 0; ti < 2; ti++)
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int mrow = m0 + wm * 64 + ti * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        uint32_t hv = __half_as_ushort(__float2half_rn(acc[ti][tj][i] + bv));
        if (lam) hv = gelu_div_h(hv, lv);        // fp16(gelu(y) / lam)
        if (mrow < M) y[(size_t)mrow * N + bcol[tj]] = __ushort_as_half((unsigned short)hv);
      }
  }
}

// Few token rows (the weight-streaming regime, M <= 256): one workgroup per 32 output columns
// and a slab of up to 128 rows (MT tiles of 32; blockIdx.y picks the slab), so each weight row
// is read once per slab, in its packed layout (half the bytes of the 6-bit container).  The
// four waves split K (groups w, w + 4, ...), each holding PD groups of loads in flight straight
// into registers: lane (r32, h) loads the 16 bytes of codes 32 h .. 32 h + 31 of its weight row
// and of each of its token rows, which, unpacked to 16 q with two masks and a shift, are its
// operands of the two v_mfma_i32_32x32x32_i8 of a group (the same K order on both sides).  The
// int32 result is 256 P_g exactly; the scale-product MFMA gives S = sw sx, one fma per element
// and group adds 256 P_g S, and the accumulator is scaled by 1/256 once (exact).  The waves'
// partial sums are added in LDS in wave order; wave 0 adds T L2 and the bias and stores.
template <int RB, bool BIAS, int MT>
__global__ void __launch_bounds__(NTHREADS, 2)
k_gemm2_skinny(const uint8_t* __restrict__ xq, const __half* __restrict__ xs, const __half* __restrict__ t,
               const uint8_t* __restrict__ wq, const __half* __restrict__ ws, const __half* __restrict__ l2,
               const __half* __restrict__ bias, const float* __restrict__ lam, int M, int N, int K,
               __half* __restrict__ y) {
  constexpr int R = RB * 16;
  constexpr int PD = MT <= 2 ? 4 : 2;       // groups in flight per wave
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
  // the epilogue's operands (L2 columns, bias, and T rows when MT <= 2), loaded by every wave
  // before the K loop so that their latency overlaps it (wave 0 uses them)
  constexpr int MTT = MT <= 2 ? MT : 1;
  uint32_t lv[RB > 0 ? RB : 1][8];
  uint4 tv[MTT][RB > 0 ? RB : 1];
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
  uint2 braw[4];
  float4 lam4[4];                            // with the MLP glue folded in: the next layer's factors
  const rsrc_t rl = make_rsrc(lam, lam ? (size_t)N * 4 : 0);
#pragma unroll
  for (int q = 0; q < 4; q++) {  // columns past N read the last four (their outputs are not stored)
    braw[q] = BIAS ? *reinterpret_cast<const uint2*>(bias + min(nb + 8 * q + 4 * h, N - 4)) : make_uint2(0u, 0u);
    lam4[q] = load_f4(rl, min(nb + 8 * q + 4 * h, N - 4));
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
      const bool zero = h || st < PD || st - PD >= ng;   // upper K half, or an empty slot
      const Op& cur = ring[j];
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
    __syncthreads();
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

// Up to this many token rows the weight-streaming kernel runs (in 128-row slabs).
constexpr int kSkinnyRows2 = 256;

template <int RB, bool BIAS, int MT>
static hipError_t launch_g2_skinny(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm2_skinny<RB, BIAS, MT>), dim3((a.N + 31) / 32, (a.M + 32 * MT - 1) / (32 * MT)),
                     dim3(NTHREADS), 0, s, (const uint8_t*)a.xq, (const __half*)a.xs, (const __half*)a.t,
                     (const uint8_t*)a.wq, (const __half*)a.ws, (const __half*)a.l2, (const __half*)a.bias, a.lam,
                     a.M, a.N, a.K, (__half*)a.y);
  return hipGetLastError();
}

template <int CORE, int RB, bool BIAS>
static hipError_t launch_g2(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 32) return launch_g2_skinny<RB, BIAS, 1>(a, s);
  if (a.M <= 64) return launch_g2_skinny<RB, BIAS, 2>(a, s);
  if (a.M <= kSkinnyRows2) return launch_g2_skinny<RB, BIAS, 4>(a, s);
  const int nb = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((k_gemm2<CORE, RB, BIAS>), dim3(nb), dim3(NTHREADS), 0, s, (const uint8_t*)a.xq,
                     (const __half*)a.xs, (const __half*)a.t, (const uint8_t*)a.wq, (const __half*)a.ws,
                     (const __half*)a.l2, (const __half*)a.bias, a.lam, a.M, a.N, a.K, (__half*)a.y);
  return hipGetLastError();
}

template <int CORE, bool BIAS>
static hipError_t launch_g2_r(const GemmArgs& a, hipStream_t s) {
  switch (a.r) {
    case 0: return launch_g2<CORE, 0, BIAS>(a, s);
    case 16: return launch_g2<CORE, 1, BIAS>(a, s);
    case 32: return launch_g2<CORE, 2, BIAS>(a, s);
    case 48: return launch_g2<CORE, 3, BIAS>(a, s);
    case 64: return launch_g2<CORE, 4, BIAS>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm2(const GemmArgs& a, hipStream_t s) {
  const bool b = a.bias != nullptr;
  if (a.fmt == FMT_INT4) return b ? launch_g2_r<CORE_I4, true>(a, s) : launch_g2_r<CORE_I4, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace svdq
