// Persistent LDS-DMA GEMM skeleton for gfx950, shared by the INT8 and FP4
// Kernel B variants: workgroup tile 128 x 128, four waves in 2 x 2 of 64 x 64
// (2 x 2 MFMA tiles of 32 x 32 each), two workgroups per CU, each looping over
// tiles.  K advances in stages through two LDS buffers that are filled straight
// from global memory by LDS-DMA buffer loads one stage ahead: a step reads its
// stage's operands into registers, issues the next stage's loads (the next
// tile's first stage after a tile's last step, so those loads overlap the
// epilogue), computes, waits for its loads and synchronises.
//
// The accumulators acc[tj][ti] hold the tile product with the weight tile as
// the MFMA row operand and the activation tile as the column operand: lane
// (r32, h) owns output row m = ti*32 + r32 and columns 8(v/4) + 4h + v%4 of
// tile tj.  The epilogue adds the low-rank up projection T L2 (fp16 matrix
// cores, L2 staged transposed through LDS) and the bias, rounds to fp16 and
// writes 16-byte row pieces through LDS ("sota-314", "Do this": the up
// projection shares the 4-bit kernel's output).
//
// A format supplies an operator type Op with
//   static constexpr int BUF;                       LDS bytes of one stage buffer
//   int NS;                                         stages per tile
//   struct Src; Src src(int m0, int n0);            per-lane global offsets of a tile
//   void load(const Src&, int st, uint8_t* buf);    the stage's LDS-DMA loads
//   struct Regs; void read(const uint8_t* buf, int st, Regs&);
//   void mma(const Regs&, int st, v16f (&acc)[2][2]);
//   void finish(v16f (&acc)[2][2]);                 once per tile, before the epilogue
// and, for an operator whose kernel runs the last partial round as 32 x 32 sub-tile jobs
// (operands straight into registers; used by FP4 and MXFP4):
//   int NU; static constexpr int SUB_PD;            64-column units of K; register ring depth
//   struct UR; void gload(int u, int m, int n, UR&);  unit u of lane's X row m, W row n (every
//                                                   lane loads: no branch around a load)
//   void gmma(const UR&, bool zero, v16f& acc);     acc += the unit's products (zero: the
//                                                   unit adds exactly +0)
#pragma once
#include "kernels.h"

namespace svdq {
namespace skel {

constexpr int BM = 128, BN = 128, NT = 256;
constexpr int E_YS = 136;                   // output staging: per wave 32 rows x 136 bytes

__host__ __device__ constexpr int epi_bytes(int R) {
  return BN * (R + 8) * 2 > 4 * 32 * E_YS ? BN * (R + 8) * 2 : 4 * 32 * E_YS;
}

// One wave's LDS-DMA load: lane l's 16 (4) bytes go to dst + 16 l (dst + 4 l); 2 bytes or 1 byte
// are zero-extended to the dword at dst + 4 l.  dst must be wave-uniform.  Offsets go into the
// vector or scalar offset (the immediate would move the LDS destination as well).
__device__ __forceinline__ void dma16(rsrc_t r, uint8_t* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, (int)voff, (int)soff, 0, 0);
}
__device__ __forceinline__ void dma4(rsrc_t r, uint8_t* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 4, (int)voff, (int)soff, 0, 0);
}
__device__ __forceinline__ void dma2(rsrc_t r, uint8_t* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 2, (int)voff, (int)soff, 0, 0);
}
__device__ __forceinline__ void dma1(rsrc_t r, uint8_t* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 1, (int)voff, (int)soff, 0, 0);
}

// Tile index -> output tile: contiguous ranges per XCD (workgroups are dealt round-robin to
// the 8 XCDs and keep their XCD), then 8-tile-row groups within a range.
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

// The scale-product operand of v_mfma_f32_32x32x8_f16: the row's fp16 scale in K slot 0 for
// the lower half of the lanes, zeros elsewhere, so the MFMA returns sw[n] sx[m] exactly.
typedef _Float16 v4h_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4h_t scale_operand(uint32_t s, int h) {
  return __builtin_bit_cast(v4h_t, make_uint2(h ? 0u : (s & 0xFFFFu), 0u));
}

// acc += T L2 (RB > 0), bias, fp16 store.  eb: this workgroup's epilogue LDS (epi_bytes(R)),
// free of loads in flight.  Ends with a workgroup barrier.
template <int RB, bool BIAS>
__device__ __forceinline__ void epilogue(v16f (&acc)[2][2], uint8_t* eb, const __half* __restrict__ t,
                                         const __half* __restrict__ l2, const __half* __restrict__ bias,
                                         const float* __restrict__ lam, int M, int N, int m0, int n0,
                                         __half* __restrict__ y) {
  constexpr int R = RB * 16;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, r32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
  if (RB > 0) {
    // L2[:, n0:n0+128] transposed into LDS as [n][k] (row stride R + 8 halves); row operand
    // L2^T (columns n), column operand T (rows m, 8 consecutive k per lane)
    constexpr int LS2 = (R + 8) * 2;
    for (int idx = tid; idx < R * (BN / 8); idx += NT) {
      const int k = idx % R, c8 = idx / R;
      const int n = n0 + c8 * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (n < N) v = *reinterpret_cast<const uint4*>(l2 + (size_t)k * N + n);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; e++)
        *reinterpret_cast<uint16_t*>(eb + (c8 * 8 + e) * LS2 + k * 2) = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    }
    uint4 top[RB > 0 ? RB : 1][2];
#pragma unroll
    for (int kb = 0; kb < RB; kb++)
#pragma unroll
      for (int ti = 0; ti < 2; ti++) {
        const int m = min(m0 + wm * 64 + ti * 32 + r32, M - 1);
        top[kb][ti] = *reinterpret_cast<const uint4*>(t + (size_t)m * R + kb * 16 + 8 * h);
      }
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < RB; kb++)
#pragma unroll
      for (int tj = 0; tj < 2; tj++) {
        const uint4 lo = *reinterpret_cast<const uint4*>(eb + (wn * 64 + tj * 32 + r32) * LS2 + (kb * 16 + 8 * h) * 2);
#pragma unroll
        for (int ti = 0; ti < 2; ti++)
          acc[tj][ti] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(lo), as_h8(top[kb][ti]), acc[tj][ti], 0, 0, 0);
      }
    __syncthreads();                         // the output staging reuses the L2 staging bytes
  }
  float bv[2][4][4];
#pragma unroll
  for (int tj = 0; tj < 2; tj++)
#pragma unroll
    for (int q = 0; q < 4; q++) {
#pragma unroll
      for (int j = 0; j < 4; j++) bv[tj][q][j] = 0.f;
      if (BIAS) {
        const int n = n0 + wn * 64 + tj * 32 + 8 * q + 4 * h;
        if (n < N) {
          const uint2 braw = *reinterpret_cast<const uint2*>(bias + n);
          bv[tj][q][0] = __half2float(__ushort_as_half((unsigned short)(braw.x & 0xFFFFu)));
          bv[tj][q][1] = __half2float(__ushort_as_half((unsigned short)(braw.x >> 16)));
          bv[tj][q][2] = __half2float(__ushort_as_half((unsigned short)(braw.y & 0xFFFFu)));
          bv[tj][q][3] = __half2float(__ushort_as_half((unsigned short)(braw.y >> 16)));
        }
      }
    }
  // with the MLP glue folded in, the next layer's factors of the 8 columns this lane stores
  const rsrc_t rl = make_rsrc(lam, lam ? (size_t)N * 4 : 0);
  const float4 la = load_f4(rl, n0 + wn * 64 + (lane & 7) * 8), lb = load_f4(rl, n0 + wn * 64 + (lane & 7) * 8 + 4);
  uint8_t* ys = eb + wave * 32 * E_YS;
#pragma unroll
  for (int ti = 0; ti < 2; ti++) {
#pragma unroll
    for (int tj = 0; tj < 2; tj++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int nl = tj * 32 + 8 * q + 4 * h;    // column within the wave's 64
        uint32_t hv[4];
#pragma unroll
        for (int j = 0; j < 4; j++) hv[j] = __half_as_ushort(__float2half_rn(acc[tj][ti][4 * q + j] + bv[tj][q][j]));
        *reinterpret_cast<uint2*>(ys + r32 * E_YS + nl * 2) = make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int it = 0; it < 4; it++) {
      const int rl = it * 8 + (lane >> 3), c = (lane & 7) * 8;   // row within the 32, column
      uint2 a = *reinterpret_cast<const uint2*>(ys + rl * E_YS + c * 2);
      uint2 b = *reinterpret_cast<const uint2*>(ys + rl * E_YS + c * 2 + 8);
      if (lam) {                             // the MLP glue folded in: fp16(gelu(y) / lam)
        a.x = gelu_div_h(a.x & 0xFFFFu, la.x) | (gelu_div_h(a.x >> 16, la.y) << 16);
        a.y = gelu_div_h(a.y & 0xFFFFu, la.z) | (gelu_div_h(a.y >> 16, la.w) << 16);
        b.x = gelu_div_h(b.x & 0xFFFFu, lb.x) | (gelu_div_h(b.x >> 16, lb.y) << 16);
        b.y = gelu_div_h(b.y & 0xFFFFu, lb.z) | (gelu_div_h(b.y >> 16, lb.w) << 16);
      }
      const int m = m0 + wm * 64 + ti * 32 + rl, n = n0 + wn * 64 + c;
      if (m < M && n < N) *reinterpret_cast<uint4*>(y + (size_t)m * N + n) = make_uint4(a.x, a.y, b.x, b.y);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  __syncthreads();                           // the buffer is refilled by the next tile's loads
}

// The persistent loop: tiles blockIdx.x, blockIdx.x + gridDim.x, ... below tiles_run.
// lds: 2 Op::BUF bytes; the epilogue uses buffer 1 (buffer 0 already receives the next
// tile's stage 0).
template <class Op, int RB, bool BIAS>
__device__ __forceinline__ void persistent(Op& op, uint8_t* lds, const __half* __restrict__ t,
                                           const __half* __restrict__ l2, const __half* __restrict__ bias,
                                           const float* __restrict__ lam, int M, int N, int tiles_run,
                                           __half* __restrict__ y) {
  static_assert(Op::BUF >= epi_bytes(RB * 16), "the epilogue must fit one stage buffer");
  static_assert(Op::BUF % 16 == 0, "16-byte aligned buffers");
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int tiles = tiles_m * tiles_n;
  const int NS = op.NS;
  const int NSE = (NS + 1) & ~1;             // rounded up to even: stage s uses buffer s % 2
  auto origin = [&](int tile, int* m0, int* n0) {
    int tm, tn;
    tile_of(tile, tiles, tiles_m, tiles_n, &tm, &tn);
    *m0 = tm * BM;
    *n0 = tn * BN;
  };
  auto wait_loads = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  int tile = blockIdx.x;
  int m0, n0;
  origin(tile, &m0, &n0);
  typename Op::Src cur = op.src(m0, n0);
  op.load(cur, 0, lds);
  typename Op::Regs regs;
  v16f acc[2][2];
  while (true) {
    const int next = tile + (int)gridDim.x;
    const bool has_next = next < tiles_run;
    int m1, n1;
    origin(has_next ? next : tile, &m1, &n1);
    const typename Op::Src nxt = op.src(m1, n1);
    wait_loads();
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
      for (int b = 0; b < 2; b++)
#pragma unroll
        for (int i = 0; i < 16; i++) acc[a][b][i] = 0.f;

    auto step = [&](int st, int buf) {
      if (st < NS) op.read(lds + buf * Op::BUF, st, regs);
      __builtin_amdgcn_sched_barrier(0);
      if (st + 1 < NS) op.load(cur, st + 1, lds + (buf ^ 1) * Op::BUF);
      else if (st + 1 == NSE && has_next) op.load(nxt, 0, lds + (buf ^ 1) * Op::BUF);
      __builtin_amdgcn_sched_barrier(0);
      if (st < NS) op.mma(regs, st, acc);
      if (st + 1 < NSE) wait_loads();        // the last step's loads land during the epilogue
      __syncthreads();
    };
    for (int st = 0; st < NSE; st += 2) {
      step(st, 0);
      step(st + 1, 1);
    }
    op.finish(acc);
    epilogue<RB, BIAS>(acc, lds + Op::BUF, t, l2, bias, lam, M, N, m0, n0, y);
    if (!has_next) break;
    tile = next;
    m0 = m1;
    n0 = n1;
    cur = nxt;
  }
}

// One 32 x 32 sub-tile job of the last partial round (tiles past tiles_run, cut into 16 sub-tiles
// each): the four waves split K (units w, w + 4, ...) through a register ring of PD units and
// add their partial sums in LDS (red, 12 KB of the workgroup's LDS) in a fixed order, so the
// result is deterministic.  Step s of the ring processes slot s % PD, which holds the wave's
// unit s - PD (none for s < PD: zeroed slots, added as exactly +0), then refills it with unit s
// (past the last one it re-reads the last one): no prologue and no branch in the loop, so the
// compiler's wait counts let each slot wait for its own loads only.  The epilogue's operands
// are loaded before the K loop.  Ends with a workgroup barrier (red is reused).
template <class Op, int RB, bool BIAS>
__device__ __forceinline__ void subtile_job(const Op& op, float (*red)[16][64], const __half* __restrict__ t,
                                            const __half* __restrict__ l2, const __half* __restrict__ bias,
                                            const float* __restrict__ lam, int M, int N, int tile0, int job,
                                            __half* __restrict__ y) {
  constexpr int R = RB * 16;
  constexpr int PD = Op::SUB_PD;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, r32 = lane & 31;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_of(tile0 + (job >> 4), tiles_m * tiles_n, tiles_m, tiles_n, &tm, &tn);
  const int sub = job & 15;
  const int nb = tn * BN + (sub >> 2) * 32, mb = tm * BM + (sub & 3) * 32;   // sub-tile origin
  const int m = min(mb + r32, M - 1), n = min(nb + r32, N - 1);           // this lane's operand rows
  uint4 tv[RB > 0 ? RB : 1];
  uint32_t lv[RB > 0 ? RB : 1][8];
#pragma unroll
  for (int kb = 0; kb < RB; kb++) {
    tv[kb] = *reinterpret_cast<const uint4*>(t + (size_t)m * R + kb * 16 + 8 * h);
#pragma unroll
    for (int e = 0; e < 8; e++) lv[kb][e] = __half_as_ushort(l2[(size_t)(kb * 16 + 8 * h + e) * N + n]);
  }
  uint2 braw[4];
  float4 lam4[4];                            // with the MLP glue folded in: the next layer's factors
  const rsrc_t rl = make_rsrc(lam, lam ? (size_t)N * 4 : 0);
#pragma unroll
  for (int q = 0; q < 4; q++) {  // columns past N read the last four (their outputs are not stored)
    braw[q] = BIAS ? *reinterpret_cast<const uint2*>(bias + min(nb + 8 * q + 4 * h, N - 4)) : make_uint2(0u, 0u);
    lam4[q] = load_f4(rl, min(nb + 8 * q + 4 * h, N - 4));
  }
  v16f acc;
#pragma unroll
  for (int i = 0; i < 16; i++) acc[i] = 0.f;
  const int NU = op.NU;
  const int nu = wave < NU ? (NU - 1 - wave) / 4 + 1 : 0;   // this wave's units
  typename Op::UR ring[PD];
#pragma unroll
  for (int j = 0; j < PD; j++) ring[j] = typename Op::UR{};
  for (int s0 = 0; s0 < nu + PD; s0 += PD) {
    // the step number, hidden from loop analysis: "st < PD" holds on the first pass only, and
    // the compiler would peel that pass (its zeroed slots fold to constants) and issue its
    // loads as one block ordered by type, which merged wait counts then impose on every pass
    int s0o = s0;
    asm volatile("" : "+s"(s0o));
#pragma unroll
    for (int j = 0; j < PD; j++) {
      const int st = s0o + j;
      op.gmma(ring[j], st < PD || st - PD >= nu, acc);
      op.gload(nu > 0 ? wave + 4 * min(st, nu - 1) : 0, m, n, ring[j]);
      __builtin_amdgcn_sched_barrier(0);     // keep the slots in order: each waits for its own loads only
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < 16; i++) red[wave - 1][i][lane] = acc[i];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 16; i++) acc[i] = ((acc[i] + red[0][i][lane]) + red[1][i][lane]) + red[2][i][lane];
    // up projection: row operand L2^T (columns n), column operand T (rows m)
#pragma unroll
    for (int kb = 0; kb < RB; kb++) {
      const uint4 lw = make_uint4(lv[kb][0] | (lv[kb][1] << 16), lv[kb][2] | (lv[kb][3] << 16),
                                  lv[kb][4] | (lv[kb][5] << 16), lv[kb][6] | (lv[kb][7] << 16));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(lw), as_h8(tv[kb]), acc, 0, 0, 0);
    }
    // lane owns row mb + r32 and columns nb + 8 q + 4 h + j (reg 4 q + j)
    const int mo = mb + r32;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int no = nb + 8 * q + 4 * h;
      if (mo >= M || no >= N) continue;
      float bv[4] = {0.f, 0.f, 0.f, 0.f};
      if (BIAS) {
        bv[0] = __half2float(__ushort_as_half((unsigned short)(braw[q].x & 0xFFFFu)));
        bv[1] = __half2float(__ushort_as_half((unsigned short)(braw[q].x >> 16)));
        bv[2] = __half2float(__ushort_as_half((unsigned short)(braw[q].y & 0xFFFFu)));
        bv[3] = __half2float(__ushort_as_half((unsigned short)(braw[q].y >> 16)));
      }
      uint32_t hv[4];
#pragma unroll
      for (int j = 0; j < 4; j++) hv[j] = __half_as_ushort(__float2half_rn(acc[4 * q + j] + bv[j]));
      if (lam) {                             // the MLP glue folded in: fp16(gelu(y) / lam)
        const float lq[4] = {lam4[q].x, lam4[q].y, lam4[q].z, lam4[q].w};
#pragma unroll
        for (int j = 0; j < 4; j++) hv[j] = gelu_div_h(hv[j], lq[j]);
      }
      *reinterpret_cast<uint2*>(y + (size_t)mo * N + no) = make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
    }
  }
  __syncthreads();
}

// The tiles past tiles_run (a last partial round) as sub-tile jobs, taken by the workgroups as
// they finish their full tiles.  lds: the workgroup's LDS, free (no loads in flight).
template <class Op, int RB, bool BIAS>
__device__ __forceinline__ void subtile_jobs(const Op& op, uint8_t* lds, const __half* __restrict__ t,
                                             const __half* __restrict__ l2, const __half* __restrict__ bias,
                                             const float* __restrict__ lam, int M, int N, int tiles_run,
                                             __half* __restrict__ y) {
  static_assert(2 * Op::BUF >= 3 * 16 * 64 * 4, "the sub-tile partial sums must fit the LDS ring");
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int n_sub = (tiles - tiles_run) * 16;
  for (int job = blockIdx.x; job < n_sub; job += gridDim.x)
    subtile_job<Op, RB, BIAS>(op, reinterpret_cast<float (*)[16][64]>(lds), t, l2, bias, lam, M, N, tiles_run, job,
                              y);
}

// Full rounds of the persistent loop, then (when the remainder is at most a quarter of a
// round) the remaining tiles as sub-tile jobs in the same launch.  Returns the tiles the
// persistent loop takes; *nb gets the grid size.
inline int persistent_split(int M, int N, int* nb) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int slots = resident_workgroups();
  const int rem = tiles % slots;
  const int main_tiles = (tiles > slots && rem > 0 && 4 * rem <= slots) ? tiles - rem : tiles;
  *nb = main_tiles < slots ? main_tiles : slots;
  return main_tiles;
}

}  // namespace skel
}  // namespace svdq
