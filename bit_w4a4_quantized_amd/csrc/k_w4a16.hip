// W4A16 control: Y = fp16( X deq(W)^T + b ) with fp16 activations X [M, K] and
// SVDQ_INT4_G64 weights (packed nibbles, group-major [K/64][N][32 bytes]; fp16
// scales group-major [K/64][N]), no low-rank branch.  Practice page "sota-314", sections "Do this" and "What it
// buys": the W4A16 baseline the W4A4 layer is compared with, and the layers that
// stay W4A16.
//
// Arithmetic: each weight is dequantized once to fp16, w = fp16_rne(q s), as a
// weight-only kernel does before its 16-bit matrix multiply; products and sums
// are fp32 on v_mfma_f32_32x32x16_f16.  The codes become exact fp16 integers
// with the bit trick fp16(0x6400 | (u ^ 8)) - 1032 = q (u the nibble), then one
// packed fp16 multiply by the column's scale.
//
// Work decomposition (gfx950, wave64): workgroup tile 128 x 128, each of the four
// waves owning 32 output columns over all 128 rows (so each weight is dequantized
// once per tile), two workgroups per CU, persistent over tiles.  K advances
// one group of 64 at a time through two LDS buffers, filled straight from global
// memory by LDS-DMA buffer loads one group ahead.  The MFMA K order is permuted
// the same way for both operands: at k-step ks the upper-half lanes carry
// columns 32 + 8 ks .. +7 and the lower-half lanes 8 ks .. +7, so a lane's
// weight nibbles for the whole group are one 16-byte chunk.  LDS slots are
// XOR-swizzled against bank conflicts.  Each lane's accumulators belong to one
// output row; the epilogue adds the bias, rounds to fp16 and writes 16-byte row
// pieces through LDS.
#include "kernels.h"

namespace svdq {

namespace {

constexpr int BM = 128, BN = 128, NT = 256;
constexpr int L_X = 0;                      // X: [128 rows][8 slots of 16 bytes]
constexpr int L_W = 16384;                  // W: [128 rows][2 slots of 16 bytes]
constexpr int L_S = 20480;                  // scales: one dword (fp16, zero-extended) per row
constexpr int GROUP = L_S + 512;            // 20992
constexpr int RING = 2 * GROUP;
constexpr int E_Y = GROUP;                  // epilogue: buffer 1, per wave 32 rows x 80 bytes
constexpr int E_YS = 80;
static_assert(E_Y + 4 * 32 * E_YS <= RING, "output staging must fit buffer 1");

// LDS-DMA loads: lane l's 16 bytes go to dst + 16 l, its 2 bytes zero-extended to dst + 4 l
__device__ __forceinline__ void dma16(rsrc_t r, uint8_t* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, (int)voff, (int)soff, 0, 0);
}
__device__ __forceinline__ void dma2(rsrc_t r, uint8_t* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 2, (int)voff, (int)soff, 0, 0);
}

__device__ __forceinline__ int xslot(int row, int b) { return row * 128 + 16 * (b ^ (row & 7)); }
__device__ __forceinline__ int wslot(int row, int c) { return row * 32 + 16 * (c ^ ((row >> 3) & 1)); }

// Tile index -> output tile: contiguous ranges per XCD, 8-tile-row groups within a range.
__device__ __forceinline__ void tile_of_w(int bid, int nblocks, int tiles_m, int tiles_n, int* tm, int* tn) {
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

// Eight nibbles (codes j = 0..7, two per byte, low first) times the fp16 scale pair s2:
// four packed fp16 pairs (code 2i, code 2i+1).
__device__ __forceinline__ uint4 dequant8(uint32_t w, uint32_t s2) {
  const uint32_t lo = w & 0x0F0F0F0Fu;          // codes 0, 2, 4, 6 (one per byte)
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // codes 1, 3, 5, 7
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    // bytes: lo.b_i -> low half, hi.b_i -> high half, upper bytes zero
    const uint32_t sel = 0x0C000C00u | (uint32_t)i | ((uint32_t)(4 + i) << 16);
    const uint32_t u = __builtin_amdgcn_perm(hi, lo, sel) ^ 0x64086408u;   // fp16 1024 + (u ^ 8)
    __half2 hv;
    __builtin_memcpy(&hv, &u, 4);
    hv = __hsub2(hv, __half2half2(__ushort_as_half((unsigned short)0x6408u)));   // - 1032: exact q
    __half2 sv;
    __builtin_memcpy(&sv, &s2, 4);
    hv = __hmul2(hv, sv);                                                          // fp16(q s)
    __builtin_memcpy(&r[i], &hv, 4);
  }
  return make_uint4(r[0], r[1], r[2], r[3]);
}

}  // namespace

template <bool BIAS>
__global__ void __launch_bounds__(NT, 2)
k_w4a16(const __half* __restrict__ x, const uint8_t* __restrict__ wq, const __half* __restrict__ ws,
        const __half* __restrict__ bias, int M, int N, int K, __half* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[RING];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, r32 = lane & 31;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int tiles = tiles_m * tiles_n;
  const int G = K >> 6;
  const int GE = (G + 1) & ~1;               // group g goes through LDS buffer g % 2

  // ---- loads.  X: each wave 4 instructions of 8 rows x 128 bytes (lane -> row lane/8 of the 8,
  // slot lane%8 -> 16-byte block (lane%8) ^ (row%8)).  W: one instruction per wave, rows
  // 32 w + lane/2, slot lane%2.  Scales: waves 0, 1, rows 64 w + lane.
  const rsrc_t rxb = make_rsrc(x, (size_t)M * K * 2);
  const rsrc_t rwb = make_rsrc(wq, (size_t)N * K / 2);
  const rsrc_t rsb = make_rsrc(ws, (size_t)N * G * 2);
  const int xr = lane >> 3, xb = (lane & 7);
  const int wr = wave * 32 + (lane >> 1), wc = (lane & 1) ^ ((wr >> 3) & 1);
  const int sr = (wave & 1) * 64 + lane;
  struct Src {
    uint32_t vx[4], vw, vs;
  };
  auto tile_src = [&](int tile) {
    int tm_, tn_;
    tile_of_w(tile, tiles, tiles_m, tiles_n, &tm_, &tn_);
    const int m0_ = tm_ * BM, n0_ = tn_ * BN;
    Src r;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int row = wave * 32 + i * 8 + xr;
      const int m = min(m0_ + row, M - 1);
      r.vx[i] = (uint32_t)m * K * 2 + 16u * (uint32_t)(xb ^ (row & 7));
    }
    r.vw = (uint32_t)min(n0_ + wr, N - 1) * 32u + 16u * wc;   // codes [K/64][N][32]
    r.vs = (uint32_t)min(n0_ + sr, N - 1) * 2u;                // scales [K/64][N]
    return r;
  };
  auto load_group = [&](const Src& src, int g, int buf) {
    g = min(g, G - 1);                       // a group past the end re-reads the last one (unused)
    uint8_t* b = lds + buf * GROUP;
#pragma unroll
    for (int i = 0; i < 4; i++) dma16(rxb, b + L_X + (wave * 32 + i * 8) * 128, src.vx[i], (uint32_t)g * 128);
    dma16(rwb, b + L_W + wave * 1024, src.vw, (uint32_t)g * (uint32_t)N * 32u);
    if (wave < 2) dma2(rsb, b + L_S + wave * 256, src.vs, (uint32_t)g * (uint32_t)N * 2u);
  };
  auto wait_loads = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // per-lane LDS read offsets: X rows i*32 + r32 (row tile i; the swizzle depends on the row
  // only through r32 % 8, so row tile i is +4096 bytes), this wave's 32 weight rows
  int xo[4];
#pragma unroll
  for (int ks = 0; ks < 4; ks++) xo[ks] = L_X + xslot(r32, 4 * h + ks);
  const int wo = L_W + wslot(wave * 32 + r32, h);
  const int so = L_S + (wave * 32 + r32) * 4;
  v16f acc[4];                               // [row tile i]: lane -> row i*32 + r32, this wave's 32 columns

  int tile = blockIdx.x;
  Src cur = tile_src(tile);
  load_group(cur, 0, 0);
  while (true) {
    const int next = tile + (int)gridDim.x;
    const bool has_next = next < tiles;
    const Src nxt = tile_src(has_next ? next : tile);
    int tm, tn;
    tile_of_w(tile, tiles, tiles_m, tiles_n, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;
    wait_loads();
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[a][i] = 0.f;

    auto step = [&](int g, int buf) {
      uint4 wd[4];
      uint4 xv[4][4];
      if (g < G) {
        const uint8_t* b = lds + buf * GROUP;
        const uint4 w = *reinterpret_cast<const uint4*>(b + wo);
        const uint32_t sc = *reinterpret_cast<const uint32_t*>(b + so);
        const uint32_t s2 = sc | (sc << 16);
        wd[0] = dequant8(w.x, s2);
        wd[1] = dequant8(w.y, s2);
        wd[2] = dequant8(w.z, s2);
        wd[3] = dequant8(w.w, s2);
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
          for (int ks = 0; ks < 4; ks++) xv[i][ks] = *reinterpret_cast<const uint4*>(b + xo[ks] + i * 4096);
      }
      __builtin_amdgcn_sched_barrier(0);
      const bool nx = g + 1 >= G;
      if (!nx) load_group(cur, g + 1, buf ^ 1);
      else if (g + 1 == GE && has_next) load_group(nxt, 0, buf ^ 1);
      __builtin_amdgcn_sched_barrier(0);
      if (g < G) {
#pragma unroll
        for (int ks = 0; ks < 4; ks++)
#pragma unroll
          for (int i = 0; i < 4; i++)
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(wd[ks]), as_h8(xv[i][ks]), acc[i], 0, 0, 0);
      }
      if (g + 1 < GE) wait_loads();
      __syncthreads();
    };
    for (int g = 0; g < GE; g += 2) {
      step(g, 0);
      step(g + 1, 1);
    }

    // ---- epilogue in buffer 1: bias, fp16, 16-byte row stores through LDS (per wave 32 rows of
    // its 32 columns at a time)
    uint8_t* ys = lds + E_Y + wave * 32 * E_YS;
    float bv[4][4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
#pragma unroll
      for (int j = 0; j < 4; j++) bv[q][j] = 0.f;
      if (BIAS) {
        const int n = n0 + wave * 32 + 8 * q + 4 * h;
        if (n < N) {
          const uint2 braw = *reinterpret_cast<const uint2*>(bias + n);
          bv[q][0] = __half2float(__ushort_as_half((unsigned short)(braw.x & 0xFFFFu)));
          bv[q][1] = __half2float(__ushort_as_half((unsigned short)(braw.x >> 16)));
          bv[q][2] = __half2float(__ushort_as_half((unsigned short)(braw.y & 0xFFFFu)));
          bv[q][3] = __half2float(__ushort_as_half((unsigned short)(braw.y >> 16)));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int nl = 8 * q + 4 * h;        // column within the wave's 32
        uint32_t hv[4];
#pragma unroll
        for (int j = 0; j < 4; j++) hv[j] = __half_as_ushort(__float2half_rn(acc[i][4 * q + j] + bv[q][j]));
        *reinterpret_cast<uint2*>(ys + r32 * E_YS + nl * 2) = make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int it = 0; it < 2; it++) {
        const int rl = it * 16 + (lane >> 2), c = (lane & 3) * 8;   // row within the 32, column
        const uint2 a = *reinterpret_cast<const uint2*>(ys + rl * E_YS + c * 2);
        const uint2 b = *reinterpret_cast<const uint2*>(ys + rl * E_YS + c * 2 + 8);
        const int m = m0 + i * 32 + rl, n = n0 + wave * 32 + c;
        if (m < M && n < N) *reinterpret_cast<uint4*>(y + (size_t)m * N + n) = make_uint4(a.x, a.y, b.x, b.y);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    __syncthreads();                         // buffer 1 is rewritten by the next tile's group 1
    if (!has_next) break;
    tile = next;
    cur = nxt;
  }
}


hipError_t launch_w4a16(const void* x, const void* wq, const void* ws, const void* bias, int M, int N,
                        int K, void* y, hipStream_t s) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int nb = tiles < resident_workgroups() ? tiles : resident_workgroups();
  if (bias)
    hipLaunchKernelGGL(k_w4a16<true>, dim3(nb), dim3(NT), 0, s, (const __half*)x, (const uint8_t*)wq,
                       (const __half*)ws, (const __half*)bias, M, N, K, (__half*)y);
  else
    hipLaunchKernelGGL(k_w4a16<false>, dim3(nb), dim3(NT), 0, s, (const __half*)x, (const uint8_t*)wq,
                       (const __half*)ws, (const __half*)nullptr, M, N, K, (__half*)y);
  return hipGetLastError();
}

}  // namespace svdq
