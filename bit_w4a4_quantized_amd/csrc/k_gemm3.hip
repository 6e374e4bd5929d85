// Kernel B for the 6-bit container format (SVDQ_INT4_G64_E2M3): low-bit GEMM on
// the FP6 matrix cores, per-group rescale into fp32, up projection and bias in
// the epilogue, fp16 store.
//
// Practice page "sota-314", section "Do this": the up projection is fused
// with the 4-bit compute because both write the same output.
//
//   Y[m,n] = fp16_rne( sum_g sx[m,g] sw[n,g] P_g[m,n] + (T L2)[m,n] + b[n] )
//   P_g    = sum_{k in group g} q_x[m,k] q_w[n,k]   (exact)
//
// Each INT4 code q is held as the E2M3 subnormal of q/8, so 32 codes of a row
// (one half of a group) are the six-dword operand of
// v_mfma_scale_f32_32x32x64_f8f6f4 in FP6 mode, and one MFMA per 32 x 32 tile
// and group returns P_g / 64 in fp32 exactly.  The scale products
// S = sw sx^T of a tile come from one v_mfma_f32_32x32x16_f16 whose operands
// carry the scales in K slot 0 and zeros elsewhere (exact), so the vector ALU
// spends one fma per output element and group: acc += P_g * S.
//
// The MFMAs take the weight tile as the row operand and the activation tile as
// the column operand, so each lane's accumulators belong to one output row
// (token m) and 4 runs of 4 consecutive columns: the epilogue's stores are
// 8-byte pieces, assembled through LDS into 16-byte row-contiguous stores.
//
// Work decomposition (gfx950, wave64): workgroup tile 128 x 128, four waves in
// 2 x 2 of 64 x 64 (2 x 2 MFMA tiles), two workgroups per CU.  K advances in
// stages of two groups.  Global -> LDS staging goes through registers: buffer
// loads whose per-group offset is a scalar, so the address arithmetic costs no
// vector instructions; while the waves compute stage s from LDS, stage s+1 is
// written to the other LDS buffer and the loads of stage s+2 are in flight.
// The grid is persistent (two workgroups per CU, each looping over tiles): the
// last step of a tile already loads the next tile's first stage, so the next
// tile's start overlaps this tile's epilogue and its stores.
// LDS keeps, per group and operand, bytes 0..15 of each (row, half) in one
// 16-byte slot and bytes 16..23 in one 8-byte slot (the slot order swizzled
// against bank conflicts), so every MFMA operand is
// one 16-byte and one 8-byte LDS read straight into its registers.  Scale
// slots are 8 bytes, [scale, 0, 0, 0] as fp16, read by the lanes of the lower K
// half; the upper-half lanes read a zero block that is written once.
// The block index is remapped so that each XCD (own L2) works on a contiguous
// range of tiles, rastered in groups of 8 tile rows.
#include "kernels.h"

namespace svdq {

namespace {

constexpr int BM = 128, BN = 128, NT = 256, KC = 2;
constexpr int GB = 48;                      // container bytes per (row, group)
// LDS layout of one group (byte offsets)
constexpr int L_XP0 = 0;                    // X: bytes 0..15 of each half, [128 rows][2 slots] x 16
constexpr int L_XP1 = 4096;                 // X: bytes 16..23 of each half, [128 rows][2 slots] x 8
constexpr int L_WP0 = 6144;                 // W: as X
constexpr int L_WP1 = 10240;
constexpr int L_S = 12288;                  // scale slots: [128 X rows + 128 W rows] x 8, then 256 zero bytes
constexpr int L_Z = L_S + 2048;
constexpr int GROUP = L_Z + 256;            // 14592
constexpr int STAGE = KC * GROUP;
constexpr int RING = 2 * STAGE;             // 58368 bytes
// epilogue reuse of the ring
constexpr int E_Y = 20480;                  // per-wave fp16 output staging, 64 rows x 136 bytes
constexpr int E_YS = 136;
static_assert(E_Y + 4 * 64 * E_YS <= RING, "epilogue staging must fit the ring");

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, size_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)n, 0x00020000);
}

// An opaque copy: LDS reads from distinct bases are not merged into paired reads whose
// halves would then have to be moved into the MFMA operand registers.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ uint4 ld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  v4i v = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

__device__ __forceinline__ uint2 ld8(rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef int v2i_t __attribute__((ext_vector_type(2)));
  v2i_t v = __builtin_bit_cast(v2i_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
  return make_uint2((uint32_t)v[0], (uint32_t)v[1]);
}

// LDS position of (row, half) in the 16-byte and 8-byte slot arrays: the two halves of a
// row are neighbours, swapped on a row-bit pattern so that both the writers (neighbouring
// lanes = the two halves of one row) and the readers (neighbouring lanes = consecutive
// rows, one half) touch distinct banks, with 32 or with 64 four-byte banks.
__device__ __forceinline__ int slot16(int row, int half) {
  return row * 32 + 16 * (half ^ (((row >> 2) ^ (row >> 3)) & 1));
}
__device__ __forceinline__ int slot8(int row, int half) {
  return row * 16 + 8 * (half ^ (((row >> 3) ^ (row >> 4)) & 1));
}

// Launch index -> output tile: contiguous ranges per XCD (blocks are dealt
// round-robin to the 8 XCDs), then 8-tile-row groups within a range.
__device__ __forceinline__ void tile_of3(int bid, int nblocks, int tiles_m, int tiles_n, int* tm, int* tn) {
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

template <int RB, bool BIAS>
__global__ void __launch_bounds__(NT, 2)
k_gemm3(const uint8_t* __restrict__ xq, const __half* __restrict__ xs, const __half* __restrict__ t,
        const uint8_t* __restrict__ wq, const __half* __restrict__ ws, const __half* __restrict__ l2,
        const __half* __restrict__ bias, int M, int N, int K, __half* __restrict__ y) {
  constexpr int R = RB * 16;
  __shared__ __attribute__((aligned(16))) uint8_t lds[RING];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, r32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int tiles = tiles_m * tiles_n;
  const int G = K >> 6;
  const int NS = (G + KC - 1) / KC;          // stages of a tile
  const int NSE = (NS + 1) & ~1;             // rounded up to even (the loop takes two per pass)
  const uint32_t gx_step = (uint32_t)M * GB, gw_step = (uint32_t)N * GB;   // bytes between groups

  // ---- staging assignment: thread -> (row tid/2, half tid%2) of both code tiles (a row's
  // 48 bytes come from two neighbouring lanes); rows past the edge re-read the tile's last
  // valid row (their outputs are never stored).  Scales (group-major [G, rows]): waves 0-1
  // stage sx of rows m0 + tid, waves 2-3 sw of columns n0 + tid - 128.
  const int srow = tid >> 1, shalf = tid & 1;
  const bool s_x = wave < 2;
  const int s_stride = s_x ? M : N;
  struct Src {                               // where one tile's operands are read from
    rsrc_t rx, rw, rs;
    uint32_t vx, vw, vs;
  };
  auto tile_src = [&](int tile) {
    int tm_, tn_;
    tile_of3(tile, tiles, tiles_m, tiles_n, &tm_, &tn_);
    const int m0_ = tm_ * BM, n0_ = tn_ * BN;
    const int mr = min(BM, M - m0_), nr = min(BN, N - n0_);
    const int sr = s_x ? mr : nr;
    Src r;
    // codes are group-major [G][rows][48]: a tile's rows of one group are contiguous
    r.rx = make_rsrc(xq + (size_t)m0_ * GB, ((size_t)(G - 1) * M + mr) * GB);
    r.rw = make_rsrc(wq + (size_t)n0_ * GB, ((size_t)(G - 1) * N + nr) * GB);
    r.rs = make_rsrc(s_x ? (const void*)(xs + m0_) : (const void*)(ws + n0_), ((size_t)(G - 1) * s_stride + sr) * 2);
    r.vx = (uint32_t)min(srow, mr - 1) * GB + 24u * shalf;
    r.vw = (uint32_t)min(srow, nr - 1) * GB + 24u * shalf;
    r.vs = (uint32_t)min(tid & 127, sr - 1) * 2;
    return r;
  };

  // one register slot of staged global data; stage s of a tile goes through LDS buffer s % 2
  uint4 xlo[KC], wlo[KC];
  uint2 xhi[KC], whi[KC];
  uint32_t sv[KC];
  auto load_stage = [&](const Src& src, int st) {
#pragma unroll
    for (int k = 0; k < KC; k++) {
      const int g = min(st * KC + k, G - 1);   // a group past the end re-reads the last one (unused)
      const uint32_t sox = (uint32_t)g * gx_step, sow = (uint32_t)g * gw_step;
      xlo[k] = ld16(src.rx, src.vx, sox);
      xhi[k] = ld8(src.rx, src.vx + 16, sox);
      wlo[k] = ld16(src.rw, src.vw, sow);
      whi[k] = ld8(src.rw, src.vw + 16, sow);
      sv[k] = __builtin_amdgcn_raw_buffer_load_b16(src.rs, (int)src.vs, (int)((uint32_t)g * s_stride * 2), 0);
    }
  };
  const int w_p0 = slot16(srow, shalf), w_p1 = slot8(srow, shalf);
  const int w_s = tid * 8;    // slot of X row tid (waves 0-1) or W row tid - 128 (waves 2-3)
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int k = 0; k < KC; k++) {
      uint8_t* b = lds + buf * STAGE + k * GROUP;
      *reinterpret_cast<uint4*>(b + L_XP0 + w_p0) = xlo[k];
      *reinterpret_cast<uint2*>(b + L_XP1 + w_p1) = xhi[k];
      *reinterpret_cast<uint4*>(b + L_WP0 + w_p0) = wlo[k];
      *reinterpret_cast<uint2*>(b + L_WP1 + w_p1) = whi[k];
      *reinterpret_cast<uint2*>(b + L_S + w_s) = make_uint2(sv[k], 0u);   // K slots 0..3: s, 0, 0, 0
    }
  };


  // per-lane LDS read bases (tile offsets and stage offsets are immediates)
  int rx_p0[2], rx_p1[2], rw_p0[2], rw_p1[2], rs_x[2], rs_w[2];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    rx_p0[i] = slot16(wm * 64 + i * 32 + r32, h);
    rw_p0[i] = slot16(wn * 64 + i * 32 + r32, h);
    rx_p1[i] = opaque(slot8(wm * 64 + i * 32 + r32, h));
    rw_p1[i] = opaque(slot8(wn * 64 + i * 32 + r32, h));
    rs_x[i] = opaque(h ? L_Z - L_S + r32 * 8 : (wm * 64 + i * 32 + r32) * 8);
    rs_w[i] = opaque(h ? L_Z - L_S + r32 * 8 : (128 + wn * 64 + i * 32 + r32) * 8);
  }
  // MFMA operands of one group.  Scale operands: only the first two dwords are reloaded,
  // the rest stays zero; code operands: dwords 6 and 7 are not read by the FP6 MFMA.
  struct Ops {
    v8i xo[2], wo[2];
    uint4 sxo[2], swo[2];
  };
  Ops ops;
#pragma unroll
  for (int i = 0; i < 2; i++) {
#pragma unroll
    for (int e = 0; e < 8; e++) { ops.xo[i][e] = 0; ops.wo[i][e] = 0; }
    ops.sxo[i] = make_uint4(0, 0, 0, 0);
    ops.swo[i] = make_uint4(0, 0, 0, 0);
  }
  v16f acc[2][2];   // [tj][ti]: lane -> row m = ti*32 + r32, reg v -> column 8(v/4) + 4h + v%4 of tile tj

  auto read_ops = [&](const uint8_t* b, Ops& o) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const uint4 x0 = *reinterpret_cast<const uint4*>(b + L_XP0 + rx_p0[i]);
      const uint2 x1 = *reinterpret_cast<const uint2*>(b + L_XP1 + rx_p1[i]);
      const uint4 w0 = *reinterpret_cast<const uint4*>(b + L_WP0 + rw_p0[i]);
      const uint2 w1 = *reinterpret_cast<const uint2*>(b + L_WP1 + rw_p1[i]);
      o.xo[i][0] = (int)x0.x; o.xo[i][1] = (int)x0.y; o.xo[i][2] = (int)x0.z; o.xo[i][3] = (int)x0.w;
      o.xo[i][4] = (int)x1.x; o.xo[i][5] = (int)x1.y;
      o.wo[i][0] = (int)w0.x; o.wo[i][1] = (int)w0.y; o.wo[i][2] = (int)w0.z; o.wo[i][3] = (int)w0.w;
      o.wo[i][4] = (int)w1.x; o.wo[i][5] = (int)w1.y;
      const uint2 sxv = *reinterpret_cast<const uint2*>(b + L_S + rs_x[i]);
      const uint2 swv = *reinterpret_cast<const uint2*>(b + L_S + rs_w[i]);
      o.sxo[i].x = sxv.x; o.sxo[i].y = sxv.y;
      o.swo[i].x = swv.x; o.swo[i].y = swv.y;
    }
  };
  auto mma_ops = [&](const Ops& o) {
#pragma unroll
    for (int tj = 0; tj < 2; tj++)
#pragma unroll
      for (int ti = 0; ti < 2; ti++) {
        const v16f p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(o.wo[tj], o.xo[ti], v16f{}, 2, 2, 0, 127, 0, 127);
        const v16f sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(o.swo[tj]), as_h8(o.sxo[ti]), v16f{}, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 16; i++) acc[tj][ti][i] = __builtin_fmaf(p[i], sc[i], acc[tj][ti][i]);
      }
  };

  // ---- persistent loop over tiles: tile, tile + gridDim.x, ...  The stages of a tile run
  // through the register slot and two LDS buffers; during its last step the loads already
  // fetch the next tile's stage 0, so that the next tile's start overlaps this tile's
  // epilogue.  The global loads inside the stage loop are unconditional (a stage
  // past the end re-reads the last group): loads under a branch would make the wait-count
  // analysis wait for every load; the scheduling barriers keep each stage's loads together
  // for the same reason.
  int tile = blockIdx.x;
  Src ld = tile_src(tile);                   // the tile whose stages are being fetched
  load_stage(ld, 0);
  __builtin_amdgcn_sched_barrier(0);
  while (true) {
    const int next = tile + (int)gridDim.x;
    const bool has_next = next < tiles;
    const Src nxt = tile_src(has_next ? next : tile);
    int tm, tn;
    tile_of3(tile, tiles, tiles_m, tiles_n, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // the zero bytes read by the upper-K-half lanes (the previous epilogue used the ring)
    if (tid < 32) {
#pragma unroll
      for (int b = 0; b < 2 * KC; b++) *reinterpret_cast<uint2*>(lds + b * GROUP + L_Z + tid * 8) = make_uint2(0u, 0u);
    }
    // stage 0 -> LDS buffer 0, stage 1 in flight
    store_stage(0);
    __builtin_amdgcn_sched_barrier(0);
    load_stage(ld, 1);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();

#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
      for (int b = 0; b < 2; b++)
#pragma unroll
        for (int i = 0; i < 16; i++) acc[a][b][i] = 0.f;

    int lbase = 0;                           // stage index of ld = step + 2 - lbase
    auto step = [&](int st, int buf, bool do_load) {
      if (st < NS) {
#pragma unroll
        for (int k = 0; k < KC; k++)
          if (st * KC + k < G) {
            read_ops(lds + buf * STAGE + k * GROUP, ops);
            mma_ops(ops);
          }
      }
      // keep the next stage's LDS writes (and their wait on the global loads) after this compute
      __builtin_amdgcn_sched_barrier(0);
      if (st + 1 < NS) store_stage(buf ^ 1);
      if (do_load) {
        if (st + 2 == NSE && has_next) {
          ld = nxt;
          lbase = NSE;
        }
        load_stage(ld, st + 2 - lbase);
      }
      __syncthreads();
    };
    for (int st = 0; st + 2 < NSE; st += 2) {
      step(st, 0, true);
      step(st + 1, 1, true);
    }
    step(NSE - 2, 0, true);
    step(NSE - 1, 1, false);

    // ---- epilogue.  The ring is free (every wave passed the last barrier).
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
      for (int b = 0; b < 2; b++)
#pragma unroll
        for (int i = 0; i < 16; i++) acc[a][b][i] *= 64.0f;   // P_g / 64 -> P_g (exact)

    if (RB > 0) {
      // L2[:, n0:n0+128] transposed into LDS as [n][k] (row stride (R+8) halves), then
      // acc += L2^T T^T on v_mfma_f32_32x32x16_f16: row operand L2^T (columns n), column
      // operand T (rows m, 8 consecutive k per lane: one 16-byte load)
      constexpr int LS2 = (R + 8) * 2;
      static_assert(BN * LS2 <= E_Y, "L2 staging overlaps the output staging");
      for (int idx = tid; idx < R * (BN / 8); idx += NT) {
        const int k = idx % R, c8 = idx / R;   // neighbouring lanes write neighbouring k
        const int n = n0 + c8 * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (n < N) v = *reinterpret_cast<const uint4*>(l2 + (size_t)k * N + n);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; e++)
          *reinterpret_cast<uint16_t*>(lds + (c8 * 8 + e) * LS2 + k * 2) = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
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
          const uint4 lo = *reinterpret_cast<const uint4*>(lds + (wn * 64 + tj * 32 + r32) * LS2 + (kb * 16 + 8 * h) * 2);
#pragma unroll
          for (int ti = 0; ti < 2; ti++)
            acc[tj][ti] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(lo), as_h8(top[kb][ti]), acc[tj][ti], 0, 0, 0);
        }
    }

    // bias, RNE to fp16, 8-byte pieces into this wave's LDS staging, 16-byte row stores
    uint8_t* ys = lds + E_Y + wave * 64 * E_YS;
#pragma unroll
    for (int tj = 0; tj < 2; tj++) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int nl = tj * 32 + 8 * q + 4 * h;    // column within the wave's 64
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if (BIAS) {
          const int n = n0 + wn * 64 + nl;
          if (n < N) {
            const uint2 braw = *reinterpret_cast<const uint2*>(bias + n);
            bv[0] = __half2float(__ushort_as_half((unsigned short)(braw.x & 0xFFFFu)));
            bv[1] = __half2float(__ushort_as_half((unsigned short)(braw.x >> 16)));
            bv[2] = __half2float(__ushort_as_half((unsigned short)(braw.y & 0xFFFFu)));
            bv[3] = __half2float(__ushort_as_half((unsigned short)(braw.y >> 16)));
          }
        }
#pragma unroll
        for (int ti = 0; ti < 2; ti++) {
          uint32_t hv[4];
#pragma unroll
          for (int j = 0; j < 4; j++)
            hv[j] = __half_as_ushort(__float2half_rn(acc[tj][ti][4 * q + j] + bv[j]));
          *reinterpret_cast<uint2*>(ys + (ti * 32 + r32) * E_YS + nl * 2) =
              make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int it = 0; it < 8; it++) {
      const int rl = it * 8 + (lane >> 3), c = (lane & 7) * 8;   // row within the wave's 64, column
      const uint2 a = *reinterpret_cast<const uint2*>(ys + rl * E_YS + c * 2);
      const uint2 b = *reinterpret_cast<const uint2*>(ys + rl * E_YS + c * 2 + 8);
      const int m = m0 + wm * 64 + rl, n = n0 + wn * 64 + c;
      if (m < M && n < N) *reinterpret_cast<uint4*>(y + (size_t)m * N + n) = make_uint4(a.x, a.y, b.x, b.y);
    }
    __syncthreads();                         // the ring is rewritten by the next tile's stage 0
    if (!has_next) break;
    tile = next;

  }
}

// Workgroups that fit on the device at once (two per CU), cached per device.
static int resident_blocks() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached[dev] = 2 * cus;
  }
  return cached[dev];
}

template <int RB, bool BIAS>
static hipError_t launch_g3(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const int nb = tiles < resident_blocks() ? tiles : resident_blocks();
  hipLaunchKernelGGL((k_gemm3<RB, BIAS>), dim3(nb), dim3(NT), 0, s, (const uint8_t*)a.xq,
                     (const __half*)a.xs, (const __half*)a.t, (const uint8_t*)a.wq, (const __half*)a.ws,
                     (const __half*)a.l2, (const __half*)a.bias, a.M, a.N, a.K, (__half*)a.y);
  return hipGetLastError();
}

template <bool BIAS>
static hipError_t launch_g3_r(const GemmArgs& a, hipStream_t s) {
  switch (a.r) {
    case 0: return launch_g3<0, BIAS>(a, s);
    case 16: return launch_g3<1, BIAS>(a, s);
    case 32: return launch_g3<2, BIAS>(a, s);
    case 48: return launch_g3<3, BIAS>(a, s);
    case 64: return launch_g3<4, BIAS>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm3(const GemmArgs& a, hipStream_t s) {
  if (a.fmt != FMT_INT4_E2M3) return hipErrorInvalidValue;
  return a.bias != nullptr ? launch_g3_r<true>(a, s) : launch_g3_r<false>(a, s);
}

}  // namespace svdq
