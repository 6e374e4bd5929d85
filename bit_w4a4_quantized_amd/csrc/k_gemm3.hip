// Kernel B for the 6-bit container format (SVDQ_INT4_G64_E2M3): low-bit GEMM on
// the FP6 matrix cores, per-group rescale into fp32, up projection and bias in
// the epilogue, fp16 store.
//
// Practice page "sota-314", section "Do this": the up projection is fused
// with the 4-bit compute since both produce Y.
//
//   Y[m,n] = fp16_rne( sum_g sx[m,g] sw[n,g] P_g[m,n] + (T L2)[m,n] + b[n] )
//   P_g    = sum_{k in group g} q_x[m,k] q_w[n,k]   (exact)
//
// Each INT4 code q is held as the E2M3 subnormal of q/8, so 32 codes of a row
// (one half of a group) are the six-dword operand of
// v_mfma_scale_f32_32x32x64_f8f6f4 in FP6 mode, and one MFMA per 32 x 32 tile
// and group returns a power-of-two multiple of P_g in fp32 exactly: the products of the E2M3
// values are P_g / 64, and the instruction's block scale for the A operand (E8M0) multiplies by
// a power of two exactly.  The scale products S = sw sx^T of a tile come from one
// v_mfma_f32_32x32x8_f16 whose operands carry the scales in K slots 0 and 4 (one from each
// lane half) and zeros elsewhere, so it returns 2 S exactly; with the FP6 MFMA returning
// P_g / 2 (E8M0 132 = 2^5), the vector ALU spends one fma per output element and group,
// acc += (P_g / 2) (2 S), whose product is exactly P_g S.
//
// The MFMAs take the weight tile as the row operand and the activation tile as
// the column operand, so each lane's accumulators belong to one output row
// (token m) and 4 runs of 4 consecutive columns: the epilogue's stores are
// 8-byte pieces, assembled through LDS into 16-byte row-contiguous stores.
//
// Work decomposition (gfx950, wave64): workgroup tile 128 x 128, four waves in
// 2 x 2 of 64 x 64 (2 x 2 MFMA tiles), two workgroups per CU, persistent (each
// workgroup loops over tiles).  K advances in stages of three groups through two
// LDS buffers.  Operands go from global memory straight into LDS (buffer loads
// with the LDS-DMA form: no registers, no LDS store instructions), issued one
// stage ahead; each wave first reads all of a stage's MFMA operands into
// registers, then issues the next stage's loads, then computes, so its LDS reads
// never wait on loads in flight.  The last step of a tile loads the next tile's
// first stage, which thus overlaps this tile's epilogue.
// The container keeps, per (row, group), half 0's bytes 0..15, half 1's bytes
// 0..15 and both halves' bytes 16..23 as three 16-byte chunks; LDS keeps each
// chunk kind as an array over the tile's rows, so a row costs three 16-byte
// loads, every MFMA operand is one 16-byte and one 8-byte LDS read straight into
// its registers, and both the loads and the reads touch contiguous bytes (no
// bank conflicts).  Scales arrive as one dword per row (the 2-byte
// DMA form zero-extends), which with a zero register is the scale MFMA's operand
// (K slot 0 for lanes of the lower K half, slot 4 for the upper; both halves read the
// same dword, a broadcast).
// Tile order: each XCD (own L2) works on a contiguous range of tiles, rastered
// in groups of 8 tile rows.
#include "kernels.h"

namespace svdq {

namespace {

constexpr int BM = 128, BN = 128, NT = 256, KC = 3;   // 3 groups a stage: fewer barriers; 2 x 79872 B of LDS per CU
constexpr int GB = 48;                      // container bytes per (row, group)
// LDS layout of one group (byte offsets): per operand the three 16-byte chunks of each row's
// 48 container bytes (half 0 bytes 0..15 | half 1 bytes 0..15 | both halves' bytes 16..23),
// each chunk kind an array [128 rows] x 16
constexpr int L_X = 0;                      // X chunks 0, 1, 2 at L_X + 2048 c
constexpr int L_W = 6144;                   // W chunks
constexpr int L_SX = 12288;                 // X scales, one dword (fp16, zero-extended) per row
constexpr int L_SW = 12800;                 // W scales
constexpr int GROUP = 13312;
constexpr int STAGE = KC * GROUP;
constexpr int RING = 2 * STAGE;             // 79872 bytes
// epilogue: buffer 1 of the ring (buffer 0 already receives the next tile's stage 0)
constexpr int E_L2 = STAGE;                 // L2^T staging, 128 columns x (r + 8) halves
constexpr int E_Y = STAGE;                  // fp16 output staging, per wave 32 rows x 136 bytes
constexpr int E_YS = 136;
static_assert(E_Y + 4 * 32 * E_YS <= RING, "output staging must fit buffer 1");
static_assert(STAGE % 16 == 0 && GROUP % 16 == 0, "16-byte aligned buffers");


// One wave's LDS-DMA load: lane l's 16 bytes (or 2 bytes, zero-extended to a dword) go to
// dst + 16 l (dst + 4 l).  dst must be wave-uniform.
// (The instruction's immediate offset would move the LDS destination too; offsets go into the
// vector or scalar offset, which move only the global address.)
__device__ __forceinline__ void dma16(rsrc_t r, uint8_t* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, (int)voff, (int)soff, 0, 0);
}
__device__ __forceinline__ void dma2(rsrc_t r, uint8_t* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 2, (int)voff, (int)soff, 0, 0);
}

// An opaque copy: LDS reads from distinct bases are not merged into paired reads whose
// halves would then have to be moved into the MFMA operand registers.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Tile index -> output tile: contiguous ranges per XCD (workgroups are dealt round-robin to
// the 8 XCDs and keep their XCD), then 8-tile-row groups within a range.
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

// The last, partial round of tiles: when only a few tiles remain after the full rounds of
// the persistent loop, each of them is cut into 16 sub-tiles of 32 x 32, and each sub-tile is
// one job for a whole workgroup, taken by the persistent workgroups once their full tiles are
// done: its four waves split K (groups w, w + 4, ...) and add their partial sums in LDS (red,
// 12 KB of the workgroup's LDS) in a fixed order, so the result is deterministic and no
// global scratch is needed.  Operands come straight from global memory into registers, four
// groups ahead.  Ends with a barrier (red is reused by the next job).
template <int RB, bool BIAS>
__device__ __forceinline__ void gemm3_subtile(const uint8_t* __restrict__ xq, const __half* __restrict__ xs,
                                              const __half* __restrict__ t, const uint8_t* __restrict__ wq,
                                              const __half* __restrict__ ws, const __half* __restrict__ l2,
                                              const __half* __restrict__ bias, const float* __restrict__ lam,
                                              int M, int N, int K, __half* __restrict__ y, int tile0, int job,
                                              float (*red)[16][64]) {
  constexpr int R = RB * 16;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, r32 = lane & 31;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int tiles = tiles_m * tiles_n;
  const int G = K >> 6;
  int tm, tn;
  tile_of3(tile0 + (job >> 4), tiles, tiles_m, tiles_n, &tm, &tn);
  const int sub = job & 15;
  const int nb = tn * BN + (sub >> 2) * 32, mb = tm * BM + (sub & 3) * 32;   // sub-tile origin
  const int m = min(mb + r32, M - 1), n = min(nb + r32, N - 1);           // this lane's operand rows

  typedef _Float16 v4h_t __attribute__((ext_vector_type(4)));
  struct Op { uint4 x0, w0; uint2 x1, w1; uint32_t sx, sw; };
  // buffer loads: the group's offset is wave-uniform (scalar offset), the lane's row offset a
  // vector offset.  (As intrinsics, not plain loads, they are also kept where they are
  // written: plain loads feeding the ring's loop-carried values get merged into one load
  // at the use.)
  const rsrc_t rxq = make_rsrc(xq, (size_t)G * M * GB), rwq = make_rsrc(wq, (size_t)G * N * GB);
  const rsrc_t rxs = make_rsrc(xs, (size_t)G * M * 2), rws = make_rsrc(ws, (size_t)G * N * 2);
  const uint32_t vx = (uint32_t)m * GB + 16u * h, vw = (uint32_t)n * GB + 16u * h;
  const uint32_t vx1 = (uint32_t)m * GB + 32u + 8u * h, vw1 = (uint32_t)n * GB + 32u + 8u * h;
  auto load = [&](int g, Op& o) {
    const uint32_t sx = (uint32_t)g * (uint32_t)M, sw = (uint32_t)g * (uint32_t)N;
    o.x0 = as_u4(__builtin_amdgcn_raw_buffer_load_b128(rxq, (int)vx, (int)(sx * GB), 0));
    o.x1 = as_u2(__builtin_amdgcn_raw_buffer_load_b64(rxq, (int)vx1, (int)(sx * GB), 0));
    o.w0 = as_u4(__builtin_amdgcn_raw_buffer_load_b128(rwq, (int)vw, (int)(sw * GB), 0));
    o.w1 = as_u2(__builtin_amdgcn_raw_buffer_load_b64(rwq, (int)vw1, (int)(sw * GB), 0));
    // every lane loads (no branch around a load); the upper K half's scale is zeroed at use
    o.sx = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rxs, (int)((uint32_t)m * 2u), (int)(sx * 2u), 0);
    o.sw = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rws, (int)((uint32_t)n * 2u), (int)(sw * 2u), 0);
  };
  // the epilogue's operands (T rows, L2 columns, bias), loaded by every wave before the K loop
  // so that their latency overlaps it (wave 0 uses them)
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
  // a ring of PD slots of loads in flight per wave (groups wave, wave + 4, ...): step s
  // (s = 0, 1, ...) processes slot s % PD, which holds the wave's group s - PD (none for
  // s < PD: the slots start zeroed and count with a zero scale product, exactly +0), then
  // refills it with the wave's group s (past the last one it re-reads the last one).  There
  // is no prologue and no branch in the loop: otherwise the compiler's wait counts, merged
  // over paths with different loads in flight, make each slot wait for every load issued.
  constexpr int PD = 4;
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
      const v8i xo = v8i{(int)cur.x0.x, (int)cur.x0.y, (int)cur.x0.z, (int)cur.x0.w, (int)cur.x1.x, (int)cur.x1.y, 0, 0};
      const v8i wo = v8i{(int)cur.w0.x, (int)cur.w0.y, (int)cur.w0.z, (int)cur.w0.w, (int)cur.w1.x, (int)cur.w1.y, 0, 0};
      const v16f p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wo, xo, v16f{}, 2, 2, 0, 133, 0, 127);
      // K slot 0 holds the scale for the lower-K-half lanes; the upper half contributes zeros
      const v16f sc = __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(v4h_t, make_uint2(zero ? 0u : cur.sw, 0u)),
                                                            __builtin_bit_cast(v4h_t, make_uint2(zero ? 0u : cur.sx, 0u)),
                                                            v16f{}, 0, 0, 0);
      // refill the slot once the MFMAs have read it (loading it earlier would make the
      // compiler copy the operands, and the copy waits for every load in flight)
      load(ng > 0 ? wave + 4 * min(st, ng - 1) : 0, ring[j]);
#pragma unroll
      for (int i = 0; i < 16; i++) acc[i] = __builtin_fmaf(p[i], sc[i], acc[i]);
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
    // up projection on the 32 x 32 sub-tile: row operand L2^T (columns n), column operand T (rows m)
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
      if (mo >= M) break;
      const int no = nb + 8 * q + 4 * h;
      if (no >= N) continue;
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

template <int RB, bool BIAS>
__global__ void __launch_bounds__(NT, 2)
k_gemm3(const uint8_t* __restrict__ xq, const __half* __restrict__ xs, const __half* __restrict__ t,
        const uint8_t* __restrict__ wq, const __half* __restrict__ ws, const __half* __restrict__ l2,
        const __half* __restrict__ bias, const float* __restrict__ lam, int M, int N, int K,
        __half* __restrict__ y, int tiles_run) {
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
  const int NSE = (NS + 1) & ~1;             // rounded up to even: stage s uses buffer s % 2

  // ---- load assignment: wave w loads rows 64 (w%2) + lane of the X (waves 0, 1) or W (waves
  // 2, 3) tile: the three code chunks of the row and its scale.  Rows past the edge re-read
  // the tile's last valid row (their outputs are never stored).
  const bool s_x = wave < 2;
  const int lrow = (wave & 1) * 64 + lane;
  const uint32_t c_step = (uint32_t)(s_x ? M : N) * GB;   // bytes between groups
  const uint32_t s_step = (uint32_t)(s_x ? M : N) * 2;
  struct Src {                               // where this wave reads one tile's operands
    rsrc_t rc, rs;
    uint32_t vc, vs;
  };
  auto tile_src = [&](int tile) {
    int tm_, tn_;
    tile_of3(tile, tiles, tiles_m, tiles_n, &tm_, &tn_);
    const int m0_ = tm_ * BM, n0_ = tn_ * BN;
    const int mr = min(BM, M - m0_), nr = min(BN, N - n0_);
    const int sr = s_x ? mr : nr;
    Src r;
    // codes are group-major [G][rows][48]: a tile's rows of one group are contiguous
    r.rc = s_x ? make_rsrc(xq + (size_t)m0_ * GB, ((size_t)(G - 1) * M + mr) * GB)
               : make_rsrc(wq + (size_t)n0_ * GB, ((size_t)(G - 1) * N + nr) * GB);
    r.rs = make_rsrc(s_x ? (const void*)(xs + m0_) : (const void*)(ws + n0_),
                     ((size_t)(G - 1) * (s_x ? M : N) + sr) * 2);
    r.vc = (uint32_t)min(lrow, sr - 1) * GB;
    r.vs = (uint32_t)min(lrow, sr - 1) * 2;
    return r;
  };
  // all loads of one stage into LDS buffer buf (4 per wave and group)
  auto load_stage = [&](const Src& src, int st, int buf) {
#pragma unroll
    for (int k = 0; k < KC; k++) {
      const int g = min(st * KC + k, G - 1);   // a group past the end re-reads the last one (unused)
      uint8_t* b = lds + buf * STAGE + k * GROUP + (s_x ? L_X : L_W) + (wave & 1) * 1024;
      const uint32_t so = (uint32_t)g * c_step;
      dma16(src.rc, b, src.vc, so);
      dma16(src.rc, b + 2048, src.vc, so + 16);
      dma16(src.rc, b + 4096, src.vc, so + 32);
      dma2(src.rs, lds + buf * STAGE + k * GROUP + (s_x ? L_SX : L_SW) + (wave & 1) * 256, src.vs,
           (uint32_t)g * s_step);
    }
  };
  auto wait_loads = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // per-lane LDS read bases (tile, group and stage offsets are immediates)
  // (operand of lane (row, half h): chunk h of the row, then the 8 bytes at 8 h of chunk 2)
  int rx_p0[2], rx_p1[2], rw_p0[2], rw_p1[2], rs_x[2], rs_w[2];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    rx_p0[i] = L_X + 2048 * h + (wm * 64 + i * 32 + r32) * 16;
    rw_p0[i] = L_W + 2048 * h + (wn * 64 + i * 32 + r32) * 16;
    rx_p1[i] = opaque(L_X + 4096 + (wm * 64 + i * 32 + r32) * 16 + 8 * h);
    rw_p1[i] = opaque(L_W + 4096 + (wn * 64 + i * 32 + r32) * 16 + 8 * h);
    rs_x[i] = opaque(L_SX + (wm * 64 + i * 32 + r32) * 4);   // both lane halves: one address
    rs_w[i] = opaque(L_SW + (wn * 64 + i * 32 + r32) * 4);
  }
  // MFMA operands of one group.  Scale operands: the second dword stays zero; code operands:
  // six dwords.
  struct Ops {
    v8i xo[2], wo[2];
    uint2 sxo[2], swo[2];
  };
  Ops ops[KC];
#pragma unroll
  for (int k = 0; k < KC; k++)
#pragma unroll
    for (int i = 0; i < 2; i++) {
#pragma unroll
      for (int e = 0; e < 8; e++) { ops[k].xo[i][e] = 0; ops[k].wo[i][e] = 0; }
      ops[k].sxo[i] = make_uint2(0, 0);
      ops[k].swo[i] = make_uint2(0, 0);
    }
  v16f acc[2][2];   // [tj][ti]: lane -> row m = ti*32 + r32, reg v -> column 8(v/4) + 4h + v%4 of tile tj

  auto read_ops = [&](const uint8_t* b, Ops& o) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const uint4 x0 = *reinterpret_cast<const uint4*>(b + rx_p0[i]);
      const uint2 x1 = *reinterpret_cast<const uint2*>(b + rx_p1[i]);
      const uint4 w0 = *reinterpret_cast<const uint4*>(b + rw_p0[i]);
      const uint2 w1 = *reinterpret_cast<const uint2*>(b + rw_p1[i]);
      o.xo[i][0] = (int)x0.x; o.xo[i][1] = (int)x0.y; o.xo[i][2] = (int)x0.z; o.xo[i][3] = (int)x0.w;
      o.xo[i][4] = (int)x1.x; o.xo[i][5] = (int)x1.y;
      o.wo[i][0] = (int)w0.x; o.wo[i][1] = (int)w0.y; o.wo[i][2] = (int)w0.z; o.wo[i][3] = (int)w0.w;
      o.wo[i][4] = (int)w1.x; o.wo[i][5] = (int)w1.y;
      o.sxo[i].x = *reinterpret_cast<const uint32_t*>(b + rs_x[i]);
      o.swo[i].x = *reinterpret_cast<const uint32_t*>(b + rs_w[i]);
    }
  };
  typedef _Float16 v4h_t __attribute__((ext_vector_type(4)));
  auto mma_ops = [&](const Ops& o) {
#pragma unroll
    for (int tj = 0; tj < 2; tj++)
#pragma unroll
      for (int ti = 0; ti < 2; ti++) {
        // P_g / 2 and 2 S (the scales sit in both K halves): the fma's product is exactly P_g S
        const v16f p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(o.wo[tj], o.xo[ti], v16f{}, 2, 2, 0, 132, 0, 127);
        const v16f sc = __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(v4h_t, o.swo[tj]),
                                                              __builtin_bit_cast(v4h_t, o.sxo[ti]), v16f{}, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 16; i++) acc[tj][ti][i] = __builtin_fmaf(p[i], sc[i], acc[tj][ti][i]);
      }
  };

  // ---- persistent loop over tiles: tile, tile + gridDim.x, ...
  int tile = blockIdx.x;
  Src cur = tile_src(tile);
  load_stage(cur, 0, 0);
  while (true) {
    const int next = tile + (int)gridDim.x;
    const bool has_next = next < tiles_run;
    const Src nxt = tile_src(has_next ? next : tile);
    int tm, tn;
    tile_of3(tile, tiles, tiles_m, tiles_n, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // stage 0 of this tile is in flight or landed in buffer 0
    wait_loads();
    __syncthreads();

#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
      for (int b = 0; b < 2; b++)
#pragma unroll
        for (int i = 0; i < 16; i++) acc[a][b][i] = 0.f;

    // step st: read stage st's operands (buffer buf), start the loads of the following
    // stage into the other buffer (this tile's st + 1, or the next tile's stage 0 after the
    // last step), compute, then wait for the loads and synchronise.
    auto step = [&](int st, int buf) {
      if (st < NS) {
#pragma unroll
        for (int k = 0; k < KC; k++)
          if (st * KC + k < G) read_ops(lds + buf * STAGE + k * GROUP, ops[k]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (st + 1 < NS) load_stage(cur, st + 1, buf ^ 1);
      else if (st + 1 == NSE && has_next) load_stage(nxt, 0, buf ^ 1);
      __builtin_amdgcn_sched_barrier(0);
      if (st < NS) {
#pragma unroll
        for (int k = 0; k < KC; k++)
          if (st * KC + k < G) mma_ops(ops[k]);
      }
      if (st + 1 < NSE) {                    // the last step's loads land during the epilogue
        wait_loads();
      }
      __syncthreads();
    };
    for (int st = 0; st < NSE; st += 2) {
      step(st, 0);
      step(st + 1, 1);
    }

    // ---- epilogue in buffer 1 of the ring (every wave passed the last barrier)

    if (RB > 0) {
      // L2[:, n0:n0+128] transposed into LDS as [n][k] (row stride (R+8) halves), then
      // acc += L2^T T^T on v_mfma_f32_32x32x16_f16: row operand L2^T (columns n), column
      // operand T (rows m, 8 consecutive k per lane: one 16-byte load)
      constexpr int LS2 = (R + 8) * 2;
      static_assert(E_L2 + BN * LS2 <= RING, "L2 staging must fit buffer 1");
      uint8_t* l2s = lds + E_L2;
      for (int idx = tid; idx < R * (BN / 8); idx += NT) {
        const int k = idx % R, c8 = idx / R;   // neighbouring lanes write neighbouring k
        const int n = n0 + c8 * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (n < N) v = *reinterpret_cast<const uint4*>(l2 + (size_t)k * N + n);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; e++)
          *reinterpret_cast<uint16_t*>(l2s + (c8 * 8 + e) * LS2 + k * 2) = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
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
          const uint4 lo = *reinterpret_cast<const uint4*>(l2s + (wn * 64 + tj * 32 + r32) * LS2 + (kb * 16 + 8 * h) * 2);
#pragma unroll
          for (int ti = 0; ti < 2; ti++)
            acc[tj][ti] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(lo), as_h8(top[kb][ti]), acc[tj][ti], 0, 0, 0);
        }
      __syncthreads();                       // the output staging reuses the L2 staging bytes
    }

    // bias, RNE to fp16, 8-byte pieces into this wave's LDS staging (32 rows at a time),
    // 16-byte row stores
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
    uint8_t* ys = lds + E_Y + wave * 32 * E_YS;
#pragma unroll
    for (int ti = 0; ti < 2; ti++) {
#pragma unroll
      for (int tj = 0; tj < 2; tj++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int nl = tj * 32 + 8 * q + 4 * h;    // column within the wave's 64
          uint32_t hv[4];
#pragma unroll
          for (int j = 0; j < 4; j++)
            hv[j] = __half_as_ushort(__float2half_rn(acc[tj][ti][4 * q + j] + bv[tj][q][j]));
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
        if (lam) {                           // the MLP glue folded in: fp16(gelu(y) / lam)
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
    __syncthreads();                         // buffer 1 is rewritten by the next tile's stage 1
    if (!has_next) break;
    tile = next;
    cur = nxt;
  }

  // ---- the tiles past tiles_run (a last, partial round) as 32 x 32 sub-tile jobs, taken as
  // the workgroups finish their full tiles; their partial sums use the ring's first 12 KB
  // (no loads are in flight: the last tile started none)
  const int n_sub = (tiles - tiles_run) * 16;
  for (int job = blockIdx.x; job < n_sub; job += gridDim.x)
    gemm3_subtile<RB, BIAS>(xq, xs, t, wq, ws, l2, bias, lam, M, N, K, y, tiles_run, job,
                            reinterpret_cast<float (*)[16][64]>(lds));
}

// Few token rows (weight-streaming regime): one workgroup per 32 output columns and a slab of
// up to 128 rows (MT tiles of 32; blockIdx.y picks the slab), so each weight row is read once
// per slab; its four waves split K
// (groups w, w + 4, ...), holding PD groups of loads in flight straight into registers, and add
// their partial sums in LDS in a fixed order, one row tile at a time; wave 0 then applies the up
// projection and the bias and stores.
template <int RB, bool BIAS, int MT, int PD>
__global__ void __launch_bounds__(NT, 2)
k_gemm3_skinny(const uint8_t* __restrict__ xq, const __half* __restrict__ xs, const __half* __restrict__ t,
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
  struct Op { uint4 w0; uint2 w1; uint32_t sw; uint4 x0[MT]; uint2 x1[MT]; uint32_t sx[MT]; };
  // buffer loads as in gemm3_subtile (group offset scalar, row offset per lane)
  const rsrc_t rxq = make_rsrc(xq, (size_t)G * M * GB), rwq = make_rsrc(wq, (size_t)G * N * GB);
  const rsrc_t rxs = make_rsrc(xs, (size_t)G * M * 2), rws = make_rsrc(ws, (size_t)G * N * 2);
  const uint32_t vw = (uint32_t)n * GB + 16u * h, vw1 = (uint32_t)n * GB + 32u + 8u * h;
  auto load = [&](int g, Op& o) {
    const uint32_t sx = (uint32_t)g * (uint32_t)M, sw = (uint32_t)g * (uint32_t)N;
    o.w0 = as_u4(__builtin_amdgcn_raw_buffer_load_b128(rwq, (int)vw, (int)(sw * GB), 0));
    o.w1 = as_u2(__builtin_amdgcn_raw_buffer_load_b64(rwq, (int)vw1, (int)(sw * GB), 0));
    // every lane loads (no branch around a load); the upper K half's scale is zeroed at use
    o.sw = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rws, (int)((uint32_t)n * 2u), (int)(sw * 2u), 0);
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      const uint32_t vr = (uint32_t)mrow[mt] * GB;
      o.x0[mt] = as_u4(__builtin_amdgcn_raw_buffer_load_b128(rxq, (int)(vr + 16u * h), (int)(sx * GB), 0));
      o.x1[mt] = as_u2(__builtin_amdgcn_raw_buffer_load_b64(rxq, (int)(vr + 32u + 8u * h), (int)(sx * GB), 0));
      o.sx[mt] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rxs, (int)((uint32_t)mrow[mt] * 2u), (int)(sx * 2u), 0);
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
  // the ring of gemm3_subtile: step s processes slot s % PD (the wave's group s - PD, or a
  // zeroed slot with a zero scale product) and refills it with the wave's group s
  const int ng = wave < G ? (G - 1 - wave) / 4 + 1 : 0;   // this wave's groups
  Op ring[PD];
#pragma unroll
  for (int j = 0; j < PD; j++) ring[j] = Op{};
  for (int s0 = 0; s0 < ng + PD; s0 += PD) {
#pragma unroll
    for (int j = 0; j < PD; j++) {
      const int st = s0 + j;
      // (skipping the work of the empty slots behind a wave-uniform branch measured slower here)
      const bool zero = h || st < PD || st - PD >= ng;   // upper K half, or an empty slot
      const Op& cur = ring[j];
      const v8i wo = v8i{(int)cur.w0.x, (int)cur.w0.y, (int)cur.w0.z, (int)cur.w0.w, (int)cur.w1.x, (int)cur.w1.y, 0, 0};
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        const v8i xo = v8i{(int)cur.x0[mt].x, (int)cur.x0[mt].y, (int)cur.x0[mt].z, (int)cur.x0[mt].w,
                           (int)cur.x1[mt].x, (int)cur.x1[mt].y, 0, 0};
        const v16f p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wo, xo, v16f{}, 2, 2, 0, 133, 0, 127);
        // K slot 0 holds the scale for the lower-K-half lanes; the upper half contributes zeros
        const v16f sc = __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(v4h_t, make_uint2(zero ? 0u : cur.sw, 0u)),
                                                              __builtin_bit_cast(v4h_t, make_uint2(zero ? 0u : cur.sx[mt], 0u)),
                                                              v16f{}, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 16; i++) acc[mt][i] = __builtin_fmaf(p[i], sc[i], acc[mt][i]);
      }
      // refill the slot once the MFMAs have read it (see gemm3_subtile)
      load(ng > 0 ? wave + 4 * min(st, ng - 1) : 0, ring[j]);
      __builtin_amdgcn_sched_barrier(0);     // keep the slots in order: each waits for its own loads only
    }
  }
  // the four waves' partials, added in wave order, one row tile at a time
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
    if (wave > 0) {
#pragma unroll
      for (int i = 0; i < 16; i++) red[wave - 1][i][lane] = acc[mt][i];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int i = 0; i < 16; i++) acc[mt][i] = ((acc[mt][i] + red[0][i][lane]) + red[1][i][lane]) + red[2][i][lane];
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


// Up to this many token rows the weight-streaming kernel runs (in 128-row slabs).
constexpr int kSkinnyRows = 256;

template <int RB, bool BIAS, int MT, int PD = (MT <= 2 ? 4 : 2)>
static hipError_t launch_g3_skinny(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm3_skinny<RB, BIAS, MT, PD>), dim3((a.N + 31) / 32, (a.M + 32 * MT - 1) / (32 * MT)),
                     dim3(NT), 0, s, (const uint8_t*)a.xq,
                     (const __half*)a.xs, (const __half*)a.t, (const uint8_t*)a.wq, (const __half*)a.ws,
                     (const __half*)a.l2, (const __half*)a.bias, a.lam, a.M, a.N, a.K, (__half*)a.y);
  return hipGetLastError();
}

template <int RB, bool BIAS>
static hipError_t launch_g3(const GemmArgs& a, hipStream_t s) {
  // few token rows: the weight-streaming kernel
  // ring depth: two groups in flight per wave (one for 128-row slabs) get each wave's data
  // sooner than four (two) did
  if (a.M <= 32) return launch_g3_skinny<RB, BIAS, 1, 2>(a, s);
  if (a.M <= 64) return launch_g3_skinny<RB, BIAS, 2, 2>(a, s);
  if (a.M <= kSkinnyRows) return launch_g3_skinny<RB, BIAS, 4, 1>(a, s);
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const int slots = resident_workgroups();
  const int rem = tiles % slots;
  const int main_tiles = (tiles > slots && rem > 0 && 4 * rem <= slots) ? tiles - rem : tiles;
  const int nb = main_tiles < slots ? main_tiles : slots;
  hipLaunchKernelGGL((k_gemm3<RB, BIAS>), dim3(nb), dim3(NT), 0, s, (const uint8_t*)a.xq,
                     (const __half*)a.xs, (const __half*)a.t, (const uint8_t*)a.wq, (const __half*)a.ws,
                     (const __half*)a.l2, (const __half*)a.bias, a.lam, a.M, a.N, a.K, (__half*)a.y, main_tiles);
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
