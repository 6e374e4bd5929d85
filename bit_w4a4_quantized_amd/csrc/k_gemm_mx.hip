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
// Two kernels.  128 x 128 tiles: stages of four 64-K chunks on the shared persistent skeleton
// (two chunks a stage left each stage waiting on the next one's loads: 142 -> 129 us at the fc1
// shape).  Per chunk and workgroup: each operand's 128 rows x 32 code bytes arrive by 16-byte
// LDS-DMA loads into 16-byte slots swapped by row (slot c of row r at c ^ ((r / 8) % 2)), and
// the rows' 2 scale bytes by 2-byte loads into 4-byte slots.  Lane half h reads the chunk's codes
// 32 h .. 32 h + 31 (one 16-byte read) and scale byte h.  256 x 256 tiles on four waves for
// large M, N and K (k_gemm_mxw, below); launch_gemm_mx picks the cheaper.
#include "gemm_skel.h"

namespace svdq {

namespace {

using namespace skel;

typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

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

namespace {

// ---------------------------------------------------------------------------------------------
// Large tiles.  With 128 x 128 tiles each CU stages 17 KB per chunk (LDS-DMA) for 32 tile-groups
// and its waves read 32 KB of operand fragments from LDS.  Here one workgroup of WM x WN waves
// per CU owns a BM x BN tile and each wave a TI x TJ block of 32 x 32 tiles: at 256 x 256 with
// 4 x 4 per wave (four waves), 18 KB of LDS-DMA per chunk serve 64 tile-groups, and each wave
// reads 8 fragments for 16 MFMAs.  The accumulators stay with the matrix cores (no vector work
// per chunk).  Codes sit in the 128 x 128 kernel's swapped 16-byte slots; each row's two scale
// bytes of a chunk arrive by one 2-byte LDS-DMA lane into a dword of their own (zero-extended),
// from which a lane shifts out its byte.  K goes through a ring of four LDS buffers (below).
// Chunks are added in the same order and the epilogue makes the same operations, so the output
// is bit-identical to the 128 x 128 kernel's.
template <int WM_, int WN_, int TI_, int TJ_, int KC_>
struct Big {
  static constexpr int WM = WM_, WN = WN_, TI = TI_, TJ = TJ_, KC = KC_;
  static constexpr int NW = WM * WN, NTH = 64 * NW;
  static constexpr int BM = WM * TI * 32, BN = WN * TJ * 32;
  // per chunk: codes X [BM][32 bytes], W [BN][32 bytes]; scales one dword per row (bytes 0 and
  // 1: the row's two groups), X [BM], W [BN]
  static constexpr int L_X = 0, L_W = BM * 32, L_SX = L_W + BN * 32, L_SW = L_SX + BM * 4;
  static constexpr int CHUNK = L_SW + BN * 4;
  static constexpr int BUF = KC * CHUNK;
  // LDS-DMA instructions per chunk: 32 code rows, or 64 scale rows, each
  static constexpr int NX = BM / 32, NWC = BN / 32, NSX = BM / 64, NSW = BN / 64;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "whole 64-row scale loads");
};

template <class C>
struct BigOp {
  // a wave's LDS-DMA instructions per chunk: code slots j (instruction wave + j NW of the NX
  // X-row and NWC W-row ones, 32 rows each) and scale slots (of the NSX + NSW, 64 rows each);
  // the kind of each slot is fixed for the wave, so its resource, LDS offset and chunk stride
  // are set once
  static constexpr int NCODE = C::NX + C::NWC, NSCALE = C::NSX + C::NSW;
  static constexpr int PC = (NCODE + C::NW - 1) / C::NW, PS = (NSCALE + C::NW - 1) / C::NW;
  static_assert(NCODE % C::NW == 0 && NSCALE % C::NW == 0, "every wave issues as many loads");
  int M, N, C_, NS;
  int lane, h, wave, wm, wn;
  rsrc_t crs[PC], srs[PS];
  int cdst[PC], sdst[PS];                    // LDS offsets within a chunk
  uint32_t cstr[PC], sstr[PS];               // global bytes per chunk
  struct Frag {
    uint4 x[C::TI], w[C::TJ];
    uint32_t sx[C::TI], sw[C::TJ];
  };
  struct Src {
    uint32_t c[PC], s[PS];
  };

  __device__ BigOp(const uint8_t* xq, const uint8_t* xs, const uint8_t* wq, const uint8_t* ws, int M_, int N_, int K)
      : M(M_), N(N_) {
    C_ = K >> 6;
    NS = (C_ + C::KC - 1) / C::KC;
    lane = threadIdx.x & 63;
    h = lane >> 5;
    wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    wm = wave / C::WN;
    wn = wave % C::WN;
    const rsrc_t rx = make_rsrc(xq, (size_t)M * K / 2), rw = make_rsrc(wq, (size_t)N * K / 2);
    const rsrc_t rsx = make_rsrc(xs, (size_t)M * K / 32), rsw = make_rsrc(ws, (size_t)N * K / 32);
#pragma unroll
    for (int j = 0; j < PC; j++) {
      const int i = wave + j * C::NW;
      const bool isx = i < C::NX;
      crs[j] = isx ? rx : rw;
      cdst[j] = isx ? C::L_X + i * 1024 : C::L_W + (i - C::NX) * 1024;
      cstr[j] = (uint32_t)(isx ? M : N) * 32u;
    }
#pragma unroll
    for (int j = 0; j < PS; j++) {
      const int i = wave + j * C::NW;
      const bool isx = i < C::NSX;
      srs[j] = isx ? rsx : rsw;
      sdst[j] = isx ? C::L_SX + i * 256 : C::L_SW + (i - C::NSX) * 256;
      sstr[j] = (uint32_t)(isx ? M : N) * 2u;
    }
  }

  // per-lane global offsets of the slots for the tile at (m0, n0): a code slot's lane l moves
  // row 32 i' + l / 2 (i' its instruction within X or W), into LDS slot l % 2, which holds piece
  // (l % 2) ^ ((row / 8) % 2); a scale slot's lane l moves the two bytes of row 64 i' + l.  Rows
  // past the edge re-read the last row.
  __device__ Src src(int m0, int n0) const {
    Src o;
#pragma unroll
    for (int j = 0; j < PC; j++) {
      const int i = wave + j * C::NW;
      const bool isx = i < C::NX;
      const int row = (isx ? i : i - C::NX) * 32 + (lane >> 1);
      const int piece = (lane & 1) ^ ((row >> 3) & 1);
      o.c[j] = (uint32_t)(isx ? min(m0 + row, M - 1) : min(n0 + row, N - 1)) * 32u + 16u * (uint32_t)piece;
    }
#pragma unroll
    for (int j = 0; j < PS; j++) {
      const int i = wave + j * C::NW;
      const bool isx = i < C::NSX;
      const int row = (isx ? i : i - C::NSX) * 64 + lane;
      o.s[j] = (uint32_t)(isx ? min(m0 + row, M - 1) : min(n0 + row, N - 1)) * 2u;
    }
    return o;
  }
  // step st's chunks; a chunk past the end of K reads as zeros (an offset past the buffer's
  // range): zero codes add exactly +0 whatever the scales
  __device__ void load(const Src& v, int st, uint8_t* buf) const {
#pragma unroll
    for (int k = 0; k < C::KC; k++) {
      const int ci = st * C::KC + k;
      const bool past = ci >= C_;
      const uint32_t c = (uint32_t)min(ci, C_ - 1);
      uint8_t* b = buf + k * C::CHUNK;
#pragma unroll
      for (int j = 0; j < PC; j++) dma16(crs[j], b + cdst[j], past ? 0x80000000u : v.c[j], c * cstr[j]);
#pragma unroll
      for (int j = 0; j < PS; j++) dma2(srs[j], b + sdst[j], past ? 0x80000000u : v.s[j], c * sstr[j]);
    }
  }
  // lane (r32, h) reads codes 32 h .. 32 h + 31 (one 16-byte slot) of its rows and byte h of
  // their scale dwords (the MFMA's scale operand: the E8M0 byte in the low byte).  In two parts:
  // part 0 the X fragments and scales and the first half of the W fragments, part 1 the rest of
  // the W fragments and the W scales.
  __device__ void read(const uint8_t* b, Frag& f, int part) const {
    const int r32 = lane & 31;
    const int xr = wm * C::TI * 32 + r32, wr = wn * C::TJ * 32 + r32;
    const int xo = C::L_X + xr * 32 + 16 * (h ^ ((xr >> 3) & 1));   // + 1024 per 32-row tile
    const int wo = C::L_W + wr * 32 + 16 * (h ^ ((wr >> 3) & 1));
    const uint32_t* sx = reinterpret_cast<const uint32_t*>(b + C::L_SX) + xr;   // + 32 per tile
    const uint32_t* sw = reinterpret_cast<const uint32_t*>(b + C::L_SW) + wr;
    if (part == 0) {
#pragma unroll
      for (int ti = 0; ti < C::TI; ti++) f.x[ti] = *reinterpret_cast<const uint4*>(b + xo + ti * 1024);
#pragma unroll
      for (int ti = 0; ti < C::TI; ti++) f.sx[ti] = (sx[ti * 32] >> (8 * h)) & 0xFFu;
    }
#pragma unroll
    for (int tj = part * C::TJ / 2; tj < (part + 1) * C::TJ / 2; tj++)
      f.w[tj] = *reinterpret_cast<const uint4*>(b + wo + tj * 1024);
    if (part == 1) {
#pragma unroll
      for (int tj = 0; tj < C::TJ; tj++) f.sw[tj] = (sw[tj * 32] >> (8 * h)) & 0xFFu;
    }
  }
  // the MFMAs of W tiles part * TJ / 2 .. (part + 1) * TJ / 2 - 1
  __device__ void mma(const Frag& f, v16f (&acc)[C::TJ][C::TI], int part) const {
#pragma unroll
    for (int tj = part * C::TJ / 2; tj < (part + 1) * C::TJ / 2; tj++)
#pragma unroll
      for (int ti = 0; ti < C::TI; ti++) acc[tj][ti] = mx_mma(f.w[tj], f.x[ti], f.sw[tj], f.sx[ti], acc[tj][ti]);
  }
};

// A workgroup barrier that leaves loads from global memory in flight (a __syncthreads() would
// wait for every LDS-DMA load of the ring): the wave's LDS operations complete.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// A workgroup barrier after waiting for the wave's LDS operations and for all but its N most
// recent vector-memory operations, written with the builtins (not inline asm) so that the
// compiler's own wait insertion knows what has completed: it then adds no wait of its own for
// fragments read before the barrier.  The empty asm statements keep memory accesses from
// moving across.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));   // vmcnt(N) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Scheduling groups: an MFMA, then (while they last) one LDS read and one vector-memory load,
// NM times.
template <int I, int NM, int NR, int NV>
__device__ __forceinline__ void interleave() {
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (I < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if constexpr (I < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    interleave<I + 1, NM, NR, NV>();
  }
}

template <int V>
struct IC {
  static constexpr int value = V;
};

// The epilogue's operands from global memory: the tile's columns of L2 (staged through LDS) and
// the wave's rows of T, loaded before the tile's last step so that their latency hides behind its
// MFMAs (up to rank 32); the bias of the lane's columns and, with the MLP glue folded in, the next
// layer's factors, loaded as the epilogue starts (earlier, their registers would spill).
template <class C, int RB>
struct BigEpiIn {
  static constexpr int R = RB * 16;
  static constexpr int L2P = RB > 0 ? (R * (C::BN / 8) + C::NTH - 1) / C::NTH : 1;   // 8-column pieces per thread
  static constexpr int NG = (C::TJ + 1) / 2;   // output column groups of (up to) two tiles
  uint4 lv[L2P];
  uint4 top[RB > 0 ? RB : 1][C::TI];
  uint2 braw[C::TJ][4];                       // the bias of the lane's columns
  float4 la[NG], lb[NG];                      // with the MLP glue folded in: the next layer's factors
};

template <class C, int RB>
__device__ __forceinline__ void big_epi_load(BigEpiIn<C, RB>& e, const __half* __restrict__ t,
                                             const __half* __restrict__ l2, int M, int N, int m0, int n0) {
  constexpr int R = RB * 16;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, r32 = lane & 31;
  const int mw = m0 + (wave / C::WN) * C::TI * 32;
  if (RB > 0) {
#pragma unroll
    for (int j = 0; j < BigEpiIn<C, RB>::L2P; j++) {
      const int idx = tid + j * C::NTH;
      const int k = idx % R, c8 = idx / R;
      const int n = n0 + c8 * 8;
      e.lv[j] = make_uint4(0, 0, 0, 0);
      if (idx < R * (C::BN / 8) && n < N) e.lv[j] = *reinterpret_cast<const uint4*>(l2 + (size_t)k * N + n);
    }
#pragma unroll
    for (int kb = 0; kb < RB; kb++)
#pragma unroll
      for (int ti = 0; ti < C::TI; ti++) {
        const int m = min(mw + ti * 32 + r32, M - 1);
        e.top[kb][ti] = *reinterpret_cast<const uint4*>(t + (size_t)m * R + kb * 16 + 8 * h);
      }
  }
}

template <class C, int RB, bool BIAS>
__device__ __forceinline__ void big_epi_load_bias(BigEpiIn<C, RB>& e, const __half* __restrict__ bias,
                                                  const float* __restrict__ lam, int N, int n0) {
  const int lane = threadIdx.x & 63, h = lane >> 5;
  const int nw = n0 + (__builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) % C::WN) * C::TJ * 32;
#pragma unroll
  for (int tj = 0; tj < C::TJ; tj++)
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int n = nw + tj * 32 + 8 * q + 4 * h;
      e.braw[tj][q] = make_uint2(0u, 0u);
      if (BIAS && n < N) e.braw[tj][q] = *reinterpret_cast<const uint2*>(bias + n);
    }
  // the factors of the 8 columns this lane stores per group (loaded only with the glue: a load
  // whose result no path uses would stay pending into the next tile, and the compiler's wait
  // before its registers are rewritten would wait for every load)
  const rsrc_t rl = make_rsrc(lam, lam ? (size_t)N * 4 : 0);
#pragma unroll
  for (int g = 0; g < BigEpiIn<C, RB>::NG; g++) {
    e.la[g] = make_float4(0.f, 0.f, 0.f, 0.f);
    e.lb[g] = e.la[g];
  }
  if (lam) {
#pragma unroll
    for (int g = 0; g < BigEpiIn<C, RB>::NG; g++) {
      const int pr = (C::TJ - 2 * g >= 2 ? 2 : 1) * 4;
      const int cl = (lane % pr) * 8;
      e.la[g] = load_f4(rl, nw + g * 64 + cl);
      e.lb[g] = load_f4(rl, nw + g * 64 + cl + 4);
    }
  }
}

// acc += T L2 (RB > 0), bias, fp16 store: the 128 x 128 epilogue's operations for a TI x TJ block
// of tiles per wave, with L2 and T from e.  eb: epilogue LDS, free.  Ends with the wave's LDS
// work done but no barrier.
template <class C, int RB, bool BIAS>
__device__ __forceinline__ void big_epilogue(v16f (&acc)[C::TJ][C::TI], uint8_t* eb, const BigEpiIn<C, RB>& e,
                                             const float* __restrict__ lam, int M, int N, int m0, int n0,
                                             __half* __restrict__ y) {
  constexpr int R = RB * 16;
  constexpr int LS2 = (R + 8) * 2;           // L2 staged transposed: [n][k], row stride R + 8 halves
  constexpr int L2P = BigEpiIn<C, RB>::L2P;
  constexpr int NG = (C::TJ + 1) / 2;        // output column groups of (up to) two tiles
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, r32 = lane & 31;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int mw = m0 + wm * C::TI * 32, nw = n0 + wn * C::TJ * 32;   // the wave's block
  if (RB > 0) {
#pragma unroll
    for (int j = 0; j < L2P; j++) {
      const int idx = tid + j * C::NTH;
      const int k = idx % R, c8 = idx / R;
      if (idx < R * (C::BN / 8)) {
        const uint32_t w[4] = {e.lv[j].x, e.lv[j].y, e.lv[j].z, e.lv[j].w};
#pragma unroll
        for (int e = 0; e < 8; e++)
          *reinterpret_cast<uint16_t*>(eb + (c8 * 8 + e) * LS2 + k * 2) = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
      }
    }
    lds_barrier();
#pragma unroll
    for (int kb = 0; kb < RB; kb++)
#pragma unroll
      for (int tj = 0; tj < C::TJ; tj++) {
        const uint4 lo =
            *reinterpret_cast<const uint4*>(eb + (wn * C::TJ * 32 + tj * 32 + r32) * LS2 + (kb * 16 + 8 * h) * 2);
#pragma unroll
        for (int ti = 0; ti < C::TI; ti++)
          acc[tj][ti] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(lo), as_h8(e.top[kb][ti]), acc[tj][ti], 0, 0, 0);
      }
    lds_barrier();                           // the output staging reuses the L2 staging bytes
  }
  // columns in groups of two tiles (64 columns; a lone tile last when TJ is odd): each lane
  // stages its 16 values per tile as fp16 row pieces, then the group's rows leave as 16-byte
  // pieces.  Two staging slots per wave, used in turn, so that one wait per block of rows
  // covers both its staging writes and the reads of the slot's previous use.
  static_assert(C::BUF >= 2 * C::NW * 32 * E_YS, "two staging slots per wave");
  // the wave's output rows from mw on: a store at an offset past M - mw rows is dropped
  const rsrc_t ry = make_rsrc(y + (size_t)mw * N, mw < M ? (size_t)(M - mw) * N * 2 : 0);
#pragma unroll
  for (int g = 0; g < NG; g++) {
    const int g0 = 2 * g;
    const int gt = C::TJ - g0 >= 2 ? 2 : 1;   // tiles in the group
    const int pr = gt * 4;                    // 16-byte pieces per staged row
    const int cl = (lane % pr) * 8;           // this lane's 8 columns within the group
    float bv[2][4][4];                        // the bias of the lane's columns, once per group
#pragma unroll
    for (int u = 0; u < 2; u++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const uint2 br = e.braw[u < gt ? g0 + u : g0][q];
        bv[u][q][0] = __half2float(__ushort_as_half((unsigned short)(br.x & 0xFFFFu)));
        bv[u][q][1] = __half2float(__ushort_as_half((unsigned short)(br.x >> 16)));
        bv[u][q][2] = __half2float(__ushort_as_half((unsigned short)(br.y & 0xFFFFu)));
        bv[u][q][3] = __half2float(__ushort_as_half((unsigned short)(br.y >> 16)));
      }
#pragma unroll
    for (int ti = 0; ti < C::TI; ti++) {
      uint8_t* ys = eb + (wave * 2 + ((g * C::TI + ti) & 1)) * 32 * E_YS;
#pragma unroll
      for (int u = 0; u < 2; u++) {
        if (u >= gt) continue;
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const v2f lo = {acc[g0 + u][ti][4 * q] + bv[u][q][0], acc[g0 + u][ti][4 * q + 1] + bv[u][q][1]};
          const v2f hi = {acc[g0 + u][ti][4 * q + 2] + bv[u][q][2], acc[g0 + u][ti][4 * q + 3] + bv[u][q][3]};
          const int nl = u * 32 + 8 * q + 4 * h;
          *reinterpret_cast<uint2*>(ys + r32 * E_YS + nl * 2) =    // two round-to-nearest-even pairs
              make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, v2h)),
                         __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, v2h)));
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's staging writes are done
      __builtin_amdgcn_wave_barrier();
      // the block's rows leave in NP passes of 64 / pr rows: every read first, the glue (one
      // branch) on all of them, then buffer stores that drop what lies past the edge (no branch
      // per store: a branch between a read and its store made each read wait for the last)
      constexpr int NP = 32 * 8 / 64;         // passes (pr pieces per row, 64 lanes)
      static_assert(C::TJ % 2 == 0, "two-tile groups");
      uint2 pa[NP], pb[NP];
#pragma unroll
      for (int it = 0; it < NP; it++) {
        const int rl = it * (64 / pr) + lane / pr;
        pa[it] = *reinterpret_cast<const uint2*>(ys + rl * E_YS + cl * 2);
        pb[it] = *reinterpret_cast<const uint2*>(ys + rl * E_YS + cl * 2 + 8);
      }
      if (lam) {                             // the MLP glue folded in: fp16(gelu(y) / lam)
#pragma unroll
        for (int it = 0; it < NP; it++) {
          uint2& a = pa[it];
          uint2& b = pb[it];
          a.x = gelu_div_h(a.x & 0xFFFFu, e.la[g].x) | (gelu_div_h(a.x >> 16, e.la[g].y) << 16);
          a.y = gelu_div_h(a.y & 0xFFFFu, e.la[g].z) | (gelu_div_h(a.y >> 16, e.la[g].w) << 16);
          b.x = gelu_div_h(b.x & 0xFFFFu, e.lb[g].x) | (gelu_div_h(b.x >> 16, e.lb[g].y) << 16);
          b.y = gelu_div_h(b.y & 0xFFFFu, e.lb[g].z) | (gelu_div_h(b.y >> 16, e.lb[g].w) << 16);
        }
      }
      const int n = nw + g0 * 32 + cl;
#pragma unroll
      for (int it = 0; it < NP; it++) {
        const int rr = ti * 32 + it * (64 / pr) + lane / pr;   // row within the wave's block
        const uint32_t off = n < N ? ((uint32_t)rr * (uint32_t)N + (uint32_t)n) * 2u : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4_t{pa[it].x, pa[it].y, pb[it].x, pb[it].y}, ry, (int)off, 0, 0);
      }
    }
  }
}

}  // namespace

// Four waves per CU, one per SIMD, each owning a 128 x 128 block (4 x 4 tiles of 32 x 32, its
// 256 accumulators in the matrix cores' registers), with the LDS reads one step ahead of the
// MFMAs: while a step's MFMAs run on fragments already in registers, the next step's fragment
// reads and the step's LDS-DMA loads go out one after each MFMA, so the matrix core works while
// the LDS serves the reads.  Per chunk and CU the LDS carries 18 KB of DMA writes and 40 KB of
// fragment and scale reads for 64 tile-MFMAs (eight waves of 64 x 128 would read 60 KB).  Ring of four buffers,
// loads four steps ahead: a buffer is read into registers one step before its MFMAs, so the
// step after that may load it again.  At a tile's end the ring carries on into the next tile:
// the tile's last four steps load the next tile's first three and the last step loads nothing
// and reads nothing; the epilogue works in the last step's buffer, then the next tile's first
// fragments are read and its fourth step loaded into that buffer.
template <class C, int RB, bool BIAS>
__global__ void __launch_bounds__(C::NTH, 1)
k_gemm_mxw(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, const __half* __restrict__ t,
           const uint8_t* __restrict__ wq, const uint8_t* __restrict__ ws, const __half* __restrict__ l2,
           const __half* __restrict__ bias, const float* __restrict__ lam, int M, int N, int K,
           __half* __restrict__ y) {
  using Op = BigOp<C>;
  using Frag = typename Op::Frag;
  constexpr int LPS = C::KC * (Op::PC + Op::PS);   // LDS-DMA instructions per wave and step
  static_assert(2 * LPS < 64, "vmcnt range");
  static_assert(C::BUF >= C::NW * 32 * E_YS && C::BUF >= C::BN * (RB * 16 + 8) * 2, "the epilogue must fit a buffer");
  __shared__ __attribute__((aligned(16))) uint8_t b0[C::BUF];
  __shared__ __attribute__((aligned(16))) uint8_t b1[C::BUF];
  __shared__ __attribute__((aligned(16))) uint8_t b2[C::BUF];
  __shared__ __attribute__((aligned(16))) uint8_t b3[C::BUF];
  Op op(xq, xs, wq, ws, M, N, K);
  const int tiles_m = (M + C::BM - 1) / C::BM, tiles_n = (N + C::BN - 1) / C::BN;
  const int tiles = tiles_m * tiles_n;
  const int NS = op.NS;
  const int NSE = (NS + 3) & ~3;             // steps per tile: a multiple of the ring's four
  auto origin = [&](int tile, int* m0, int* n0) {
    int tm, tn;
    tile_of(tile, tiles, tiles_m, tiles_n, &tm, &tn);
    *m0 = tm * C::BM;
    *n0 = tn * C::BN;
  };
  auto read_step = [&](const uint8_t* b, Frag (&f)[C::KC]) {
#pragma unroll
    for (int k = 0; k < C::KC; k++) {
      op.read(b + k * C::CHUNK, f[k], 0);
      op.read(b + k * C::CHUNK, f[k], 1);
    }
  };

  int tile = blockIdx.x;
  int m0, n0;
  origin(tile, &m0, &n0);
  typename Op::Src cur = op.src(m0, n0);
  op.load(cur, 0, b0);
  op.load(cur, 1, b1);
  op.load(cur, 2, b2);
  op.load(cur, 3, b3);
  Frag fa[C::KC], fb[C::KC];
  wait_barrier<2 * LPS>();                   // steps 0 and 1 are in
  read_step(b0, fa);
  wait_barrier<63>();                        // b0 is read before step 0 loads step 4 into it
  v16f acc[C::TJ][C::TI];
  while (true) {
    const int next = tile + (int)gridDim.x;
    const bool has_next = next < tiles;
    int m1, n1;
    origin(has_next ? next : tile, &m1, &n1);   // without a next tile its loads re-read this one (unused)
    const typename Op::Src nxt = op.src(m1, n1);
#pragma unroll
    for (int a = 0; a < C::TJ; a++)
#pragma unroll
      for (int b = 0; b < C::TI; b++)
#pragma unroll
        for (int i = 0; i < 16; i++) acc[a][b][i] = 0.f;

    // step: the MFMAs on fc; with NEXT, the next step's fragment reads (from nb into fn) and
    // step lst's loads (of ls, into ob) go out one after each MFMA, and the step ends waiting
    // for all but the two most recent steps' loads and synchronising.  Chunks past the end of K
    // (and padding steps) are loaded as zeros and computed like the others: no step branches.
    auto step = [&](auto next_c, const uint8_t* nb, uint8_t* ob, const Frag (&fc)[C::KC], Frag (&fn)[C::KC],
                    const typename Op::Src& ls, int lst) {
      constexpr bool NEXT = decltype(next_c)::value;
#pragma unroll
      for (int k = 0; k < C::KC; k++) {
        op.mma(fc[k], acc, 0);
        if (NEXT) op.read(nb + k * C::CHUNK, fn[k], 0);
        op.mma(fc[k], acc, 1);
        if (NEXT) op.read(nb + k * C::CHUNK, fn[k], 1);
      }
      if constexpr (NEXT) {
        op.load(ls, lst, ob);
        interleave<0, C::KC * C::TI * C::TJ, C::KC * (C::TI + C::TJ + 4), LPS>();
      }
      // the step's MFMAs stay in the step (the compiler would otherwise move the last steps'
      // down to the epilogue, where all their fragments would be live at once)
#pragma unroll
      for (int a = 0; a < C::TJ; a++)
#pragma unroll
        for (int b = 0; b < C::TI; b++) asm volatile("" ::"a"(acc[a][b]));
      if constexpr (NEXT) wait_barrier<2 * LPS>();
    };
    int st = 0;
    do {                                       // NSE >= 8: at least once
      step(IC<1>{}, b1, b0, fa, fb, cur, st + 4);
      step(IC<1>{}, b2, b1, fb, fa, cur, st + 5);
      step(IC<1>{}, b3, b2, fa, fb, cur, st + 6);
      step(IC<1>{}, b0, b3, fb, fa, cur, st + 7);
      st += 4;
    } while (st < NSE - 4);
    step(IC<1>{}, b1, b0, fa, fb, nxt, 0);
    step(IC<1>{}, b2, b1, fb, fa, nxt, 1);
    step(IC<1>{}, b3, b2, fa, fb, nxt, 2);
    BigEpiIn<C, RB> ein;
    constexpr bool EARLY = RB <= 2;            // above rank 32 the registers would spill
    if (EARLY) big_epi_load<C, RB>(ein, t, l2, M, N, m0, n0);   // in flight during the last step's MFMAs
    step(IC<0>{}, b0, b3, fb, fa, nxt, 3);
    // b3 was read by the previous step (all waves: its barrier); the next tile's second step
    // must be in before the barrier below
    __builtin_amdgcn_s_waitcnt((LPS & 15) | (7 << 4) | ((LPS >> 4) << 14));   // vmcnt(LPS)
    if (!EARLY) big_epi_load<C, RB>(ein, t, l2, M, N, m0, n0);
    big_epi_load_bias<C, RB, BIAS>(ein, bias, lam, N, n0);
    big_epilogue<C, RB, BIAS>(acc, b3, ein, lam, M, N, m0, n0, y);
    if (!has_next) break;
    read_step(b0, fa);                        // the next tile's first step
    wait_barrier<63>();                       // the epilogue is done with b3, and b0 is read
    op.load(nxt, 3, b3);
    tile = next;
    m0 = m1;
    n0 = n1;
    cur = nxt;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no LDS-DMA in flight when the workgroup ends
}

// 256 x 256 tiles: four waves of 128 x 128, two chunks a step
using BigW = Big<2, 2, 4, 4, 2>;

template <class C, int RB, bool BIAS>
static hipError_t launch_mxw_t(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.M + C::BM - 1) / C::BM) * ((a.N + C::BN - 1) / C::BN);
  const int cus = resident_workgroups() / 2;
  const int nb = tiles < cus ? tiles : cus;
  hipLaunchKernelGGL((k_gemm_mxw<C, RB, BIAS>), dim3(nb), dim3(C::NTH), 0, s, (const uint8_t*)a.xq,
                     (const uint8_t*)a.xs, (const __half*)a.t, (const uint8_t*)a.wq, (const uint8_t*)a.ws,
                     (const __half*)a.l2, (const __half*)a.bias, a.lam, a.M, a.N, a.K, (__half*)a.y);
  return hipGetLastError();
}

template <class C, bool BIAS>
static hipError_t launch_mxw_r(const GemmArgs& a, hipStream_t s) {
  switch (a.r) {
    case 0: return launch_mxw_t<C, 0, BIAS>(a, s);
    case 16: return launch_mxw_t<C, 1, BIAS>(a, s);
    case 32: return launch_mxw_t<C, 2, BIAS>(a, s);
    case 48: return launch_mxw_t<C, 3, BIAS>(a, s);
    case 64: return launch_mxw_t<C, 4, BIAS>(a, s);
  }
  return hipErrorInvalidValue;
}

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

// Rounds of the 128 x 128 kernel: full rounds of its persistent loop, and a last partial round
// whole, or, when it is at most a quarter of a round, as sub-tile jobs (about a quarter of a
// round per job and workgroup).
static double rounds_128(int M, int N, int slots) {
  const long tiles = (long)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (tiles <= slots) return 1.0;
  const long full = tiles / slots, rem = tiles % slots;
  if (rem == 0) return (double)full;
  if (4 * rem <= slots) return (double)full + 0.25 * (double)((16 * rem + slots - 1) / slots);
  return (double)(full + 1);
}

// The 256 x 256 kernel's time in rounds of the 128 x 128 kernel: 1.40 of them per round of large
// tiles with every CU busy, a last partial round 0.6 + 0.4 x its share of busy CUs (with fewer
// CUs at work the chip holds a higher clock), and 0.35 for the start.  Fitted on M = 256 ... 4608
// at K = 3072 (N = 12288, 9216, 4096) and on K = 12288; it picks the faster kernel at every
// measured shape but M = 768 (K = 3072), where the two estimates tie.
static double rounds_big(long tiles, int cus) {
  const long full = tiles / cus, rem = tiles % cus;
  const double u = (double)full + (rem ? 0.6 + 0.4 * (double)rem / (double)cus : 0.0);
  return 0.35 + 1.40 * u;
}

// 256 x 256 tiles where they cost less than the 128 x 128 kernel's (large M and N; at few token
// rows most of a 256-row tile would be padding), for K >= 1024 (the ring's eight steps).
hipError_t launch_gemm_mx(const GemmArgs& a, hipStream_t s) {
  const int slots = resident_workgroups(), cus = slots / 2;
  const long big_tiles = (long)((a.M + BigW::BM - 1) / BigW::BM) * ((a.N + BigW::BN - 1) / BigW::BN);
  if (a.K >= 1024 && rounds_big(big_tiles, cus) < rounds_128(a.M, a.N, slots))
    return a.bias ? launch_mxw_r<BigW, true>(a, s) : launch_mxw_r<BigW, false>(a, s);
  return a.bias ? launch_mx_r<true>(a, s) : launch_mx_r<false>(a, s);
}

}  // namespace svdq
