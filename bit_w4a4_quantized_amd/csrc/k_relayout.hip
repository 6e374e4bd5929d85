// Codes and scales between the exchange layout and the layouts Kernel A writes and Kernel B
// reads.
//
// Exchange (canonical) layout, the one the bit-exact comparisons are stated in: row-major,
// one row per token (activations) or per output column (weights), K contiguous:
//   codes  [rows, K/2] two 4-bit codes a byte (code 2b in the low nibble), or [rows, K] for
//          INT8; the 6-bit container's INT4 codes are exchanged as INT4 nibbles;
//   scales [rows, K/G]: fp16 (INT formats), E4M3 bytes (FP4, G = 16), E8M0 bytes (MXFP4, G = 32).
// Device layouts: every format is chunk-major, the rows of one 64-wide chunk of K contiguous
// ([K/64][rows][bytes per chunk], scales [K/64][rows][scale bytes per chunk]), with the INT4
// codes of the 6-bit container held as E2M3
// fields (sign << 5 | |q|, 24 bytes per half-group, stored as half 0 bytes 0..15, half 1 bytes
// 0..15, half 0 bytes 16..23, half 1 bytes 16..23).
//
// One thread per (row, 64-wide chunk); consecutive threads take consecutive chunks of a row, so
// the exchange side is read or written contiguously.  Offline / exchange work, not on the
// layer's path.
#include "kernels.h"

namespace svdq {

namespace {

template <int FMT>
__host__ __device__ constexpr int dev_chunk_bytes() {
  return FMT == FMT_INT4_E2M3 ? 48 : (FMT == FMT_INT8 ? 64 : 32);
}
template <int FMT>
__host__ __device__ constexpr int canon_chunk_bytes() {
  return FMT == FMT_INT8 ? 64 : 32;
}
template <int FMT>
__host__ __device__ constexpr int scale_chunk_bytes() {   // scale bytes per row and 64-wide chunk
  return FMT == FMT_FP4 ? 4 : 2;                          // 4 E4M3 | 2 E8M0 | one fp16
}

// 32 INT4 codes (two's-complement nibbles, 16 bytes) <-> one half-group of E2M3 fields
// (24 bytes, field j at bits [6j, 6j + 6) little-endian)
__device__ __forceinline__ void nibbles_to_fields(const uint8_t* nib, uint8_t* f24) {
  uint64_t w[3] = {0, 0, 0};
#pragma unroll
  for (int j = 0; j < 32; j++) {
    const int n = (nib[j >> 1] >> (4 * (j & 1))) & 0xF;
    const int q = n >= 8 ? n - 16 : n;
    const uint64_t field = (uint64_t)((q < 0 ? 32 : 0) | (q < 0 ? -q : q));
    const int bit = 6 * j;
    w[bit >> 6] |= field << (bit & 63);
    if ((bit & 63) > 58) w[(bit >> 6) + 1] |= field >> (64 - (bit & 63));
  }
#pragma unroll
  for (int b = 0; b < 24; b++) f24[b] = (uint8_t)(w[b >> 3] >> (8 * (b & 7)));
}

__device__ __forceinline__ void fields_to_nibbles(const uint8_t* f24, uint8_t* nib) {
  uint64_t w[3] = {0, 0, 0};
#pragma unroll
  for (int b = 0; b < 24; b++) w[b >> 3] |= (uint64_t)f24[b] << (8 * (b & 7));
#pragma unroll
  for (int j = 0; j < 16; j++) nib[j] = 0;
#pragma unroll
  for (int j = 0; j < 32; j++) {
    const int bit = 6 * j;
    uint64_t v = w[bit >> 6] >> (bit & 63);
    if ((bit & 63) > 58) v |= w[(bit >> 6) + 1] << (64 - (bit & 63));
    const int field = (int)(v & 63);
    const int mag = field & 7;
    const int q = (field & 32) ? -mag : mag;
    nib[j >> 1] |= (uint8_t)((q & 0xF) << (4 * (j & 1)));
  }
}

template <int FMT, bool TO_CANON>
__global__ void __launch_bounds__(256)
k_relayout(const uint8_t* __restrict__ ci, const uint8_t* __restrict__ si, int rows, int K,
           uint8_t* __restrict__ co, uint8_t* __restrict__ so) {
  constexpr int CBD = dev_chunk_bytes<FMT>(), CBC = canon_chunk_bytes<FMT>(), SB = scale_chunk_bytes<FMT>();
  const int nch = K >> 6;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)rows * nch) return;
  const int row = (int)(idx / nch), c = (int)(idx % nch);
  const size_t dcode = ((size_t)c * rows + row) * CBD;
  const size_t ccode = (size_t)row * nch * CBC + (size_t)c * CBC;
  const size_t dscale = ((size_t)c * rows + row) * SB;
  const size_t cscale = ((size_t)row * nch + c) * SB;
  const uint8_t* src = ci + (TO_CANON ? dcode : ccode);
  uint8_t* dst = co + (TO_CANON ? ccode : dcode);
  uint8_t buf[64];
  if constexpr (FMT == FMT_INT4_E2M3) {
    if (TO_CANON) {
      uint8_t h[2][24];
#pragma unroll
      for (int b = 0; b < 16; b++) { h[0][b] = src[b]; h[1][b] = src[16 + b]; }
#pragma unroll
      for (int b = 0; b < 8; b++) { h[0][16 + b] = src[32 + b]; h[1][16 + b] = src[40 + b]; }
      fields_to_nibbles(h[0], buf);
      fields_to_nibbles(h[1], buf + 16);
#pragma unroll
      for (int p = 0; p < 2; p++) reinterpret_cast<uint4*>(dst)[p] = reinterpret_cast<const uint4*>(buf)[p];
    } else {
      uint8_t nib[32], h[2][24];
#pragma unroll
      for (int p = 0; p < 2; p++) reinterpret_cast<uint4*>(nib)[p] = reinterpret_cast<const uint4*>(src)[p];
      nibbles_to_fields(nib, h[0]);
      nibbles_to_fields(nib + 16, h[1]);
#pragma unroll
      for (int b = 0; b < 16; b++) { buf[b] = h[0][b]; buf[16 + b] = h[1][b]; }
#pragma unroll
      for (int b = 0; b < 8; b++) { buf[32 + b] = h[0][16 + b]; buf[40 + b] = h[1][16 + b]; }
#pragma unroll
      for (int p = 0; p < 3; p++) reinterpret_cast<uint4*>(dst)[p] = reinterpret_cast<const uint4*>(buf)[p];
    }
  } else {
#pragma unroll
    for (int p = 0; p < CBC / 16; p++) reinterpret_cast<uint4*>(dst)[p] = reinterpret_cast<const uint4*>(src)[p];
  }
  const uint8_t* ssrc = si + (TO_CANON ? dscale : cscale);
  uint8_t* sdst = so + (TO_CANON ? cscale : dscale);
#pragma unroll
  for (int b = 0; b < SB; b++) sdst[b] = ssrc[b];
}

template <int FMT>
hipError_t launch_rl(const void* ci, const void* si, int rows, int K, bool to_canon, void* co, void* so,
                     hipStream_t s) {
  const size_t n = (size_t)rows * (K >> 6);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (to_canon)
    hipLaunchKernelGGL((k_relayout<FMT, true>), grid, dim3(256), 0, s, (const uint8_t*)ci, (const uint8_t*)si, rows,
                       K, (uint8_t*)co, (uint8_t*)so);
  else
    hipLaunchKernelGGL((k_relayout<FMT, false>), grid, dim3(256), 0, s, (const uint8_t*)ci, (const uint8_t*)si, rows,
                       K, (uint8_t*)co, (uint8_t*)so);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_relayout(const void* codes_in, const void* scales_in, int rows, int K, int fmt, bool to_canonical,
                           void* codes_out, void* scales_out, hipStream_t s) {
  switch (fmt) {
    case FMT_INT4: return launch_rl<FMT_INT4>(codes_in, scales_in, rows, K, to_canonical, codes_out, scales_out, s);
    case FMT_INT8: return launch_rl<FMT_INT8>(codes_in, scales_in, rows, K, to_canonical, codes_out, scales_out, s);
    case FMT_FP4: return launch_rl<FMT_FP4>(codes_in, scales_in, rows, K, to_canonical, codes_out, scales_out, s);
    case FMT_INT4_E2M3:
      return launch_rl<FMT_INT4_E2M3>(codes_in, scales_in, rows, K, to_canonical, codes_out, scales_out, s);
    case FMT_MXFP4: return launch_rl<FMT_MXFP4>(codes_in, scales_in, rows, K, to_canonical, codes_out, scales_out, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace svdq
