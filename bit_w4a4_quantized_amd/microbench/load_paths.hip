// Microbenchmark of the three ways a GEMM operand reaches the matrix cores on gfx950, per CU:
//   1. global memory -> registers (buffer/global load, 16 bytes per lane);
//   2. global memory -> LDS by the LDS-DMA form of the buffer load (16 bytes per lane);
//   3. LDS -> registers (ds_read_b128).
// The global source is a 2 MiB buffer, resident in every XCD's L2, read with the 1 KB-per-wave
// contiguous pattern of a tile's operand rows.  Two workgroups of four waves per CU (Kernel B's
// occupancy), each wave keeping four loads in flight per iteration.  Every address is masked
// into its buffer (power-of-two sizes) and every loop is bounded.  Prints bytes per clock per CU
// at the 2.4 GHz peak clock.
//
// Build and run (gfx950):
//   python -m bit_w4a4_quantized_amd.build --microbench && bit_w4a4_quantized_amd/_build/load_paths
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>

constexpr int NT = 256;
constexpr int ITERS = 2048;
constexpr int LDS_BYTES = 32768;

typedef __attribute__((address_space(3))) void lds_void;

enum Path { GLOBAL_TO_REGS, GLOBAL_TO_LDS, LDS_TO_REGS };

template <int P>
__global__ void __launch_bounds__(NT, 2) probe(const uint4* __restrict__ buf, unsigned mask16, uint4* out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint4 acc = make_uint4(0, 0, 0, 0);
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(buf), (short)0, (int)((mask16 + 1) * 16), 0x00020000);
  const unsigned base = (blockIdx.x * 4 + wave) * 64 * 8;
  for (int i = 0; i < ITERS; i++) {
    if constexpr (P == GLOBAL_TO_REGS) {
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const unsigned idx = (base + (unsigned)(i * 4 + k) * 64 * 37 + lane) & mask16;
        const uint4 v = buf[idx];
        acc.x ^= v.x; acc.y ^= v.y; acc.z ^= v.z; acc.w ^= v.w;
      }
    } else if constexpr (P == GLOBAL_TO_LDS) {
      // lane l's 16 bytes land at the wave's destination + 16 l; one wait per iteration
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const unsigned idx = (base + (unsigned)(i * 4 + k) * 64 * 37) & mask16 & ~63u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds + wave * 8192 + k * 1024), 16, (int)(lane * 16),
                                                 (int)(idx * 16), 0, 0);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const int o = (wave * 8192 + k * 1024 + lane * 16 + i * 16) & (LDS_BYTES - 1) & ~15;
        const uint4 v = *reinterpret_cast<const uint4*>(lds + o);
        acc.x ^= v.x; acc.y ^= v.y; acc.z ^= v.z; acc.w ^= v.w;
      }
    }
  }
  if (P == GLOBAL_TO_LDS) acc.x ^= lds[threadIdx.x * 16];
  out[blockIdx.x * NT + threadIdx.x] = acc;
}

// ms per launch, best of 5 timed launches (after one untimed)
template <int P>
float run(const uint4* buf, unsigned mask16, uint4* out, int grid) {
  hipEvent_t e0, e1;
  (void)hipEventCreate(&e0);
  (void)hipEventCreate(&e1);
  float best = 1e30f;
  for (int rep = 0; rep < 6; rep++) {
    (void)hipEventRecord(e0);
    hipLaunchKernelGGL(probe<P>, dim3(grid), dim3(NT), 0, 0, buf, mask16, out);
    (void)hipEventRecord(e1);
    (void)hipEventSynchronize(e1);
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, e0, e1);
    if (rep > 0) best = std::min(best, ms);
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return best;
}

int main() {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0) != hipSuccess || cus <= 0) return 2;
  const unsigned bytes = 2u << 20;
  uint4* buf = nullptr;
  uint4* out = nullptr;
  if (hipMalloc(&buf, bytes) != hipSuccess || hipMemset(buf, 1, bytes) != hipSuccess) return 2;
  const int grid = 2 * cus;
  if (hipMalloc(&out, (size_t)grid * NT * sizeof(uint4)) != hipSuccess) return 2;
  const unsigned mask16 = bytes / 16 - 1;
  const double moved = (double)grid * NT * ITERS * 4 * 16;   // bytes per launch
  const char* names[3] = {"global -> registers (16 B per lane)", "global -> LDS (LDS-DMA, 16 B per lane)",
                          "LDS -> registers (ds_read_b128)"};
  const float ms[3] = {run<GLOBAL_TO_REGS>(buf, mask16, out, grid), run<GLOBAL_TO_LDS>(buf, mask16, out, grid),
                       run<LDS_TO_REGS>(buf, mask16, out, grid)};
  std::printf("compute units %d, 2 workgroups of 4 waves per CU\n", cus);
  for (int p = 0; p < 3; p++) {
    const double bps = moved / (ms[p] * 1e-3);
    std::printf("%-40s %8.3f ms %9.1f GB/s %7.1f B/clk/CU at 2.4 GHz\n", names[p], ms[p], bps / 1e9,
                bps / cus / 2.4e9);
  }
  const hipError_t e = hipGetLastError();
  std::printf("status: %s\n", hipGetErrorString(e));
  (void)hipFree(buf);
  (void)hipFree(out);
  return e == hipSuccess ? 0 : 1;
}
