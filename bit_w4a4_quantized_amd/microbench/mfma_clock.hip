// Microbenchmark: the sustained rate of each matrix-core instruction the kernels use, and the
// shader clock the chip holds while it runs.  Every case runs on all compute units, two
// workgroups of four waves per CU (two waves per SIMD), registers only: 8 independent
// accumulators per wave, all MFMA operands changing every iteration.  A series is 40 launches of
// ~2 ms back to back; the table gives ns per instruction per SIMD for the first and the last
// launches, and the clock measured inside the first and the last launch (shader cycles from
// s_memtime against the 100 MHz s_memrealtime counter, by one wave).
//
// Build and run (gfx950):
//   python -m bit_w4a4_quantized_amd.build --microbench && bit_w4a4_quantized_amd/_build/mfma_clock
#include <hip/hip_runtime.h>

#include <cstdio>
#include <vector>

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

constexpr int NT = 256;
constexpr int T = 8;

enum Case {
  FP4_FIXED,     // v_mfma_scale_f32_32x32x64_f8f6f4, FP4 operands, fixed scales
  FP4_SCALED,    // the same, scales changing per lane and iteration (MXFP4's Kernel B)
  FP6,           // the same instruction on FP6 operands (the 6-bit container's Kernel B)
  I8,            // v_mfma_i32_32x32x32_i8 (packed INT4 and INT8 Kernel B)
  F16,           // v_mfma_f32_32x32x16_f16 (the W4A16 control)
};

__device__ __forceinline__ int bits(unsigned s, int i) {
  return (int)((s * 0x9E3779B1u + (unsigned)i * 0x85EBCA6Bu) & 0x37373737u);
}

template <Case C>
__global__ void __launch_bounds__(NT, 2) probe(float* out, unsigned long long* clk, int iters) {
  const unsigned tid = threadIdx.x + blockIdx.x * NT;
  v8i a[T], b[T];
  v16f acc[T];
  v16i iacc[T];
#pragma unroll
  for (int t = 0; t < T; t++) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      a[t][i] = bits(tid, t * 8 + i);
      b[t][i] = bits(tid * 3u + 1u, t * 8 + i);
    }
#pragma unroll
    for (int i = 0; i < 16; i++) {
      acc[t][i] = 0.f;
      iacc[t][i] = 0;
    }
  }
  const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int t = 0; t < T; t++) {
      a[t][0] ^= it;                         // no instruction is loop-invariant
      if constexpr (C == FP4_FIXED || C == FP4_SCALED) {
        const int sa = C == FP4_SCALED ? 120 + ((it + (int)threadIdx.x) & 7) : 127;
        const int sb = C == FP4_SCALED ? 121 + ((it ^ (int)threadIdx.x) & 7) : 127;
        const v8i a4 = v8i{a[t][0], a[t][1], a[t][2], a[t][3], 0, 0, 0, 0};
        const v8i b4 = v8i{b[t][0], b[t][1], b[t][2], b[t][3], 0, 0, 0, 0};
        acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a4, b4, acc[t], 4, 4, 0, sa, 0, sb);
      } else if constexpr (C == FP6) {
        const v8i a6 = v8i{a[t][0], a[t][1], a[t][2], a[t][3], a[t][4], a[t][5], 0, 0};
        const v8i b6 = v8i{b[t][0], b[t][1], b[t][2], b[t][3], b[t][4], b[t][5], 0, 0};
        acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a6, b6, acc[t], 2, 2, 0, 132, 0, 127);
      } else if constexpr (C == I8) {
        const v4i a8 = v4i{a[t][0], a[t][1], a[t][2], a[t][3]};
        const v4i b8 = v4i{b[t][0], b[t][1], b[t][2], b[t][3]};
        iacc[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a8, b8, iacc[t], 0, 0, 0);
      } else {
        const v8h ah = __builtin_bit_cast(v8h, v4i{a[t][0], a[t][1], a[t][2], a[t][3]});
        const v8h bh = __builtin_bit_cast(v8h, v4i{b[t][0], b[t][1], b[t][2], b[t][3]});
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, acc[t], 0, 0, 0);
      }
    }
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float r = 0.f;
#pragma unroll
  for (int t = 0; t < T; t++)
#pragma unroll
    for (int i = 0; i < 16; i++) r += acc[t][i] + (float)iacc[t][i];
  out[tid] = r;
  if (tid == 0) {
    clk[0] = c1 - c0;
    clk[1] = r1 - r0;
  }
}

template <Case C>
void series(const char* name, float* out, unsigned long long* clk, int grid, int iters) {
  hipEvent_t e0, e1;
  (void)hipEventCreate(&e0);
  (void)hipEventCreate(&e1);
  std::vector<float> ns;
  std::vector<double> ghz;
  for (int rep = 0; rep < 40; rep++) {
    (void)hipEventRecord(e0);
    hipLaunchKernelGGL(probe<C>, dim3(grid), dim3(NT), 0, 0, out, clk, iters);
    (void)hipEventRecord(e1);
    (void)hipEventSynchronize(e1);
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, e0, e1);
    unsigned long long h[2] = {0, 0};
    (void)hipMemcpy(h, clk, sizeof(h), hipMemcpyDeviceToHost);
    ns.push_back(ms * 1e6f / (2.0f * iters * T));
    ghz.push_back(h[1] ? (double)h[0] / ((double)h[1] / 100e6) / 1e9 : 0.0);
  }
  std::printf("%-34s %7.2f %7.2f %7.2f  %7.2f %7.2f %7.2f   %5.2f  %5.2f\n", name, ns[0], ns[1], ns[2], ns[37], ns[38],
              ns[39], ghz[0], ghz[39]);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
}

int main() {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0) != hipSuccess || cus <= 0) return 2;
  const int grid = 2 * cus;
  float* out = nullptr;
  unsigned long long* clk = nullptr;
  if (hipMalloc(&out, (size_t)grid * NT * sizeof(float)) != hipSuccess) return 2;
  if (hipMalloc(&clk, 2 * sizeof(unsigned long long)) != hipSuccess) return 2;
  const int iters = 4000;
  std::printf("compute units %d; ns per instruction per SIMD (first three, last three of 40 launches); "
              "shader clock GHz (first, last launch)\n", cus);
  series<FP4_FIXED>("FP4 32x32x64, fixed scales", out, clk, grid, iters);
  series<FP4_SCALED>("FP4 32x32x64, changing scales", out, clk, grid, iters);
  series<FP6>("FP6 32x32x64", out, clk, grid, iters);
  series<I8>("INT8 32x32x32", out, clk, grid, iters);
  series<F16>("fp16 32x32x16", out, clk, grid, iters);
  const hipError_t e = hipGetLastError();
  std::printf("status: %s\n", hipGetErrorString(e));
  return e == hipSuccess ? 0 : 1;
}
