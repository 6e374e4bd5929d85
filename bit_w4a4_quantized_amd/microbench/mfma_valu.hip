// Microbenchmark behind Kernel B's floor: per 32 x 32 tile and 64-wide group, Kernel B issues
// one FP6 block-scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, the exact partial product P_g),
// one fp16 MFMA for the scale products (v_mfma_f32_32x32x8_f16) and 16 vector fmas (the
// rescale acc += P_g S).  This program measures, per SIMD, how long each part takes alone and
// how much of the vector work the matrix core hides when both run.
//
// Every case runs on all compute units, two workgroups of four waves per CU (two waves per
// SIMD, as Kernel B), registers only: 3 independent tiles per wave, ITERS iterations.  All
// MFMA operands differ per tile and change every iteration, so the compiler can merge or hoist
// nothing; each thread stores one value at the end (out has one float per thread).
//
// The AGPR case puts P and S in AGPRs (the form the compiler picks once a kernel uses AGPRs):
// the vector ALU cannot read AGPRs, so each result comes back with v_accvgpr_read first.
//
// Build and run (gfx950):
//   python -m bit_w4a4_quantized_amd.build --microbench && bit_w4a4_quantized_amd/_build/mfma_valu
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

constexpr int NT = 256;
constexpr int ITERS = 512;
constexpr int TILES = 3;

enum Case {
  FP6_ONLY,          // the FP6 MFMA, accumulating chains
  SCALE_ONLY,        // the scale-product MFMA, accumulating chains
  MFMA_PAIR,         // both MFMAs of a tile-group, accumulating chains
  FMA_ONLY,          // 16 independent fma chains per tile
  PAIR_AND_FMA,      // MFMA_PAIR and FMA_ONLY in one loop, independent of each other
  PAIR_AND_ADD,      // MFMA_PAIR and 16 two-operand adds per tile
  KERNEL_B_PATTERN,  // P = FP6 MFMA, S = scale MFMA (C = 0), acc += P S: Kernel B's dependency
  KERNEL_B_AGPR,     // KERNEL_B_PATTERN with P and S in AGPRs (the fmas read them back: v_accvgpr_read)
};

__device__ __forceinline__ v8i codes(unsigned s) {   // six dwords of 6-bit fields (any pattern is an FP6 value)
  v8i v;
#pragma unroll
  for (int i = 0; i < 6; i++) v[i] = (int)((s * 0x9E3779B1u + (unsigned)i * 0x85EBCA6Bu) & 0x3F3F3F3Fu);
  v[6] = 0;
  v[7] = 0;
  return v;
}

template <Case C>
__global__ void __launch_bounds__(NT, 2) probe(float* out, float fa, float fb) {
  // an AGPR clobber makes the compiler allocate AGPRs, and MFMA results then go there
  if constexpr (C == KERNEL_B_AGPR) asm volatile("" ::: "a0");
  const unsigned tid = threadIdx.x + blockIdx.x * NT;
  v8i a[TILES], b[TILES];
  v4h sa[TILES], sb[TILES];
#pragma unroll
  for (int t = 0; t < TILES; t++) {
    a[t] = codes(tid * 7u + t);
    b[t] = codes(tid * 13u + 3u * t);
    sa[t] = v4h{(_Float16)(0.5f + 0.01f * (float)((tid + t) & 15)), (_Float16)0, (_Float16)0, (_Float16)0};
    sb[t] = v4h{(_Float16)(0.25f + 0.02f * (float)((tid * 3 + t) & 15)), (_Float16)0, (_Float16)0, (_Float16)0};
  }
  v16f acc[TILES], acc2[TILES];
  float v[TILES][16];
#pragma unroll
  for (int t = 0; t < TILES; t++)
#pragma unroll
    for (int i = 0; i < 16; i++) {
      acc[t][i] = 0.f;
      acc2[t][i] = 0.f;
      v[t][i] = 1e-3f * (float)(i + t);
    }
  for (int it = 0; it < ITERS; it++) {
#pragma unroll
    for (int t = 0; t < TILES; t++) {
      // operands change every iteration (an xor of the iteration into one code dword and a
      // bit of the scale), so no MFMA is loop-invariant
      a[t][0] ^= it;
      sa[t][1] = (_Float16)(float)(it & 1);
      constexpr bool PAIR = C == MFMA_PAIR || C == PAIR_AND_FMA || C == PAIR_AND_ADD;
      if constexpr (C == FP6_ONLY || PAIR)
        acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[t], b[t], acc[t], 2, 2, 0, 132, 0, 127);
      if constexpr (C == SCALE_ONLY || PAIR)
        acc2[t] = __builtin_amdgcn_mfma_f32_32x32x8f16(sa[t], sb[t], acc2[t], 0, 0, 0);
      if constexpr (C == FMA_ONLY || C == PAIR_AND_FMA) {
#pragma unroll
        for (int i = 0; i < 16; i++) v[t][i] = __builtin_fmaf(v[t][i], fa, fb);
      }
      if constexpr (C == PAIR_AND_ADD) {
#pragma unroll
        for (int i = 0; i < 16; i++) v[t][i] = v[t][i] + fb;
      }
      if constexpr (C == KERNEL_B_PATTERN || C == KERNEL_B_AGPR) {
        const v16f p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[t], b[t], v16f{}, 2, 2, 0, 132, 0, 127);
        const v16f s = __builtin_amdgcn_mfma_f32_32x32x8f16(sa[t], sb[t], v16f{}, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 16; i++) acc[t][i] = __builtin_fmaf(p[i], s[i], acc[t][i]);
      }
    }
  }
  float r = 0.f;
#pragma unroll
  for (int t = 0; t < TILES; t++)
#pragma unroll
    for (int i = 0; i < 16; i++) r += acc[t][i] + acc2[t][i] + v[t][i];
  out[tid] = r;
}

// ns per tile-group per SIMD, best of 5 timed launches (after one untimed)
template <Case C>
float run(float* out, int grid, float waves_per_simd) {
  hipEvent_t e0, e1;
  (void)hipEventCreate(&e0);
  (void)hipEventCreate(&e1);
  float best = 1e30f;
  for (int rep = 0; rep < 6; rep++) {
    (void)hipEventRecord(e0);
    hipLaunchKernelGGL(probe<C>, dim3(grid), dim3(NT), 0, 0, out, 0.999f, 1e-4f);
    (void)hipEventRecord(e1);
    (void)hipEventSynchronize(e1);
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, e0, e1);
    if (rep > 0) best = std::min(best, ms);
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return best * 1e6f / (waves_per_simd * ITERS * TILES);
}

int main() {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0) != hipSuccess || cus <= 0) return 2;
  const int grid2 = 2 * cus, grid1 = cus;
  float* out = nullptr;
  if (hipMalloc(&out, (size_t)grid2 * NT * sizeof(float)) != hipSuccess) return 2;
  for (int i = 0; i < 20; i++) hipLaunchKernelGGL(probe<KERNEL_B_PATTERN>, dim3(grid2), dim3(NT), 0, 0, out, 0.999f, 1e-4f);
  (void)hipDeviceSynchronize();
  std::printf("compute units %d; ns per 32x32 tile-group per SIMD\n", cus);
  std::printf("%-44s %8s %8s\n", "case", "2 waves", "1 wave");
  std::printf("%-44s %8.2f %8.2f\n", "FP6 MFMA only", run<FP6_ONLY>(out, grid2, 2), run<FP6_ONLY>(out, grid1, 1));
  std::printf("%-44s %8.2f %8.2f\n", "scale MFMA only", run<SCALE_ONLY>(out, grid2, 2), run<SCALE_ONLY>(out, grid1, 1));
  std::printf("%-44s %8.2f %8.2f\n", "both MFMAs", run<MFMA_PAIR>(out, grid2, 2), run<MFMA_PAIR>(out, grid1, 1));
  std::printf("%-44s %8.2f %8.2f\n", "16 fmas", run<FMA_ONLY>(out, grid2, 2), run<FMA_ONLY>(out, grid1, 1));
  std::printf("%-44s %8.2f %8.2f\n", "both MFMAs + 16 fmas, independent", run<PAIR_AND_FMA>(out, grid2, 2),
              run<PAIR_AND_FMA>(out, grid1, 1));
  std::printf("%-44s %8.2f %8.2f\n", "both MFMAs + 16 adds, independent", run<PAIR_AND_ADD>(out, grid2, 2),
              run<PAIR_AND_ADD>(out, grid1, 1));
  std::printf("%-44s %8.2f %8.2f\n", "Kernel B pattern (P, S, acc += P S)", run<KERNEL_B_PATTERN>(out, grid2, 2),
              run<KERNEL_B_PATTERN>(out, grid1, 1));
  std::printf("%-44s %8.2f %8.2f\n", "Kernel B pattern, P and S in AGPRs", run<KERNEL_B_AGPR>(out, grid2, 2),
              run<KERNEL_B_AGPR>(out, grid1, 1));
  const hipError_t e = hipGetLastError();
  std::printf("status: %s\n", hipGetErrorString(e));
  (void)hipFree(out);
  return e == hipSuccess ? 0 : 1;
}
