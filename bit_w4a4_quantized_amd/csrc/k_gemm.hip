// Kernel B dispatch: the low-bit GEMM with the up projection and the bias in the
// epilogue, one kernel family per code format.
//
//   Y[m,n] = fp16_rne( sum_g sx[m,g] sw[n,g] P_g[m,n] + (T L2)[m,n] + b[n] )
//
//   SVDQ_INT4_G64_E2M3 : FP6 matrix cores on the 6-bit container (k_gemm3.hip)
//   SVDQ_INT4_G64      : packed nibbles widened to int8 on the INT8 matrix cores
//                        (k_gemm2.hip)
//   SVDQ_INT8_G64      : INT8 matrix cores (k_gemm_i8.hip)
//   SVDQ_FP4_G16       : exact fp16 dequantization on the fp16 matrix cores
//                        (k_gemm_f4.hip)
#include "kernels.h"

namespace svdq {

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  switch (a.fmt) {
    case FMT_INT4: return launch_gemm2(a, s);
    case FMT_INT4_E2M3: return launch_gemm3(a, s);
    case FMT_INT8: return launch_gemm_i8(a, s);
    case FMT_FP4: return launch_gemm_f4(a, s);
    case FMT_MXFP4: return launch_gemm_mx(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace svdq
