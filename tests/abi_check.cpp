// Host-side argument validation of the C ABI (include/svdq.h), exercised without a GPU in a
// build of the library's host code with AddressSanitizer and UndefinedBehaviorSanitizer.
// Every call below must return before any HIP call: error statuses, empty shapes, size
// queries.  Pointers are fake, 16-byte aligned values that are never dereferenced.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "../include/svdq.h"

namespace {

int failures = 0;

void expect(const char* what, int got, int want) {
  if (got != want) {
    std::printf("FAIL %s: status %d, expected %d\n", what, got, want);
    failures++;
  }
}

void expect_size(const char* what, size_t got, size_t want) {
  if (got != want) {
    std::printf("FAIL %s: %zu, expected %zu\n", what, got, want);
    failures++;
  }
}

void* const P = reinterpret_cast<void*>(4096);      // aligned fake device pointer
void* const MIS = reinterpret_cast<void*>(4100);    // misaligned
const float* const PF = reinterpret_cast<const float*>(4096);
const float* const MISF = reinterpret_cast<const float*>(4100);
const svdq_format F4 = SVDQ_INT4_G64, F6 = SVDQ_INT4_G64_E2M3, BAD = static_cast<svdq_format>(9);

}  // namespace

int main() {
  // sizes
  expect_size("code bytes int4", svdq_code_row_bytes(3072, F4), 1536);
  expect_size("code bytes e2m3", svdq_code_row_bytes(3072, F6), 2304);
  expect_size("code bytes bad K", svdq_code_row_bytes(100, F4), 0);
  expect_size("code bytes bad fmt", svdq_code_row_bytes(64, BAD), 0);
  expect_size("scale bytes fp4", svdq_scale_row_bytes(3072, SVDQ_FP4_G16), 192);
  expect_size("scale bytes mxfp4", svdq_scale_row_bytes(3072, SVDQ_MXFP4_G32), 96);
  expect_size("linear workspace bad K", svdq_linear_workspace_bytes(16, 100, 16, F4), 0);
  expect_size("quantize_down workspace r=0", svdq_quantize_down_workspace_bytes(4608, 3072, 0, F4), 0);
  const size_t need = svdq_linear_workspace_bytes(16, 64, 16, F4);
  if (need == 0) { std::printf("FAIL linear workspace size 0\n"); failures++; }
  // Kernel A
  expect("qd null x", svdq_quantize_down(nullptr, P, 16, 64, 16, F4, P, P, P, nullptr, 0, nullptr), SVDQ_ERR_NULL);
  expect("qd null l1t", svdq_quantize_down(P, nullptr, 16, 64, 16, F4, P, P, P, nullptr, 0, nullptr), SVDQ_ERR_NULL);
  expect("qd bad K", svdq_quantize_down(P, P, 16, 100, 16, F4, P, P, P, nullptr, 0, nullptr), SVDQ_ERR_SHAPE);
  expect("qd bad r", svdq_quantize_down(P, P, 16, 64, 8, F4, P, P, P, nullptr, 0, nullptr), SVDQ_ERR_SHAPE);
  expect("qd r too big", svdq_quantize_down(P, P, 16, 64, 80, F4, P, P, P, nullptr, 0, nullptr), SVDQ_ERR_SHAPE);
  expect("qd negative M", svdq_quantize_down(P, P, -1, 64, 16, F4, P, P, P, nullptr, 0, nullptr), SVDQ_ERR_SHAPE);
  expect("qd bad fmt", svdq_quantize_down(P, P, 16, 64, 16, BAD, P, P, P, nullptr, 0, nullptr), SVDQ_ERR_FORMAT);
  expect("qd misaligned", svdq_quantize_down(MIS, P, 16, 64, 16, F4, P, P, P, nullptr, 0, nullptr), SVDQ_ERR_ALIGN);
  expect("qd empty", svdq_quantize_down(nullptr, nullptr, 0, 64, 0, F4, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
         SVDQ_OK);
  const size_t qneed = svdq_quantize_down_workspace_bytes(1024, 3072, 16, F4);
  if (qneed) {
    expect("qd small workspace", svdq_quantize_down(P, P, 1024, 3072, 16, F4, P, P, P, P, qneed - 256, nullptr),
           SVDQ_ERR_WORKSPACE);
    expect("qd misaligned workspace", svdq_quantize_down(P, P, 1024, 3072, 16, F4, P, P, P, MIS, qneed, nullptr),
           SVDQ_ERR_ALIGN);
  }
  expect("qd smooth null lambda",
         svdq_quantize_down_smooth(P, nullptr, P, 16, 64, 16, F4, P, P, P, nullptr, 0, nullptr), SVDQ_ERR_NULL);
  expect("qd smooth misaligned lambda",
         svdq_quantize_down_smooth(P, MISF, P, 16, 64, 16, F4, P, P, P, nullptr, 0, nullptr), SVDQ_ERR_ALIGN);
  // Kernel B
  expect("gemm null y", svdq_gemm_w4a4_up(P, P, P, P, P, P, P, 16, 16, 64, 16, F4, nullptr, nullptr), SVDQ_ERR_NULL);
  expect("gemm null t", svdq_gemm_w4a4_up(P, P, nullptr, P, P, P, P, 16, 16, 64, 16, F4, P, nullptr), SVDQ_ERR_NULL);
  expect("gemm bad N", svdq_gemm_w4a4_up(P, P, P, P, P, P, P, 16, 24, 64, 16, F4, P, nullptr), SVDQ_ERR_SHAPE);
  expect("gemm huge", svdq_gemm_w4a4_up(P, P, P, P, P, P, P, 1 << 25, 16, 64, 16, F4, P, nullptr), SVDQ_ERR_SHAPE);
  expect("gemm bad fmt", svdq_gemm_w4a4_up(P, P, P, P, P, P, P, 16, 16, 64, 16, BAD, P, nullptr), SVDQ_ERR_FORMAT);
  expect("gemm misaligned bias", svdq_gemm_w4a4_up(P, P, P, P, P, P, MIS, 16, 16, 64, 16, F4, P, nullptr),
         SVDQ_ERR_ALIGN);
  expect("gemm empty", svdq_gemm_w4a4_up(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 16, 64, 16,
                                         F4, nullptr, nullptr), SVDQ_OK);
  expect("gemm gelu null lambda",
         svdq_gemm_w4a4_up_gelu_smooth(P, P, P, P, P, P, P, nullptr, 16, 16, 64, 16, F4, P, nullptr), SVDQ_ERR_NULL);
  // the layer
  expect("linear small workspace", svdq_linear(P, P, P, P, P, nullptr, 16, 16, 64, 16, F4, P, need - 1, P, nullptr),
         SVDQ_ERR_WORKSPACE);
  expect("linear null workspace", svdq_linear(P, P, P, P, P, nullptr, 16, 16, 64, 16, F4, nullptr, need, P, nullptr),
         SVDQ_ERR_NULL);
  expect("linear misaligned workspace", svdq_linear(P, P, P, P, P, nullptr, 16, 16, 64, 16, F4, MIS, need, P, nullptr),
         SVDQ_ERR_ALIGN);
  expect("linear empty", svdq_linear(P, P, P, P, P, nullptr, 0, 16, 64, 16, F4, P, need, P, nullptr), SVDQ_OK);
  const size_t uneed = svdq_linear_unfused_workspace_bytes(16, 16, 64, 16, F4);
  expect("unfused small workspace",
         svdq_linear_unfused(P, P, P, P, P, nullptr, 16, 16, 64, 16, F4, P, uneed - 1, P, nullptr), SVDQ_ERR_WORKSPACE);
  expect("folded misaligned lambda",
         svdq_linear_folded(P, MISF, P, P, P, P, nullptr, nullptr, 16, 16, 64, 16, F4, P, need, P, nullptr),
         SVDQ_ERR_ALIGN);
  expect("noalloc beyond the scratch",
         svdq_linear_noalloc(P, P, P, P, P, nullptr, 8192, 16, 12288, 32, F6, P, nullptr), SVDQ_ERR_WORKSPACE);
  expect("noalloc null y", svdq_linear_noalloc(P, P, P, P, P, nullptr, 16, 16, 64, 16, F4, nullptr, nullptr),
         SVDQ_ERR_NULL);
  expect("noalloc empty", svdq_linear_noalloc(P, P, P, P, P, nullptr, 0, 16, 64, 16, F4, P, nullptr), SVDQ_OK);
  // offline, control and glue entry points
  expect("qw null", svdq_quantize_weight(nullptr, 16, 64, F4, P, P, nullptr), SVDQ_ERR_NULL);
  expect("qw bad N", svdq_quantize_weight(PF, 15, 64, F4, P, P, nullptr), SVDQ_ERR_SHAPE);
  expect("pack fp4", svdq_pack_weight(static_cast<const int8_t*>(P), P, 16, 64, SVDQ_FP4_G16, P, P, nullptr),
         SVDQ_ERR_FORMAT);
  expect("w4a16 bad K", svdq_gemm_w4a16(P, P, P, nullptr, 4, 16, 96, P, nullptr), SVDQ_ERR_SHAPE);
  expect("gelu bad C", svdq_gelu_tanh_smooth(P, PF, 4, 12, P, nullptr), SVDQ_ERR_SHAPE);
  expect("relayout bad direction", svdq_relayout(P, P, 16, 64, F6, 2, P, P, nullptr), SVDQ_ERR_SHAPE);
  expect("relayout null", svdq_relayout(nullptr, P, 16, 64, F6, 1, P, P, nullptr), SVDQ_ERR_NULL);
  expect("relayout empty", svdq_relayout(nullptr, nullptr, 0, 64, F6, 1, nullptr, nullptr, nullptr), SVDQ_OK);
  for (int s = 0; s >= -8; s--)
    if (!svdq_status_string(static_cast<svdq_status>(s))[0]) { std::printf("FAIL status string %d\n", s); failures++; }
  if (!svdq_version()[0]) { std::printf("FAIL version\n"); failures++; }
  std::printf("%s: %d failure(s)\n", failures ? "FAILED" : "OK", failures);
  return failures ? 1 : 0;
}
