/*
 * svdq.h -- C ABI of the fused SVDQuant W4A4 linear layer for AMD Instinct
 * MI355X (gfx950).
 *
 * The layer (SVDQuant, Li, Lin, Zhang, Cai, Li, Guo, Xie, Meng, Zhu, Han 2024,
 * as described by the practice page "sota-314", section "Do this", and the
 * reading note "note-257", section "Key results"):
 *
 *     Y = X_hat L1 L2  +  Q(X_hat) Q(R)  +  b,     R = W_hat - L1 L2,
 *
 * where X_hat / W_hat are the smoothed activations / weight, L1 L2 is the
 * 16-bit rank-r branch taken off W_hat by truncated SVD, and Q() is per-group
 * symmetric quantization along the reduction axis K.  The two fusions the
 * pages name are the two kernels behind this ABI:
 *   Kernel A  (svdq_quantize_down): quantize X_hat and compute the down
 *             projection T = X_hat L1 in the same pass (same input);
 *   Kernel B  (svdq_gemm_w4a4_up):  the low-bit GEMM with the up projection
 *             T L2 and the bias in its epilogue (same output).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor pointers are DEVICE pointers, owned by the caller, row-major,
 *    16-byte aligned.  The library never allocates or frees memory and keeps
 *    no mutable global state beyond a per-device cache of the compute-unit
 *    count (set atomically on first use); calls are thread-safe.
 *  - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *    enqueued on it asynchronously; nothing synchronizes the device and there
 *    are no host<->device copies.
 *  - Arguments are validated on the host before any HIP call; a failed check
 *    returns an error status and enqueues nothing.  A launch failure reported
 *    by the runtime returns SVDQ_ERR_LAUNCH.  No C++ exception crosses the ABI.
 *  - Shapes: M >= 0 and N >= 0 (0 = nothing to do: SVDQ_OK once the format
 *    and the other dimensions check out, and the pointers may then be NULL,
 *    as a zero-size tensor's are); K > 0 with
 *    K % 64 == 0; N % 16 == 0; r % 16 == 0 and 0 <= r <= 64; M, N, K <= 2^24;
 *    the GEMM entry points also need each code operand (M and N times the
 *    format's code bytes per row) below 4 GiB, and the W4A16 control needs
 *    M * 2K and N * K/2 bytes below 4 GiB.
 *  - Non-finite inputs are undefined behaviour.
 *
 * Formats (group quantization along K; groups per token row for activations,
 * per output column for the weight; "sota-314", "Do this": INT4 group 64 with
 * 16-bit scales, NVFP4 group 16 with FP8 scales, rank 16 at 8 bits):
 *  SVDQ_INT4_G64 : codes in [-7, 7], two's-complement nibbles, two per byte
 *                  (byte b = code 2b | code 2b+1 << 4); fp16 scale per 64.
 *                  scale = fp16_rne(fp32(absmax) / 7.0f); code =
 *                  clamp(rint_half_even(fp32(v) / scale), -7, 7); scale 0 ->
 *                  codes 0.  Codes group-major [K/64][rows][32 bytes] (group g
 *                  of row i at byte (g * rows + i) * 32), fp16 scales
 *                  group-major [K/64][rows]: a GEMM tile's rows of one group
 *                  are one contiguous run.
 *  SVDQ_INT8_G64 : same rule with 127; one int8 code per byte.  Codes
 *                  group-major [K/64][rows][64 bytes] (group g of row i at
 *                  byte (g * rows + i) * 64), fp16 scales group-major
 *                  [K/64][rows]: a GEMM tile's rows of one group are one
 *                  contiguous run.
 *  SVDQ_FP4_G16  : E2M1 codes (sign<<3 | magnitude index, magnitudes
 *                  0,0.5,1,1.5,2,3,4,6), packed as INT4; one E4M3FN scale byte
 *                  per 16: scale = e4m3_rne_sat(fp32(absmax) / 6.0f); code =
 *                  nearest E2M1 to fp32(v)/scale, ties to the even mantissa,
 *                  -0 -> +0.  Codes chunk-major [K/64][rows][32 bytes] (chunk c of
 *                  row i at byte (c * rows + i) * 32, two codes per byte as
 *                  above), E4M3 bytes [K/64][rows][4].
 *  SVDQ_INT4_G64_E2M3 : the SVDQ_INT4_G64 codes and scales, bit for bit, in the
 *                  storage the gfx950 FP6 matrix cores read directly: each code
 *                  q becomes the 6-bit E2M3 pattern of q/8 (a subnormal:
 *                  sign<<5 | |q|).  A row takes 48 bytes per group of 64:
 *                  each half of the group (codes 0..31, 32..63) is a 24-byte
 *                  little-endian field string, code j of the half in bits
 *                  [6j, 6j+6); the 48 bytes hold half 0 bytes 0..15, half 1
 *                  bytes 0..15, half 0 bytes 16..23, half 1 bytes 16..23 (so
 *                  each half is one 16-byte and one 8-byte aligned piece).
 *                  Codes and scales are group-major:
 *                  codes [K/64][rows][48 bytes] (the group-g slice of row i at
 *                  byte (g * rows + i) * 48; 3K/4 bytes per row in total),
 *                  fp16 scales [K/64][rows].  The 4-bit values
 *                  sit in a 6-bit container (1.5x the bytes of SVDQ_INT4_G64)
 *                  so that the GEMM runs on the FP6 matrix cores, which return
 *                  fp32 partials and, measured on MI355X, do 1.57x the INT8
 *                  instruction's work per K element.
 *  SVDQ_MXFP4_G32 : MXFP4 (OCP Microscaling Formats v1.0), the block-scaled
 *                  format gfx950's matrix cores apply natively ("sota-314",
 *                  "Conditions": the format ranking follows the hardware's
 *                  native group support; "Quantization", "KV cache
 *                  quantization": OCP MXFP4 among the production formats).
 *                  E2M1 codes packed as SVDQ_FP4_G16, one E8M0 byte per 32
 *                  along K: e = floor(log2 absmax) - 2 clamped to [-127, 127]
 *                  (-127 for an all-zero group), byte = e + 127; code =
 *                  nearest E2M1 to v / 2^e (exact division), ties to the even
 *                  mantissa, saturating at 6, -0 -> +0.  Codes and scales are
 *                  chunk-major, so that a tile's rows of one 64-wide chunk of K
 *                  are contiguous: codes [K/64][rows][32 bytes] (chunk c of
 *                  row i at byte (c * rows + i) * 32; within it the two 16-byte
 *                  halves are the groups, two codes per byte as SVDQ_FP4_G16),
 *                  E8M0 bytes [K/64][rows][2].
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SVDQ_OK = 0,
  SVDQ_ERR_NULL = -1,      /* a required pointer is NULL                         */
  SVDQ_ERR_SHAPE = -2,     /* M/N/K/r/C outside the documented constraints       */
  SVDQ_ERR_ALIGN = -3,     /* a pointer is not 16-byte aligned                   */
  SVDQ_ERR_FORMAT = -4,    /* unknown or unsupported format for this entry point */
  SVDQ_ERR_WORKSPACE = -5, /* workspace smaller than the *_workspace_bytes value */
  SVDQ_ERR_DEVICE = -6,    /* the current device is not a gfx950 GPU             */
  SVDQ_ERR_LAUNCH = -7     /* the HIP runtime reported a launch error            */
} svdq_status;

typedef enum {
  SVDQ_INT4_G64 = 0,
  SVDQ_INT8_G64 = 1,
  SVDQ_FP4_G16 = 2,
  SVDQ_INT4_G64_E2M3 = 3,
  SVDQ_MXFP4_G32 = 4,
  /* Not formats: these two make the type span every int, so that any value a caller passes is
   * a valid value of the type (in C++ an enum holds only the values its enumerators' range
   * covers) and an unknown one is rejected with SVDQ_ERR_FORMAT. */
  SVDQ_FORMAT_INT_MIN_ = -2147483647 - 1,
  SVDQ_FORMAT_INT_MAX_ = 2147483647
} svdq_format;

/* Bytes of codes per row for K columns (K/2 for 4-bit formats, K for INT8,
 * 3K/4 for the E2M3 container; the device layouts interleave the rows group by
 * group), and bytes of scales per row (K/64 fp16 for the INT formats, K/16 E4M3
 * bytes for FP4, K/32 E8M0 bytes for MXFP4).  Returns 0 for a bad format. */
size_t svdq_code_row_bytes(int K, svdq_format fmt);
size_t svdq_scale_row_bytes(int K, svdq_format fmt);

/*
 * Kernel A: quantize + down projection ("sota-314", "Do this": the down
 * projection is fused with quantization since both consume X_hat;
 * "note-257", "Key results").
 *   x_hat : fp16 [M, K], the smoothed activations (smoothing already applied).
 *   l1t   : fp16 [r, K] = L1^T; NULL iff r == 0.
 *   xq    : out, codes, M * code_row_bytes(K) bytes in the format's layout.
 *   xs    : out, scales, M * scale_row_bytes(K) bytes in the format's layout.
 *   t     : out, fp16 [M, r] = fp16_rne(X_hat L1), fp32 accumulation; NULL iff r == 0.
 *   workspace, workspace_bytes : caller-owned device scratch for the fp32
 *           partial sums of T when the kernel slices K across workgroups
 *           (svdq_quantize_down_workspace_bytes; 16-byte aligned).  Its
 *           contents need no initialisation and are dead after the call; two
 *           calls in flight at once need two workspaces.  NULL is allowed: K
 *           is then not sliced for r > 0 (same results, slower for long K);
 *           a non-NULL workspace that is too small is SVDQ_ERR_WORKSPACE.
 * The branch reads the unquantized 16-bit X_hat.  Results do not depend on
 * the workspace: the slices' partials are added in a fixed order.
 */
svdq_status svdq_quantize_down(const void* x_hat, const void* l1t, int M, int K, int r,
                               svdq_format fmt, void* xq, void* xs, void* t, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Workspace bytes svdq_quantize_down uses to slice K (0: no slicing for this
 * shape, or r == 0, or a bad format or shape). */
size_t svdq_quantize_down_workspace_bytes(int M, int K, int r, svdq_format fmt);

/*
 * Kernel B: low-bit GEMM + up projection + bias ("sota-314", "Do this": the up
 * projection is fused with the 4-bit compute because both write the same
 * output).
 *   Y = fp16_rne( sum_g sx[m,g] sw[n,g] P_g[m,n] + T L2 + b ),
 *   P_g = sum over the group's K of q_x q_w (exact integers; fp32 accumulation
 *   of the rescaled partials).
 *   xq, xs : Kernel A's codes and scales for M rows.
 *   t      : fp16 [M, r]; NULL iff r == 0.
 *   wq     : codes of the N output columns, N * code_row_bytes(K) bytes in the
 *            format's layout (rows = output columns).
 *   ws     : their scales, N * scale_row_bytes(K) bytes in the format's layout.
 *   l2     : fp16 [r, N]; NULL iff r == 0.
 *   bias   : fp16 [N], or NULL for none.
 *   y      : out, fp16 [M, N].
 * r == 0 selects the bare low-bit GEMM (no branch).
 */
svdq_status svdq_gemm_w4a4_up(const void* xq, const void* xs, const void* t, const void* wq,
                              const void* ws, const void* l2, const void* bias, int M, int N, int K,
                              int r, svdq_format fmt, void* y, void* stream);

/* Workspace svdq_linear needs: codes, scales and T for M rows, and Kernel A's
 * partial sums (svdq_quantize_down_workspace_bytes), each part 256-byte
 * aligned.  0 for a bad format or shape. */
size_t svdq_linear_workspace_bytes(int M, int K, int r, svdq_format fmt);

/*
 * The fused layer: Kernel A then Kernel B on one stream, with codes, scales
 * and T in the caller's workspace (>= svdq_linear_workspace_bytes).
 * Arguments as for the two kernels above.
 */
svdq_status svdq_linear(const void* x_hat, const void* l1t, const void* wq, const void* ws,
                        const void* l2, const void* bias, int M, int N, int K, int r,
                        svdq_format fmt, void* workspace, size_t workspace_bytes, void* y,
                        void* stream);

/*
 * The fused layer without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): svdq_linear with its codes, scales, T and Kernel A's partial sums in a static
 * device array of SVDQ_STATIC_SCRATCH_BYTES inside the library.  Each GPU the library runs on
 * holds its own copy of the array until the process ends; the first call on a device looks up
 * that copy's address (hipGetSymbolAddress, with the device current) and keeps it.  The call
 * allocates nothing (no hipMalloc / hipFree, no allocating library routine).
 *   Limit: shapes whose svdq_linear_workspace_bytes(M, K, r, fmt) exceeds
 *   SVDQ_STATIC_SCRATCH_BYTES return SVDQ_ERR_WORKSPACE before anything is enqueued (the FLUX
 *   shapes, M = 4608 with K = 3072 or 12288, fit in every format).
 *   Concurrency: every call on one GPU shares that GPU's array and its contents persist from
 *   call to call (nothing in it needs to start at zero).  Calls that overlap on one GPU -- on
 *   two streams, or from two host threads without ordering -- race on it and give wrong
 *   results: order them on one stream.
 * Other arguments, results (bit for bit those of svdq_linear) and errors as for svdq_linear.
 */
#define SVDQ_STATIC_SCRATCH_BYTES (64u << 20)
svdq_status svdq_linear_noalloc(const void* x_hat, const void* l1t, const void* wq, const void* ws,
                                const void* l2, const void* bias, int M, int N, int K, int r,
                                svdq_format fmt, void* y, void* stream);

/*
 * Offline weight quantizer: the residual R = W_hat - L1 L2, given as
 * R^T fp32 [N, K] (K contiguous per output column), to codes wq and scales ws
 * in the layouts Kernel B reads ("sota-314", "Do this": quantize only the
 * residual; round-to-nearest-even here, where the pages' own pipeline uses
 * GPTQ).
 */
svdq_status svdq_quantize_weight(const float* r_t, int N, int K, svdq_format fmt, void* wq,
                                 void* ws, void* stream);

/*
 * Codes and scales of the residual computed elsewhere -- e.g. GPTQ on the host
 * ("sota-314", "Do this": the authors' pipeline rounds the residual with GPTQ,
 * not to nearest) -- put into the layouts Kernel B reads, for the INT
 * formats (SVDQ_INT4_G64, SVDQ_INT4_G64_E2M3, SVDQ_INT8_G64; others are
 * SVDQ_ERR_FORMAT):
 *   codes  : int8 [N, K], one code per byte (in [-7, 7] or [-127, 127]; not
 *            checked), K contiguous per output column.
 *   scales : fp16 [N, K/64].
 *   wq, ws : out, as svdq_quantize_weight writes them.
 * With round-to-nearest codes and scales this reproduces svdq_quantize_weight
 * bit for bit.  Pointers 16-byte aligned; N % 16 == 0, K % 64 == 0.
 */
svdq_status svdq_pack_weight(const int8_t* codes, const void* scales, int N, int K, svdq_format fmt,
                             void* wq, void* ws, void* stream);

/*
 * Codes and scales between the exchange layout and the layout of the format's kernels
 * (the exchange layout is the one the bit-exact comparisons with a plain implementation of
 * the quantizers are stated in; "sota-314", "Do this": INT4 group 64 with 16-bit scales,
 * NVFP4 group 16 with FP8 scales, rank 16 at 8 bits -- the formats fix codes and scales, not
 * a memory order).
 *   Exchange layout: row-major, K contiguous per row (token, or output column of a weight):
 *     codes  [rows, K/2] for the 4-bit formats (two codes a byte, code 2b in the low nibble;
 *            two's-complement INT4 for SVDQ_INT4_G64 and SVDQ_INT4_G64_E2M3, E2M1 nibbles for
 *            SVDQ_FP4_G16 and SVDQ_MXFP4_G32) or [rows, K] for SVDQ_INT8_G64;
 *     scales [rows, K/G]: fp16 (INT formats), E4M3 bytes (SVDQ_FP4_G16), E8M0 bytes
 *            (SVDQ_MXFP4_G32).
 *   Device layout: the format's layout above (chunk- or group-major).  SVDQ_INT4_G64_E2M3's INT4 codes are
 *   turned into or out of their 6-bit E2M3 fields exactly; exchange codes must lie in [-7, 7].
 *   to_canonical : 1 = device -> exchange, 0 = exchange -> device.
 *   codes_in, scales_in : the source layout; codes_out, scales_out : the destination layout
 *   (caller-allocated, svdq_code_row_bytes(K, SVDQ_INT4_G64 or fmt) and
 *   svdq_scale_row_bytes(K, fmt) bytes a row; may not alias the sources).
 *   rows >= 0 (any count), K % 64 == 0.  Offline / exchange work, not on the layer's path.
 */
svdq_status svdq_relayout(const void* codes_in, const void* scales_in, int rows, int K, svdq_format fmt,
                          int to_canonical, void* codes_out, void* scales_out, void* stream);

/* Workspace of the unfused comparison: svdq_linear's workspace plus an fp16
 * [M, N] intermediate, 256-byte aligned. */
size_t svdq_linear_unfused_workspace_bytes(int M, int N, int K, int r, svdq_format fmt);

/*
 * Unfused comparison (measurement only; "sota-314", "Do this", latency table:
 * a rank-32 branch run as separate kernels): four launches -- quantize;
 * down projection T = X_hat L1 (a second read of X_hat); the low-bit GEMM
 * writing fp16 Y0 = fp16(Q(X_hat) Q(R) + b); up projection
 * Y = fp16(Y0 + T L2) (a second read and write of the output).  Note the extra
 * fp16 rounding of Y0: results agree with svdq_linear to fp16 tolerance, not
 * bitwise.
 */
svdq_status svdq_linear_unfused(const void* x_hat, const void* l1t, const void* wq, const void* ws,
                                const void* l2, const void* bias, int M, int N, int K, int r,
                                svdq_format fmt, void* workspace, size_t workspace_bytes,
                                void* y, void* stream);

/*
 * W4A16 control ("sota-314", "Do this" and "What it buys": the W4A16
 * baseline and the layers kept at W4A16): Y = fp16_rne( X deq(W) + b ) with
 * X fp16 [M, K] unquantized, W as SVDQ_INT4_G64 codes wq and fp16 scales ws
 * (the format's layout, rows = output columns), fp32 accumulation; bias may be
 * NULL.  No branch.
 */
svdq_status svdq_gemm_w4a16(const void* x, const void* wq, const void* ws, const void* bias,
                            int M, int N, int K, void* y, void* stream);

/*
 * GELU(tanh) + smoothing glue between an MLP's two linears:
 *   out[m, c] = fp16_rne( gelu_tanh(float(y[m, c])) / lambda[c] ),
 *   gelu_tanh(v) = 0.5 v (1 + tanh( sqrt(2/pi) (v + 0.044715 v^3) )),
 *   evaluated in fp32 as gelu_div(v, lam) = v / ((1 + exp(-2u)) lam) with
 *   u = sqrt(2/pi) (v + 0.044715 v^3) (the same value; no cancellation for
 *   negative v), exp and the reciprocal from the hardware's approximations:
 *   within one fp16 ulp of the exactly rounded result.
 *   y: fp16 [M, C]; lambda: fp32 [C] (the second layer's smoothing factors);
 *   out: fp16 [M, C] (may not alias y).  C % 8 == 0.
 */
svdq_status svdq_gelu_tanh_smooth(const void* y, const float* lambda, int M, int C, void* out,
                                  void* stream);

/*
 * Folding the neighbouring steps into the two kernels.  The pages fuse the
 * branch with the low-bit kernels because the fused steps share an operand
 * ("sota-314", "Do this"); the same argument carries the steps on either side
 * of a layer into the kernels: the smoothing of the layer's input into Kernel A
 * (both read X) and an MLP's GELU + next-layer smoothing into Kernel B's
 * epilogue (both write the output).  The pages do not describe this fold.
 *
 * Kernel A on the unsmoothed activations ("sota-314", "Do this": smoothing
 * divides each input channel by its factor, X_hat = X diag(lambda)^-1):
 *   x      : fp16 [M, K], unsmoothed.
 *   lambda : fp32 [K], the layer's smoothing factors (> 0), 16-byte aligned.
 *   Every value is first replaced by X_hat = fp16_rne(fp32(x) / lambda[k])
 *   (IEEE fp32 division, then one rounding); codes, scales and T are then
 *   exactly those svdq_quantize_down gives for that X_hat.  Other arguments,
 *   the workspace rules and errors as for svdq_quantize_down; lambda NULL is
 *   SVDQ_ERR_NULL.
 */
svdq_status svdq_quantize_down_smooth(const void* x, const float* lambda, const void* l1t, int M, int K,
                                      int r, svdq_format fmt, void* xq, void* xs, void* t,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Kernel B with an MLP's glue in its epilogue: writes
 *   y[m, n] = fp16_rne( gelu_div( Y[m, n], lambda_next[n] ) ),
 * where Y is the fp16 output svdq_gemm_w4a4_up would write and gelu_div is the
 * arithmetic of svdq_gelu_tanh_smooth, so the result equals
 * svdq_gelu_tanh_smooth(svdq_gemm_w4a4_up(...), lambda_next) bit for bit
 * without the fp16 round trip of Y through memory.
 *   lambda_next : fp32 [N], the next layer's smoothing factors (> 0), 16-byte
 *                 aligned; NULL is SVDQ_ERR_NULL.
 * Other arguments and errors as for svdq_gemm_w4a4_up.
 */
svdq_status svdq_gemm_w4a4_up_gelu_smooth(const void* xq, const void* xs, const void* t, const void* wq,
                                          const void* ws, const void* l2, const void* bias,
                                          const float* lambda_next, int M, int N, int K, int r,
                                          svdq_format fmt, void* y, void* stream);

/*
 * The fused layer with either fold: svdq_linear's Kernel A then Kernel B, with
 * lambda_in != NULL taking x unsmoothed (as svdq_quantize_down_smooth) and
 * lambda_next != NULL writing fp16(gelu(Y) / lambda_next) (as
 * svdq_gemm_w4a4_up_gelu_smooth).  With both NULL it is svdq_linear.  An
 * MLP's first layer runs with both; its output is then the second layer's
 * X_hat, for svdq_linear.  Workspace as for svdq_linear
 * (svdq_linear_workspace_bytes covers the smoothing variant's plan too).
 */
svdq_status svdq_linear_folded(const void* x, const float* lambda_in, const void* l1t, const void* wq,
                               const void* ws, const void* l2, const void* bias, const float* lambda_next,
                               int M, int N, int K, int r, svdq_format fmt, void* workspace,
                               size_t workspace_bytes, void* y, void* stream);

/* Static description of a status code. */
const char* svdq_status_string(svdq_status s);

/* Library version string. */
const char* svdq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H */
