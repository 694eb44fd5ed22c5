/*
 * mxq.h — C ABI of the MI355X (gfx950) FP8 / MXFP8 training-numerics library (libmxq.so).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless stated otherwise. The caller allocates and owns every buffer; the
 *     library never allocates or frees device memory, never synchronizes, and keeps no mutable global state.
 *   - Work is enqueued on `stream` (NULL = the default stream) and the call returns immediately.
 *   - Errors found on the host (NULL pointers, shapes, alignment, workspace size) return a status at once and
 *     enqueue nothing. A failed launch returns MXQ_ERR_HIP. Device-side faults surface at the caller's next
 *     synchronization, as with any HIP kernel.
 *   - bf16 and fp16 tensors are passed as their 16-bit patterns (uint16_t); FP8 tensors as bytes.
 *   - Matrices are row-major and contiguous unless a leading dimension is given. Every pointer must be
 *     16-byte aligned and every row of a bf16 input must start on a 16-byte boundary (cols % 8 == 0).
 *   - Buffers must not overlap, except where an argument is documented as updated in place.
 *   - A call whose sizes make it empty (no output elements) returns MXQ_OK at once and enqueues nothing; its
 *     data pointers may then be NULL.
 *
 * Formats: E4M3 is OCP E4M3FN (max 448, no infinities), E5M2 is OCP E5M2 (max 57344). Conversions round to
 * nearest even and saturate at the largest finite value; a NaN input gives a NaN code. E8M0 scale bytes hold
 * 2^(byte-127); byte 0xFF (NaN) marks a 32-value block holding a NaN.
 *
 * Sources (page titles and sections):
 *   [OLMO11] "OLMo-core MoE, Section 11: MXFP8 Training" — Eq. 57, Eq. 58, Figures 47/49/50/55, Eq. 60,
 *            Sections 11.2.1, 11.3.2, 11.3.4, 11.3.5 / Table 24, 11.4.1, 11.4.4 / Table 25.
 *   [LLMSB]  "3.8 Mixed Precision, bf16 & FP8 Training" — per-tensor scaling, delayed scaling, Exercise 6,
 *            "Tensor cores accumulate in fp32" (and its caveat on FP8 accumulators).
 *   [FP8-LM] "FP8-LM: Training FP8 Large Language Models" — tensor scaling, AdamW update, Eq. 7-8.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MXQ_OK = 0,
    MXQ_ERR_NULL = 1,         /* a required pointer is NULL */
    MXQ_ERR_SHAPE = 2,        /* a size is negative, or not divisible as the operation requires */
    MXQ_ERR_ALIGN = 3,        /* a pointer is not 16-byte aligned */
    MXQ_ERR_UNSUPPORTED = 4,  /* an enum value or combination the library does not implement, or an Adam beta
                                 outside [0, 1) */
    MXQ_ERR_WORKSPACE = 5,    /* workspace missing or smaller than mxq_workspace_bytes() */
    MXQ_ERR_HIP = 6           /* a HIP launch or query failed */
} mxq_status;

typedef enum { MXQ_E4M3 = 0, MXQ_E5M2 = 1 } mxq_fp8;
typedef enum { MXQ_SCALE_RCEIL = 0, MXQ_SCALE_FLOOR = 1 } mxq_scale_rule;
typedef enum { MXQ_PER_TENSOR = 0, MXQ_MX_BLOCK32 = 1 } mxq_scaling;

/* Static, never-NULL description of a status code. */
const char* mxq_status_string(mxq_status s);
/* Version of this ABI; bumped on any incompatible change. */
int mxq_abi_version(void);

/*
 * MXFP8 quantization of a bf16 matrix x[rows][cols] ([OLMO11] Section 11.2.1, Eq. 58; orientations from
 * Section 11.3.2, Eq. 60; scale rules from Section 11.3.5, Table 24).
 *   For each block of 32 values: amax = max |x_i|;
 *     RCEIL: s = the smallest power of two with amax <= 448 * s;  FLOOR: s = 2^(floor(log2 amax) - 8);
 *     the exponent is clamped to [-127, 127] (an all-zero block gets 2^-127);
 *   q_i = E4M3(x_i / s) (exact division by a power of two, then RNE with saturation), scale byte = log2(s) + 127.
 * Row orientation (blocks along a row):      q_row[rows][cols],  s_row[rows][cols/32]; needs cols % 32 == 0.
 * Column orientation (blocks down a column), stored transposed so the block runs contiguously:
 *                                            q_col[cols][rows],  s_col[cols][rows/32]; needs rows % 32 == 0.
 * Pass NULL for both pointers of an orientation to skip it (at least one orientation is required). One pass
 * over x emits both orientations. Storage per orientation is 33/32 bytes per value (Eq. 57).
 */
mxq_status mxq_quantize(const uint16_t* x_bf16, int64_t rows, int64_t cols,
                        uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                        mxq_scale_rule rule, hipStream_t stream);

/*
 * mxq_quantize that also classifies the operand for the FP8 matrix instruction, so that scaled_gemm_ranged can pick its
 * instruction without re-reading the codes. Arguments and outputs are those of mxq_quantize, plus:
 *   wide_row (device uint32, required with q_row): 1 if any 64-value window along a row of q_row is wide, else 0;
 *   wide_col (device uint32, required with q_col): the same for the windows along a row of q_col (64 rows of x).
 * A window is wide when it holds a nonzero code and 24 or more of its codes lie more than 6 binades below its largest
 * (a code's binade: its E4M3 exponent field plus its block's scale byte): the definition scaled_gemm's range check
 * applies to its operands, so the two classify the same codes identically. Requires cols % 64 == 0 for the row
 * orientation and rows % 64 == 0 for the column orientation (whole windows). The words are cleared and set by the
 * call's own kernels; an empty x gives 0.
 */
mxq_status mxq_quantize_ranged(const uint16_t* x_bf16, int64_t rows, int64_t cols,
                               uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                               mxq_scale_rule rule, uint32_t* wide_row, uint32_t* wide_col, hipStream_t stream);

/*
 * Fused SwiGLU + MXFP8 row quantize of the routed experts' hidden representation ([OLMO11] Section 11.4.1: a fused
 * SwiGLU-plus-quantization step produces the down projection's operand with no separate BF16-to-MXFP8 pass).
 *   c_bf16[rows][2F]: the up/gate GEMM output, gate in columns [0, F), up in [F, 2F);
 *   h = silu(g) * u in fp32 with silu(g) = g / (1 + exp(-g)), each operation rounded on its own; exp is a fixed fp32
 *   sequence (Cody-Waite reduction by k ln2, degree-6 Taylor polynomial, exact scaling by 2^k; within a few ulp of the
 *   true exponential), so the result is reproducible bit for bit;
 *   q[rows][F], s[rows][F/32]: h quantized from fp32 in 32-value blocks along each row (rule as in mxq_quantize).
 * Requires F % 32 == 0.
 */
mxq_status swiglu_mx_quantize(const uint16_t* c_bf16, int64_t rows, int64_t F, uint8_t* q, uint8_t* s,
                              mxq_scale_rule rule, hipStream_t stream);

/*
 * swiglu_mx_quantize with both orientations, for a forward that saves the hidden representation for the down
 * projection's Wgrad ([OLMO11] Section 11.3.2: an activation saved in MXFP8 for Wgrad is produced explicitly in the
 * right-hand-operand layout; Section 11.4.1, fused SwiGLU plus quantization).
 *   h[r][j] = silu(c[r][j]) c[r][F + j] in fp32 exactly as swiglu_mx_quantize computes it, quantized from fp32:
 *   row: q_row[rows][F], s_row[rows][F/32] (equal to swiglu_mx_quantize's q and s);
 *   col: q_col[F][rows], s_col[F][rows/32] (blocks of 32 routed rows, stored transposed).
 * Either orientation may be NULL (not both). Requires F % 32 == 0 and rows % 32 == 0.
 */
mxq_status swiglu_mx_quantize_oriented(const uint16_t* c_bf16, int64_t rows, int64_t F, uint8_t* q_row,
                                       uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, mxq_scale_rule rule,
                                       hipStream_t stream);

/*
 * Combine backward of the routed experts: the route weighting fused with the gradient's MXFP8 quantize ([OLMO11]
 * Section 11.4.1, combine backward; Section 11.4.4 / Table 25, route weighting + gradient Q as one fusion).
 *   dy_bf16[rows][cols]: the output gradient of each routed row (in expert order); route_w: device fp32[rows], the
 *   route weight of each routed row (0 for padding rows).
 *   x[r][c] = fp32(route_w[r] * dy[r][c]) (one rounding), quantized from fp32 like mxq_quantize:
 *   row: q_row[rows][cols], s_row[rows][cols/32] (the down projection's dgrad operand);
 *   col: q_col[cols][rows], s_col[cols][rows/32] (its Wgrad operand, blocks of 32 routed rows).
 * Either orientation may be NULL (not both). Requires cols % 32 == 0 and rows % 32 == 0.
 */
mxq_status route_weighted_mx_quantize(const uint16_t* dy_bf16, const float* route_w, int64_t rows, int64_t cols,
                                      uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                                      mxq_scale_rule rule, hipStream_t stream);

/*
 * SwiGLU backward fused with the MXFP8 quantize of its gradients ([OLMO11] Section 11.4.1: qdata and scales pass
 * directly between adjacent backward stages that agree on layout, with no DQ-Q cycle).
 *   c_bf16[rows][2F]: the forward up/gate GEMM output (gate in [0, F), up in [F, 2F)); dh_bf16[rows][F]: the
 *   gradient of h = silu(g) u (the down projection's dgrad output).
 *   With sigma = 1 / (1 + e^-g), silu = g / (1 + e^-g) (the forward's value) and silu' = sigma (1 + g (1 - sigma)):
 *   dc[r][j] = (dh u) silu'(g), dc[r][F + j] = dh silu(g); every fp32 operation rounded on its own, in the order
 *   written, with swiglu_mx_quantize's fixed exponential.
 *   row: q_row[rows][2F], s_row[rows][2F/32] (the up/gate dgrad operand, K = 2F);
 *   col: q_col[2F][rows], s_col[2F][rows/32] (its Wgrad operand). Either orientation may be NULL (not both).
 * Requires F % 32 == 0 and rows % 32 == 0.
 */
mxq_status swiglu_backward_mx_quantize(const uint16_t* c_bf16, const uint16_t* dh_bf16, int64_t rows, int64_t F,
                                       uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                                       mxq_scale_rule rule, hipStream_t stream);

/*
 * Per-tensor current scaling ([FP8-LM] tensor scaling FP8(x) = cast(s x), x ~ FP8(x) / s; [LLMSB] per-tensor
 * scaling and Exercise 6's to_fp8_e4m3):
 *   amax_out[0] = max |x|   (fp32, device);
 *   scale_out[0] = (FMAX / max(amax, 1e-12)) * margin   (fp32 IEEE division and product; FMAX = 448 for E4M3,
 *                  57344 for E5M2), or *scale_in when scale_in != NULL (delayed scaling: amax_out is still written);
 *   q[rows][cols] = FP8(fp32(x * s)) and q_t[cols][rows] = its transpose; either may be NULL.
 * The scale never leaves the device. workspace: device scratch of at least mxq_workspace_bytes("pertensor", rows*cols)
 * bytes, clobbered by the call (its contents need no initialization). amax_out and scale_out are required.
 */
mxq_status fp8_quantize_pertensor(const uint16_t* x_bf16, int64_t rows, int64_t cols, mxq_fp8 fmt, float margin,
                                  const float* scale_in, float* amax_out, float* scale_out,
                                  uint8_t* q, uint8_t* q_t, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * fp8_quantize_pertensor without a workspace, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation). Arguments, outputs and errors are those of
 * fp8_quantize_pertensor without workspace and workspace_bytes. The amax pass's partial maxima go to a scratch array
 * of the library's own (2048 words, 8 KiB per GPU, kept until the process ends), which holds the partials of any
 * size; a size whose partials would not fit returns MXQ_ERR_WORKSPACE. The call allocates nothing. Its first call on
 * a GPU looks up that GPU's copy of the array (MXQ_ERR_HIP if the lookup fails). Calls that overlap on one GPU share
 * the array and race: order them on one stream, or use fp8_quantize_pertensor with workspaces of their own.
 */
mxq_status fp8_quantize_pertensor_noalloc(const uint16_t* x_bf16, int64_t rows, int64_t cols, mxq_fp8 fmt,
                                          float margin, const float* scale_in, float* amax_out, float* scale_out,
                                          uint8_t* q, uint8_t* q_t, hipStream_t stream);

/*
 * Delayed per-tensor scaling: one pass over x instead of two ([LLMSB] "Per-tensor scaling and the delayed-scaling
 * recipe", the DelayedScale sketch; [FP8-LM] Section 3.4, delayed scaling).
 *   amax_history: device float[history_len] (in/out), hist_pos: device int32[1] (in/out, 0 <= pos < history_len),
 *   1 <= history_len <= 2^20.
 *   scale_out[0] = (FMAX / max(max(amax_history), 1e-12)) * margin, from the history as it was before this call
 *                  (fp32 division and product; a NaN entry gives a NaN scale);
 *   q[rows][cols] = FP8(fp32(x * scale)) and q_t[cols][rows] its transpose; either or both may be NULL;
 *   amax_out[0] = max |x| of this call, which is then stored at amax_history[pos], and pos = (pos + 1) % history_len.
 * All of this happens on the device, in stream order; the host never sees the scale. An all-zero history gives the
 * scale FMAX / 1e-12, which saturates every nonzero value: seed the history (for example with the amax of a
 * current-scaling call) before relying on it. workspace: at least mxq_workspace_bytes("pertensor_delayed", n) bytes,
 * clobbered.
 */
mxq_status fp8_quantize_pertensor_delayed(const uint16_t* x_bf16, int64_t rows, int64_t cols, mxq_fp8 fmt,
                                          float margin, float* amax_history, int32_t* hist_pos, int64_t history_len,
                                          float* amax_out, float* scale_out, uint8_t* q, uint8_t* q_t,
                                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Auto-scaled FP8 gradient cast, the per-GPU half of the FP8 all-reduce ([FP8-LM] Section 3.4, automatic scaling
 * factor mu, Eq. 3):
 *   q[i] = FP8(fp32(mu * g[i])) with saturation; the scale of q is mu (g ~ val(q) / mu), reported in scale_out[0]
 *   (may be NULL); overflow_count[0] (device uint64) = the number of codes at the format's maximum magnitude;
 *   then mu[0] (device, in/out) <- mu / 2 if overflow_count / n > 1e-5 (0.001 %), else mu * 2^(1/1000) (the factor
 *   rounded to fp32; each product one fp32 rounding), for the next step.
 * workspace: mxq_workspace_bytes("autoscale", n) bytes, clobbered.
 */
mxq_status fp8_autoscale_cast(const uint16_t* g_bf16, int64_t n, mxq_fp8 fmt, float* mu, uint8_t* q,
                              float* scale_out, uint64_t* overflow_count, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * Re-quantize to the shared scaling factor before an FP8 all-reduce ([FP8-LM] Section 3.4, Eq. 4-6):
 *   shared_scale_out[0] = s_g = min(gathered_scales[0 .. nranks)) (the scales every rank reported for this tensor;
 *   a NaN entry gives NaN), sum_scale_out[0] = nranks * s_g (the scale of the sum of the ranks' tensors; may be NULL);
 *   q_out[i] = FP8_out(s_g * (val_in(q_in[i]) / scale_in[0])), each operation one fp32 rounding, saturating; a NaN
 *   gives the NaN code (E4M3 S.1111.111, E5M2 S.11111.10).
 * All scalars are device pointers. 1 <= nranks <= 2^24.
 */
mxq_status fp8_requantize_shared(const uint8_t* q_in, int64_t n, mxq_fp8 fmt_in, const float* scale_in,
                                 const float* gathered_scales, int64_t nranks, mxq_fp8 fmt_out, uint8_t* q_out,
                                 float* shared_scale_out, float* sum_scale_out, hipStream_t stream);

/*
 * Scaled FP8 GEMM with fp32 accumulation and a bf16 epilogue ([OLMO11] Figure 47 and Section 11.2.3:
 * block scales applied inside the matrix operation, BF16 output; [LLMSB] Exercise 6: de-scale by 1/(s_a s_b)):
 *   C[M][N] (row-major, leading dimension ldc >= N, in elements) = bf16_rne( A[M][K] * B[N][K]^T ).
 *   Both operands are K-contiguous (the "TN" layout): A row i is a_q[i*K .. i*K+K), B row j is b_q[j*K ..).
 *   PER_TENSOR: a_scale, b_scale each point to one fp32 scale s on the device (q = x*s);
 *               C = (sum_k val(a_q) val(b_q)) / (s_a s_b). a_fmt / b_fmt may each be E4M3 or E5M2.
 *   MX_BLOCK32: a_scale = E8M0 bytes [M][K/32], b_scale = [N][K/32]; a_fmt = b_fmt = E4M3;
 *               C = sum_k (val(a_q) 2^(sa-127)) (val(b_q) 2^(sb-127)).
 * Requires K % 32 == 0 and K > 0; M, N >= 1 are arbitrary; c_bf16 needs only 2-byte alignment.
 * Accuracy: every output is within 2^-7 |y| + 2^-20 sum_k |a_k b_k| of the exact product y of the dequantized
 * operands, on any input. gfx950's FP8 matrix instructions sum the products of each instruction's 64-value K window in
 * a narrow internal window (products far below the largest lose low-order bits), which keeps that bound only at large
 * K and only on operands whose windows hold values of similar magnitude. So this call takes the block-scaled FP8
 * instruction only when M, N >= 512, K >= 12288 (K % 512 == 0 for MX, K % 64 == 0 for per-tensor) and a device-side
 * check finds no 64-value window of either operand with 24 or more codes (zeros included) more than 6 binades below
 * the window's largest (a code's binade: its exponent field, plus its block's scale byte for MX; a window of zeros
 * does not count); otherwise it dequantizes both operands exactly to bf16 and uses the bf16 matrix instruction
 * (fp32-quality accumulation, half the FP8 rate). The check reads every code of A and B once ((M + N) K bytes) and
 * leaves a flag in C's second row and a gate in each 256 x 256 tile's first element before the FP8 and exact kernels
 * run as a pair, each computing only the tiles its gate names: the choice never returns to the host, and every
 * element of C is written by the call. Normally distributed operands (the workloads' data) take the FP8 instruction;
 * rare large outliers, magnitudes spread over many binades, differently scaled columns or mostly-zero operands take
 * the exact path.
 */
mxq_status scaled_gemm(const uint8_t* a_q, const void* a_scale, mxq_fp8 a_fmt,
                       const uint8_t* b_q, const void* b_scale, mxq_fp8 b_fmt,
                       int64_t M, int64_t N, int64_t K, mxq_scaling scaling,
                       uint16_t* c_bf16, int64_t ldc, hipStream_t stream);

/*
 * scaled_gemm on the exact path at every K: both operands are dequantized to bf16 in registers (every FP8 value times
 * its power-of-two block scale, or the per-tensor code, is exact in bf16), multiplied with the bf16 matrix
 * instruction and accumulated in fp32 ([LLMSB] "Tensor cores accumulate in fp32": narrow inputs, a wide accumulator;
 * the same page's caveat that an FP8 accumulator need not keep full fp32 precision is what this path avoids).
 * Arguments, layouts, requirements and outputs are those of scaled_gemm, without its range check. Where scaled_gemm's
 * check picks the exact path the two give identical bytes.
 */
mxq_status scaled_gemm_exact(const uint8_t* a_q, const void* a_scale, mxq_fp8 a_fmt,
                             const uint8_t* b_q, const void* b_scale, mxq_fp8 b_fmt,
                             int64_t M, int64_t N, int64_t K, mxq_scaling scaling,
                             uint16_t* c_bf16, int64_t ldc, hipStream_t stream);

/*
 * scaled_gemm on the block-scaled FP8 matrix instruction at every K, without the range check ([OLMO11] Figure 47 and
 * Section 11.2.3: block scales applied inside the matrix operation). Arguments, layouts, requirements and outputs are
 * those of scaled_gemm. This is the fastest form (twice the exact path's matrix rate), for callers who accept the
 * instruction's narrow window sums: the bound 2^-7 |y| + 2^-20 sum_k |a_k b_k| is NOT guaranteed. Measured on
 * MX-quantized N(0,1) operands (520 x 528 outputs), the worst |err| / bound is 2.2 at K = 1024, 0.98 at 4096, 0.89
 * at 8192, 0.70 at 12288 and 0.49 at 36864; on wide-range operands it is 4 to 29 at every K. Where scaled_gemm's
 * check picks the FP8 instruction the two give identical bytes.
 */
mxq_status scaled_gemm_fp8(const uint8_t* a_q, const void* a_scale, mxq_fp8 a_fmt,
                           const uint8_t* b_q, const void* b_scale, mxq_fp8 b_fmt,
                           int64_t M, int64_t N, int64_t K, mxq_scaling scaling,
                           uint16_t* c_bf16, int64_t ldc, hipStream_t stream);

/*
 * The MX scaled_gemm with its instruction picked from range words instead of a range check: a_wide and b_wide are
 * device uint32 words that mxq_quantize_ranged wrote for these operands (the orientation each operand was taken from).
 * When M, N >= 512, K >= 12288 and K % 512 == 0, the FP8 and exact kernels run as a pair and the words, read on the
 * device, pick the FP8 instruction if both are 0 and the exact path otherwise; other shapes take the exact path. The
 * result is byte for byte scaled_gemm's for the same operands, without reading the codes twice. Words that do not
 * belong to these operands void the accuracy statement. a_scale, b_scale are E8M0 grids [M][K/32], [N][K/32];
 * everything else is as in scaled_gemm with MX_BLOCK32 and E4M3 operands.
 */
mxq_status scaled_gemm_ranged(const uint8_t* a_q, const uint8_t* a_scale, const uint32_t* a_wide,
                              const uint8_t* b_q, const uint8_t* b_scale, const uint32_t* b_wide,
                              int64_t M, int64_t N, int64_t K, uint16_t* c_bf16, int64_t ldc, hipStream_t stream);

/*
 * Grouped MX GEMM over ragged expert groups ([OLMO11] Section 11.4.1, routed experts: the up/gate and down
 * grouped GEMMs over dispatched MXFP8 rows; Section 11.3.1 on small, uneven expert GEMMs).
 *   group_offsets: device int64[G+1], offsets[0] = 0, non-decreasing, each a multiple of 32, offsets[G] = total_rows.
 *   For each group g, rows [offsets[g], offsets[g+1]) of C = those rows of A times B[g]^T (MX_BLOCK32 semantics).
 *   a_q[total_rows][K], a_s[total_rows][K/32]; b_q[G][N][K], b_s[G][N][K/32]; c_bf16[total_rows][N].
 * Requires K % 32 == 0, N >= 1, 1 <= G <= 4096. The offsets are read on the device only (no host round trip); the
 * host cannot check them, so offsets that break the rules above give unspecified output rows (never stray writes:
 * rows are clamped to [0, total_rows)). It runs scaled_gemm_exact's exact path at every K (the routed projections'
 * K of 1024 to 2048 lies far below where the FP8 instruction could keep the bound), so every output keeps
 * scaled_gemm's bound.
 */
mxq_status grouped_scaled_gemm(const uint8_t* a_q, const uint8_t* a_s, const int64_t* group_offsets, int64_t G,
                               int64_t total_rows, const uint8_t* b_q, const uint8_t* b_s,
                               int64_t N, int64_t K, uint16_t* c_bf16, hipStream_t stream);

/*
 * The same grouped MX GEMM with a strided B operand, so the routed experts' dgrad reads the column-orientation weight
 * cache in place ([OLMO11] Section 11.4.1: dgrad uses the orientation-specific MXFP8 weight caches). Expert g's B row
 * n (n < N) is the K bytes at b_q + g*b_group_stride + n*ldb, its scales the K/32 bytes at
 * b_s + g*bs_group_stride + n*ldbs; C rows have stride ldc (bf16 elements).
 * Example: W[G][D][F] refreshed as one [G*D][F] matrix by fp8_adam_step_mx_cache has q_col[F][G*D]; the dgrad
 * dX = dY W_g takes b_q = q_col, ldb = G*D, b_group_stride = D, b_s = s_col, ldbs = G*D/32, bs_group_stride = D/32,
 * N = F, K = D.
 * Requires everything grouped_scaled_gemm requires, plus ldb >= K, ldbs >= K/32, ldc >= N, non-negative group
 * strides, and ldb and b_group_stride multiples of 16 (16-byte rows). Fastest when ldbs and bs_group_stride are
 * multiples of 16 as well.
 */
mxq_status grouped_scaled_gemm_strided(const uint8_t* a_q, const uint8_t* a_s, const int64_t* group_offsets,
                                       int64_t G, int64_t total_rows, const uint8_t* b_q, const uint8_t* b_s,
                                       int64_t ldb, int64_t b_group_stride, int64_t ldbs, int64_t bs_group_stride,
                                       int64_t N, int64_t K, uint16_t* c_bf16, int64_t ldc, hipStream_t stream);

/*
 * Routed Wgrad: one MX contraction per expert over that expert's token rows ([OLMO11] Section 11.4.1 and
 * Section 11.4.4 / Table 25: the routed Wgrad's reduction dimension is the expert's tokens). The operands are
 * column-orientation MXFP8 tensors whose 32-value blocks run along the token dimension (mxq_quantize's q_col / s_col
 * of the token-major activations and gradients, or route_weighted_mx_quantize's and swiglu_backward_mx_quantize's):
 *   a_q[M][Kt], a_s[M][Kt/32], b_q[N][Kt], b_s[N][Kt/32]; group_offsets: device int64[G+1], offsets[0] = 0,
 *   non-decreasing, multiples of 32, offsets[G] = Kt.
 *   For each expert g: C_g[m][n] = sum over k in [offsets[g], offsets[g+1]) of a_hat[m][k] b_hat[n][k] (fp32
 *   accumulation of exactly dequantized operands: equal to dequantizing to BF16 and running a BF16 grouped GEMM).
 *   Output, exactly one of: c_bf16[G][M][N] (bf16 RNE of C_g; an empty expert gives zeros), or
 *   c_f32[G][M][N] (in/out: c_f32 += C_g, one fp32 rounding per element; the FP32 gradient buffer that Wgrad
 *   outputs accumulate into, [OLMO11] Sections 11.3.4 and 11.4).
 * Requires M, N >= 1, Kt >= 0 and Kt % 32 == 0, 1 <= G <= 4096. As for grouped_scaled_gemm, the offsets are read on
 * the device only; offsets outside [0, Kt] are clamped.
 * Scale grids are read in aligned 4-byte words, so up to 3 bytes past the end of a_s or b_s (inside the word that
 * holds their last byte) may be read; nothing outside the caller's buffers is ever written.
 */
mxq_status grouped_wgrad_mx(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q, const uint8_t* b_s,
                            const int64_t* group_offsets, int64_t G, int64_t M, int64_t N, int64_t Kt,
                            uint16_t* c_bf16, float* c_f32, hipStream_t stream);

/* Adam hyper-parameters, passed by HOST pointer. step is the 1-based step count t (MXQ_ERR_SHAPE if below 1);
 * beta1 and beta2 lie in [0, 1) (MXQ_ERR_UNSUPPORTED otherwise, NaN included). Every Adam entry point checks both
 * before its early return for an empty tensor, so a call with n == 0 still reports a bad setting. */
typedef struct {
    float lr, beta1, beta2, eps, weight_decay;
    int64_t step;
} mxq_adam_hparams;

/*
 * One precision-decoupled FP8 AdamW step over n parameters held as one tensor ([FP8-LM] AdamW update rule,
 * Eq. 7-8: first moment in FP8 with a per-tensor scale, second moment in FP16, high-precision master weight):
 *   master (fp32, in/out), m_q (E4M3, in/out, m ~ val(m_q) / m_scale), m_scale (fp32[1], in/out), v_fp16 (in/out),
 *   grad_bf16 (in), w_bf16 (out, bf16 copy of the updated weight; may be NULL).
 *   m_t = b1 m + (1-b1) g;  v_t = b2 v + (1-b2) g^2;  c1 = 1/(1-b1^t), c2 = 1/(1-b2^t);
 *   theta -= lr ((m_t c1) / (sqrt(v_t c2) + eps) + wd theta);
 *   the new first-moment scale is 448 / max(amax(m_t), 1e-12) (current scaling), and m_q = E4M3(m_t * scale).
 * Every fp32 operation is rounded separately (no fused multiply-add); sqrt and division are correctly rounded; the
 * bias-correction scalars are computed on the host in double and rounded once to float, b^t as the product of t
 * factors (the host loop ends once a further factor changes neither product, so any step count costs bounded time).
 * workspace: device scratch of at least mxq_workspace_bytes("adam", n) bytes, clobbered.
 */
mxq_status fp8_adam_step(float* master, const uint16_t* grad_bf16, uint8_t* m_q, float* m_scale,
                         uint16_t* v_fp16, uint16_t* w_bf16, int64_t n, const mxq_adam_hparams* hp,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The AdamW step of fp8_adam_step fused with the refresh of the weight's MXFP8 caches ([OLMO11] Section 11.3.2 and
 * Figure 55: the cached operand orientations derive from the FP32 main weight and are rebuilt after every update).
 * The n = rows * cols parameters are the weight matrix W[rows][cols] (row-major). After the update:
 *   row orientation:    q_row[rows][cols], s_row[rows][cols/32]   (needs cols % 32 == 0), the forward operand;
 *   column orientation: q_col[cols][rows], s_col[cols][rows/32]   (needs rows % 32 == 0), the dgrad operand;
 * each 32-value block of the updated fp32 master weight quantized as mxq_quantize does (rule = rceil or floor, one
 * rounding from fp32 to E4M3). Either orientation pair may be NULL, not both. All Adam outputs are bit-identical to
 * fp8_adam_step's; w_bf16 may be NULL. Requires cols % 8 == 0. workspace: mxq_workspace_bytes("adam", rows * cols).
 */
mxq_status fp8_adam_step_mx_cache(float* master, const uint16_t* grad_bf16, uint8_t* m_q, float* m_scale,
                                  uint16_t* v_fp16, uint16_t* w_bf16, int64_t rows, int64_t cols, uint8_t* q_row,
                                  uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, mxq_scale_rule rule,
                                  const mxq_adam_hparams* hp, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * The same AdamW step with a delayed first-moment scale, in one pass over the state (no amax pre-pass; [FP8-LM]
 * Section 3.4, tensor-scaled first moment with delayed scaling):
 *   s_new = 448 / max(max(m_history), 1e-12) from the amax of m of earlier steps encodes this step's m_t;
 *   m_scale[0] <- s_new; the amax of this step's m_t is stored at m_history[pos], and pos = (pos + 1) % history_len.
 * m_history: device float[history_len], hist_pos: device int32[1], both in/out (1 <= history_len <= 2^20). Every
 * other output is computed exactly as in fp8_adam_step. An all-zero history saturates m (seed it, for example with the
 * amax one current-scaling step reports). workspace: mxq_workspace_bytes("adam_delayed", n) bytes, clobbered.
 */
mxq_status fp8_adam_step_delayed(float* master, const uint16_t* grad_bf16, uint8_t* m_q, float* m_scale,
                                 uint16_t* v_fp16, uint16_t* w_bf16, int64_t n, const mxq_adam_hparams* hp,
                                 float* m_history, int32_t* hist_pos, int64_t history_len, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes needed by op ("pertensor", "adam", "pertensor_delayed", "adam_delayed" or "autoscale") for n
 * elements; 0 for an unknown op. op is a host string. */
size_t mxq_workspace_bytes(const char* op, int64_t n);

#ifdef __cplusplus
}
#endif
#endif /* MXQ_H */
