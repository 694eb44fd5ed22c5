// C ABI of libmxq (declared in include/mxq.h): argument validation on the host, then kernel launches.
// Validation happens before any HIP call, so every error path returns without touching the device.
#include <stdint.h>
#include <string.h>

#include "launch.h"
#include "mxq.h"

namespace {

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool al4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
mxq_status hip_status(hipError_t e) { return e == hipSuccess ? MXQ_OK : MXQ_ERR_HIP; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

size_t pertensor_ws(int64_t n) { return round_up((size_t)mxq::pertensor_amax_parts(n) * 4u, 256); }
size_t adam_ws(int64_t n) { return round_up((size_t)mxq::adam_parts(n) * 4u, 256) + 256; }
constexpr size_t kDelayedWs = 256;   // delayed modes: the atomic amax word (and Adam's three constants)
constexpr int64_t kMaxHistory = 1 << 20;

constexpr int64_t kMaxGridY = 65535;

// Adam's moment decay rates lie in [0, 1): the bias corrections divide by 1 - beta^t. NaN fails both comparisons.
bool betas_ok(const mxq_adam_hparams& hp) {
    return hp.beta1 >= 0.0f && hp.beta1 < 1.0f && hp.beta2 >= 0.0f && hp.beta2 < 1.0f;
}

// Adam's host scalars in double, each rounded once to float. beta^t is the product of t factors. The loop stops
// once one more factor would change neither product: from there on every further factor returns the same values
// (0, 1, or the smallest subnormal, where beta >= 0.5 leaves it in place), so the result equals the full product
// and the time taken is bounded for any step count. A NaN product also stays NaN.
mxq::AdamConsts adam_consts(const mxq_adam_hparams& hp) {
    double p1 = 1.0, p2 = 1.0;
    for (int64_t t = 0; t < hp.step; ++t) {
        const double n1 = p1 * (double)hp.beta1, n2 = p2 * (double)hp.beta2;
        const bool fixed = (n1 == p1 || (n1 != n1 && p1 != p1)) && (n2 == p2 || (n2 != n2 && p2 != p2));
        p1 = n1;
        p2 = n2;
        if (fixed) break;
    }
    mxq::AdamConsts k;
    k.b1 = hp.beta1;
    k.ob1 = (float)(1.0 - (double)hp.beta1);
    k.b2 = hp.beta2;
    k.ob2 = (float)(1.0 - (double)hp.beta2);
    k.c1 = (float)(1.0 / (1.0 - p1));
    k.c2 = (float)(1.0 / (1.0 - p2));
    k.lr = hp.lr;
    k.eps = hp.eps;
    k.wd = hp.weight_decay;
    return k;
}

}  // namespace

extern "C" {

const char* mxq_status_string(mxq_status s) {
    switch (s) {
        case MXQ_OK: return "ok";
        case MXQ_ERR_NULL: return "a required pointer is NULL";
        case MXQ_ERR_SHAPE: return "a size is negative or not divisible as the operation requires";
        case MXQ_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case MXQ_ERR_UNSUPPORTED: return "unsupported format, rule, scaling mode or optimizer setting";
        case MXQ_ERR_WORKSPACE: return "workspace missing or too small";
        case MXQ_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

int mxq_abi_version(void) { return 1; }

size_t mxq_workspace_bytes(const char* op, int64_t n) {
    if (!op || n < 0) return 0;
    if (strcmp(op, "pertensor") == 0) return pertensor_ws(n);
    if (strcmp(op, "adam") == 0) return adam_ws(n);
    if (strcmp(op, "pertensor_delayed") == 0 || strcmp(op, "adam_delayed") == 0 || strcmp(op, "autoscale") == 0)
        return kDelayedWs;
    return 0;
}

mxq_status mxq_quantize(const uint16_t* x_bf16, int64_t rows, int64_t cols, uint8_t* q_row, uint8_t* s_row,
                        uint8_t* q_col, uint8_t* s_col, mxq_scale_rule rule, hipStream_t stream) {
    if ((q_row == nullptr) != (s_row == nullptr) || (q_col == nullptr) != (s_col == nullptr)) return MXQ_ERR_NULL;
    const bool row = q_row != nullptr, col = q_col != nullptr;
    if (!row && !col) return MXQ_ERR_NULL;
    if (rule != MXQ_SCALE_RCEIL && rule != MXQ_SCALE_FLOOR) return MXQ_ERR_UNSUPPORTED;
    if (rows < 0 || cols < 0 || cols % 8 != 0) return MXQ_ERR_SHAPE;
    if ((row && cols % 32 != 0) || (col && rows % 32 != 0)) return MXQ_ERR_SHAPE;
    if ((rows + 127) / 128 > kMaxGridY) return MXQ_ERR_SHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;                 // empty: nothing to read or write
    if (!x_bf16) return MXQ_ERR_NULL;
    if (!al16(x_bf16) || (row && !al16(q_row)) || (col && !al16(q_col))) return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_mx_quantize(x_bf16, rows, cols, q_row, s_row, q_col, s_col, (int)rule, stream));
}

mxq_status mxq_quantize_ranged(const uint16_t* x_bf16, int64_t rows, int64_t cols, uint8_t* q_row, uint8_t* s_row,
                               uint8_t* q_col, uint8_t* s_col, mxq_scale_rule rule, uint32_t* wide_row,
                               uint32_t* wide_col, hipStream_t stream) {
    if ((q_row == nullptr) != (s_row == nullptr) || (q_col == nullptr) != (s_col == nullptr)) return MXQ_ERR_NULL;
    const bool row = q_row != nullptr, col = q_col != nullptr;
    if (!row && !col) return MXQ_ERR_NULL;
    if ((row && !wide_row) || (col && !wide_col)) return MXQ_ERR_NULL;
    if (rule != MXQ_SCALE_RCEIL && rule != MXQ_SCALE_FLOOR) return MXQ_ERR_UNSUPPORTED;
    if (rows < 0 || cols < 0 || cols % 8 != 0) return MXQ_ERR_SHAPE;
    if ((row && cols % 64 != 0) || (col && rows % 64 != 0)) return MXQ_ERR_SHAPE;   // whole 64-value windows
    if ((rows + 127) / 128 > kMaxGridY) return MXQ_ERR_SHAPE;
    if ((row && !al4(wide_row)) || (col && !al4(wide_col))) return MXQ_ERR_ALIGN;
    if (rows == 0 || cols == 0) {
        // nothing to quantize; the words still say "no wide window"
        return hip_status(mxq::launch_mx_quantize_ranged(x_bf16, 0, 0, q_row, s_row, q_col, s_col, (int)rule,
                                                         wide_row, wide_col, stream));
    }
    if (!x_bf16) return MXQ_ERR_NULL;
    if (!al16(x_bf16) || (row && !al16(q_row)) || (col && !al16(q_col))) return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_mx_quantize_ranged(x_bf16, rows, cols, q_row, s_row, q_col, s_col, (int)rule,
                                                     wide_row, wide_col, stream));
}

mxq_status swiglu_mx_quantize(const uint16_t* c_bf16, int64_t rows, int64_t F, uint8_t* q, uint8_t* s,
                              mxq_scale_rule rule, hipStream_t stream) {
    if (rule != MXQ_SCALE_RCEIL && rule != MXQ_SCALE_FLOOR) return MXQ_ERR_UNSUPPORTED;
    if (rows < 0 || F < 0 || F % 32 != 0) return MXQ_ERR_SHAPE;
    if (rows == 0 || F == 0) return MXQ_OK;
    if (!c_bf16 || !q || !s) return MXQ_ERR_NULL;
    if (!al16(c_bf16) || !al16(q)) return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_swiglu_mx_quantize(c_bf16, rows, F, q, s, (int)rule, stream));
}

mxq_status swiglu_mx_quantize_oriented(const uint16_t* c_bf16, int64_t rows, int64_t F, uint8_t* q_row,
                                       uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, mxq_scale_rule rule,
                                       hipStream_t stream) {
    if ((q_row == nullptr) != (s_row == nullptr) || (q_col == nullptr) != (s_col == nullptr)) return MXQ_ERR_NULL;
    if (q_row == nullptr && q_col == nullptr) return MXQ_ERR_NULL;
    if (rule != MXQ_SCALE_RCEIL && rule != MXQ_SCALE_FLOOR) return MXQ_ERR_UNSUPPORTED;
    if (rows < 0 || F < 0 || F % 32 != 0 || rows % 32 != 0) return MXQ_ERR_SHAPE;
    if ((rows + 63) / 64 > kMaxGridY) return MXQ_ERR_SHAPE;
    if (rows == 0 || F == 0) return MXQ_OK;
    if (!c_bf16) return MXQ_ERR_NULL;
    if (!al16(c_bf16) || (q_row && !al16(q_row)) || (q_col && !al16(q_col))) return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_swiglu_mx_quantize_oriented(c_bf16, rows, F, q_row, s_row, q_col, s_col, (int)rule,
                                                              stream));
}

mxq_status route_weighted_mx_quantize(const uint16_t* dy_bf16, const float* route_w, int64_t rows, int64_t cols,
                                      uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                                      mxq_scale_rule rule, hipStream_t stream) {
    if ((q_row == nullptr) != (s_row == nullptr) || (q_col == nullptr) != (s_col == nullptr)) return MXQ_ERR_NULL;
    if (q_row == nullptr && q_col == nullptr) return MXQ_ERR_NULL;
    if (rule != MXQ_SCALE_RCEIL && rule != MXQ_SCALE_FLOOR) return MXQ_ERR_UNSUPPORTED;
    if (rows < 0 || cols < 0 || cols % 32 != 0 || rows % 32 != 0) return MXQ_ERR_SHAPE;
    if ((rows + 63) / 64 > kMaxGridY) return MXQ_ERR_SHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!dy_bf16 || !route_w) return MXQ_ERR_NULL;
    if (!al16(dy_bf16) || !al4(route_w) || (q_row && !al16(q_row)) || (q_col && !al16(q_col))) return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_route_weighted_mx_quantize(dy_bf16, route_w, rows, cols, q_row, s_row, q_col, s_col,
                                                             (int)rule, stream));
}

mxq_status swiglu_backward_mx_quantize(const uint16_t* c_bf16, const uint16_t* dh_bf16, int64_t rows, int64_t F,
                                       uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                                       mxq_scale_rule rule, hipStream_t stream) {
    if ((q_row == nullptr) != (s_row == nullptr) || (q_col == nullptr) != (s_col == nullptr)) return MXQ_ERR_NULL;
    if (q_row == nullptr && q_col == nullptr) return MXQ_ERR_NULL;
    if (rule != MXQ_SCALE_RCEIL && rule != MXQ_SCALE_FLOOR) return MXQ_ERR_UNSUPPORTED;
    if (rows < 0 || F < 0 || F % 32 != 0 || rows % 32 != 0) return MXQ_ERR_SHAPE;
    if ((rows + 63) / 64 > kMaxGridY) return MXQ_ERR_SHAPE;
    if (rows == 0 || F == 0) return MXQ_OK;
    if (!c_bf16 || !dh_bf16) return MXQ_ERR_NULL;
    if (!al16(c_bf16) || !al16(dh_bf16) || (q_row && !al16(q_row)) || (q_col && !al16(q_col))) return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_swiglu_bwd_mx_quantize(c_bf16, dh_bf16, rows, F, q_row, s_row, q_col, s_col,
                                                         (int)rule, stream));
}

mxq_status fp8_quantize_pertensor(const uint16_t* x_bf16, int64_t rows, int64_t cols, mxq_fp8 fmt, float margin,
                                  const float* scale_in, float* amax_out, float* scale_out, uint8_t* q, uint8_t* q_t,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!amax_out || !scale_out) return MXQ_ERR_NULL;
    if (fmt != MXQ_E4M3 && fmt != MXQ_E5M2) return MXQ_ERR_UNSUPPORTED;
    if (rows < 0 || cols < 0 || cols % 8 != 0) return MXQ_ERR_SHAPE;
    if (q_t && rows % 32 != 0) return MXQ_ERR_SHAPE;
    if ((rows + 127) / 128 > kMaxGridY) return MXQ_ERR_SHAPE;
    if (rows * cols > 0 && !x_bf16) return MXQ_ERR_NULL;       // an empty x still yields amax 0 and its scale
    if (!al16(x_bf16) || (q && !al16(q)) || (q_t && !al16(q_t))) return MXQ_ERR_ALIGN;
    if (!al4(amax_out) || !al4(scale_out) || (scale_in && !al4(scale_in))) return MXQ_ERR_ALIGN;
    const int64_t n = rows * cols;
    if (!workspace || workspace_bytes < pertensor_ws(n)) return MXQ_ERR_WORKSPACE;
    if (!al16(workspace)) return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_pertensor_quantize(x_bf16, rows, cols, (int)fmt, margin, scale_in, amax_out,
                                                     scale_out, q, q_t, static_cast<uint32_t*>(workspace), stream));
}

mxq_status fp8_quantize_pertensor_noalloc(const uint16_t* x_bf16, int64_t rows, int64_t cols, mxq_fp8 fmt,
                                          float margin, const float* scale_in, float* amax_out, float* scale_out,
                                          uint8_t* q, uint8_t* q_t, hipStream_t stream) {
    if (!amax_out || !scale_out) return MXQ_ERR_NULL;
    if (fmt != MXQ_E4M3 && fmt != MXQ_E5M2) return MXQ_ERR_UNSUPPORTED;
    if (rows < 0 || cols < 0 || cols % 8 != 0) return MXQ_ERR_SHAPE;
    if (q_t && rows % 32 != 0) return MXQ_ERR_SHAPE;
    if ((rows + 127) / 128 > kMaxGridY) return MXQ_ERR_SHAPE;
    if (rows * cols > 0 && !x_bf16) return MXQ_ERR_NULL;
    if (!al16(x_bf16) || (q && !al16(q)) || (q_t && !al16(q_t))) return MXQ_ERR_ALIGN;
    if (!al4(amax_out) || !al4(scale_out) || (scale_in && !al4(scale_in))) return MXQ_ERR_ALIGN;
    uint32_t* scratch = nullptr;
    size_t scratch_bytes = 0;
    if (mxq::pertensor_scratch(stream, &scratch, &scratch_bytes) != hipSuccess) return MXQ_ERR_HIP;
    if (pertensor_ws(rows * cols) > scratch_bytes) return MXQ_ERR_WORKSPACE;   // partials would not fit
    return hip_status(mxq::launch_pertensor_quantize(x_bf16, rows, cols, (int)fmt, margin, scale_in, amax_out,
                                                     scale_out, q, q_t, scratch, stream));
}

mxq_status fp8_quantize_pertensor_delayed(const uint16_t* x_bf16, int64_t rows, int64_t cols, mxq_fp8 fmt,
                                          float margin, float* amax_history, int32_t* hist_pos, int64_t history_len,
                                          float* amax_out, float* scale_out, uint8_t* q, uint8_t* q_t,
                                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!amax_out || !scale_out || !amax_history || !hist_pos) return MXQ_ERR_NULL;
    if (fmt != MXQ_E4M3 && fmt != MXQ_E5M2) return MXQ_ERR_UNSUPPORTED;
    if (rows < 0 || cols < 0 || cols % 8 != 0) return MXQ_ERR_SHAPE;
    if (q_t && rows % 32 != 0) return MXQ_ERR_SHAPE;
    if ((rows + 127) / 128 > kMaxGridY) return MXQ_ERR_SHAPE;
    if (history_len < 1 || history_len > kMaxHistory) return MXQ_ERR_SHAPE;
    if (rows * cols > 0 && !x_bf16) return MXQ_ERR_NULL;
    if (!al16(x_bf16) || (q && !al16(q)) || (q_t && !al16(q_t))) return MXQ_ERR_ALIGN;
    if (!al4(amax_out) || !al4(scale_out) || !al4(amax_history) || !al4(hist_pos)) return MXQ_ERR_ALIGN;
    if (!workspace || workspace_bytes < kDelayedWs) return MXQ_ERR_WORKSPACE;
    if (!al16(workspace)) return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_pertensor_quantize_delayed(x_bf16, rows, cols, (int)fmt, margin, amax_history,
                                                             hist_pos, (int)history_len, amax_out, scale_out, q, q_t,
                                                             static_cast<uint32_t*>(workspace), stream));
}

mxq_status fp8_autoscale_cast(const uint16_t* g_bf16, int64_t n, mxq_fp8 fmt, float* mu, uint8_t* q,
                              float* scale_out, uint64_t* overflow_count, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    if (!mu || !overflow_count) return MXQ_ERR_NULL;
    if (fmt != MXQ_E4M3 && fmt != MXQ_E5M2) return MXQ_ERR_UNSUPPORTED;
    if (n < 0) return MXQ_ERR_SHAPE;
    if (n > 0 && (!g_bf16 || !q)) return MXQ_ERR_NULL;
    if (!al16(g_bf16) || !al16(q) || !al4(mu) || (scale_out && !al4(scale_out)) ||
        (reinterpret_cast<uintptr_t>(overflow_count) & 7u))
        return MXQ_ERR_ALIGN;
    if (!workspace || workspace_bytes < kDelayedWs) return MXQ_ERR_WORKSPACE;
    if (!al16(workspace)) return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_autoscale_cast(g_bf16, n, (int)fmt, mu, q, scale_out,
                                                 reinterpret_cast<unsigned long long*>(overflow_count),
                                                 static_cast<unsigned long long*>(workspace), stream));
}

mxq_status fp8_requantize_shared(const uint8_t* q_in, int64_t n, mxq_fp8 fmt_in, const float* scale_in,
                                 const float* gathered_scales, int64_t nranks, mxq_fp8 fmt_out, uint8_t* q_out,
                                 float* shared_scale_out, float* sum_scale_out, hipStream_t stream) {
    if ((fmt_in != MXQ_E4M3 && fmt_in != MXQ_E5M2) || (fmt_out != MXQ_E4M3 && fmt_out != MXQ_E5M2))
        return MXQ_ERR_UNSUPPORTED;
    if (n < 0 || nranks < 1 || nranks > (int64_t(1) << 24)) return MXQ_ERR_SHAPE;
    if (!scale_in || !gathered_scales || !shared_scale_out) return MXQ_ERR_NULL;
    if (n > 0 && (!q_in || !q_out)) return MXQ_ERR_NULL;
    if (!al16(q_in) || !al16(q_out) || !al4(scale_in) || !al4(gathered_scales) || !al4(shared_scale_out) ||
        (sum_scale_out && !al4(sum_scale_out)))
        return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_requantize_shared(q_in, n, (int)fmt_in, scale_in, gathered_scales, (int)nranks,
                                                    (int)fmt_out, q_out, shared_scale_out, sum_scale_out, stream));
}

}  // extern "C"

namespace {

mxq_status scaled_gemm_impl(const uint8_t* a_q, const void* a_scale, mxq_fp8 a_fmt, const uint8_t* b_q,
                            const void* b_scale, mxq_fp8 b_fmt, int64_t M, int64_t N, int64_t K, mxq_scaling scaling,
                            uint16_t* c_bf16, int64_t ldc, int path, hipStream_t stream,
                            const uint32_t* a_wide = nullptr, const uint32_t* b_wide = nullptr) {
    if (scaling != MXQ_PER_TENSOR && scaling != MXQ_MX_BLOCK32) return MXQ_ERR_UNSUPPORTED;
    if ((a_fmt != MXQ_E4M3 && a_fmt != MXQ_E5M2) || (b_fmt != MXQ_E4M3 && b_fmt != MXQ_E5M2)) return MXQ_ERR_UNSUPPORTED;
    if (scaling == MXQ_MX_BLOCK32 && (a_fmt != MXQ_E4M3 || b_fmt != MXQ_E4M3)) return MXQ_ERR_UNSUPPORTED;
    if (M < 0 || N < 0 || K <= 0 || K % 32 != 0 || ldc < N) return MXQ_ERR_SHAPE;
    if (M == 0 || N == 0) return MXQ_OK;                       // empty output: nothing enqueued
    if (!a_q || !b_q || !a_scale || !b_scale || !c_bf16) return MXQ_ERR_NULL;
    if (!al16(a_q) || !al16(b_q) || (reinterpret_cast<uintptr_t>(c_bf16) & 1u)) return MXQ_ERR_ALIGN;
    if (scaling == MXQ_MX_BLOCK32 ? (!al16(a_scale) || !al16(b_scale)) : (!al4(a_scale) || !al4(b_scale)))
        return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_scaled_gemm(a_q, a_scale, (int)a_fmt, b_q, b_scale, (int)b_fmt, M, N, K,
                                              scaling == MXQ_MX_BLOCK32 ? 1 : 0, c_bf16, ldc, path, a_wide, b_wide,
                                              stream));
}

}  // namespace

extern "C" {

mxq_status scaled_gemm(const uint8_t* a_q, const void* a_scale, mxq_fp8 a_fmt, const uint8_t* b_q,
                       const void* b_scale, mxq_fp8 b_fmt, int64_t M, int64_t N, int64_t K, mxq_scaling scaling,
                       uint16_t* c_bf16, int64_t ldc, hipStream_t stream) {
    return scaled_gemm_impl(a_q, a_scale, a_fmt, b_q, b_scale, b_fmt, M, N, K, scaling, c_bf16, ldc,
                            mxq::GEMM_PATH_CHECKED, stream);
}

mxq_status scaled_gemm_exact(const uint8_t* a_q, const void* a_scale, mxq_fp8 a_fmt, const uint8_t* b_q,
                             const void* b_scale, mxq_fp8 b_fmt, int64_t M, int64_t N, int64_t K, mxq_scaling scaling,
                             uint16_t* c_bf16, int64_t ldc, hipStream_t stream) {
    return scaled_gemm_impl(a_q, a_scale, a_fmt, b_q, b_scale, b_fmt, M, N, K, scaling, c_bf16, ldc,
                            mxq::GEMM_PATH_EXACT, stream);
}

mxq_status scaled_gemm_fp8(const uint8_t* a_q, const void* a_scale, mxq_fp8 a_fmt, const uint8_t* b_q,
                           const void* b_scale, mxq_fp8 b_fmt, int64_t M, int64_t N, int64_t K, mxq_scaling scaling,
                           uint16_t* c_bf16, int64_t ldc, hipStream_t stream) {
    return scaled_gemm_impl(a_q, a_scale, a_fmt, b_q, b_scale, b_fmt, M, N, K, scaling, c_bf16, ldc,
                            mxq::GEMM_PATH_FP8, stream);
}

mxq_status scaled_gemm_ranged(const uint8_t* a_q, const uint8_t* a_scale, const uint32_t* a_wide,
                              const uint8_t* b_q, const uint8_t* b_scale, const uint32_t* b_wide, int64_t M,
                              int64_t N, int64_t K, uint16_t* c_bf16, int64_t ldc, hipStream_t stream) {
    if (!a_wide || !b_wide) return MXQ_ERR_NULL;
    if (!al4(a_wide) || !al4(b_wide)) return MXQ_ERR_ALIGN;
    return scaled_gemm_impl(a_q, a_scale, MXQ_E4M3, b_q, b_scale, MXQ_E4M3, M, N, K, MXQ_MX_BLOCK32, c_bf16, ldc,
                            mxq::GEMM_PATH_RANGED, stream, a_wide, b_wide);
}

mxq_status grouped_scaled_gemm(const uint8_t* a_q, const uint8_t* a_s, const int64_t* group_offsets, int64_t G,
                               int64_t total_rows, const uint8_t* b_q, const uint8_t* b_s, int64_t N, int64_t K,
                               uint16_t* c_bf16, hipStream_t stream) {
    if (G < 1 || G > 4096 || total_rows < 0 || N < 1 || K <= 0 || K % 32 != 0) return MXQ_ERR_SHAPE;
    if (!group_offsets || !b_q || !b_s) return MXQ_ERR_NULL;
    if (total_rows == 0) return MXQ_OK;
    if (!a_q || !a_s || !c_bf16) return MXQ_ERR_NULL;
    if (!al16(a_q) || !al16(a_s) || !al16(b_q) || !al16(b_s) || (reinterpret_cast<uintptr_t>(c_bf16) & 1u) ||
        (reinterpret_cast<uintptr_t>(group_offsets) & 7u))
        return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_grouped_gemm(a_q, a_s, group_offsets, G, total_rows, b_q, b_s, K, N * K, K / 32,
                                               N * (K / 32), N, K, c_bf16, N, stream));
}

mxq_status grouped_scaled_gemm_strided(const uint8_t* a_q, const uint8_t* a_s, const int64_t* group_offsets,
                                       int64_t G, int64_t total_rows, const uint8_t* b_q, const uint8_t* b_s,
                                       int64_t ldb, int64_t b_group_stride, int64_t ldbs, int64_t bs_group_stride,
                                       int64_t N, int64_t K, uint16_t* c_bf16, int64_t ldc, hipStream_t stream) {
    if (G < 1 || G > 4096 || total_rows < 0 || N < 1 || K <= 0 || K % 32 != 0) return MXQ_ERR_SHAPE;
    if (ldb < K || ldbs < K / 32 || ldc < N || b_group_stride < 0 || bs_group_stride < 0) return MXQ_ERR_SHAPE;
    if (ldb % 16 != 0 || b_group_stride % 16 != 0) return MXQ_ERR_ALIGN;
    if (!group_offsets || !b_q || !b_s) return MXQ_ERR_NULL;
    if (total_rows == 0) return MXQ_OK;
    if (!a_q || !a_s || !c_bf16) return MXQ_ERR_NULL;
    if (!al16(a_q) || !al16(a_s) || !al16(b_q) || !al16(b_s) || (reinterpret_cast<uintptr_t>(c_bf16) & 1u) ||
        (reinterpret_cast<uintptr_t>(group_offsets) & 7u))
        return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_grouped_gemm(a_q, a_s, group_offsets, G, total_rows, b_q, b_s, ldb, b_group_stride,
                                               ldbs, bs_group_stride, N, K, c_bf16, ldc, stream));
}

mxq_status grouped_wgrad_mx(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q, const uint8_t* b_s,
                            const int64_t* group_offsets, int64_t G, int64_t M, int64_t N, int64_t Kt,
                            uint16_t* c_bf16, float* c_f32, hipStream_t stream) {
    if (G < 1 || G > 4096 || M < 1 || N < 1 || Kt < 0 || Kt % 32 != 0) return MXQ_ERR_SHAPE;
    if ((c_bf16 == nullptr) == (c_f32 == nullptr)) return MXQ_ERR_NULL;       // exactly one output
    if (!group_offsets) return MXQ_ERR_NULL;
    if (Kt > 0 && (!a_q || !a_s || !b_q || !b_s)) return MXQ_ERR_NULL;
    if (!al16(a_q) || !al16(a_s) || !al16(b_q) || !al16(b_s) || (c_bf16 && !al16(c_bf16)) ||
        (c_f32 && !al16(c_f32)) || (reinterpret_cast<uintptr_t>(group_offsets) & 7u))
        return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_grouped_wgrad(a_q, a_s, b_q, b_s, group_offsets, G, M, N, Kt, c_bf16, c_f32,
                                                stream));
}

mxq_status fp8_adam_step(float* master, const uint16_t* grad_bf16, uint8_t* m_q, float* m_scale, uint16_t* v_fp16,
                         uint16_t* w_bf16, int64_t n, const mxq_adam_hparams* hp, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
    if (!hp) return MXQ_ERR_NULL;
    if (n < 0 || hp->step < 1) return MXQ_ERR_SHAPE;
    if (!betas_ok(*hp)) return MXQ_ERR_UNSUPPORTED;
    if (n == 0) return MXQ_OK;                                 // empty: no element and no scale changes
    if (!master || !grad_bf16 || !m_q || !m_scale || !v_fp16) return MXQ_ERR_NULL;
    if (!al16(master) || !al16(grad_bf16) || !al16(m_q) || !al16(v_fp16) || (w_bf16 && !al16(w_bf16)) || !al4(m_scale))
        return MXQ_ERR_ALIGN;
    if (!workspace || workspace_bytes < adam_ws(n)) return MXQ_ERR_WORKSPACE;
    if (!al16(workspace)) return MXQ_ERR_ALIGN;
    const mxq::AdamConsts k = adam_consts(*hp);
    const size_t part_bytes = round_up((size_t)mxq::adam_parts(n) * 4u, 256);
    uint32_t* partial = static_cast<uint32_t*>(workspace);
    float* consts = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + part_bytes);
    return hip_status(mxq::launch_adam(master, grad_bf16, m_q, m_scale, v_fp16, w_bf16, n, k, partial, consts, stream));
}

mxq_status fp8_adam_step_mx_cache(float* master, const uint16_t* grad_bf16, uint8_t* m_q, float* m_scale,
                                  uint16_t* v_fp16, uint16_t* w_bf16, int64_t rows, int64_t cols, uint8_t* q_row,
                                  uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, mxq_scale_rule rule,
                                  const mxq_adam_hparams* hp, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
    if (!hp) return MXQ_ERR_NULL;
    if ((q_row == nullptr) != (s_row == nullptr) || (q_col == nullptr) != (s_col == nullptr)) return MXQ_ERR_NULL;
    const bool row = q_row != nullptr, col = q_col != nullptr;
    if (!row && !col) return MXQ_ERR_NULL;
    if (rule != MXQ_SCALE_RCEIL && rule != MXQ_SCALE_FLOOR) return MXQ_ERR_UNSUPPORTED;
    if (rows < 0 || cols < 0 || cols % 8 != 0 || hp->step < 1) return MXQ_ERR_SHAPE;
    if ((row && cols % 32 != 0) || (col && rows % 32 != 0)) return MXQ_ERR_SHAPE;
    if (!betas_ok(*hp)) return MXQ_ERR_UNSUPPORTED;
    if ((rows + 63) / 64 > kMaxGridY) return MXQ_ERR_SHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!master || !grad_bf16 || !m_q || !m_scale || !v_fp16) return MXQ_ERR_NULL;
    if (!al16(master) || !al16(grad_bf16) || !al16(m_q) || !al16(v_fp16) || (w_bf16 && !al16(w_bf16)) ||
        !al4(m_scale) || (row && !al16(q_row)) || (col && !al16(q_col)))
        return MXQ_ERR_ALIGN;
    const int64_t n = rows * cols;
    if (!workspace || workspace_bytes < adam_ws(n)) return MXQ_ERR_WORKSPACE;
    if (!al16(workspace)) return MXQ_ERR_ALIGN;
    const mxq::AdamConsts k = adam_consts(*hp);
    const size_t part_bytes = round_up((size_t)mxq::adam_parts(n) * 4u, 256);
    uint32_t* partial = static_cast<uint32_t*>(workspace);
    float* consts = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + part_bytes);
    return hip_status(mxq::launch_adam_weight_cache(master, grad_bf16, m_q, m_scale, v_fp16, w_bf16, rows, cols, q_row,
                                                    s_row, q_col, s_col, (int)rule, k, partial, consts, stream));
}

mxq_status fp8_adam_step_delayed(float* master, const uint16_t* grad_bf16, uint8_t* m_q, float* m_scale,
                                 uint16_t* v_fp16, uint16_t* w_bf16, int64_t n, const mxq_adam_hparams* hp,
                                 float* m_history, int32_t* hist_pos, int64_t history_len, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    if (!hp) return MXQ_ERR_NULL;
    if (n < 0 || hp->step < 1 || history_len < 1 || history_len > kMaxHistory) return MXQ_ERR_SHAPE;
    if (!betas_ok(*hp)) return MXQ_ERR_UNSUPPORTED;
    if (n == 0) return MXQ_OK;
    if (!master || !grad_bf16 || !m_q || !m_scale || !v_fp16 || !m_history || !hist_pos) return MXQ_ERR_NULL;
    if (!al16(master) || !al16(grad_bf16) || !al16(m_q) || !al16(v_fp16) || (w_bf16 && !al16(w_bf16)) ||
        !al4(m_scale) || !al4(m_history) || !al4(hist_pos))
        return MXQ_ERR_ALIGN;
    if (!workspace || workspace_bytes < kDelayedWs) return MXQ_ERR_WORKSPACE;
    if (!al16(workspace)) return MXQ_ERR_ALIGN;
    const mxq::AdamConsts k = adam_consts(*hp);
    uint32_t* amax_word = static_cast<uint32_t*>(workspace);
    float* consts = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + 16);
    return hip_status(mxq::launch_adam_delayed(master, grad_bf16, m_q, m_scale, v_fp16, w_bf16, n, k, m_history,
                                               hist_pos, (int)history_len, consts, amax_word, stream));
}

}  // extern "C"
