// Host-side launchers of the gfx950 kernels (internal to libmxq; the public C ABI is include/mxq.h).
// Each launcher enqueues on `stream` and returns the launch status; arguments are validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

struct AdamConsts {
    float b1, ob1, b2, ob2, c1, c2, lr, eps, wd;
};

hipError_t launch_mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q_row, uint8_t* s_row,
                              uint8_t* q_col, uint8_t* s_col, int rule, hipStream_t stream);

// mxq_quantize plus the range words of each emitted orientation (1 if a 64-value window is wide, else 0).
hipError_t launch_mx_quantize_ranged(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q_row, uint8_t* s_row,
                                     uint8_t* q_col, uint8_t* s_col, int rule, uint32_t* wide_row,
                                     uint32_t* wide_col, hipStream_t stream);

int pertensor_amax_parts(int64_t n);
// The device scratch of the allocation-free per-tensor quantize on the stream's device, and its size in bytes.
hipError_t pertensor_scratch(hipStream_t stream, uint32_t** ptr, size_t* bytes);
hipError_t launch_pertensor_quantize(const uint16_t* x, int64_t rows, int64_t cols, int fmt, float margin,
                                     const float* scale_in, float* amax_out, float* scale_out, uint8_t* q,
                                     uint8_t* q_t, uint32_t* partial, hipStream_t stream);

hipError_t launch_pertensor_quantize_delayed(const uint16_t* x, int64_t rows, int64_t cols, int fmt, float margin,
                                             float* hist, int32_t* pos, int H, float* amax_out, float* scale_out,
                                             uint8_t* q, uint8_t* q_t, uint32_t* amax_word, hipStream_t stream);

hipError_t launch_swiglu_mx_quantize(const uint16_t* c, int64_t rows, int64_t F, uint8_t* q, uint8_t* s, int rule,
                                     hipStream_t stream);

// GEMM paths: CHECKED takes the FP8 instruction only for large tiles at K >= 12288 whose operands pass the device-side
// range check (else the exact path); RANGED decides the same way from the operands' range words (a_wide, b_wide)
// instead of checking; EXACT dequantizes to bf16 for the bf16 instruction at every K; FP8 takes the FP8 instruction
// at every K.
enum : int { GEMM_PATH_CHECKED = 0, GEMM_PATH_EXACT = 1, GEMM_PATH_FP8 = 2, GEMM_PATH_RANGED = 3 };
hipError_t launch_scaled_gemm(const uint8_t* a_q, const void* a_scale, int a_fmt, const uint8_t* b_q,
                              const void* b_scale, int b_fmt, int64_t M, int64_t N, int64_t K, int mx,
                              uint16_t* c, int64_t ldc, int path, const uint32_t* a_wide, const uint32_t* b_wide,
                              hipStream_t stream);

hipError_t launch_grouped_gemm(const uint8_t* a_q, const uint8_t* a_s, const int64_t* offsets, int64_t G,
                               int64_t total_rows, const uint8_t* b_q, const uint8_t* b_s, int64_t ldb,
                               int64_t b_gstride, int64_t ldsb, int64_t sb_gstride, int64_t N, int64_t K,
                               uint16_t* c, int64_t ldc, hipStream_t stream);
hipError_t launch_grouped_wgrad(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q, const uint8_t* b_s,
                                const int64_t* offsets, int64_t G, int64_t M, int64_t N, int64_t Kt, uint16_t* c,
                                float* cf, hipStream_t stream);

hipError_t launch_route_weighted_mx_quantize(const uint16_t* dy, const float* p, int64_t rows, int64_t cols,
                                             uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, int rule,
                                             hipStream_t stream);
hipError_t launch_swiglu_mx_quantize_oriented(const uint16_t* c, int64_t rows, int64_t F, uint8_t* q_row,
                                              uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, int rule,
                                              hipStream_t stream);
hipError_t launch_swiglu_bwd_mx_quantize(const uint16_t* c, const uint16_t* dh, int64_t rows, int64_t F,
                                         uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, int rule,
                                         hipStream_t stream);

hipError_t launch_autoscale_cast(const uint16_t* g, int64_t n, int fmt, float* mu, uint8_t* q, float* scale_out,
                                 unsigned long long* overflow, unsigned long long* count, hipStream_t stream);
hipError_t launch_requantize_shared(const uint8_t* q_in, int64_t n, int fmt_in, const float* scale_in,
                                    const float* scales, int nranks, int fmt_out, uint8_t* q_out, float* shared_out,
                                    float* sum_out, hipStream_t stream);

int adam_parts(int64_t n);
hipError_t launch_adam(float* master, const uint16_t* grad, uint8_t* m_q, float* m_scale, uint16_t* v16, uint16_t* w,
                       int64_t n, const AdamConsts& k, uint32_t* partial, float* consts, hipStream_t stream);
hipError_t launch_adam_weight_cache(float* master, const uint16_t* grad, uint8_t* m_q, float* m_scale, uint16_t* v16,
                                    uint16_t* w, int64_t rows, int64_t cols, uint8_t* q_row, uint8_t* s_row,
                                    uint8_t* q_col, uint8_t* s_col, int rule, const AdamConsts& k, uint32_t* partial,
                                    float* consts, hipStream_t stream);
hipError_t launch_adam_delayed(float* master, const uint16_t* grad, uint8_t* m_q, float* m_scale, uint16_t* v16,
                               uint16_t* w, int64_t n, const AdamConsts& k, float* hist, int32_t* pos, int H,
                               float* consts, uint32_t* amax_word, hipStream_t stream);

}  // namespace mxq
