// Routed-expert backward quantizers for gfx950 ("OLMo-core MoE, Section 11: MXFP8 Training", Section 11.4.1,
// backward of the routed experts, and Section 11.4.4, Table 25: route weighting fused with the gradient quantize;
// MXFP8 qdata and scales passed straight between adjacent backward stages that agree on layout).
//
// The kernels produce fp32 values in registers and quantize them to MXFP8 in both orientations in the same pass:
//   route_weighted_mx_kernel  x[r][c] = p[r] * dy[r][c]  (the combine backward's route weighting)
//   swiglu_bwd_mx_kernel      (d_gate | d_up) of h = silu(g) u for the incoming gradient dh
//   swiglu_fwd_mx_kernel      h = silu(g) u itself, when the forward also saves h for the down projection's Wgrad
// The row orientation (blocks along the row) feeds the next dgrad; the column orientation (blocks of 32 routed rows,
// stored transposed) feeds the Wgrad contraction over each expert's token rows.
//
// Tiles: 64 rows x 128 columns per 256-thread workgroup. Thread t owns 8 consecutive columns (t % 16) of rows
// t / 16 + 16 j (j < 4), loaded with 16-byte accesses; the 4 lanes of a quad cover one 32-value row block. Column
// blocks go through an fp32 LDS tile: thread t reads column t % 128, rows 32 (t / 128) .. +31.
// Every fp32 operation is rounded on its own: contraction into fused multiply-adds is disabled for this file.
#pragma clang fp contract(off)
#include "mxq_device.h"
#include "launch.h"

namespace mxq {

constexpr int MT_ROWS = 64, MT_COLS = 128, MT_THREADS = 256;

// Column orientation of one 32-row block: the fp32 values d[0..31] of tile column c (rows grow .. grow+31) become
// one E8M0 byte and 32 codes, stored at output column oc0 + c (skipped for columns at or past climit and for a
// block past the last row).
template <int RULE>
__device__ __forceinline__ void mx_col_block_out(const float (&d)[32], int64_t c0, int c, int64_t grow, int64_t climit,
                                                 int64_t oc0, int64_t rows, uint8_t* __restrict__ q_col,
                                                 uint8_t* __restrict__ s_col) {
    uint32_t m = 0;
#pragma unroll
    for (int r = 0; r < 32; ++r) m = max(m, __float_as_uint(d[r]) & 0x7FFFFFFFu);
    const uint32_t byte = mx_scale_byte_f32(m, RULE);
    const float f = mx_inv_scale_f32(byte);
    uint32_t out[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float y0 = clamp_keep_nan(d[4 * q] * f, 448.0f), y1 = clamp_keep_nan(d[4 * q + 1] * f, 448.0f);
        const float y2 = clamp_keep_nan(d[4 * q + 2] * f, 448.0f), y3 = clamp_keep_nan(d[4 * q + 3] * f, 448.0f);
        out[q] = cvt_f32_pair<FMT_E4M3, true>(cvt_f32_pair<FMT_E4M3, false>(0u, y0, y1), y2, y3);
    }
    if (c0 + c < climit && grow + 32 <= rows) {
        const int64_t ocol = oc0 + c;
        uint4* q = reinterpret_cast<uint4*>(q_col + ocol * rows + grow);
        q[0] = make_uint4(out[0], out[1], out[2], out[3]);
        q[1] = make_uint4(out[4], out[5], out[6], out[7]);
        s_col[ocol * (rows / 32) + grow / 32] = (uint8_t)byte;
    }
}

// Quantize the tile's fp32 values x[j][e] (row r0 + t/16 + 16 j, column c0 + 8 (t % 16) + e of the input) into the
// output matrix [rows][ocols] at output column oc0 + (column - c0). Columns at or past climit are outside the input
// (their x are 0 and nothing is stored for them). climit and ocols are multiples of 32, rows a multiple of 32.
template <int RULE, bool ROW, bool COL>
__device__ __forceinline__ void mx_tile_out(const float (&x)[4][8], float* tile, int64_t r0, int64_t c0,
                                            int64_t climit, int64_t oc0, int64_t rows, int64_t ocols,
                                            uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
                                            uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col) {
    const int tid = threadIdx.x;
    const int ch = tid & 15, rr = tid >> 4;
    const bool col_ok = c0 + 8 * ch < climit;
    const int64_t oc = oc0 + 8 * ch;
    if constexpr (ROW) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t gr = r0 + rr + 16 * j;
            uint32_t m = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) m = max(m, __float_as_uint(x[j][e]) & 0x7FFFFFFFu);
            m = quad_max(m);
            const uint32_t byte = mx_scale_byte_f32(m, RULE);
            const float f = mx_inv_scale_f32(byte);
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = clamp_keep_nan(x[j][e] * f, 448.0f);
            const uint32_t lo = cvt_f32_pair<FMT_E4M3, true>(cvt_f32_pair<FMT_E4M3, false>(0u, y[0], y[1]), y[2], y[3]);
            const uint32_t hi = cvt_f32_pair<FMT_E4M3, true>(cvt_f32_pair<FMT_E4M3, false>(0u, y[4], y[5]), y[6], y[7]);
            if (col_ok && gr < rows) {
                stnt8(q_row + gr * ocols + oc, make_uint2(lo, hi));
                if ((ch & 3) == 0) s_row[gr * (ocols / 32) + oc / 32] = (uint8_t)byte;
            }
        }
    }
    if constexpr (COL) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float* dst = &tile[(rr + 16 * j) * MT_COLS + 8 * ch];
            *reinterpret_cast<float4*>(dst) = make_float4(x[j][0], x[j][1], x[j][2], x[j][3]);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(x[j][4], x[j][5], x[j][6], x[j][7]);
        }
        __syncthreads();
        const int c = tid & (MT_COLS - 1), b = tid >> 7;
        float d[32];
#pragma unroll
        for (int r = 0; r < 32; ++r) d[r] = tile[(32 * b + r) * MT_COLS + c];
        __syncthreads();                                      // the tile may be refilled after this
        mx_col_block_out<RULE>(d, c0, c, r0 + 32 * b, climit, oc0, rows, q_col, s_col);
    }
}

// ---------------------------------------------------------------------------------------- route-weighted gradient
template <int RULE, bool ROW, bool COL>
__global__ __launch_bounds__(MT_THREADS) void route_weighted_mx_kernel(const uint16_t* __restrict__ dy,
                                                                      const float* __restrict__ p, int64_t rows,
                                                                      int64_t cols, uint8_t* q_row, uint8_t* s_row,
                                                                      uint8_t* q_col, uint8_t* s_col) {
    // The column orientation keeps the tile's bf16 gradient and its rows' route weights in LDS (16.25 KiB, so twice
    // as many workgroups fit on a CU as with an fp32 tile) and forms each product again: p * dy is one fp32
    // multiply, so both orientations quantize the same values.
    __shared__ __attribute__((aligned(16))) uint16_t tile[COL ? MT_ROWS * MT_COLS : 1];
    __shared__ float pw[COL ? MT_ROWS : 1];
    const int tid = threadIdx.x;
    const int ch = tid & 15, rr = tid >> 4;
    const int64_t r0 = (int64_t)blockIdx.y * MT_ROWS, c0 = (int64_t)blockIdx.x * MT_COLS;
    const int64_t gc = c0 + 8 * ch;
    float x[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t gr = r0 + rr + 16 * j;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        float w = 0.0f;
        if (gr < rows) w = p[gr];
        if (gc < cols && gr < rows) v = ldnt16(dy + gr * cols + gc);
        const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) x[j][e] = w * ((e & 1) ? bf16_hi(vw[e >> 1]) : bf16_lo(vw[e >> 1]));
        if constexpr (COL) {
            *reinterpret_cast<uint4*>(&tile[(rr + 16 * j) * MT_COLS + 8 * ch]) = v;
            if (ch == 0) pw[rr + 16 * j] = w;
        }
    }
    if constexpr (ROW) mx_tile_out<RULE, true, false>(x, nullptr, r0, c0, cols, c0, rows, cols, q_row, s_row, q_col, s_col);
    if constexpr (COL) {
        __syncthreads();
        const int c = tid & (MT_COLS - 1), b = tid >> 7;
        float d[32];
#pragma unroll
        for (int r = 0; r < 32; ++r) {
            const uint32_t h = tile[(32 * b + r) * MT_COLS + c];
            d[r] = pw[32 * b + r] * __uint_as_float(h << 16);
        }
        mx_col_block_out<RULE>(d, c0, c, r0 + 32 * b, cols, c0, rows, q_col, s_col);
    }
}

// ---------------------------------------------------------------------------------------- SwiGLU forward, saved
// h = silu(g) u of the forward, quantized in both orientations in one pass: the row orientation feeds the down
// projection, the column orientation is the down projection's Wgrad operand, saved explicitly in the RHS layout.
template <int RULE, bool ROW, bool COL>
__global__ __launch_bounds__(MT_THREADS) void swiglu_fwd_mx_kernel(const uint16_t* __restrict__ c, int64_t rows,
                                                                  int64_t F, uint8_t* q_row, uint8_t* s_row,
                                                                  uint8_t* q_col, uint8_t* s_col) {
    __shared__ __attribute__((aligned(16))) float tile[COL ? MT_ROWS * MT_COLS : 1];
    const int tid = threadIdx.x;
    const int ch = tid & 15, rr = tid >> 4;
    const int64_t r0 = (int64_t)blockIdx.y * MT_ROWS, c0 = (int64_t)blockIdx.x * MT_COLS;
    const int64_t gc = c0 + 8 * ch;
    float x[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t gr = r0 + rr + 16 * j;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[j][e] = 0.0f;
        if (gc < F && gr < rows) {
            const uint4 gv = ldnt16(c + gr * 2 * F + gc);
            const uint4 uv = ldnt16(c + gr * 2 * F + F + gc);
            const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w}, uw[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float g = (e & 1) ? bf16_hi(gw[e >> 1]) : bf16_lo(gw[e >> 1]);
                const float u = (e & 1) ? bf16_hi(uw[e >> 1]) : bf16_lo(uw[e >> 1]);
                x[j][e] = swiglu_f32(g, u);
            }
        }
    }
    mx_tile_out<RULE, ROW, COL>(x, tile, r0, c0, F, c0, rows, F, q_row, s_row, q_col, s_col);
}

// ---------------------------------------------------------------------------------------- SwiGLU backward
// h = silu(g) u, silu(g) = g / (1 + e^-g) (the forward's value), sigma = 1 / (1 + e^-g),
// silu'(g) = sigma (1 + g (1 - sigma)); d_gate = (dh u) silu'(g), d_up = dh silu(g). One rounding per operation,
// in this order.
__device__ __forceinline__ void swiglu_bwd_f32(float g, float u, float dh, float& d_gate, float& d_up) {
    const float e = exp_fixed(-g);
    const float d = 1.0f + e;
    const float silu = g / d;
    const float sig = 1.0f / d;
    const float one_m = 1.0f - sig;
    float t = g * one_m;
    t = 1.0f + t;
    const float ds = sig * t;
    const float du = dh * u;
    d_gate = du * ds;
    d_up = dh * silu;
}

// A tile covers columns c0 .. c0+127 of the gate and of the up halves: the gate half's gradients go to output
// columns c0 + ..., the up half's to F + c0 + ... of dc[rows][2F]; g, u and dh are each read once.
template <int RULE, bool ROW, bool COL>
__global__ __launch_bounds__(MT_THREADS) void swiglu_bwd_mx_kernel(const uint16_t* __restrict__ c,
                                                                  const uint16_t* __restrict__ dh, int64_t rows,
                                                                  int64_t F, uint8_t* q_row, uint8_t* s_row,
                                                                  uint8_t* q_col, uint8_t* s_col) {
    __shared__ __attribute__((aligned(16))) float tile[COL ? MT_ROWS * MT_COLS : 1];
    const int tid = threadIdx.x;
    const int ch = tid & 15, rr = tid >> 4;
    const int64_t r0 = (int64_t)blockIdx.y * MT_ROWS, c0 = (int64_t)blockIdx.x * MT_COLS;
    const int64_t gc = c0 + 8 * ch;
    float xg[4][8], xu[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t gr = r0 + rr + 16 * j;
#pragma unroll
        for (int e = 0; e < 8; ++e) { xg[j][e] = 0.0f; xu[j][e] = 0.0f; }
        if (gc < F && gr < rows) {
            const uint4 gv = ldnt16(c + gr * 2 * F + gc);
            const uint4 uv = ldnt16(c + gr * 2 * F + F + gc);
            const uint4 hv = ldnt16(dh + gr * F + gc);
            const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w}, uw[4] = {uv.x, uv.y, uv.z, uv.w};
            const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float g = (e & 1) ? bf16_hi(gw[e >> 1]) : bf16_lo(gw[e >> 1]);
                const float u = (e & 1) ? bf16_hi(uw[e >> 1]) : bf16_lo(uw[e >> 1]);
                const float h = (e & 1) ? bf16_hi(hw[e >> 1]) : bf16_lo(hw[e >> 1]);
                swiglu_bwd_f32(g, u, h, xg[j][e], xu[j][e]);
            }
        }
    }
    mx_tile_out<RULE, ROW, COL>(xg, tile, r0, c0, F, c0, rows, 2 * F, q_row, s_row, q_col, s_col);
    mx_tile_out<RULE, ROW, COL>(xu, tile, r0, c0, F, F + c0, rows, 2 * F, q_row, s_row, q_col, s_col);
}

// ---------------------------------------------------------------------------------------- launchers
#define MXQ_MT_DISPATCH(KERNEL, GRID, ...)                                                                  \
    do {                                                                                                   \
        if (rule == RULE_FLOOR) {                                                                          \
            if (row && col) hipLaunchKernelGGL((KERNEL<RULE_FLOOR, true, true>), GRID, dim3(MT_THREADS), 0, stream, __VA_ARGS__); \
            else if (row) hipLaunchKernelGGL((KERNEL<RULE_FLOOR, true, false>), GRID, dim3(MT_THREADS), 0, stream, __VA_ARGS__); \
            else hipLaunchKernelGGL((KERNEL<RULE_FLOOR, false, true>), GRID, dim3(MT_THREADS), 0, stream, __VA_ARGS__); \
        } else {                                                                                           \
            if (row && col) hipLaunchKernelGGL((KERNEL<RULE_RCEIL, true, true>), GRID, dim3(MT_THREADS), 0, stream, __VA_ARGS__); \
            else if (row) hipLaunchKernelGGL((KERNEL<RULE_RCEIL, true, false>), GRID, dim3(MT_THREADS), 0, stream, __VA_ARGS__); \
            else hipLaunchKernelGGL((KERNEL<RULE_RCEIL, false, true>), GRID, dim3(MT_THREADS), 0, stream, __VA_ARGS__); \
        }                                                                                                  \
    } while (0)

hipError_t launch_route_weighted_mx_quantize(const uint16_t* dy, const float* p, int64_t rows, int64_t cols,
                                             uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, int rule,
                                             hipStream_t stream) {
    const bool row = q_row != nullptr, col = q_col != nullptr;
    const dim3 grid((unsigned)((cols + MT_COLS - 1) / MT_COLS), (unsigned)((rows + MT_ROWS - 1) / MT_ROWS));
    MXQ_MT_DISPATCH(route_weighted_mx_kernel, grid, dy, p, rows, cols, q_row, s_row, q_col, s_col);
    return hipGetLastError();
}

hipError_t launch_swiglu_bwd_mx_quantize(const uint16_t* c, const uint16_t* dh, int64_t rows, int64_t F,
                                         uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, int rule,
                                         hipStream_t stream) {
    const bool row = q_row != nullptr, col = q_col != nullptr;
    const dim3 grid((unsigned)((F + MT_COLS - 1) / MT_COLS), (unsigned)((rows + MT_ROWS - 1) / MT_ROWS));
    MXQ_MT_DISPATCH(swiglu_bwd_mx_kernel, grid, c, dh, rows, F, q_row, s_row, q_col, s_col);
    return hipGetLastError();
}

hipError_t launch_swiglu_mx_quantize_oriented(const uint16_t* c, int64_t rows, int64_t F, uint8_t* q_row,
                                              uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, int rule,
                                              hipStream_t stream) {
    const bool row = q_row != nullptr, col = q_col != nullptr;
    const dim3 grid((unsigned)((F + MT_COLS - 1) / MT_COLS), (unsigned)((rows + MT_ROWS - 1) / MT_ROWS));
    MXQ_MT_DISPATCH(swiglu_fwd_mx_kernel, grid, c, rows, F, q_row, s_row, q_col, s_col);
    return hipGetLastError();
}

#undef MXQ_MT_DISPATCH

}  // namespace mxq
