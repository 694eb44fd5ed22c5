// Operand quantization kernels for gfx950: MXFP8 (32-value blocks, E8M0 scales, row and column orientation)
// and per-tensor scaled E4M3/E5M2 (current or delayed scaling).
//
// MXFP8 follows "OLMo-core MoE, Section 11: MXFP8 Training": Eq. 58 (q = E4M3(x/s), power-of-two s per block of
// 32 along the reduction dimension), Section 11.3.5 / Table 24 (rceil and floor scale rules) and Eq. 60 (forward,
// dgrad and wgrad need both orientations). Per-tensor scaling follows "3.8 Mixed Precision, bf16 & FP8 Training"
// (per-tensor scale from amax, Exercise 6) and the tensor-scaling formula of the FP8-LM summary page.
//
// Design (HBM-bound): one workgroup owns a 128 x 128 bf16 tile. 16-byte coalesced loads land in registers; the
// row orientation is encoded straight from registers (a 32-value block spans 4 lanes; its amax is a DPP quad max)
// while the tile is also written to LDS, from which each thread re-reads a column pair of 32 rows for the column
// orientation, stored transposed so each block's 32 codes are contiguous. One pass over x emits both.
#include <mutex>

#include "mxq_device.h"
#include "launch.h"

namespace mxq {

constexpr int QT = 128;            // tile rows and columns
constexpr int QTHREADS = 256;

enum : int { QM_MX_RCEIL = 0, QM_MX_FLOOR = 1, QM_PT_E4M3 = 2, QM_PT_E5M2 = 3 };

struct QuantArgs {
    const uint16_t* x;
    int64_t rows, cols;
    uint8_t* q_row;     // MX: q_row ; per-tensor: q
    uint8_t* s_row;     // MX only
    uint8_t* q_col;     // MX: q_col ; per-tensor: q_t
    uint8_t* s_col;     // MX only
    const float* scale; // per-tensor only
    int srow_words;     // s_row rows hold whole 4-byte words per 128-column tile (cols % 128 == 0, 4-aligned)
    int scol_words;     // s_col likewise (rows % 128 == 0, 4-aligned)
    uint32_t* amax_word;  // AMAX: running max of |x| as a bf16 magnitude pattern (atomic max, one per workgroup)
    uint32_t* wide_row;   // RANGE: set to 1 if a 64-value window of the row orientation is wide (cleared before)
    uint32_t* wide_col;   // RANGE: likewise for the column orientation
};

// RANGE: one atomic per workgroup that found a wide window, skipped once the flag is seen set.
__device__ __forceinline__ void raise_wide(uint32_t* word) {
    if (__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) atomicOr(word, 1u);
}

// RANGE: the byte-replicated threshold below which a code magnitude byte lies more than kWideBinades binades under
// its window's top, for a block with scale byte `byte`; `top` is the window's largest binade + 1 (0 when the window
// holds no nonzero code). Clamped to [0, 128]: 0 counts no code, 128 every code (bit 7 of a magnitude byte is 0).
__device__ __forceinline__ uint32_t wide_th4(int top, int byte) {
    const int t = min(max(top - 1 - kWideBinades - byte, 0), 16) << 3;
    return __builtin_amdgcn_perm(0u, (uint32_t)t, 0u);       // byte 0 of t in all four bytes
}

template <int MODE>
__device__ __forceinline__ uint32_t pt_cvt_quad(float s, uint32_t p0, uint32_t p1) {
    constexpr int FMT = MODE == QM_PT_E4M3 ? FMT_E4M3 : FMT_E5M2;
    constexpr float FMAX = MODE == QM_PT_E4M3 ? 448.0f : 57344.0f;
    float a = clamp_keep_nan(bf16_lo(p0) * s, FMAX), b = clamp_keep_nan(bf16_hi(p0) * s, FMAX);
    float c = clamp_keep_nan(bf16_lo(p1) * s, FMAX), d = clamp_keep_nan(bf16_hi(p1) * s, FMAX);
    return cvt_f32_pair<FMT, true>(cvt_f32_pair<FMT, false>(0u, a, b), c, d);
}

// RANGE (MX only): also classify every 64-value window of each emitted orientation as the GEMM's range check does
// (kWideBinades, kWideCount) from the codes and scale bytes just formed, and raise wide_row / wide_col if any is wide.
// Row windows are 8 lanes of a tile row (two quads); column windows are the 32-row blocks b and b ^ 1 of a column,
// held by threads tid and tid ^ 64, which trade their block's top binade and small-code count through LDS.
template <int MODE, bool ROW, bool COL, bool AMAX = false, bool RANGE = false>
__global__ __launch_bounds__(QTHREADS) void quant_tile_kernel(QuantArgs a) {
    constexpr bool MX = MODE == QM_MX_RCEIL || MODE == QM_MX_FLOOR;
    constexpr int RULE = MODE == QM_MX_FLOOR ? RULE_FLOOR : RULE_RCEIL;
    static_assert(!RANGE || MX, "range words are computed for MX operands");
    __shared__ uint32_t lds[COL ? QT * QT / 2 : 1];
    int wide_r = 0, wide_c = 0;

    const int tid = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.y * QT, c0 = (int64_t)blockIdx.x * QT;
    const int ch = tid & 15;                     // 16-byte chunk within a tile row (8 bf16)
    const int64_t gc = c0 + ch * 8;
    const bool col_ok = gc < a.cols;             // cols % 8 == 0, so a chunk is all in or all out
    float pt_scale = 0.0f;
    if constexpr (!MX) pt_scale = *a.scale;

    // chunk j of this thread: tile row (tid >> 4) + 16 j, 8 values from column gc; pointers advance 16 rows per chunk
    const int64_t rows_in_tile = a.rows - r0;                // may exceed QT
    uint4 v[8];
    {
        const uint16_t* xp = a.x + (r0 + (tid >> 4)) * a.cols + gc;
        const int64_t xstep = 16 * a.cols;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (col_ok && (tid >> 4) + 16 * j < rows_in_tile)
                v[j] = ldnt16(xp);
            else
                v[j] = make_uint4(0u, 0u, 0u, 0u);
            xp += xstep;
        }
    }

    // AMAX: this thread's max |x| (bf16 magnitude patterns; NaN patterns sort above infinity; padding loaded as 0);
    // the workgroup's reduction waits until its stores are issued, so no wave stalls on it before converting.
    uint32_t amax_local = 0;
    if constexpr (AMAX) {
#pragma unroll
        for (int j = 0; j < 8; ++j) amax_local = max(amax_local, amax_bits8(v[j]));
    }

    if constexpr (COL) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int row = (tid >> 4) + 16 * j;
            *reinterpret_cast<uint4*>(&lds[row * (QT / 2) + ch * 4]) = v[j];
        }
    }

    if constexpr (ROW) {
        // This thread's row of chunk j is lrow + 16 j; its code and scale pointers advance 16 rows per chunk (no 64-bit
        // index arithmetic per chunk).
        const int lrow = tid >> 4;
        const int64_t rows_left = rows_in_tile;
        uint8_t* qr = a.q_row + (r0 + lrow) * a.cols + gc;
        const int64_t qr_step = 16 * a.cols;
        uint8_t* sr = nullptr;
        int64_t sr_step = 0;
        if constexpr (MX) {
            sr = a.s_row + (r0 + lrow) * (a.cols / 32) + (a.srow_words ? c0 / 32 : gc / 32);
            sr_step = 16 * (a.cols / 32);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool ok = col_ok && lrow + 16 * j < rows_left;
            uint32_t lo, hi;
            if constexpr (MX) {
                uint32_t m = quad_max(amax_bits8(v[j]));
                uint32_t byte = mx_scale_byte(m, RULE);
                float s = scale_operand(byte);
                lo = cvt_mx_quad(v[j].x, v[j].y, s);
                hi = cvt_mx_quad(v[j].z, v[j].w, s);
                if (RULE == RULE_FLOOR || m >= 0x7F80u) {
                    uint32_t thr = mx_sat_threshold(byte);
                    lo = mx_patch4(lo, v[j].x, v[j].y, thr);
                    hi = mx_patch4(hi, v[j].z, v[j].w, thr);
                }
                if constexpr (RANGE) {
                    // window = chunks 8w .. 8w + 7 of the tile row: this quad's block and the one at chunk ^ 4. A
                    // block's top is 0 when all its codes are 0, else its largest binade + 1, so the window's top is
                    // 0 exactly when the window holds no nonzero code.
                    const uint32_t ml = lo & 0x7F7F7F7Fu, mh = hi & 0x7F7F7F7Fu;
                    const uint32_t qm = quad_max(max_code_mag8(ml, mh));
                    const int tb = qm ? (int)(qm >> 3) + (int)byte + 1 : 0;
                    const int top = max(tb, __shfl_xor(tb, 4, 16));
                    const uint32_t th4 = wide_th4(top, (int)byte);
                    int cnt = count_below4(ml, th4) + count_below4(mh, th4);
                    cnt += __builtin_amdgcn_mov_dpp(cnt, 0xB1, 0xF, 0xF, false);
                    cnt += __builtin_amdgcn_mov_dpp(cnt, 0x4E, 0xF, 0xF, false);
                    cnt += __shfl_xor(cnt, 4, 16);
                    wide_r |= (top > 0 && cnt >= kWideCount) ? 1 : 0;
                }
                // The 16 lanes of a tile row hold its 4 block bytes at chunks 0, 4, 8, 12; chunk 0 gathers them with
                // row shifts (lane i reads lane i + 4, i + 8, i + 12 of its 16-lane row).
                const uint32_t b4 = (uint32_t)__builtin_amdgcn_mov_dpp((int)byte, 0x104, 0xF, 0xF, false);
                const uint32_t b8 = (uint32_t)__builtin_amdgcn_mov_dpp((int)byte, 0x108, 0xF, 0xF, false);
                const uint32_t b12 = (uint32_t)__builtin_amdgcn_mov_dpp((int)byte, 0x10C, 0xF, 0xF, false);
                if (ok) {
                    stnt8(qr, make_uint2(lo, hi));
                    if (a.srow_words) {
                        if (ch == 0) *reinterpret_cast<uint32_t*>(sr) = byte | (b4 << 8) | (b8 << 16) | (b12 << 24);
                    } else if ((tid & 3) == 0) {
                        *sr = (uint8_t)byte;
                    }
                }
                sr += sr_step;
            } else {
                lo = pt_cvt_quad<MODE>(pt_scale, v[j].x, v[j].y);
                hi = pt_cvt_quad<MODE>(pt_scale, v[j].z, v[j].w);
                if (ok) stnt8(qr, make_uint2(lo, hi));
            }
            qr += qr_step;
        }
    }

    if constexpr (COL) {
        __syncthreads();
        const int p = tid & 63;                  // column pair within the tile
        const int b = tid >> 6;                  // 32-row block within the tile
        uint32_t d[32];
#pragma unroll
        for (int r = 0; r < 32; ++r) d[r] = lds[(32 * b + r) * (QT / 2) + p];
        uint32_t out0[8], out1[8];
        uint32_t sb0 = 0, sb1 = 0;
        if constexpr (MX) {
            uint32_t m = 0;
#pragma unroll
            for (int r = 0; r < 32; ++r) m = max_u16x2(m, d[r] & 0x7FFF7FFFu);
            const uint32_t m0 = m & 0xFFFFu, m1 = m >> 16;
            sb0 = mx_scale_byte(m0, RULE);
            sb1 = mx_scale_byte(m1, RULE);
            const float s0 = scale_operand(sb0), s1 = scale_operand(sb1);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                // pairs down the column: lo halves -> column 2p, hi halves -> column 2p+1
                uint32_t a0 = __builtin_amdgcn_perm(d[4 * i + 1], d[4 * i + 0], 0x05040100u);
                uint32_t a1 = __builtin_amdgcn_perm(d[4 * i + 3], d[4 * i + 2], 0x05040100u);
                uint32_t h0 = __builtin_amdgcn_perm(d[4 * i + 1], d[4 * i + 0], 0x07060302u);
                uint32_t h1 = __builtin_amdgcn_perm(d[4 * i + 3], d[4 * i + 2], 0x07060302u);
                out0[i] = cvt_mx_quad(a0, a1, s0);
                out1[i] = cvt_mx_quad(h0, h1, s1);
                if (RULE == RULE_FLOOR || m0 >= 0x7F80u) out0[i] = mx_patch4(out0[i], a0, a1, mx_sat_threshold(sb0));
                if (RULE == RULE_FLOOR || m1 >= 0x7F80u) out1[i] = mx_patch4(out1[i], h0, h1, mx_sat_threshold(sb1));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                uint32_t a0 = __builtin_amdgcn_perm(d[4 * i + 1], d[4 * i + 0], 0x05040100u);
                uint32_t a1 = __builtin_amdgcn_perm(d[4 * i + 3], d[4 * i + 2], 0x05040100u);
                uint32_t h0 = __builtin_amdgcn_perm(d[4 * i + 1], d[4 * i + 0], 0x07060302u);
                uint32_t h1 = __builtin_amdgcn_perm(d[4 * i + 3], d[4 * i + 2], 0x07060302u);
                out0[i] = pt_cvt_quad<MODE>(pt_scale, a0, a1);
                out1[i] = pt_cvt_quad<MODE>(pt_scale, h0, h1);
            }
        }
        // RANGE: this thread's two column blocks (rows 32b .. 32b+31 of columns 2p, 2p+1): top binade and, after the
        // trade with the other block of the window (thread tid ^ 64), the small-code count against the window's top.
        // The trades use LDS words past the transposed codes and scale bytes (which end at byte QT*QT + 4*QT).
        // (a block's top is 0 when all its codes are 0, else its largest binade + 1, as in the row path)
        int ctop[2] = {0, 0};
        if constexpr (RANGE) {
            uint32_t mm[2] = {0u, 0u};
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                const uint32_t e0 = out0[i] & 0x7F7F7F7Fu, e1 = out0[i + 1] & 0x7F7F7F7Fu;
                const uint32_t f0 = out1[i] & 0x7F7F7F7Fu, f1 = out1[i + 1] & 0x7F7F7F7Fu;
                mm[0] = max(mm[0], max_code_mag8(e0, e1));
                mm[1] = max(mm[1], max_code_mag8(f0, f1));
            }
            ctop[0] = mm[0] ? (int)(mm[0] >> 3) + (int)sb0 + 1 : 0;
            ctop[1] = mm[1] ? (int)(mm[1] >> 3) + (int)sb1 + 1 : 0;
        }
        // Transpose the codes once more through LDS so that the global stores write whole 128-byte lines: output
        // row c (column c of x) is 128 bytes; its 16-byte chunk k sits at chunk k ^ ((c >> 1) & 7) to spread the
        // writes of neighbouring columns over the banks.
        __syncthreads();                                           // every thread has read its input column pair
        int* xtop = reinterpret_cast<int*>(lds) + (QT * QT + 4 * QT) / 4;   // [256][2] block tops
        int* xcnt = xtop + 2 * QTHREADS;                                    // [256][2] small counts
        int wtop[2] = {0, 0};                                               // the windows' tops
        if constexpr (RANGE) {
            xtop[2 * tid] = ctop[0];
            xtop[2 * tid + 1] = ctop[1];
            __syncthreads();
            const int partner = tid ^ 64;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                wtop[h] = max(ctop[h], xtop[2 * partner + h]);
                const uint32_t th4 = wide_th4(wtop[h], (int)(h ? sb1 : sb0));
                int cnt = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) cnt += count_below4((h ? out1[i] : out0[i]) & 0x7F7F7F7Fu, th4);
                xcnt[2 * tid + h] = cnt;
            }
        }
        uint8_t* obuf = reinterpret_cast<uint8_t*>(lds);           // 128 x 128 codes, then 128 x 4 scale bytes
        {
            const int c_even = 2 * p, c_odd = 2 * p + 1;
            const int k0 = 2 * b, k1 = 2 * b + 1;                  // the two 16-byte chunks of rows 32b .. 32b+31
            uint4* e = reinterpret_cast<uint4*>(obuf + c_even * QT);
            uint4* o = reinterpret_cast<uint4*>(obuf + c_odd * QT);
            e[k0 ^ ((c_even >> 1) & 7)] = make_uint4(out0[0], out0[1], out0[2], out0[3]);
            e[k1 ^ ((c_even >> 1) & 7)] = make_uint4(out0[4], out0[5], out0[6], out0[7]);
            o[k0 ^ ((c_odd >> 1) & 7)] = make_uint4(out1[0], out1[1], out1[2], out1[3]);
            o[k1 ^ ((c_odd >> 1) & 7)] = make_uint4(out1[4], out1[5], out1[6], out1[7]);
            if constexpr (MX) {
                obuf[QT * QT + c_even * 4 + b] = (uint8_t)sb0;
                obuf[QT * QT + c_odd * 4 + b] = (uint8_t)sb1;
            }
        }
        __syncthreads();
        if constexpr (RANGE) {
            if ((b & 1) == 0) {                                    // the window's first block decides
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int cnt = xcnt[2 * tid + h] + xcnt[2 * (tid ^ 64) + h];
                    wide_c |= (wtop[h] > 0 && cnt >= kWideCount) ? 1 : 0;
                }
            }
        }
        {
            // output row c = 32 pass + tid / 8 (column c0 + c of x), bytes 16 k .. 16 k + 15 of its 128
            const int k = tid & 7;
            const int64_t cols_in_tile = a.cols - c0;
            const bool row_ok = 16 * k < rows_in_tile;             // rows % 32 == 0: a 16-row chunk is whole
            uint8_t* qc = a.q_col + (c0 + (tid >> 3)) * a.rows + r0 + 16 * k;
            const int64_t qc_step = 32 * a.rows;
#pragma unroll
            for (int pass = 0; pass < QT / 32; ++pass) {           // 32 output rows (x columns) per pass
                const int c = 32 * pass + (tid >> 3);
                if (c < cols_in_tile && row_ok) {
                    const uint4 val = *reinterpret_cast<const uint4*>(obuf + c * QT + 16 * (k ^ ((c >> 1) & 7)));
                    *reinterpret_cast<uint4*>(qc) = val;
                }
                qc += qc_step;
            }
        }
        if constexpr (MX) {
            if (tid < QT) {
                const int c = tid;
                const int64_t gc2 = c0 + c;
                if (gc2 < a.cols) {
                    const uint32_t w = *reinterpret_cast<const uint32_t*>(obuf + QT * QT + 4 * c);
                    uint8_t* dst = a.s_col + gc2 * (a.rows / 32) + r0 / 32;
                    if (a.scol_words) {
                        *reinterpret_cast<uint32_t*>(dst) = w;
                    } else {
                        for (int bb = 0; bb < 4 && r0 + 32 * bb < a.rows; ++bb) dst[bb] = (uint8_t)(w >> (8 * bb));
                    }
                }
            }
        }
    }
    if constexpr (RANGE) {
        if constexpr (COL) {
            // per-wave flags in LDS words past the column trades (no extra LDS, so occupancy stays at 5 per CU)
            int* flags = reinterpret_cast<int*>(lds) + (QT * QT + 4 * QT) / 4 + 4 * QTHREADS;
            const bool fr = __ballot(wide_r) != 0, fc = __ballot(wide_c) != 0;
            if ((tid & 63) == 0) {
                flags[2 * (tid >> 6)] = fr ? 1 : 0;
                flags[2 * (tid >> 6) + 1] = fc ? 1 : 0;
            }
            __syncthreads();
            if (tid == 0) {
                if (ROW && (flags[0] | flags[2] | flags[4] | flags[6])) raise_wide(a.wide_row);
                if (flags[1] | flags[3] | flags[5] | flags[7]) raise_wide(a.wide_col);
            }
        } else {
            if (__syncthreads_or(wide_r) && tid == 0) raise_wide(a.wide_row);
        }
    }
    if constexpr (AMAX) {
        __shared__ uint32_t red[QTHREADS / 64];
        uint32_t m = amax_local;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
        if ((tid & 63) == 0) red[tid >> 6] = m;
        __syncthreads();
        if (tid == 0) {
            m = max(max(red[0], red[1]), max(red[2], red[3]));
            // the running maximum only grows: most tiles find theirs already covered and skip the atomic
            if (m > __hip_atomic_load(a.amax_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(a.amax_word, m);
        }
    }
}

template <int MODE>
static hipError_t launch_quant_mode(const QuantArgs& a, bool row, bool col, hipStream_t stream) {
    dim3 grid((unsigned)((a.cols + QT - 1) / QT), (unsigned)((a.rows + QT - 1) / QT));
    if (row && col) hipLaunchKernelGGL((quant_tile_kernel<MODE, true, true>), grid, dim3(QTHREADS), 0, stream, a);
    else if (row) hipLaunchKernelGGL((quant_tile_kernel<MODE, true, false>), grid, dim3(QTHREADS), 0, stream, a);
    else hipLaunchKernelGGL((quant_tile_kernel<MODE, false, true>), grid, dim3(QTHREADS), 0, stream, a);
    return hipGetLastError();
}

__global__ void clear_words_kernel(uint32_t* w0, uint32_t* w1) {
    if (w0) *w0 = 0u;
    if (w1) *w1 = 0u;
}

template <int MODE>
static hipError_t launch_quant_ranged(const QuantArgs& a, bool row, bool col, hipStream_t stream) {
    hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(1), 0, stream, row ? a.wide_row : nullptr,
                       col ? a.wide_col : nullptr);
    if (a.rows == 0 || a.cols == 0) return hipGetLastError();
    dim3 grid((unsigned)((a.cols + QT - 1) / QT), (unsigned)((a.rows + QT - 1) / QT));
    if (row && col) hipLaunchKernelGGL((quant_tile_kernel<MODE, true, true, false, true>), grid, dim3(QTHREADS), 0, stream, a);
    else if (row) hipLaunchKernelGGL((quant_tile_kernel<MODE, true, false, false, true>), grid, dim3(QTHREADS), 0, stream, a);
    else hipLaunchKernelGGL((quant_tile_kernel<MODE, false, true, false, true>), grid, dim3(QTHREADS), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_mx_quantize_ranged(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q_row, uint8_t* s_row,
                                     uint8_t* q_col, uint8_t* s_col, int rule, uint32_t* wide_row,
                                     uint32_t* wide_col, hipStream_t stream) {
    QuantArgs a{x, rows, cols, q_row, s_row, q_col, s_col, nullptr, 0, 0, nullptr, wide_row, wide_col};
    a.srow_words = cols % QT == 0 && (reinterpret_cast<uintptr_t>(s_row) & 3) == 0;
    a.scol_words = rows % QT == 0 && (reinterpret_cast<uintptr_t>(s_col) & 3) == 0;
    bool row = q_row != nullptr, col = q_col != nullptr;
    return rule == RULE_FLOOR ? launch_quant_ranged<QM_MX_FLOOR>(a, row, col, stream)
                              : launch_quant_ranged<QM_MX_RCEIL>(a, row, col, stream);
}

hipError_t launch_mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q_row, uint8_t* s_row,
                              uint8_t* q_col, uint8_t* s_col, int rule, hipStream_t stream) {
    QuantArgs a{x, rows, cols, q_row, s_row, q_col, s_col, nullptr, 0, 0, nullptr};
    a.srow_words = cols % QT == 0 && (reinterpret_cast<uintptr_t>(s_row) & 3) == 0;
    a.scol_words = rows % QT == 0 && (reinterpret_cast<uintptr_t>(s_col) & 3) == 0;
    bool row = q_row != nullptr, col = q_col != nullptr;
    return rule == RULE_FLOOR ? launch_quant_mode<QM_MX_FLOOR>(a, row, col, stream)
                              : launch_quant_mode<QM_MX_RCEIL>(a, row, col, stream);
}

// ---------------------------------------------------------------------------------------- per-tensor amax
constexpr int AMAX_THREADS = 256;

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
    return v;
}

__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* sh) {
    v = wave_max(v);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) sh[w] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < (int)(blockDim.x >> 6); ++i) v = max(v, sh[i]);
    }
    return v;
}

// Partial max of |x| (bf16 magnitude bit patterns; NaN patterns sort above infinity) per workgroup.
__global__ __launch_bounds__(AMAX_THREADS) void pt_amax_partial_kernel(const uint4* __restrict__ x, int64_t nchunks,
                                                                      uint32_t* __restrict__ partial) {
    __shared__ uint32_t sh[AMAX_THREADS / 64];
    uint32_t m = 0;
    const int64_t stride = (int64_t)gridDim.x * AMAX_THREADS;
    int64_t i = (int64_t)blockIdx.x * AMAX_THREADS + threadIdx.x;
    for (; i + 3 * stride < nchunks; i += 4 * stride) {
        uint4 a0 = ldnt16(x + i), a1 = ldnt16(x + i + stride);
        uint4 a2 = ldnt16(x + i + 2 * stride), a3 = ldnt16(x + i + 3 * stride);
        m = max(m, max(max(amax_bits8(a0), amax_bits8(a1)), max(amax_bits8(a2), amax_bits8(a3))));
    }
    for (; i < nchunks; i += stride) m = max(m, amax_bits8(ldnt16(x + i)));
    m = block_max(m, sh);
    if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// amax_out = max|x| (fp32), scale_out = (FMAX / max(amax, 1e-12)) * margin, or *scale_in in delayed mode.
__global__ __launch_bounds__(AMAX_THREADS) void pt_finalize_kernel(const uint32_t* __restrict__ partial, int nparts,
                                                                  float fmax, float margin,
                                                                  const float* __restrict__ scale_in,
                                                                  float* __restrict__ amax_out,
                                                                  float* __restrict__ scale_out) {
    __shared__ uint32_t sh[AMAX_THREADS / 64];
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nparts; i += AMAX_THREADS) m = max(m, partial[i]);
    m = block_max(m, sh);
    if (threadIdx.x == 0) {
        float amax = __uint_as_float(m << 16);
        float s;
        if (scale_in) {
            s = *scale_in;
        } else {
            float a = amax < 1e-12f ? 1e-12f : amax;
            s = fmax / a;
            s = s * margin;
        }
        *amax_out = amax;
        *scale_out = s;
    }
}

int pertensor_amax_parts(int64_t n) {
    int64_t chunks = n / 8;
    int64_t parts = (chunks + AMAX_THREADS * 8 - 1) / (AMAX_THREADS * 8);
    if (parts < 1) parts = 1;
    if (parts > 2048) parts = 2048;
    return (int)parts;
}

hipError_t launch_pertensor_quantize(const uint16_t* x, int64_t rows, int64_t cols, int fmt, float margin,
                                     const float* scale_in, float* amax_out, float* scale_out, uint8_t* q,
                                     uint8_t* q_t, uint32_t* partial, hipStream_t stream) {
    const int64_t n = rows * cols;
    const int parts = pertensor_amax_parts(n);
    hipLaunchKernelGGL(pt_amax_partial_kernel, dim3(parts), dim3(AMAX_THREADS), 0, stream,
                       reinterpret_cast<const uint4*>(x), n / 8, partial);
    hipLaunchKernelGGL(pt_finalize_kernel, dim3(1), dim3(AMAX_THREADS), 0, stream, partial, parts,
                       fmt == FMT_E4M3 ? 448.0f : 57344.0f, margin, scale_in, amax_out, scale_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // an empty tensor still gets amax 0 and its scale; there are no codes to write
    if ((!q && !q_t) || rows == 0 || cols == 0) return hipSuccess;
    QuantArgs a{x, rows, cols, q, nullptr, q_t, nullptr, scale_out, 0, 0, nullptr};
    return fmt == FMT_E4M3 ? launch_quant_mode<QM_PT_E4M3>(a, q != nullptr, q_t != nullptr, stream)
                           : launch_quant_mode<QM_PT_E5M2>(a, q != nullptr, q_t != nullptr, stream);
}

// ------------------------------------------------------------------------ allocation-free per-tensor quantize
// fp8_quantize_pertensor_noalloc keeps the amax pass's partial maxima in this file-scope device array instead of a
// caller workspace. pertensor_amax_parts never exceeds 2048, so the array holds the partials of any size; each GPU
// keeps its own copy until the process ends. Calls that overlap on one GPU share it and race; every partial is written
// by its workgroup before the finalize kernel reads it, so nothing has to be cleared between calls.
constexpr int kScratchWords = 2048;
static __device__ __align__(256) uint32_t scratch[kScratchWords];

constexpr int kMaxScratchDevices = 64;
static std::mutex g_scratch_mu;
static uint32_t* g_scratch[kMaxScratchDevices] = {};

// Device address of `scratch` on the device of `stream` (the current device for the null stream), found once per
// device with that device current. In host code the array's name is only a stand-in, so kernels get this address.
hipError_t pertensor_scratch(hipStream_t stream, uint32_t** ptr, size_t* bytes) {
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = static_cast<uint32_t*>(p);
    }
    *ptr = g_scratch[dev];
    *bytes = sizeof(uint32_t) * kScratchWords;
    return hipSuccess;
}

// ---------------------------------------------------------------------------------------- delayed scaling
// Scale from the amax history of earlier calls ("3.8 Mixed Precision, bf16 & FP8 Training", delayed-scaling recipe):
// max over the history (any NaN entry makes it NaN), clamped below at 1e-12, FMAX over it, times the margin. Also
// clears the word the cast kernel's workgroups take the atomic max of |x| into.
__global__ __launch_bounds__(AMAX_THREADS) void pt_delayed_prep_kernel(const float* __restrict__ hist, int H, float fmax,
                                                                      float margin, float* __restrict__ scale_out,
                                                                      uint32_t* __restrict__ amax_word) {
    __shared__ float shm[AMAX_THREADS / 64];
    __shared__ int shn[AMAX_THREADS / 64];
    float m = 0.0f;
    int nan = 0;
    for (int i = threadIdx.x; i < H; i += AMAX_THREADS) {
        const float h = hist[i];
        if (h != h) nan = 1;
        else if (h > m) m = h;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        m = fmaxf(m, __shfl_xor(m, off, 64));
        nan |= __shfl_xor(nan, off, 64);
    }
    if ((threadIdx.x & 63) == 0) { shm[threadIdx.x >> 6] = m; shn[threadIdx.x >> 6] = nan; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < AMAX_THREADS / 64; ++w) { m = fmaxf(m, shm[w]); nan |= shn[w]; }
        float a = nan ? __uint_as_float(0x7FC00000u) : m;
        a = a < 1e-12f ? 1e-12f : a;                 // a NaN stays NaN
        float s = fmax / a;
        s = s * margin;
        *scale_out = s;
        *amax_word = 0u;
    }
}

// amax_out = max |x| of this call; it goes to the history at the ring position, which then advances.
__global__ void pt_delayed_finalize_kernel(const uint32_t* __restrict__ amax_word, float* __restrict__ hist,
                                           int32_t* __restrict__ pos, int H, float* __restrict__ amax_out) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        const float amax = __uint_as_float(*amax_word << 16);
        *amax_out = amax;
        int p = *pos;
        p = ((p % H) + H) % H;                        // an out-of-range position never writes outside the history
        hist[p] = amax;
        *pos = (p + 1) % H;
    }
}

template <int MODE>
static hipError_t launch_quant_delayed_mode(const QuantArgs& a, bool row, bool col, hipStream_t stream) {
    dim3 grid((unsigned)((a.cols + QT - 1) / QT), (unsigned)((a.rows + QT - 1) / QT));
    if (row && col) hipLaunchKernelGGL((quant_tile_kernel<MODE, true, true, true>), grid, dim3(QTHREADS), 0, stream, a);
    else if (row) hipLaunchKernelGGL((quant_tile_kernel<MODE, true, false, true>), grid, dim3(QTHREADS), 0, stream, a);
    else if (col) hipLaunchKernelGGL((quant_tile_kernel<MODE, false, true, true>), grid, dim3(QTHREADS), 0, stream, a);
    else hipLaunchKernelGGL((quant_tile_kernel<MODE, false, false, true>), grid, dim3(QTHREADS), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_pertensor_quantize_delayed(const uint16_t* x, int64_t rows, int64_t cols, int fmt, float margin,
                                             float* hist, int32_t* pos, int H, float* amax_out, float* scale_out,
                                             uint8_t* q, uint8_t* q_t, uint32_t* amax_word, hipStream_t stream) {
    hipLaunchKernelGGL(pt_delayed_prep_kernel, dim3(1), dim3(AMAX_THREADS), 0, stream, (const float*)hist, H,
                       fmt == FMT_E4M3 ? 448.0f : 57344.0f, margin, scale_out, amax_word);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (rows > 0 && cols > 0) {
        QuantArgs a{x, rows, cols, q, nullptr, q_t, nullptr, scale_out, 0, 0, amax_word};
        e = fmt == FMT_E4M3 ? launch_quant_delayed_mode<QM_PT_E4M3>(a, q != nullptr, q_t != nullptr, stream)
                            : launch_quant_delayed_mode<QM_PT_E5M2>(a, q != nullptr, q_t != nullptr, stream);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(pt_delayed_finalize_kernel, dim3(1), dim3(64), 0, stream, (const uint32_t*)amax_word, hist, pos,
                       H, amax_out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------- fused SwiGLU + MX
// The routed experts' hidden representation ("OLMo-core MoE, Section 11: MXFP8 Training", Section 11.4.1: a fused
// SwiGLU-plus-quantization step feeds the down projection without a separate BF16-to-MXFP8 pass). C[rows][2F]
// holds the gate in columns [0, F) and up in [F, 2F); h = silu(g) * u in fp32 (exp_fixed), quantized from fp32 in
// 32-value blocks along each row.

// One thread per 8 consecutive outputs of a row; the 4 lanes of a quad cover one 32-value block (F % 32 == 0, so
// quads never straddle rows and the chunk count is a multiple of 4).
template <int RULE>
__global__ __launch_bounds__(256) void swiglu_mx_kernel(const uint16_t* __restrict__ c, int64_t rows, int64_t F,
                                                       uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
    const int64_t per_row = F / 8, total = rows * per_row;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
        const int64_t r = i / per_row, j = (i - r * per_row) * 8;
        const uint4 gv = ldnt16(c + r * 2 * F + j);
        const uint4 uv = ldnt16(c + r * 2 * F + F + j);
        const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w}, uw[4] = {uv.x, uv.y, uv.z, uv.w};
        float h[8];
        uint32_t m = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float g = (e & 1) ? bf16_hi(gw[e >> 1]) : bf16_lo(gw[e >> 1]);
            const float u = (e & 1) ? bf16_hi(uw[e >> 1]) : bf16_lo(uw[e >> 1]);
            h[e] = swiglu_f32(g, u);
            m = max(m, __float_as_uint(h[e]) & 0x7FFFFFFFu);
        }
        m = quad_max(m);
        const uint32_t byte = mx_scale_byte_f32(m, RULE);
        const float f = mx_inv_scale_f32(byte);
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = clamp_keep_nan(h[e] * f, 448.0f);
        const uint32_t lo = cvt_f32_pair<FMT_E4M3, true>(cvt_f32_pair<FMT_E4M3, false>(0u, y[0], y[1]), y[2], y[3]);
        const uint32_t hi = cvt_f32_pair<FMT_E4M3, true>(cvt_f32_pair<FMT_E4M3, false>(0u, y[4], y[5]), y[6], y[7]);
        stnt8(q + r * F + j, make_uint2(lo, hi));
        if ((j & 31) == 0) s[r * (F / 32) + j / 32] = (uint8_t)byte;
    }
}

hipError_t launch_swiglu_mx_quantize(const uint16_t* c, int64_t rows, int64_t F, uint8_t* q, uint8_t* s, int rule,
                                     hipStream_t stream) {
    const int64_t total = rows * (F / 8);
    int64_t blocks = (total + 255) / 256;
    if (blocks > (int64_t(1) << 30)) blocks = int64_t(1) << 30;     // one chunk per thread (the loop is a guard)
    if (rule == RULE_FLOOR)
        hipLaunchKernelGGL(swiglu_mx_kernel<RULE_FLOOR>, dim3((unsigned)blocks), dim3(256), 0, stream, c, rows, F, q, s);
    else
        hipLaunchKernelGGL(swiglu_mx_kernel<RULE_RCEIL>, dim3((unsigned)blocks), dim3(256), 0, stream, c, rows, F, q, s);
    return hipGetLastError();
}

}  // namespace mxq
