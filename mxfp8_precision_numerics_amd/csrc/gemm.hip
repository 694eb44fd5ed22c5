// Scaled FP8 GEMM for gfx950: C[M][N] (bf16) = A[M][K] * B[N][K]^T with fp32 accumulation.
//
// MX_BLOCK32 applies one E8M0 scale per 32 values along K inside the matrix instruction ("OLMo-core MoE,
// Section 11: MXFP8 Training", Figure 47 and Section 11.2.3: native block-scaled GEMM, BF16 operator output).
// PER_TENSOR multiplies the fp32 accumulator by 1 / (s_a s_b) ("3.8 Mixed Precision, bf16 & FP8 Training",
// Exercise 6: de-scale by 1/(s_x s_w)). The grouped variants run the same tiles over ragged expert row groups
// (Section 11.4.1, routed experts: forward, and dgrad with a strided expert operand) and over ragged expert ranges of
// K with one output per expert (the routed Wgrad, whose contraction runs over each expert's tokens).
//
// FP8 matrix instruction of the large-tile kernel: v_mfma_scale_f32_32x32x64_f8f6f4. Operand layout (per lane l,
// g = l / 32): row l % 32;
// bytes 0-15 hold k = 16g .. 16g+15 and bytes 16-31 hold k = 32+16g .. 32+16g+15 of the 64-wide K window. The
// E8M0 scale for (row r, 32-block b of the window) comes from lane r + 32b, byte chosen by op_sel. Output: lane l,
// register j -> row 8(j/4) + 4g + j%4, column l % 32. The kernel feeds B as the instruction's first operand and A
// as its second, so a lane's four consecutive accumulator registers are four consecutive n of one output row m
// (8-byte bf16 stores).
//
// Paths (see the path-selection notes below): scaled_gemm takes the FP8 instruction only on large tiles at
// K >= 12288 when a device-side range check of both operands allows it, and otherwise the exact path (operands
// dequantized to bf16 exactly, bf16 instruction, fp32 accumulation); scaled_gemm_exact always takes the exact path,
// scaled_gemm_fp8 always the FP8 instruction. The grouped variants take the exact path.
//
// Small-tile kernel (gemm_kernel): 256 threads (4 waves, 2 x 2), a 128 x 128 output tile, waves own 64 x 64, as
// 4 x 4 v_mfma_scale_f32_16x16x128_f8f6f4 on the FP8 path or 2 x 2 v_mfma_f32_32x32x16_bf16 on operands dequantized
// to bf16 (the exact path). K advances 128 bytes per stage; stages are double-buffered in LDS. LDS rows are 128 bytes
// with the 16-byte chunk index XOR-swizzled by (row & 7), so the 16-byte fragment reads of 8 consecutive rows hit
// distinct banks. The large-tile kernel (gemm_big_kernel) is described where it is defined.
#include <type_traits>

#include "mxq_device.h"
#include "launch.h"

namespace mxq {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int GTHREADS = 256;
constexpr int GROUP_M = 8;

// Group modes: none; expert groups of A rows, each against its own B (forward and dgrad of routed experts); expert
// ranges of K, each with its own output (routed Wgrad: the contraction runs over the expert's token rows).
enum : int { GM_NONE = 0, GM_ROWS = 1, GM_TOKENS = 2 };

struct GemmArgs {
    const uint8_t* a;
    const uint8_t* b;
    const uint8_t* sa;   // MX: E8M0 per 32 values of K, row stride ldsa
    const uint8_t* sb;   // MX: likewise for B, row stride ldsb
    const float* pa;     // per-tensor scales
    const float* pb;
    uint16_t* c;         // bf16 output, row stride ldc
    float* cf;           // token groups only: fp32 output that the result is added to (when c is null)
    int64_t M, N, K, ldc;
    int64_t lda, ldb, ldsa, ldsb;      // operand row strides in bytes (qdata) and scale bytes
    int64_t b_gstride, sb_gstride;     // row groups: distance from one expert's B (and B scales) to the next
    int64_t c_gstride;                 // token groups: distance from one expert's output to the next
    const int64_t* offsets;            // grouped only: [G+1]
    int64_t G;
    int gate;                          // large tiles, no groups: 0 = always run; 1 (FP8) / 2 (exact) = run the tile
                                       // only if its first output element holds kGateFp8 / kGateExact; 3 (FP8) /
                                       // 4 (exact) = run only if the range words *wa | *wb are 0 / nonzero
    const uint32_t* wa;                // gates 3, 4: the operands' range words
    const uint32_t* wb;
};

// Tile gates of the checked path (bf16 NaN patterns the epilogue never writes for finite results).
constexpr uint16_t kGateFp8 = 0x7FA1u, kGateExact = 0x7FA2u;

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 4); }

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));

// 8 FP8 codes (E4M3 when FMT == 0, E5M2 when 1) -> 8 bf16 equal to code * 2^E, where E is the exponent field of
// `scale` (exact whenever the product is representable in bf16).
template <int FMT>
__device__ __forceinline__ v8bf dequant8_bf16(uint2 x, float scale) {
    v2bf_t p0, p1, p2, p3;
    if constexpr (FMT == 0) {
        p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x.x, scale, false);
        p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x.x, scale, true);
        p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x.y, scale, false);
        p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x.y, scale, true);
    } else {
        p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)x.x, scale, false);
        p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)x.x, scale, true);
        p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)x.y, scale, false);
        p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)x.y, scale, true);
    }
    return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Row-grouped GEMMs: the expert group that holds row tile t (tiles of TH rows, numbered group by group, each group's
// rows [off[q], off[q+1]) clamped to [0, M) and cut into ceil(rows / TH) tiles). Each wave scans 64 groups at a time:
// lane l loads group base + l's offsets, a wave prefix sum of the tile counts finds the group, so a workgroup pays one
// round of loads per 64 groups instead of a dependent load per group. grp = -1 when t lies past the last tile.
struct RowTile {
    int64_t grp, lo, hi;      // group, first row of the tile, end of the group's rows
};

template <int TH>
__device__ __forceinline__ RowTile find_row_tile(const GemmArgs& g, int64_t t) {
    const int lane = threadIdx.x & 63;
    RowTile r{-1, 0, 0};
    int64_t before = 0;                          // tiles of the groups already scanned
    for (int64_t base = 0; base < g.G; base += 64) {
        const int64_t q = base + lane;
        int64_t a0 = 0, a1 = 0;
        int nt = 0;
        if (q < g.G) {
            a0 = g.offsets[q];
            a1 = g.offsets[q + 1];
            a0 = a0 < 0 ? 0 : (a0 > g.M ? g.M : a0);
            a1 = a1 < a0 ? a0 : (a1 > g.M ? g.M : a1);
            nt = (int)((a1 - a0 + TH - 1) / TH);
        }
        int incl = nt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_up(incl, off, 64);
            if (lane >= off) incl += v;
        }
        const uint64_t hit = __ballot(before + incl > t);
        if (hit) {
            const int L = __ffsll((unsigned long long)hit) - 1;
            const int64_t excl = before + __shfl(incl - nt, L, 64);
            r.grp = base + L;
            r.lo = __shfl(a0, L, 64) + (t - excl) * TH;
            r.hi = __shfl(a1, L, 64);
            return r;
        }
        before += __shfl(incl, 63, 64);
    }
    return r;
}

template <bool MX, int FA, int FB, int GM, int MF>
__global__ __launch_bounds__(GTHREADS) void gemm_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * BK];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * BK];
    __shared__ uint32_t sSA[2][BM];
    __shared__ uint32_t sSB[2][BN];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int tiles_n = (int)((g.N + BN - 1) / BN);

    // ------------------------------------------------------------------ tile -> (rows, n0, K range)
    int64_t m0, m_end, n0;
    int64_t K = g.K;                                  // this tile's contraction length
    const uint8_t* Aq = g.a;
    const uint8_t* As = g.sa;
    const uint8_t* Bq = g.b;
    const uint8_t* Bs = g.sb;
    uint16_t* Cb = g.c;
    float* Cf = g.cf;
    if constexpr (GM == GM_ROWS) {
        const int64_t bid = blockIdx.x;
        const int64_t t = bid / tiles_n;
        n0 = (bid % tiles_n) * BN;
        const RowTile rt = find_row_tile<BM>(g, t);
        const int64_t grp = rt.grp, lo = rt.lo, hi = rt.hi;
        if (grp < 0) return;                          // more workgroups than tiles: nothing to do
        m0 = lo;
        m_end = (lo + BM < hi) ? lo + BM : hi;
        Bq = g.b + grp * g.b_gstride;
        Bs = MX ? g.sb + grp * g.sb_gstride : nullptr;
    } else {
        const int tiles_m = (int)((g.M + BM - 1) / BM);
        int64_t bid = blockIdx.x;
        if constexpr (GM == GM_TOKENS) {
            // expert-major order: every expert's tiles share its K range; its A and B columns are read once per tile
            const int64_t per = (int64_t)tiles_m * tiles_n;
            const int64_t grp = bid / per;
            bid -= grp * per;
            int64_t k0 = g.offsets[grp], k1 = g.offsets[grp + 1];
            k0 = k0 < 0 ? 0 : (k0 > g.K ? g.K : k0);
            k1 = k1 < k0 ? k0 : (k1 > g.K ? g.K : k1);
            K = k1 - k0;
            Aq = g.a + k0;
            Bq = g.b + k0;
            As = g.sa + k0 / 32;
            Bs = g.sb + k0 / 32;
            if (Cb) Cb += grp * g.c_gstride;
            if (Cf) Cf += grp * g.c_gstride;
        }
        const int per_group = GROUP_M * tiles_n;
        const int first_m = ((int)bid / per_group) * GROUP_M;
        const int gm = min(GROUP_M, tiles_m - first_m);
        const int r = (int)bid % per_group;
        m0 = (int64_t)(first_m + r % gm) * BM;
        n0 = (int64_t)(r / gm) * BN;
        m_end = (m0 + BM < g.M) ? m0 + BM : g.M;
    }
    const int64_t kblocks = K / 32;
    const int64_t n_end = (n0 + BN < g.N) ? n0 + BN : g.N;

    // ------------------------------------------------------------------ global -> registers (one stage)
    uint4 ra[4], rb[4];
    uint32_t rs = 0x7F7F7F7Fu;

    auto load_stage = [&](int64_t k0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = (tid >> 3) + 32 * j, ch = tid & 7;
            const int64_t kk = k0 + ch * 16;
            const int64_t ar = m0 + row, br = n0 + row;
            ra[j] = (ar < m_end && kk < K) ? *reinterpret_cast<const uint4*>(Aq + ar * g.lda + kk) : make_uint4(0, 0, 0, 0);
            rb[j] = (br < n_end && kk < K) ? *reinterpret_cast<const uint4*>(Bq + br * g.ldb + kk) : make_uint4(0, 0, 0, 0);
        }
        if constexpr (MX) {
            const int row = tid & 127;
            const bool isA = tid < 128;
            const int64_t rr = isA ? m0 + row : n0 + row;
            const bool ok = isA ? rr < m_end : rr < n_end;
            const uint8_t* sp = isA ? As + rr * g.ldsa : Bs + rr * g.ldsb;    // this row's scales
            const int64_t kb = k0 / 32;
            if (ok && kb + 4 <= kblocks && (reinterpret_cast<uintptr_t>(sp + kb) & 3) == 0) {
                rs = *reinterpret_cast<const uint32_t*>(sp + kb);
            } else {
                uint32_t v = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uint32_t byte = (ok && kb + i < kblocks) ? sp[kb + i] : 127u;
                    v |= byte << (8 * i);
                }
                rs = v;
            }
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = (tid >> 3) + 32 * j, ch = tid & 7;
            *reinterpret_cast<uint4*>(&sA[buf][swz(row, ch)]) = ra[j];
            *reinterpret_cast<uint4*>(&sB[buf][swz(row, ch)]) = rb[j];
        }
        if constexpr (MX) {
            if (tid < 128) sSA[buf][tid] = rs; else sSB[buf][tid - 128] = rs;
        }
    };

    // accumulators: MF 2 (exact path) -> 2 x 2 tiles of 32x32 (16 regs); MF 1 (FP8) -> 4 x 4 tiles of 16x16 (4 regs)
    v16f acc[2][2];
    v4f acc4[4][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc4[i][j] = v4f{};

    const int nk = (int)((K + BK - 1) / BK);
    const int fr = lane & 31, fg = lane >> 5;

    load_stage(0);
    store_stage(0);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_stage((int64_t)(kt + 1) * BK);

        if constexpr (MF == 2) {
            // Exact-accumulation variant: dequantize the FP8 codes (times their E8M0 block scale) to bf16 in
            // registers and use v_mfma_f32_32x32x16_bf16 (lane l: row l % 32, k = 8(l/32) .. +7 of a 16-wide window).
            // Window t of the 128-byte stage is LDS chunk t; lane half g reads its bytes 8g .. 8g+7.
            uint32_t sa_w[2], sb_w[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) sa_w[j] = MX ? sSA[buf][wm * 64 + j * 32 + fr] : 0x7F7F7F7Fu;
#pragma unroll
            for (int i = 0; i < 2; ++i) sb_w[i] = MX ? sSB[buf][wn * 64 + i * 32 + fr] : 0x7F7F7F7Fu;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                v8bf fa[2], fb[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int row = wm * 64 + j * 32 + fr;
                    const uint2 x = *reinterpret_cast<const uint2*>(&sA[buf][swz(row, t) + 8 * fg]);
                    fa[j] = dequant8_bf16<FA>(x, scale_operand((sa_w[j] >> (8 * (t >> 1))) & 0xFFu));
                }
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int row = wn * 64 + i * 32 + fr;
                    const uint2 x = *reinterpret_cast<const uint2*>(&sB[buf][swz(row, t) + 8 * fg]);
                    fb[i] = dequant8_bf16<FB>(x, scale_operand((sb_w[i] >> (8 * (t >> 1))) & 0xFFu));
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[i], fa[j], acc[i][j], 0, 0, 0);
            }
        } else {
            // 16x16x128: lane l holds row l % 16; bytes 0-15 = k 16q..16q+15, bytes 16-31 = k 64+16q.. (q = l / 16);
            // its scale byte is block q of that row.
            const int r16 = lane & 15, q16 = lane >> 4;
            uint32_t sa_reg[4], sb_reg[4];
            v8i fa[4], fb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = wm * 64 + j * 16 + r16;
                sa_reg[j] = MX ? (sSA[buf][row] >> (8 * q16)) : 0x7F7F7F7Fu;
                uint4 x0 = *reinterpret_cast<const uint4*>(&sA[buf][swz(row, q16)]);
                uint4 x1 = *reinterpret_cast<const uint4*>(&sA[buf][swz(row, 4 + q16)]);
                fa[j] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wn * 64 + i * 16 + r16;
                sb_reg[i] = MX ? (sSB[buf][row] >> (8 * q16)) : 0x7F7F7F7Fu;
                uint4 x0 = *reinterpret_cast<const uint4*>(&sB[buf][swz(row, q16)]);
                uint4 x1 = *reinterpret_cast<const uint4*>(&sB[buf][swz(row, 4 + q16)]);
                fb[i] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc4[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[i], fa[j], acc4[i][j], FB, FA, 0,
                                                                                 (int)sb_reg[i], 0, (int)sa_reg[j]);
        }

        if (kt + 1 < nk) store_stage(buf ^ 1);
        __syncthreads();
    }

    // ------------------------------------------------------------------ epilogue: fp32 -> bf16, store
    float post = 1.0f;
    if constexpr (!MX) post = 1.0f / (g.pa[0] * g.pb[0]);
    const bool vec_ok = (g.ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(Cb) & 7) == 0;
    const bool vec_ok_f = (g.ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(Cf) & 15) == 0;
    auto store4 = [&](int64_t m, int64_t n, float v0, float v1, float v2, float v3) {
        if (m >= m_end) return;
        float v[4] = {v0, v1, v2, v3};
        if constexpr (GM == GM_TOKENS) {
            if (Cb == nullptr) {                      // add to the fp32 output: one rounding of old + sum
                float* dst = Cf + m * g.ldc + n;
                if (vec_ok_f && n + 4 <= n_end) {
                    const float4 o = *reinterpret_cast<const float4*>(dst);
                    *reinterpret_cast<float4*>(dst) = make_float4(o.x + v[0], o.y + v[1], o.z + v[2], o.w + v[3]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < n_end) dst[e] = dst[e] + v[e];
                }
                return;
            }
        }
        uint16_t h4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float x = v[e];
            if constexpr (!MX) x = x * post;
            h4[e] = __builtin_bit_cast(uint16_t, (__bf16)x);
        }
        uint16_t* dst = Cb + m * g.ldc + n;
        if (vec_ok && n + 4 <= n_end) {
            *reinterpret_cast<uint2*>(dst) = make_uint2((uint32_t)h4[0] | ((uint32_t)h4[1] << 16),
                                                        (uint32_t)h4[2] | ((uint32_t)h4[3] << 16));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n + e < n_end) dst[e] = h4[e];
        }
    };
    if constexpr (MF == 2) {
        // 32x32 output: lane -> m = l % 32; register 4q+e -> n = 8q + 4(l/32) + e
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    store4(m0 + wm * 64 + j * 32 + fr, n0 + wn * 64 + i * 32 + 8 * q + 4 * fg, acc[i][j][4 * q],
                           acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
    } else {
        // 16x16 output: lane -> m = l % 16; register e -> n = 4(l/16) + e
        const int r16 = lane & 15, q16 = lane >> 4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                store4(m0 + wm * 64 + j * 16 + r16, n0 + wn * 64 + i * 16 + 4 * q16, acc4[i][j][0], acc4[i][j][1],
                       acc4[i][j][2], acc4[i][j][3]);
    }
}


// ---------------------------------------------------------------------------------------------------------------
// Large-tile kernel: a 256 x 256 output tile per workgroup, one workgroup per CU (4 waves, 2 x 2, each 128 x 128 as
// 4 x 4 tiles of 32 x 32 matrix instructions). K advances 64 bytes per stage; trip t multiplies stage t from
// fragments read into registers during trip t - 1, while reading stage t + 1's fragments.
// LDS: per operand two 32 KiB regions of two stages each, as 32 blocks of 1 KiB: block b holds rows 8b .. 8b+7 of the
// region's first stage in its first 512 bytes and of its second stage in the last 512 (64 bytes per row).
// Copies go straight from global memory to LDS (buffer_load_dwordx4 ... lds) and every copy instruction fetches whole
// 128-byte lines: 8 rows x 128 bytes of K, the same rows of two consecutive stages (lanes 0-31 the first stage,
// lanes 32-63 the second), half the cache-line requests of 64-byte rows. A's stage pairs are (2q, 2q+1) and B's
// (2q+1, 2q+2); trip t copies one pair, A's (t+3, t+4) on odd t and B's on even t, into the region whose two stages
// were read by the end of trip t - 1. Stage t + 2 must have landed at the end of trip t, so only the current trip's
// copies stay in flight across that wait, and every stage has one to two trips to land.
// Within a block, position p of a row holds chunk p ^ swz8(row), so the 16-byte fragment reads of 16 consecutive
// rows hit distinct banks. Rows past the end of an operand are clamped to its last row (their outputs are never
// stored), so every access stays inside the caller's buffers.
// MX scales: on the FP8 instruction's path a group covers SGM = 16 stages, 32 scale bytes per row, copied as two
// 16-byte halves by a pair of lanes (32 rows per copy instruction, so each instruction touches half as many rows'
// cache lines as one 16-byte lane per row would); the exact path and token groups keep groups of SG = 8 stages, one
// 16-byte lane per row. The groups are double-buffered and a group's copies are issued four trips before its first
// stage is read.
// Tile order: each XCD (which receives every eighth workgroup) walks a contiguous run of a grouped-M order, so its
// resident workgroups share A and B tiles in its L2. Row groups take their tiles group by group; token groups run
// expert-major in launch order (see the token-group notes in the kernel).
constexpr int TB = 256;
constexpr int KS = 64;
constexpr int SG = 8;
constexpr int SGM = 16;
constexpr int GROUP_M2 = 4;
constexpr int64_t kXcdChunk = 32;   // CUs per XCD: the workgroups of the large-tile kernel one XCD holds at once
// Issue slot (of the 16 matrix instructions of a stage) after which each of a trip's 8 copy instructions goes.
constexpr int kCopySlot[8] = {1, 3, 5, 7, 9, 11, 13, 15};

__device__ __forceinline__ int swz8(int row) { return (row >> 2) & 3; }

// Raw buffer resource (base, stride 0, 2^31 - 1 bytes, raw untyped access) for a workgroup-uniform address. The
// address is moved to scalar registers explicitly: values derived from the tile index are computed with vector
// instructions, and the descriptor must live in scalar registers.
// With `records` set, accesses at or past that many bytes from the base are out of range: loads return zero and
// nothing outside the buffer is touched.
__device__ __forceinline__ v4i buffer_rsrc(const void* p, uint32_t records = 0x7FFFFFFFu) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return v4i{(int)lo, (int)(hi & 0xFFFFu), (int)__builtin_amdgcn_readfirstlane(records), 0x00020000};
}

// LDS offset (the low 32 bits of a shared-aperture address) of an LDS location, made wave-uniform.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(p));
}

// Asynchronous copy global -> LDS: each lane reads BYTES (16 or 4) at base + voff + soff and the wave's results land
// in consecutive slots starting at LDS offset `lds` (M0). Written as inline assembly on purpose: the compiler does
// not then treat the copy as an LDS write, so LDS reads of other stages are not made to wait for it. The kernel
// orders copies itself (wait_copies_barrier): a stage is read only after its copies have completed on every wave,
// and a buffer is refilled only after every wave has finished reading it.
template <int BYTES>
__device__ __forceinline__ void dma_to_lds(v4i rsrc, uint32_t lds, int voff, int soff) {
    if constexpr (BYTES == 16)
        asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
                     :: "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds) : "memory");
    else
        asm volatile("buffer_load_dword %0, %1, %2 offen lds"
                     :: "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds) : "memory");
}

// Wait until at most N of this wave's copies are still outstanding (vector-memory counter, which retires in issue
// order) and all its LDS reads have returned, then join the workgroup barrier. One asm statement with a memory
// clobber, so the compiler keeps LDS accesses on their side of it.
template <int N>
__device__ __forceinline__ void wait_copies_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
}

// One output tile (workgroup-uniform index bid) of the large-tile kernel; returning ends the tile.
template <bool MX, int FA, int FB, int GM, int MF>
__device__ __forceinline__ void gemm_big_tile(const GemmArgs& g, const int bid_in) {
    // Token groups: every expert has its own K range (a multiple of 32, not of the 64-byte stage) and scale rows of
    // any byte alignment; they run the exact path only.
    constexpr bool TOK = GM == GM_TOKENS;
    static_assert(!TOK || (MX && MF == 2), "token-grouped contractions are MX on the exact path");
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][2 * TB * KS];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][2 * TB * KS];
    // MX scales, double-buffered by group of SGX stages (2 blocks per stage). Rows: [row][SCW words]. Token groups:
    // [word][row], 5 words from the 4-byte-aligned address at or below the row's first scale byte of the group.
    constexpr int SGX = (TOK || MF == 2) ? SG : SGM;
    constexpr int SCW = TOK ? 5 : SGX / 2;
    __shared__ __attribute__((aligned(16))) uint32_t sSA[2][MX ? TB * SCW : 1];
    __shared__ __attribute__((aligned(16))) uint32_t sSB[2][MX ? TB * SCW : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS copy bases go to M0
    const int wm = wave & 1, wn = wave >> 1;
    int64_t K = g.K;                                   // this tile's contraction length
    const int tiles_n = (int)((g.N + TB - 1) / TB);

    int64_t m0, m_end, n0;
    int64_t k0 = 0;                                    // token groups: first column of the expert's K range
    const uint8_t* Aq = g.a;
    const uint8_t* Bq = g.b;
    const uint8_t* Bs = g.sb;
    uint16_t* Cb = g.c;
    float* Cf = g.cf;
    if constexpr (TOK) {
        // Expert-major order in workgroup order (no XCD remap: consecutive workgroups go to different XCDs, so every
        // XCD shares the large experts at the front), grouped by GROUP_M2 row tiles of one expert.
        const int tiles_m = (int)((g.M + TB - 1) / TB);
        const int tiles_mm = (int)g.G * tiles_m;
        const int v = bid_in;
        const int per_group = GROUP_M2 * tiles_n;
        const int first_m = (v / per_group) * GROUP_M2;
        const int gm = min(GROUP_M2, tiles_mm - first_m);
        const int r = v % per_group;
        const int mt = first_m + r % gm;
        const int64_t grp = mt / tiles_m;
        m0 = (int64_t)(mt - grp * tiles_m) * TB;
        n0 = (int64_t)(r / gm) * TB;
        m_end = (m0 + TB < g.M) ? m0 + TB : g.M;
        int64_t a0 = g.offsets[grp], a1 = g.offsets[grp + 1];
        a0 = a0 < 0 ? 0 : (a0 > g.K ? g.K : a0);
        a1 = a1 < a0 ? a0 : (a1 > g.K ? g.K : a1);
        k0 = a0;
        K = a1 - a0;
        Aq = g.a + k0;
        Bq = g.b + k0;
        if (Cb) Cb += grp * g.c_gstride;
        if (Cf) Cf += grp * g.c_gstride;
    } else if constexpr (GM == GM_ROWS) {
        // XCD-aware order: workgroup b runs on XCD b % 8, and each XCD in turn takes a chunk of kXcdChunk consecutive
        // tiles (one per CU of the XCD), so the workgroups resident on an XCD share an expert's weight tiles and row
        // tiles in its L2. Workgroups past the last whole round keep their own index (the map stays a bijection).
        const int64_t nb = gridDim.x, b = bid_in, round = 8 * kXcdChunk;
        const int64_t bid = b < (nb / round) * round
                                ? (b >> 3) / kXcdChunk * round + (b & 7) * kXcdChunk + (b >> 3) % kXcdChunk
                                : b;
        const int64_t t = bid / tiles_n;
        n0 = (bid % tiles_n) * TB;
        const RowTile rt = find_row_tile<TB>(g, t);
        const int64_t grp = rt.grp, lo = rt.lo, hi = rt.hi;
        if (grp < 0) return;
        m0 = lo;
        m_end = (lo + TB < hi) ? lo + TB : hi;
        Bq = g.b + grp * g.b_gstride;
        Bs = MX ? g.sb + grp * g.sb_gstride : nullptr;
    } else {
        const int tiles_m = (int)((g.M + TB - 1) / TB);
        const int T = tiles_m * tiles_n;
        const int bid = bid_in;
        const int T8 = T & ~7;
        const int v = bid < T8 ? (bid & 7) * (T8 >> 3) + (bid >> 3) : bid;
        const int per_group = GROUP_M2 * tiles_n;
        const int first_m = (v / per_group) * GROUP_M2;
        const int gm = min(GROUP_M2, tiles_m - first_m);
        const int r = v % per_group;
        m0 = (int64_t)(first_m + r % gm) * TB;
        n0 = (int64_t)(r / gm) * TB;
        m_end = (m0 + TB < g.M) ? m0 + TB : g.M;
        if (g.gate == 1 || g.gate == 2) {
            // Checked path: the tile's first output element names the kernel that computes it (written by
            // gate_broadcast_kernel; only this workgroup writes the tile, and only after this read).
            const uint32_t v = __builtin_amdgcn_readfirstlane((uint32_t)Cb[m0 * g.ldc + n0]);
            if (v != (g.gate == 1 ? kGateFp8 : kGateExact)) return;
        } else if (g.gate) {
            // Ranged path: the operands' range words, written by the quantizers, pick the kernel.
            const uint32_t wide = __builtin_amdgcn_readfirstlane(*g.wa | *g.wb);
            if ((wide != 0u) != (g.gate == 4)) return;
        }
    }
    const int64_t n_end = (n0 + TB < g.N) ? n0 + TB : g.N;

    // ------------------------------------------------------------------ copies global -> LDS
    // One resource per operand based at the tile's first row; 32-bit per-lane offsets (row * K + byte, below 2^31
    // because the host requires 256 K < 2^31); a pair's k offset goes in the scalar offset. Copy instruction c of a
    // wave fills block 4c + wave of a region.
    const int half_lane = lane >> 5;                       // which stage of a pair this lane carries
    const int brow = (lane & 31) >> 2;                     // row within the 8-row block
    // chunk this lane fetches: its position ^ swz8(row); rows 8 (4c + wave) + brow have swz8 = (2 wave + brow / 4) & 3
    const int bchunk = (lane & 3) ^ ((2 * wave + (brow >> 2)) & 3);
    // Token groups: a half-filled last stage reads up to 32 bytes past the expert's range; the record counts end
    // the resources at the operands' last byte, so such reads past the matrix return zero (and are never used).
    const v4i rA = TOK ? buffer_rsrc(Aq + m0 * g.lda, (uint32_t)((g.M - m0) * g.lda - k0))
                       : buffer_rsrc(Aq + m0 * g.lda);
    const v4i rB = TOK ? buffer_rsrc(Bq + n0 * g.ldb, (uint32_t)((g.N - n0) * g.ldb - k0))
                       : buffer_rsrc(Bq + n0 * g.ldb);
    int a_off[8], b_off[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int row = 8 * (4 * c + wave) + brow;
        const int ar = (m0 + row < m_end) ? row : (int)(m_end - 1 - m0);
        const int br = (n0 + row < n_end) ? row : (int)(n_end - 1 - n0);
        a_off[c] = ar * (int)g.lda + KS * half_lane + 16 * bchunk;
        b_off[c] = br * (int)g.ldb + KS * half_lane + 16 * bchunk;
    }
    v4i rSA = rA, rSB = rB;
    int sa_off = 0, sb_off = 0;
    int sa_off2[2] = {0, 0}, sb_off2[2] = {0, 0};
    if constexpr (TOK) {
        // Scale bytes of row r for the expert start at byte r * lds + k0 / 32 of the grid (any alignment). Each lane
        // copies 4-byte words from the aligned address at or below it; a word holding a byte of the grid lies in
        // the grid's last page, and words past the grid's rounded-up end read as zero.
        const int row = 64 * wave + lane;
        const int ar = (m0 + row < m_end) ? row : (int)(m_end - 1 - m0);
        const int br = (n0 + row < n_end) ? row : (int)(n_end - 1 - n0);
        rSA = buffer_rsrc(g.sa, (uint32_t)((g.M * g.ldsa + 3) & ~int64_t(3)));
        rSB = buffer_rsrc(g.sb, (uint32_t)((g.N * g.ldsb + 3) & ~int64_t(3)));
        sa_off = (int)(((m0 + ar) * g.ldsa + k0 / 32) & ~int64_t(3));
        sb_off = (int)(((n0 + br) * g.ldsb + k0 / 32) & ~int64_t(3));
    } else if constexpr (MX && SGX == SGM) {
        // copy k (0, 1) of a wave: rows 32 (2 wave + k) + lane / 2, bytes 16 (lane % 2) .. + 15 of the row's group
        rSA = buffer_rsrc(g.sa + m0 * g.ldsa);
        rSB = buffer_rsrc(Bs + n0 * g.ldsb);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int row = 32 * (2 * wave + k) + (lane >> 1);
            const int ar = (m0 + row < m_end) ? row : (int)(m_end - 1 - m0);
            const int br = (n0 + row < n_end) ? row : (int)(n_end - 1 - n0);
            sa_off2[k] = ar * (int)g.ldsa + 16 * (lane & 1);
            sb_off2[k] = br * (int)g.ldsb + 16 * (lane & 1);
        }
    } else if constexpr (MX) {
        const int row = 64 * wave + lane;
        const int ar = (m0 + row < m_end) ? row : (int)(m_end - 1 - m0);
        const int br = (n0 + row < n_end) ? row : (int)(n_end - 1 - n0);
        rSA = buffer_rsrc(g.sa + m0 * g.ldsa);
        rSB = buffer_rsrc(Bs + n0 * g.ldsb);
        sa_off = ar * (int)g.ldsa;
        sb_off = br * (int)g.ldsb;
    }
    // Token groups: a K range of 32 mod 64 ends in a half stage, of which only the first 32-value block is summed.
    const int nk = TOK ? (int)((K + KS - 1) / KS) : (int)(K / KS);
    const bool half_last = TOK && (K % KS) != 0;
    // Byte shift of the fragment rows' scale words (token groups): the low two bits of each row's first scale byte,
    // two bits per row, A rows j at bits 2j, B rows i at bits 8 + 2i (v_alignbyte reads only the low two bits).
    uint32_t shifts = 0;
    if constexpr (TOK) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = wm * 128 + 32 * j + (lane & 31);
            const int ar = (m0 + row < m_end) ? row : (int)(m_end - 1 - m0);
            shifts |= (uint32_t)(((m0 + ar) * g.ldsa + k0 / 32) & 3) << (2 * j);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = wn * 128 + 32 * i + (lane & 31);
            const int br = (n0 + row < n_end) ? row : (int)(n_end - 1 - n0);
            shifts |= (uint32_t)(((n0 + br) * g.ldsb + k0 / 32) & 3) << (8 + 2 * i);
        }
    }
    // Region of stage s: A (s / 2) % 2, B ((s + 1) / 2) % 2; its half: A s % 2, B (s + 1) % 2.
    // Copy instruction c of the pair of operand A (IS_A) or B whose first stage is s0, into region `region`. When the
    // pair's second stage lies past K only the first-stage lanes copy.
    // WHOLE: the pair is known at compile time to lie inside K.
    auto copy_pair = [&](auto is_a, auto whole_c, int region, int s0, int c) {
        constexpr bool IS_A = decltype(is_a)::value;
        const uint32_t lds = lds_offset(IS_A ? &sA[region][1024 * wave] : &sB[region][1024 * wave]) + 4096 * c;
        if (decltype(whole_c)::value || s0 + 1 < nk)
            dma_to_lds<16>(IS_A ? rA : rB, lds, IS_A ? a_off[c] : b_off[c], s0 * KS);
        else if (half_lane == 0)
            dma_to_lds<16>(IS_A ? rA : rB, lds, IS_A ? a_off[c] : b_off[c], s0 * KS);
    };
    auto copy_scales = [&](int s) {                       // the scale group whose first stage is s
        const int gb = (s / SGX) & 1;
        if constexpr (TOK) {
#pragma unroll
            for (int w = 0; w < 5; ++w) {
                dma_to_lds<4>(rSA, lds_offset(&sSA[gb][TB * w + 64 * wave]), sa_off, s * KS / 32 + 4 * w);
                dma_to_lds<4>(rSB, lds_offset(&sSB[gb][TB * w + 64 * wave]), sb_off, s * KS / 32 + 4 * w);
            }
        } else {
            if constexpr (SGX == SGM) {
                // a half whose 8 stages lie past K is not read (K is a whole number of 8-stage halves)
                const bool half_in = s + 8 * (lane & 1) < nk;
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    if (half_in) {
                        dma_to_lds<16>(rSA, lds_offset(&sSA[gb][32 * (2 * wave + k) * SCW]), sa_off2[k], s * KS / 32);
                        dma_to_lds<16>(rSB, lds_offset(&sSB[gb][32 * (2 * wave + k) * SCW]), sb_off2[k], s * KS / 32);
                    }
                }
            } else {
                dma_to_lds<16>(rSA, lds_offset(&sSA[gb][256 * wave]), sa_off, s * KS / 32);
                dma_to_lds<16>(rSB, lds_offset(&sSB[gb][256 * wave]), sb_off, s * KS / 32);
            }
        }
    };
    constexpr int kScaleCopies = TOK ? 10 : (SGX == SGM ? 4 : 2);
    // Copy instruction c of trip t: the pair starting at stage t + 3 (A on odd t, B on even t), if any. PH = t % 4 when
    // known at compile time (then the pair exists in full), else -1.
    auto trip_copy = [&](auto ph_c, int t, int c) {
        constexpr int PH = decltype(ph_c)::value;
        const int s0 = t + 3;
        if constexpr (PH >= 0) {
            if constexpr (PH & 1) copy_pair(std::true_type{}, std::true_type{}, ((PH + 3) >> 1) & 1, s0, c);
            else copy_pair(std::false_type{}, std::true_type{}, ((PH + 4) >> 1) & 1, s0, c);
        } else if (s0 < nk) {
            if (t & 1) copy_pair(std::true_type{}, std::false_type{}, (s0 >> 1) & 1, s0, c);
            else copy_pair(std::false_type{}, std::false_type{}, ((s0 + 1) >> 1) & 1, s0, c);
        }
    };
    // Scale copies of trip t (issued after its pair): the group starting at stage t + 4. Returns whether issued.
    auto trip_scales = [&](int t) -> bool {
        if constexpr (MX) {
            const int s = t + 4;
            if (s % SGX == 0 && s < nk) { copy_scales(s); return true; }
        }
        return false;
    };
    // Wait at the end of trip t: only the copies issued in trip t may remain in flight.
    auto trip_wait = [&](int t, bool scales) {
        if (t + 3 >= nk) wait_copies_barrier<0>();
        else if (scales) wait_copies_barrier<8 + kScaleCopies>();
        else wait_copies_barrier<8>();
    };

    // ------------------------------------------------------------------ fragments
    // 32 x 32 x 64 operand of lane l: row l % 32, global chunks g and 2 + g of the 64-byte stage row (g = l / 32),
    // i.e. k = 16g .. 16g+15 and 32+16g .. 32+16g+15. Its scale operand is the scale of (row, block g), stage word
    // (st % SGX) / 2, byte 2 (st % 2) + g.
    const int fr = lane & 31, fg = lane >> 5;
    const int fsw = swz8(fr);                  // rows wm*128 + 32j + fr share bits 2..3 with fr
    const int frow = (fr >> 3) * 1024 + (fr & 7) * KS;   // lane's row within its 32-row group (block, row in block)
    const int fch0 = 16 * (fg ^ fsw), fch1 = 16 * ((2 + fg) ^ fsw);
    // Byte offset, within an operand's LDS, of chunk half h (0: chunk g, 1: chunk 2 + g) of the lane's row in 32-row
    // group `grp` (0..7) of stage s. SP = s % 4 when known at compile time, else -1.
    auto frag_off = [&](auto is_a, auto sp_c, int s, int grp, int h) {
        constexpr bool IS_A = decltype(is_a)::value;
        constexpr int SP = decltype(sp_c)::value;
        const int sp = SP < 0 ? (s & 3) : SP;
        const int region = IS_A ? ((sp >> 1) & 1) : (((sp + 1) >> 1) & 1);
        const int half = IS_A ? (sp & 1) : ((sp + 1) & 1);
        return region * (2 * TB * KS) + grp * 4096 + half * 512 + frow + (h ? fch1 : fch0);
    };
    auto frag = [&](auto is_a, auto sp_c, int s, int grp) {
        constexpr bool IS_A = decltype(is_a)::value;
        const uint8_t* base = IS_A ? &sA[0][0] : &sB[0][0];
        const uint4 x0 = *reinterpret_cast<const uint4*>(base + frag_off(is_a, sp_c, s, grp, 0));
        const uint4 x1 = *reinterpret_cast<const uint4*>(base + frag_off(is_a, sp_c, s, grp, 1));
        return v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    };
    auto read_scales = [&](int st, uint32_t* sa, uint32_t* sb) {
        if constexpr (TOK) {
            // word w of the group = bytes 4w .. 4w+3 after the row's shift
            const uint32_t* cSA = sSA[(st / SGX) & 1];
            const uint32_t* cSB = sSB[(st / SGX) & 1];
            const int w = (st % SGX) >> 1;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = wm * 128 + 32 * j + fr;
                sa[j] = __builtin_amdgcn_alignbyte(cSA[TB * (w + 1) + row], cSA[TB * w + row], shifts >> (2 * j));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wn * 128 + 32 * i + fr;
                sb[i] = __builtin_amdgcn_alignbyte(cSB[TB * (w + 1) + row], cSB[TB * w + row], shifts >> (8 + 2 * i));
            }
        } else if constexpr (MX) {
            const uint32_t* cSA = sSA[(st / SGX) & 1];
            const uint32_t* cSB = sSB[(st / SGX) & 1];
            const int w = (st % SGX) >> 1;
#pragma unroll
            for (int j = 0; j < 4; ++j) sa[j] = cSA[(wm * 128 + 32 * j + fr) * SCW + w];
#pragma unroll
            for (int i = 0; i < 4; ++i) sb[i] = cSB[(wn * 128 + 32 * i + fr) * SCW + w];
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) { sa[j] = 0x7F7F7F7Fu; sb[j] = 0x7F7F7F7Fu; }
        }
        if constexpr (MF == 2) {
            // exact path: the stage's bf16-conversion scale operands, block-major: [4 blk + j]
            uint32_t wa[4], wb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) { wa[j] = sa[j]; wb[j] = sb[j]; }
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                const int sh = 8 * (2 * (st & 1) + blk);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    sa[4 * blk + j] = __float_as_uint(scale_operand((wa[j] >> sh) & 0xFFu));
                    sb[4 * blk + j] = __float_as_uint(scale_operand((wb[j] >> sh) & 0xFFu));
                }
            }
        }
    };
    auto read_stage = [&](auto sp_c, int st, v8i* fa, v8i* fb, uint32_t* sa, uint32_t* sb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) fa[j] = frag(std::true_type{}, sp_c, st, 4 * wm + j);
#pragma unroll
        for (int i = 0; i < 4; ++i) fb[i] = frag(std::false_type{}, sp_c, st, 4 * wn + i);
        read_scales(st, sa, sb);
    };

    v16f acc16[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc16[i][j] = v16f{};

    // The matrix instructions of one stage, from fragments in registers.
    auto mma_stage = [&](auto par_c, int kt, const v8i* fa, const v8i* fb, const uint32_t* sa, const uint32_t* sb) {
        constexpr int PAR = decltype(par_c)::value;                // kt & 1 when known at compile time, else -1
        if constexpr (MF == 1) {
            const int odd = PAR < 0 ? (kt & 1) : PAR;
            const int sh = 8 * (2 * odd + fg);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc16[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        fb[i], fa[j], acc16[i][j], FB, FA, 0, (int)(sb[i] >> sh), 0, (int)(sa[j] >> sh));
        } else {
            // Exact path: dequantize to bf16 and use the bf16 instruction. k-step s takes bytes 8s .. 8s+7 of each
            // lane's 32 (A and B lanes hold the same k values, so the product sums every k of the stage once);
            // steps 0, 1 lie in the stage's first 32-block, steps 2, 3 in its second. The two blocks' scale operands
            // were formed when the stage's scale words were read, a trip ahead (read_scales).
            float xa[2][4], xb[2][4];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
                for (int j = 0; j < 4; ++j) xa[blk][j] = __uint_as_float(sa[4 * blk + j]);
#pragma unroll
                for (int i = 0; i < 4; ++i) xb[blk][i] = __uint_as_float(sb[4 * blk + i]);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                v8bf da[4], db[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    da[j] = dequant8_bf16<FA>(make_uint2((uint32_t)fa[j][2 * s], (uint32_t)fa[j][2 * s + 1]),
                                              xa[s >> 1][j]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    db[i] = dequant8_bf16<FB>(make_uint2((uint32_t)fb[i][2 * s], (uint32_t)fb[i][2 * s + 1]),
                                              xb[s >> 1][i]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc16[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(db[i], da[j], acc16[i][j], 0, 0, 0);
            }
        }
    };

    // The matrix instructions are pure, so the optimizer may otherwise sink them past the (asm) waits and barriers.
    // This empty statement reads every accumulator, so all of a stage's instructions are issued before the wait
    // that follows it.
    auto pin_accumulators = [&]() {
        asm volatile("" :: "a"(acc16[0][0]), "a"(acc16[0][1]), "a"(acc16[0][2]), "a"(acc16[0][3]),
                           "a"(acc16[1][0]), "a"(acc16[1][1]), "a"(acc16[1][2]), "a"(acc16[1][3]),
                           "a"(acc16[2][0]), "a"(acc16[2][1]), "a"(acc16[2][2]), "a"(acc16[2][3]),
                           "a"(acc16[3][0]), "a"(acc16[3][1]), "a"(acc16[3][2]), "a"(acc16[3][3]));
    };

    // Scheduling pattern for a stage of the exact path: four matrix instructions, then the next LDS read (MX: two),
    // so the next stage's fragment reads trickle out between the matrix instructions instead of queueing ahead.
    auto interleave_reads = [&]() {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);                // matrix instructions
            __builtin_amdgcn_sched_group_barrier(0x100, MX ? 2 : 1, 0);        // LDS reads
        }
    };

    // ------------------------------------------------------------------ prologue: stages 0 .. 3
    // (token groups: an expert without tokens skips straight to its zero output)
    if (!TOK || nk > 0) {
    if constexpr (MX) copy_scales(0);
#pragma unroll
    for (int c = 0; c < 8; ++c) copy_pair(std::true_type{}, std::false_type{}, 0, 0, c);       // A (0, 1)
#pragma unroll
    for (int c = 0; c < 8; ++c) {                                                       // B (-1, 0): stage 0 only
        const uint32_t lds = lds_offset(&sB[0][1024 * wave]) + 4096 * c;
        if (half_lane == 1) dma_to_lds<16>(rB, lds, b_off[c] - KS, 0);
    }
    if (nk > 1) {
#pragma unroll
        for (int c = 0; c < 8; ++c) copy_pair(std::false_type{}, std::false_type{}, 1, 1, c);  // B (1, 2)
    }
    if (nk > 2) {
#pragma unroll
        for (int c = 0; c < 8; ++c) copy_pair(std::true_type{}, std::false_type{}, 1, 2, c);   // A (2, 3)
    }
    // The zeroed accumulators are written here, while the first stages are in flight, rather than after the wait
    // (where the compiler would otherwise put their 256 register writes, just before the first matrix instruction).
    // The statement reads and rewrites each one, so the sixteen zero blocks stay distinct registers.
    asm volatile("" : "+a"(acc16[0][0]), "+a"(acc16[0][1]), "+a"(acc16[0][2]), "+a"(acc16[0][3]),
                      "+a"(acc16[1][0]), "+a"(acc16[1][1]), "+a"(acc16[1][2]), "+a"(acc16[1][3]),
                      "+a"(acc16[2][0]), "+a"(acc16[2][1]), "+a"(acc16[2][2]), "+a"(acc16[2][3]),
                      "+a"(acc16[3][0]), "+a"(acc16[3][1]), "+a"(acc16[3][2]), "+a"(acc16[3][3]));
    if (nk > 2) wait_copies_barrier<8>();                       // stages 0 and 1 have landed
    else wait_copies_barrier<0>();
    if constexpr (MF == 2) {
    // Exact path, pipelined over the stage's four 16-value k-steps. k-step s takes bytes 8s .. 8s+7 of each lane's
    // 32 (steps 0, 1 lie in the stage's first 32-block, 2, 3 in its second). While k-step s's 16 matrix instructions
    // run, k-step s + 1 is converted to bf16 (two conversions per matrix instruction), and the next stage's fragments
    // stream into the registers of k-steps already converted: bytes 0-15 during k-step 0, bytes 16-31 during k-step 2;
    // k-step 3 converts the next stage's k-step 0. One fragment register set thus serves both stages, which leaves
    // room for two sets of converted operands.
    v8i F[8];                                  // F[j]: A rows wm*128 + 32j + (lane % 32); F[4 + i]: B rows wn*128 + 32i
    uint32_t SA[2][8], SB[2][8];               // conversion scale operands [4 blk + j] of the current and next stage
    v8bf CV[2][8];                             // converted k-steps: CV[s & 1][j] A, [4 + i] B
    // chunk half h (bytes 16h .. 16h+15) of all eight fragments of stage st
    auto read_chunk = [&](auto sp_c, int st, auto h_c) {
        constexpr int H = decltype(h_c)::value;
#pragma unroll
        for (int f = 0; f < 8; ++f) {
            const uint4 x = f < 4 ? *reinterpret_cast<const uint4*>(&sA[0][0] + frag_off(std::true_type{}, sp_c, st,
                                                                                          4 * wm + f, H))
                                  : *reinterpret_cast<const uint4*>(&sB[0][0] + frag_off(std::false_type{}, sp_c, st,
                                                                                          4 * wn + f - 4, H));
            F[f][4 * H] = (int)x.x; F[f][4 * H + 1] = (int)x.y; F[f][4 * H + 2] = (int)x.z; F[f][4 * H + 3] = (int)x.w;
        }
    };
    // fragment f's k-step s, with the scale operands of its block
    auto convert = [&](int s, int f, const uint32_t* sa, const uint32_t* sb, v8bf* cv) {
        const uint2 x = make_uint2((uint32_t)F[f][2 * s], (uint32_t)F[f][2 * s + 1]);
        if (f < 4) cv[f] = dequant8_bf16<FA>(x, __uint_as_float(sa[4 * (s >> 1) + f]));
        else cv[f] = dequant8_bf16<FB>(x, __uint_as_float(sb[4 * (s >> 1) + f - 4]));
    };
    // Raw scale words of stage st for the fragment rows (LDS reads only; the operands are formed later, by
    // scale_op, so no wait for these reads sits between matrix instructions): MX rows word w of the group in
    // ra[j] / rb[i]; token groups words w and w + 1 in [j] and [4 + j]; per-tensor unit scales.
    auto scale_words = [&](int st, uint32_t* ra, uint32_t* rb) {
        const int w = (st % SGX) >> 1;
        if constexpr (TOK) {
            const uint32_t* cSA = sSA[(st / SGX) & 1];
            const uint32_t* cSB = sSB[(st / SGX) & 1];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = wm * 128 + 32 * j + fr;
                ra[j] = cSA[TB * w + row];
                ra[4 + j] = cSA[TB * (w + 1) + row];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wn * 128 + 32 * i + fr;
                rb[i] = cSB[TB * w + row];
                rb[4 + i] = cSB[TB * (w + 1) + row];
            }
        } else if constexpr (MX) {
            const uint32_t* cSA = sSA[(st / SGX) & 1];
            const uint32_t* cSB = sSB[(st / SGX) & 1];
#pragma unroll
            for (int j = 0; j < 4; ++j) ra[j] = cSA[(wm * 128 + 32 * j + fr) * SCW + w];
#pragma unroll
            for (int i = 0; i < 4; ++i) rb[i] = cSB[(wn * 128 + 32 * i + fr) * SCW + w];
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) { ra[j] = 0x7F7F7F7Fu; rb[j] = 0x7F7F7F7Fu; }
        }
    };
    // Conversion scale operand e (0 .. 15; A [4 blk + j] for e < 8, B [4 blk + i] after) of stage st from its raw
    // words, as read_scales forms it.
    auto scale_op = [&](int st, const uint32_t* ra, const uint32_t* rb, int e, uint32_t* sa, uint32_t* sb) {
        const bool is_a = e < 8;
        const int blk = (e >> 2) & 1, r = e & 3;
        const uint32_t* raw = is_a ? ra : rb;
        uint32_t word;
        if constexpr (TOK) word = __builtin_amdgcn_alignbyte(raw[4 + r], raw[r], shifts >> ((is_a ? 0 : 8) + 2 * r));
        else word = raw[r];
        const uint32_t v = __float_as_uint(scale_operand((word >> (8 * (2 * (st & 1) + blk))) & 0xFFu));
        if (is_a) sa[4 * blk + r] = v;
        else sb[4 * blk + r] = v;
    };
    // k-step S: its 16 matrix instructions from CV[S & 1]. Between them: the conversion of k-step CS (0 .. 3 of the
    // stage whose scales are csa/csb; -1 none) into CV[(S + 1) & 1], one fragment per two instructions; if
    // RH >= 0, chunk half RH of the next stage's fragments (stage st_next, position SPN), one fragment per two;
    // with XS, the next stage's scale operand q after instruction q (from the raw words xra / xrb into xsa / xsb);
    // with CP >= 0, the trip's copy instructions CP .. CP + NC - 1 (copy(c)), spread evenly (copy c after
    // instruction (16 / NC) (c + 1/2) - 1), fenced so each stays between its matrix instructions: a copy that finds
    // the memory queue full then stalls the wave while a matrix instruction is still running.
    auto kstep = [&](auto s_c, auto cs_c, const uint32_t* csa, const uint32_t* csb, auto rh_c, auto spn_c,
                     int st_next, auto xs_c, const uint32_t* xra, const uint32_t* xrb, uint32_t* xsa,
                     uint32_t* xsb, auto cp_c, auto nc_c, auto&& copy) {
        constexpr int S = decltype(s_c)::value, CS = decltype(cs_c)::value, RH = decltype(rh_c)::value;
        constexpr bool XS = decltype(xs_c)::value;
        constexpr int CP = decltype(cp_c)::value, NC = decltype(nc_c)::value;
        auto read_f = [&](int f) {
            const uint4 x = f < 4 ? *reinterpret_cast<const uint4*>(&sA[0][0] +
                                        frag_off(std::true_type{}, spn_c, st_next, 4 * wm + f, RH))
                                  : *reinterpret_cast<const uint4*>(&sB[0][0] +
                                        frag_off(std::false_type{}, spn_c, st_next, 4 * wn + f - 4, RH));
            F[f][4 * RH] = (int)x.x; F[f][4 * RH + 1] = (int)x.y;
            F[f][4 * RH + 2] = (int)x.z; F[f][4 * RH + 3] = (int)x.w;
        };
        auto slot = [&](int q) {
            const int i = q >> 2, j = q & 3;
            acc16[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(CV[S & 1][4 + i], CV[S & 1][j], acc16[i][j], 0, 0, 0);
            if constexpr (CS >= 0) {
                if (q & 1) convert(CS, q >> 1, csa, csb, CV[(S + 1) & 1]);
            }
            if constexpr (RH >= 0) {
                if ((q & 1) == 0 && q > 0) read_f((q >> 1) - 1);   // the fragment whose last conversion just issued
            }
            if constexpr (XS) scale_op(st_next, xra, xrb, q, xsa, xsb);
        };
        constexpr int NV = (CS >= 0 ? 2 : 0) + (XS ? 2 : 0);
        auto groups = [&](int q0, int q1) {                     // the scheduling pattern of instructions q0 .. q1
#pragma unroll
            for (int q = q0; q <= q1; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // one matrix instruction
                if constexpr (RH >= 0) {
                    if ((q & 1) == 0 && q > 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // a fragment read
                }
                if constexpr (NV > 0) __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);  // conversions, scales
            }
        };
        if constexpr (CP < 0) {
#pragma unroll
            for (int q = 0; q < 16; ++q) slot(q);
            if constexpr (RH >= 0) read_f(7);
            groups(0, 15);
        } else {
            constexpr int D = 16 / NC;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int q0 = c == 0 ? 0 : D * c - D / 2, q1 = D * c + D / 2 - 1;
#pragma unroll
                for (int q = q0; q <= q1; ++q) slot(q);
                groups(q0, q1);
                __builtin_amdgcn_sched_barrier(0);
                copy(CP + c);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int q = 16 - D / 2; q < 16; ++q) slot(q);
            if constexpr (RH >= 0) read_f(7);
            groups(16 - D / 2, 15);
        }
        __builtin_amdgcn_sched_barrier(0);                                            // k-steps do not mix
    };
    // The next stage's k-step 0 operands and its scale operands, used after the trip's wait: this empty statement
    // keeps the compiler from moving their conversions past the branch of the next trip's scale copy, which would
    // put them all between two matrix instructions instead of spread over k-step 3.
    auto pin_converted = [&](const uint32_t* nsa, const uint32_t* nsb) {
        asm volatile("" :: "v"(CV[0][0]), "v"(CV[0][1]), "v"(CV[0][2]), "v"(CV[0][3]),
                           "v"(CV[0][4]), "v"(CV[0][5]), "v"(CV[0][6]), "v"(CV[0][7]));
        asm volatile("" :: "v"(nsa[0]), "v"(nsa[1]), "v"(nsa[2]), "v"(nsa[3]), "v"(nsa[4]), "v"(nsa[5]),
                           "v"(nsa[6]), "v"(nsa[7]));
        asm volatile("" :: "v"(nsb[0]), "v"(nsb[1]), "v"(nsb[2]), "v"(nsb[3]), "v"(nsb[4]), "v"(nsb[5]),
                           "v"(nsb[6]), "v"(nsb[7]));
    };
    // k-step without scale operands
    auto no_copy = [](int) {};
    using NOCP = std::integral_constant<int, -1>;
    auto kstep_ = [&](auto s_c, auto cs_c, const uint32_t* csa, const uint32_t* csb, auto rh_c, auto spn_c,
                      int st_next) {
        kstep(s_c, cs_c, csa, csb, rh_c, spn_c, st_next, std::false_type{}, nullptr, nullptr, nullptr, nullptr,
              NOCP{}, NOCP{}, no_copy);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using NONE = std::integral_constant<int, -1>;
    // Trip kt (kt + 1 < nk): stage kt's four k-steps with the trip's copies (two per k-step) and stage kt + 1's
    // fragments, scale operands and k-step 0 conversion folded in, then the scale copies and the wait until stage
    // kt + 2 has landed.
    auto trip = [&](auto ph_c, int kt, uint32_t* csa, uint32_t* csb, uint32_t* nsa, uint32_t* nsb) {
        constexpr int PH = decltype(ph_c)::value;
        using SP = std::integral_constant<int, PH < 0 ? -1 : (PH + 1) % 4>;     // stage kt + 1 mod 4
        // stage kt + 1's scale words, read ahead of the trip's fragment reads: LDS reads return in order, so the
        // wait before their use in k-step 1 does not hold for the fragment reads issued after them
        uint32_t ra[8], rb[8];
        scale_words(kt + 1, ra, rb);
        __builtin_amdgcn_sched_barrier(0);
        auto copy = [&](int c) { trip_copy(ph_c, kt, c); };
        using C2 = std::integral_constant<int, 2>;
        // bytes 0-15 of stage kt + 1 follow their conversions, bytes 16-31 likewise; the trip's copies go two per
        // k-step; k-step 3 converts the next stage's k-step 0 (its bytes arrived during k-step 0) with its scales
        kstep(I0{}, I1{}, csa, csb, I0{}, SP{}, kt + 1, std::false_type{}, nullptr, nullptr, nullptr, nullptr, I0{},
              C2{}, copy);
        kstep(I1{}, I2{}, csa, csb, NONE{}, SP{}, kt + 1, std::true_type{}, ra, rb, nsa, nsb, I2{}, C2{}, copy);
        kstep(I2{}, I3{}, csa, csb, I1{}, SP{}, kt + 1, std::false_type{}, nullptr, nullptr, nullptr, nullptr,
              std::integral_constant<int, 4>{}, C2{}, copy);
        kstep(I3{}, I0{}, nsa, nsb, NONE{}, SP{}, kt + 1, std::false_type{}, nullptr, nullptr, nullptr, nullptr,
              std::integral_constant<int, 6>{}, C2{}, copy);
        pin_accumulators();
        pin_converted(nsa, nsb);
        // the scale copies (a branch) go last, so the trip's matrix instructions share one basic block
        const bool scales = trip_scales(kt);
        if constexpr (PH >= 0) {
            if (scales) wait_copies_barrier<8 + kScaleCopies>();
            else wait_copies_barrier<8>();
        } else {
            trip_wait(kt, scales);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
    };
    // The last stage (its fragments, scales and k-step 0 conversion are in registers; no copy is outstanding).
    auto last_stage = [&](uint32_t* csa, uint32_t* csb) {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (TOK) {
            // A half last stage sums only its first block: the second block's codes become 0 and its scale bytes
            // 2^0, so k-steps 2 and 3 add exact zeros whatever lies past the expert's range (selects, not branches).
            const uint32_t keep = half_last ? 0u : 0xFFFFFFFFu;
            const uint32_t one = __float_as_uint(scale_operand(127u));
#pragma unroll
            for (int f = 0; f < 8; ++f)
#pragma unroll
                for (int e = 4; e < 8; ++e) F[f][e] = (int)((uint32_t)F[f][e] & keep);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                csa[4 + j] = half_last ? one : csa[4 + j];
                csb[4 + j] = half_last ? one : csb[4 + j];
            }
        }
        kstep_(I0{}, I1{}, csa, csb, NONE{}, NONE{}, 0);
        kstep_(I1{}, I2{}, csa, csb, NONE{}, NONE{}, 0);
        kstep_(I2{}, I3{}, csa, csb, NONE{}, NONE{}, 0);
        kstep_(I3{}, NONE{}, csa, csb, NONE{}, NONE{}, 0);
    };
    // prologue: stage 0's fragments, scales and k-step 0
    read_chunk(I0{}, 0, I0{});
    read_chunk(I0{}, 0, I1{});
    read_scales(0, SA[0], SB[0]);
    // Stage 0's regions are refilled by the first trips: every wave's reads of them must have returned.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
#pragma unroll
    for (int f = 0; f < 8; ++f) convert(0, f, SA[0], SB[0], CV[0]);
    using dyn = std::integral_constant<int, -1>;
    int kt = 0;
    for (; kt + 7 < nk; kt += 4) {                               // kt % 4 == 0; every pair of these trips is whole
        trip(I0{}, kt, SA[0], SB[0], SA[1], SB[1]);
        trip(I1{}, kt + 1, SA[1], SB[1], SA[0], SB[0]);
        trip(I2{}, kt + 2, SA[0], SB[0], SA[1], SB[1]);
        trip(I3{}, kt + 3, SA[1], SB[1], SA[0], SB[0]);
    }
    for (; kt + 2 < nk; kt += 2) {
        trip(dyn{}, kt, SA[0], SB[0], SA[1], SB[1]);
        trip(dyn{}, kt + 1, SA[1], SB[1], SA[0], SB[0]);
    }
    if (kt + 1 < nk) {
        trip(dyn{}, kt, SA[0], SB[0], SA[1], SB[1]);
#pragma unroll
        for (int e = 0; e < 8; ++e) { SA[0][e] = SA[1][e]; SB[0][e] = SB[1][e]; }
    }
    last_stage(SA[0], SB[0]);
    } else {
    v8i fa[4], fb[4];
    constexpr int SAN = MF == 2 ? 8 : 4;                  // scale registers per operand (exact path: operands)
    uint32_t sa[SAN], sb[SAN];
    read_stage(std::integral_constant<int, 0>{}, 0, fa, fb, sa, sb);
    // Stage 0's regions are refilled by the first trips: every wave's reads of them must have returned.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // The asm waits are invisible to the compiler; this visible lgkmcnt(0) (vmcnt 63 and expcnt 7: no wait) tells it
    // that the fragment reads so far have returned, so it does not hold matrix instructions for them later.
    __builtin_amdgcn_s_waitcnt(0xC07F);

    // ------------------------------------------------------------------ trips
    // Trip kt (kt + 1 < nk): copy the trip's pair, read stage kt + 1's fragments, multiply stage kt, then wait until
    // stage kt + 2 has landed. Two fragment register sets ping-pong between trips (no copies between iterations).
    v8i fa2[4], fb2[4];
    uint32_t sa2[SAN], sb2[SAN];
    // PH_C: kt % 4 as a std::integral_constant when known (then the trip's pair exists in full), else -1.
    auto steady = [&](auto ph_c, int kt, v8i* ca, v8i* cb, uint32_t* csa, uint32_t* csb, v8i* na, v8i* nb,
                      uint32_t* nsa, uint32_t* nsb) {
        constexpr int PH = decltype(ph_c)::value;
        using SP = std::integral_constant<int, PH < 0 ? -1 : (PH + 1) % 4>;     // stage kt + 1 mod 4
        bool scales = false;
        if constexpr (MF == 1) {
            // FP8 path: 16 issue slots, each one matrix instruction; the 16 fragment reads of stage kt + 1 go two per
            // slot in the first 8 slots and (MX) its 8 scale reads two per slot in the next 4, so they have returned
            // well before the wait that ends the trip; the trip's 8 copy instructions go in the slots kCopySlot names,
            // and a scale group's copies (every SGM trips) after slot 7, not at the end of the trip where a stall on
            // them would hold the wave back from the barrier. Spreading the copies keeps a wave that finds the memory
            // queue full from stalling its matrix instructions behind a burst of copy issues. The scheduling barriers
            // keep the slots in this order.
            const int odd = PH < 0 ? (kt & 1) : (PH & 1);
            const int sh = 8 * (2 * odd + fg);
            const uint32_t* cSA = sSA[((kt + 1) / SGX) & 1];
            const uint32_t* cSB = sSB[((kt + 1) / SGX) & 1];
            const int sw = ((kt + 1) % SGX) >> 1;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int i = q >> 2, j = q & 3;
                acc16[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    cb[i], ca[j], acc16[i][j], FB, FA, 0, (int)(csb[i] >> sh), 0, (int)(csa[j] >> sh));
#pragma unroll
                for (int pc = 2 * q; pc < 2 * q + 2; ++pc) {
                    if (pc >= 16) break;
                    const int f = pc >> 1, h = pc & 1;
                    uint4 x;
                    if (f < 4)
                        x = *reinterpret_cast<const uint4*>(&sA[0][0] +
                                                            frag_off(std::true_type{}, SP{}, kt + 1, 4 * wm + f, h));
                    else
                        x = *reinterpret_cast<const uint4*>(&sB[0][0] +
                                                            frag_off(std::false_type{}, SP{}, kt + 1, 4 * wn + f - 4, h));
                    v8i& d = f < 4 ? na[f & 3] : nb[f & 3];
                    d[4 * h] = (int)x.x; d[4 * h + 1] = (int)x.y; d[4 * h + 2] = (int)x.z; d[4 * h + 3] = (int)x.w;
                }
                if constexpr (MX) {
                    // A scale word holds the bytes of two stages: an odd stage reuses its even neighbour's words.
                    constexpr bool REUSE = PH >= 0 && ((PH + 1) & 1) == 1;
                    if constexpr (REUSE) {
                        if (q == 8) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) { nsa[e] = csa[e]; nsb[e] = csb[e]; }
                        }
                    } else if (q >= 8 && q < 12) {
#pragma unroll
                        for (int e = 2 * (q - 8); e < 2 * (q - 8) + 2; ++e) {
                            if (e < 4) nsa[e] = cSA[(wm * 128 + 32 * e + fr) * SCW + sw];
                            else nsb[e - 4] = cSB[(wn * 128 + 32 * (e - 4) + fr) * SCW + sw];
                        }
                    }
                } else if (q == 0) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) { nsa[e] = 0x7F7F7F7Fu; nsb[e] = 0x7F7F7F7Fu; }
                }
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    if (q == kCopySlot[c]) trip_copy(ph_c, kt, c);
                if (q == 7) scales = trip_scales(kt);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) trip_copy(ph_c, kt, c);
            scales = trip_scales(kt);
            read_stage(SP{}, kt + 1, na, nb, nsa, nsb);
            mma_stage(std::integral_constant<int, PH < 0 ? -1 : PH % 2>{}, kt, ca, cb, csa, csb);
            interleave_reads();
        }
        pin_accumulators();
        if constexpr (PH >= 0) {
            if (scales) wait_copies_barrier<8 + kScaleCopies>();
            else wait_copies_barrier<8>();
        } else {
            trip_wait(kt, scales);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
    };
    using dyn = std::integral_constant<int, -1>;
    int kt = 0;
    for (; kt + 7 < nk; kt += 4) {                               // kt % 4 == 0; every pair of these trips is whole
        steady(std::integral_constant<int, 0>{}, kt, fa, fb, sa, sb, fa2, fb2, sa2, sb2);
        steady(std::integral_constant<int, 1>{}, kt + 1, fa2, fb2, sa2, sb2, fa, fb, sa, sb);
        steady(std::integral_constant<int, 2>{}, kt + 2, fa, fb, sa, sb, fa2, fb2, sa2, sb2);
        steady(std::integral_constant<int, 3>{}, kt + 3, fa2, fb2, sa2, sb2, fa, fb, sa, sb);
    }
    for (; kt + 2 < nk; kt += 2) {
        steady(dyn{}, kt, fa, fb, sa, sb, fa2, fb2, sa2, sb2);
        steady(dyn{}, kt + 1, fa2, fb2, sa2, sb2, fa, fb, sa, sb);
    }
    if (kt + 1 < nk) {
        steady(dyn{}, kt, fa, fb, sa, sb, fa2, fb2, sa2, sb2);
        ++kt;
#pragma unroll
        for (int j = 0; j < 4; ++j) { fa[j] = fa2[j]; fb[j] = fb2[j]; }
#pragma unroll
        for (int j = 0; j < SAN; ++j) { sa[j] = sa2[j]; sb[j] = sb2[j]; }
    }
    // Last stage (kt == nk - 1): its fragments are in registers and no copy is outstanding.
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (TOK) {
        // A half last stage sums only its first block: the second block's codes become 0 and its scale bytes 2^0,
        // so those k-steps add exact zeros whatever lies past the expert's range (selects, not branches, so the
        // accumulators keep one path).
        const uint32_t keep = half_last ? 0u : 0xFFFFFFFFu;
        const uint32_t one = __float_as_uint(scale_operand(127u));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int e = 4; e < 8; ++e) {
                fa[j][e] = (int)((uint32_t)fa[j][e] & keep);
                fb[j][e] = (int)((uint32_t)fb[j][e] & keep);
            }
            sa[4 + j] = half_last ? one : sa[4 + j];
            sb[4 + j] = half_last ? one : sb[4 + j];
        }
    }
    mma_stage(dyn{}, kt, fa, fb, sa, sb);
    }
    }

    // ------------------------------------------------------------------ epilogue
    // Lane l holds, for output row m (l % 32), the columns 8q + 4g + 0..3 (g = l / 32) of each 32-column block in
    // accumulator registers 4q .. 4q+3. After rounding to bf16 pairs, swapping register sets q = 2p + 1 of the lower
    // half-wave with q = 2p of the upper (v_permlane32_swap) leaves lane l with the 8 consecutive columns
    // 16p + 8g .. 16p + 8g + 7 (p = 0, 1) of its row. A second swap between 16-lane rows (v_permlane16_swap: lanes
    // l and l + 16 of each half-wave trade lane l's p = 1 set for lane l + 16's p = 0 set) leaves lane l with
    // columns 16h + 8g .. + 7 (h = (l / 16) % 2) of rows r and 16 + r (r = l % 16). Each 16-byte store then writes 64
    // contiguous bytes into each of 16 rows, rather than 32 bytes into each of 32, which halves the partial-line
    // write requests per store.
    float post = 1.0f;
    if constexpr (!MX) post = 1.0f / (g.pa[0] * g.pb[0]);
    if constexpr (TOK) {
        if (Cb == nullptr) {
            // fp32 gradient sink: c += sum, one rounding per element; lane l adds its 4 consecutive n of row m
            const bool vec_f = (g.ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(Cf) & 15) == 0;
            if (vec_f && m_end - m0 == TB && n_end - n0 == TB) {
                // whole tile, one column block i at a time: block i + 1's 16 loads are in flight while block i is
                // added and stored. Lanes l and l + 16 of each half-wave trade register sets (v_permlane16_swap) so
                // that lane l holds columns 16 h2 + 4 (2 h + g) .. + 3 (h = (l / 16) % 2) of rows r and 16 + r
                // (r = l % 16): each 16-byte access then covers 64 contiguous bytes in each of 16 rows rather than
                // 32 bytes in each of 32.
                const int hk = 2 * ((lane >> 4) & 1) + fg;
                // accumulators permuted in place first: register set 4q .. 4q + 3 holds columns 8q + 4g .. + 3 of
                // row fr; after the swap set 2 h2 + rh holds columns 16 h2 + 4 hk .. + 3 of row 16 rh + r
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const auto r = __builtin_amdgcn_permlane16_swap(
                                    __float_as_uint(acc16[i][j][8 * h2 + e]), __float_as_uint(acc16[i][j][8 * h2 + 4 + e]),
                                    false, false);
                                acc16[i][j][8 * h2 + e] = __uint_as_float(r[0]);
                                acc16[i][j][8 * h2 + 4 + e] = __uint_as_float(r[1]);
                            }
                auto sink_ptr = [&](int i, int j, int rh, int h2) {
                    return Cf + (m0 + wm * 128 + j * 32 + 16 * rh + (fr & 15)) * g.ldc + n0 + wn * 128 + i * 32 +
                           16 * h2 + 4 * hk;
                };
                float4 o[2][4][4];                             // [buffer][j][2 rh + h2]
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int x = 0; x < 4; ++x)
                        o[0][j][x] = *reinterpret_cast<const float4*>(sink_ptr(0, j, x >> 1, x & 1));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (i + 1 < 4) {
#pragma unroll
                        for (int j = 0; j < 4; ++j)
#pragma unroll
                            for (int x = 0; x < 4; ++x)
                                o[(i + 1) & 1][j][x] =
                                    *reinterpret_cast<const float4*>(sink_ptr(i + 1, j, x >> 1, x & 1));
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int rh = 0; rh < 2; ++rh)
#pragma unroll
                            for (int h2 = 0; h2 < 2; ++h2) {
                                const float4 s = o[i & 1][j][2 * rh + h2];
                                const int x = 4 * (2 * h2 + rh);
                                *reinterpret_cast<float4*>(sink_ptr(i, j, rh, h2)) =
                                    make_float4(s.x + acc16[i][j][x], s.y + acc16[i][j][x + 1],
                                                s.z + acc16[i][j][x + 2], s.w + acc16[i][j][x + 3]);
                            }
                }
                return;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t m = m0 + wm * 128 + j * 32 + fr;
                    if (m >= m_end) continue;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int64_t n = n0 + wn * 128 + i * 32 + 8 * q + 4 * fg;
                        float* dst = Cf + m * g.ldc + n;
                        const float v[4] = {acc16[i][j][4 * q], acc16[i][j][4 * q + 1], acc16[i][j][4 * q + 2],
                                            acc16[i][j][4 * q + 3]};
                        if (vec_f && n + 4 <= n_end) {
                            const float4 o = *reinterpret_cast<const float4*>(dst);
                            *reinterpret_cast<float4*>(dst) = make_float4(o.x + v[0], o.y + v[1], o.z + v[2], o.w + v[3]);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (n + e < n_end) dst[e] = dst[e] + v[e];
                        }
                    }
                }
            return;
        }
    }
    const bool vec_ok = (g.ldc & 7) == 0 && (reinterpret_cast<uintptr_t>(Cb) & 15) == 0;
    auto pack2 = [&](float x0, float x1) {
        if constexpr (!MX) { x0 = x0 * post; x1 = x1 * post; }
        return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x0) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x1) << 16);
    };
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t w[4][2];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int h = 0; h < 2; ++h) w[q][h] = pack2(acc16[i][j][4 * q + 2 * h], acc16[i][j][4 * q + 2 * h + 1]);
#pragma unroll
            for (int pq = 0; pq < 2; ++pq)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const auto r = __builtin_amdgcn_permlane32_swap(w[2 * pq][h], w[2 * pq + 1][h], false, false);
                    w[2 * pq][h] = r[0];
                    w[2 * pq + 1][h] = r[1];
                }
            // d[p]: columns 16p + 8g .. + 7 of row fr; after the swap d[rh]: columns 16h + 8g .. + 7 of row 16rh + r
            uint32_t d[2][4] = {{w[0][0], w[0][1], w[1][0], w[1][1]}, {w[2][0], w[2][1], w[3][0], w[3][1]}};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const auto r = __builtin_amdgcn_permlane16_swap(d[0][e], d[1][e], false, false);
                d[0][e] = r[0];
                d[1][e] = r[1];
            }
#pragma unroll
            for (int rh = 0; rh < 2; ++rh) {
                const int64_t m = m0 + wm * 128 + j * 32 + 16 * rh + (fr & 15);
                if (m >= m_end) continue;
                const int64_t n = n0 + wn * 128 + i * 32 + 16 * ((lane >> 4) & 1) + 8 * fg;
                uint16_t* dst = Cb + m * g.ldc + n;
                const uint32_t* v4 = d[rh];
                if (vec_ok && n + 8 <= n_end) {
                    *reinterpret_cast<uint4*>(dst) = make_uint4(v4[0], v4[1], v4[2], v4[3]);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (n + e < n_end) dst[e] = (uint16_t)(v4[e >> 1] >> (16 * (e & 1)));
                }
            }
        }
}

template <bool MX, int FA, int FB, int GM, int MF>
__global__ __launch_bounds__(GTHREADS, 1) void gemm_big_kernel(GemmArgs g) {
    gemm_big_tile<MX, FA, FB, GM, MF>(g, blockIdx.x);
}

// The exact half of the checked path's kernel pair on a persistent grid: each workgroup walks tiles blockIdx.x,
// blockIdx.x + gridDim.x, ... and computes those its gate names. When the check picks the FP8 instruction (the usual
// case) this launch is one gate read per tile on a grid of one workgroup per CU, instead of a full grid of
// workgroups that each hold 144 KiB of LDS only to read their gate.
template <bool MX, int FA, int FB>
__global__ __launch_bounds__(GTHREADS, 1) void gemm_big_gated_loop_kernel(GemmArgs g, int tiles) {
    for (int t = blockIdx.x; t < tiles; t += gridDim.x) {
        __syncthreads();                           // the previous tile's LDS reads are done before new copies land
        gemm_big_tile<MX, FA, FB, GM_NONE, 2>(g, t);
    }
}

// Path selection. The FP8 matrix instructions (v_mfma_scale_*_f8f6f4; the older *_fp8_fp8 forms measure alike) do
// not sum their K window exactly. Measured on probes of cancelling pairs and small products (matched bit for bit by
// a model in the tests): each product is truncated to 13 binades below the largest product of its group of 8
// consecutive K values, and each 32-value block's sum to 25 binades below the block's largest product; block sums,
// instructions and the fp32 accumulator then add without loss. A product 7 or more binades below its group's
// largest thus loses low-order bits (its significand has 8), up to ~2^-12 of sum |a b| per group on wide-range
// data. The bf16 instruction accumulates at fp32 quality. Measured on MX-quantized N(0,1) operands against the
// bound |err| <= 2^-7 |y| + 2^-20 sum|a b|, the FP8 path's worst ratio is 2.2-2.4 at K = 1024, 1.0-1.1 at 4096,
// 0.89 at 8192, 0.65-0.70 at 12288 and 0.49 at 36864 (0.5 is bf16 output rounding alone); on operands whose
// windows mix magnitudes far apart (rare large outliers, values spread over many binades, many zeros) it exceeds
// the bound at every K. The checked path (scaled_gemm) therefore takes the FP8 instruction only from K >= kFp8MinK
// and only when no 64-value window of either operand holds kWideCount or more codes (zeros included) more than
// kWideBinades binades below the window's largest (range_check_kernel); otherwise the exact path: operands
// dequantized to bf16 (exact) for the bf16 instruction.
constexpr int64_t kFp8MinK = 12288;

// ------------------------------------------------------------------ operand range check (checked path)
// Every 64-value window of K (the large-tile kernel's stage, one FP8 instruction's K span) of either operand is
// checked. A code's binade is its exponent field (E4M3: bits 6..3, E5M2: bits 6..2; zeros and subnormals read 0)
// plus, for MX, its 32-block's scale byte; the window is wide if it holds a nonzero code and at least kWideCount
// codes lie more than kWideBinades binades below the window's largest. A window of zeros is never wide (its products
// are exact). Any wide window sets *word (one atomic per workgroup that found one). Reads every code once:
// (M + N) K bytes, plus (M + N) K / 32 scale bytes for MX.
struct RangeOperand {
    const uint8_t* q;      // [rows][K] codes: window w is bytes 64 w .. 64 w + 63
    const uint8_t* s;      // MX: [rows][K/32] E8M0 bytes: window w's two blocks are bytes 2 w, 2 w + 1
    int64_t windows;       // rows * K / 64
    int sh;                // exponent field shift: 3 (E4M3) or 2 (E5M2)
};

// Workgroups [0, blocks_a) take A's windows, the rest B's; a workgroup takes 256 consecutive windows (windows are
// contiguous in memory, so a window's bytes and its scale bytes follow from its index alone). Four lanes share a
// window: lane quarter k holds bytes 16k .. 16k + 15 (quarters 0-1 the first 32-block, 2-3 the second), so each load
// instruction of a wave reads 1 KiB contiguous. With mag the code's magnitude (bits 6..0) and e = mag >> sh,
// "e + scale < top - kWideBinades" is "mag < (top - kWideBinades - scale) << sh", compared four bytes at a time.
template <bool MX>
__global__ __launch_bounds__(256) void range_check_kernel(RangeOperand a, RangeOperand b, int64_t blocks_a,
                                                          uint32_t* __restrict__ word) {
    constexpr int U = 4;                                   // 64 windows per workgroup per trip, 4 trips
    const bool isa = (int64_t)blockIdx.x < blocks_a;
    const RangeOperand o = isa ? a : b;
    const int64_t w0 = ((int64_t)blockIdx.x - (isa ? 0 : blocks_a)) * 256;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, quarter = lane & 3;
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t w = w0 + 64 * u + 16 * wave + (lane >> 2);
        v[u] = w < o.windows ? ldnt16(o.q + 64 * w + 16 * quarter) : make_uint4(0u, 0u, 0u, 0u);
    }
    int wide = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t w = w0 + 64 * u + 16 * wave + (lane >> 2);
        const uint32_t m0 = v[u].x & 0x7F7F7F7Fu, m1 = v[u].y & 0x7F7F7F7Fu;
        const uint32_t m2 = v[u].z & 0x7F7F7F7Fu, m3 = v[u].w & 0x7F7F7F7Fu;
        uint32_t nz = m0 | m1 | m2 | m3;
        uint32_t lo = max_u16x2_pk(max_u16x2_pk(m0 & 0x00FF00FFu, m1 & 0x00FF00FFu),
                                   max_u16x2_pk(m2 & 0x00FF00FFu, m3 & 0x00FF00FFu));
        uint32_t hi = max_u16x2_pk(max_u16x2_pk(m0 & 0xFF00FF00u, m1 & 0xFF00FF00u),
                                   max_u16x2_pk(m2 & 0xFF00FF00u, m3 & 0xFF00FF00u));
        uint32_t bm = max(max(lo & 0xFFFFu, lo >> 16), max(hi & 0xFFFFu, hi >> 16) >> 8);
        bm = max(bm, (uint32_t)__builtin_amdgcn_mov_dpp((int)bm, 0xB1, 0xF, 0xF, false));   // the block's two lanes
        int sx = 0;
        if constexpr (MX) sx = w < o.windows ? (int)o.s[2 * w + (quarter >> 1)] : 0;
        int top = (int)(bm >> o.sh) + sx;
        top = max(top, __builtin_amdgcn_mov_dpp(top, 0x4E, 0xF, 0xF, false));             // the other block
        const int th = min(min(max(top - kWideBinades - sx, 0), 32) << o.sh, 128);
        const uint32_t th4 = (uint32_t)th * 0x01010101u;
        int cnt = 16 - __builtin_popcount(((m0 | 0x80808080u) - th4) & 0x80808080u)
                     - __builtin_popcount(((m1 | 0x80808080u) - th4) & 0x80808080u)
                     - __builtin_popcount(((m2 | 0x80808080u) - th4) & 0x80808080u)
                     - __builtin_popcount(((m3 | 0x80808080u) - th4) & 0x80808080u);
        cnt += __builtin_amdgcn_mov_dpp(cnt, 0xB1, 0xF, 0xF, false);
        cnt += __builtin_amdgcn_mov_dpp(cnt, 0x4E, 0xF, 0xF, false);
        nz |= (uint32_t)__builtin_amdgcn_mov_dpp((int)nz, 0xB1, 0xF, 0xF, false);
        nz |= (uint32_t)__builtin_amdgcn_mov_dpp((int)nz, 0x4E, 0xF, 0xF, false);
        wide |= (nz != 0 && cnt >= kWideCount) ? 1 : 0;
    }
    // One atomic per workgroup that found a wide window, skipped once the flag is seen set (an agent-scope load,
    // so a set flag is seen from any XCD): on wide-range operands most workgroups find one, and same-address atomics
    // from all of them would serialize.
    if (__syncthreads_or(wide) && threadIdx.x == 0 &&
        __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u)
        atomicOr(word, 1u);
}

__global__ void gate_clear_kernel(uint32_t* __restrict__ word) { *word = 0u; }

// Writes each large tile's gate into its first output element: kGateExact if a wide window was found, else
// kGateFp8. The flag word lies in output row 1, which holds no tile's first element.
__global__ __launch_bounds__(256) void gate_broadcast_kernel(const uint32_t* __restrict__ word, uint16_t* c,
                                                             int64_t ldc, int64_t tiles_m, int64_t tiles_n) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= tiles_m * tiles_n) return;
    const uint16_t v = *word ? kGateExact : kGateFp8;
    const int64_t tm = t / tiles_n;
    c[tm * TB * ldc + (t - tm * tiles_n) * TB] = v;
}

// Large tiles when K is a whole number of 64-byte stages, the output spans at least a few tiles, and a tile's
// 256 rows stay below 2^31 bytes (the kernel's 32-bit buffer offsets). Its copies move 16-byte pieces, so operand row
// strides (and, for row groups, the distance between experts) are multiples of 16 bytes. MX operands also need K to
// be a whole number of 16-byte scale pieces (SG stages, 16 scale bytes per row; a group copies two) and 16-byte scale
// rows.
static bool use_big(const GemmArgs& a, bool mx, bool grouped) {
    constexpr int64_t kLim = int64_t(1) << 23;                  // 256 rows x stride < 2^31
    if (a.K % (mx ? KS * SG : KS) != 0 || a.M < 512 || a.N < 512 || a.K > (int64_t(1) << 22)) return false;
    if (a.lda % 16 || a.ldb % 16 || a.lda >= kLim || a.ldb >= kLim) return false;
    if (mx && (a.ldsa % 16 || a.ldsb % 16)) return false;
    if (grouped && (a.b_gstride % 16 || (mx && a.sb_gstride % 16))) return false;
    return true;
}

// Token groups on the large tiles: at least one whole tile each way, and every operand and scale byte offset of a
// tile below 2^31 (32-bit buffer offsets and record counts).
static bool use_big_tokens(const GemmArgs& a) {
    constexpr int64_t kLim = int64_t(1) << 31;
    return a.M >= TB && a.N >= TB && a.lda % 16 == 0 && a.ldb % 16 == 0 && a.M * a.lda < kLim && a.N * a.ldb < kLim;
}

template <bool MX, int FA, int FB, int GM>
static hipError_t launch_gemm_t(const GemmArgs& a, unsigned blocks_small, unsigned blocks_big, int path,
                                hipStream_t stream) {
    if constexpr (GM == GM_TOKENS) {
        // Expert K ranges differ, so every expert runs the exact path (which meets the bound at any K).
        if (blocks_big > 0 && use_big_tokens(a))
            hipLaunchKernelGGL((gemm_big_kernel<MX, FA, FB, GM, 2>), dim3(blocks_big), dim3(GTHREADS), 0, stream, a);
        else
            hipLaunchKernelGGL((gemm_kernel<MX, FA, FB, GM, 2>), dim3(blocks_small), dim3(GTHREADS), 0, stream, a);
    } else {
        const bool big = use_big(a, MX, GM == GM_ROWS);
        if (GM == GM_NONE && path == GEMM_PATH_CHECKED && big && a.K >= kFp8MinK) {
            // Checked path: clear the flag word (in output row 1), check both operands, write every tile's gate,
            // then the FP8 and exact kernels as a pair; each tile runs in the one its gate names.
            uint32_t* word = reinterpret_cast<uint32_t*>((reinterpret_cast<uintptr_t>(a.c + a.ldc + 2) + 3) & ~uintptr_t(3));
            const int64_t tiles_m = (a.M + TB - 1) / TB, tiles_n = (a.N + TB - 1) / TB;
            RangeOperand ra{a.a, a.sa, a.M * (a.K / 64), FA == FMT_E4M3 ? 3 : 2};
            RangeOperand rb{a.b, a.sb, a.N * (a.K / 64), FB == FMT_E4M3 ? 3 : 2};
            const int64_t blocks_a = (ra.windows + 255) / 256, blocks_b = (rb.windows + 255) / 256;
            hipLaunchKernelGGL(gate_clear_kernel, dim3(1), dim3(1), 0, stream, word);
            hipLaunchKernelGGL((range_check_kernel<MX>), dim3((unsigned)(blocks_a + blocks_b)), dim3(256), 0, stream,
                               ra, rb, blocks_a, word);
            hipLaunchKernelGGL(gate_broadcast_kernel, dim3((unsigned)((tiles_m * tiles_n + 255) / 256)), dim3(256), 0,
                               stream, word, a.c, a.ldc, tiles_m, tiles_n);
            GemmArgs g1 = a, g2 = a;
            g1.gate = 1;
            g2.gate = 2;
            const int tiles = (int)(tiles_m * tiles_n);
            hipLaunchKernelGGL((gemm_big_kernel<MX, FA, FB, GM, 1>), dim3(blocks_big), dim3(GTHREADS), 0, stream, g1);
            hipLaunchKernelGGL((gemm_big_gated_loop_kernel<MX, FA, FB>), dim3((unsigned)(tiles < 256 ? tiles : 256)),
                               dim3(GTHREADS), 0, stream, g2, tiles);
        } else if (GM == GM_NONE && path == GEMM_PATH_RANGED && big && a.K >= kFp8MinK) {
            // Ranged path: the FP8 and exact kernels as a pair, picked by the operands' range words on the device.
            const int64_t tiles = ((a.M + TB - 1) / TB) * ((a.N + TB - 1) / TB);
            GemmArgs g1 = a, g2 = a;
            g1.gate = 3;
            g2.gate = 4;
            hipLaunchKernelGGL((gemm_big_kernel<MX, FA, FB, GM, 1>), dim3(blocks_big), dim3(GTHREADS), 0, stream, g1);
            hipLaunchKernelGGL((gemm_big_gated_loop_kernel<MX, FA, FB>), dim3((unsigned)(tiles < 256 ? tiles : 256)),
                               dim3(GTHREADS), 0, stream, g2, (int)tiles);
        } else if (GM == GM_NONE && path == GEMM_PATH_FP8) {
            if (big) hipLaunchKernelGGL((gemm_big_kernel<MX, FA, FB, GM, 1>), dim3(blocks_big), dim3(GTHREADS), 0, stream, a);
            else hipLaunchKernelGGL((gemm_kernel<MX, FA, FB, GM, 1>), dim3(blocks_small), dim3(GTHREADS), 0, stream, a);
        } else {
            if (big) hipLaunchKernelGGL((gemm_big_kernel<MX, FA, FB, GM, 2>), dim3(blocks_big), dim3(GTHREADS), 0, stream, a);
            else hipLaunchKernelGGL((gemm_kernel<MX, FA, FB, GM, 2>), dim3(blocks_small), dim3(GTHREADS), 0, stream, a);
        }
    }
    return hipGetLastError();
}

hipError_t launch_scaled_gemm(const uint8_t* a_q, const void* a_scale, int a_fmt, const uint8_t* b_q,
                              const void* b_scale, int b_fmt, int64_t M, int64_t N, int64_t K, int mx,
                              uint16_t* c, int64_t ldc, int path, const uint32_t* a_wide, const uint32_t* b_wide,
                              hipStream_t stream) {
    GemmArgs a{};
    a.a = a_q; a.b = b_q; a.c = c; a.M = M; a.N = N; a.K = K; a.ldc = ldc; a.wa = a_wide; a.wb = b_wide;
    a.lda = K; a.ldb = K; a.ldsa = K / 32; a.ldsb = K / 32;
    if (mx) { a.sa = (const uint8_t*)a_scale; a.sb = (const uint8_t*)b_scale; }
    else { a.pa = (const float*)a_scale; a.pb = (const float*)b_scale; }
    const int64_t small = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int64_t big = ((M + TB - 1) / TB) * ((N + TB - 1) / TB);
    if (small > 0x7FFFFFFF) return hipErrorInvalidValue;
    const unsigned bs = (unsigned)small, bb = (unsigned)big;
    if (mx) return launch_gemm_t<true, 0, 0, GM_NONE>(a, bs, bb, path, stream);
    if (a_fmt == FMT_E4M3 && b_fmt == FMT_E4M3) return launch_gemm_t<false, 0, 0, GM_NONE>(a, bs, bb, path, stream);
    if (a_fmt == FMT_E5M2 && b_fmt == FMT_E4M3) return launch_gemm_t<false, 1, 0, GM_NONE>(a, bs, bb, path, stream);
    if (a_fmt == FMT_E4M3 && b_fmt == FMT_E5M2) return launch_gemm_t<false, 0, 1, GM_NONE>(a, bs, bb, path, stream);
    return launch_gemm_t<false, 1, 1, GM_NONE>(a, bs, bb, path, stream);
}

hipError_t launch_grouped_gemm(const uint8_t* a_q, const uint8_t* a_s, const int64_t* offsets, int64_t G,
                               int64_t total_rows, const uint8_t* b_q, const uint8_t* b_s, int64_t ldb,
                               int64_t b_gstride, int64_t ldsb, int64_t sb_gstride, int64_t N, int64_t K,
                               uint16_t* c, int64_t ldc, hipStream_t stream) {
    GemmArgs a{};
    a.a = a_q; a.sa = a_s; a.b = b_q; a.sb = b_s; a.c = c;
    a.M = total_rows; a.N = N; a.K = K; a.ldc = ldc; a.offsets = offsets; a.G = G;
    a.lda = K; a.ldsa = K / 32; a.ldb = ldb; a.ldsb = ldsb; a.b_gstride = b_gstride; a.sb_gstride = sb_gstride;
    // each group adds at most one partial row tile
    const int64_t small = ((total_rows + BM - 1) / BM + G) * ((N + BN - 1) / BN);
    const int64_t big = ((total_rows + TB - 1) / TB + G) * ((N + TB - 1) / TB);
    if (small > 0x7FFFFFFF) return hipErrorInvalidValue;
    return launch_gemm_t<true, 0, 0, GM_ROWS>(a, (unsigned)small, (unsigned)big, GEMM_PATH_EXACT, stream);
}

hipError_t launch_grouped_wgrad(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q, const uint8_t* b_s,
                                const int64_t* offsets, int64_t G, int64_t M, int64_t N, int64_t Kt, uint16_t* c,
                                float* cf, hipStream_t stream) {
    GemmArgs a{};
    a.a = a_q; a.sa = a_s; a.b = b_q; a.sb = b_s; a.c = c; a.cf = cf;
    a.M = M; a.N = N; a.K = Kt; a.ldc = N; a.offsets = offsets; a.G = G;
    a.lda = Kt; a.ldb = Kt; a.ldsa = Kt / 32; a.ldsb = Kt / 32; a.c_gstride = M * N;
    const int64_t blocks = G * ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int64_t big = G * ((M + TB - 1) / TB) * ((N + TB - 1) / TB);
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    return launch_gemm_t<true, 0, 0, GM_TOKENS>(a, (unsigned)blocks, (unsigned)big, GEMM_PATH_EXACT, stream);
}

}  // namespace mxq
