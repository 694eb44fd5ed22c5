/*
 * mxq oracle: a plain, slow CPU reference of FP8 / MXFP8 training numerics.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call this file. Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg use it. It shares no source, header, table or
 * helper with the GPU library.
 *
 * Built by gcc with -O2 -ffp-contract=off and without fast-math, so every float operation below is one IEEE
 * binary32 operation rounded to nearest even, and every double operation one IEEE binary64 operation.
 * Threads only split independent outputs; no sum is reordered.
 *
 * Pages cited (by title and section):
 *   [FP8-LM]   "FP8-LM: Training FP8 Large Language Models" (paper summary page): the tensor-scaling formula
 *              FP8(x) = cast(s*x) and its inverse, and the AdamW update rule with the precision-decoupled
 *              optimizer of Eq. 7-8 (FP8 first moment with a tensor scale, FP16 second moment).
 *   [LLMSB]    "3.8 Mixed Precision, bf16 & FP8 Training" (llm-stack-book): the fp32->bf16 conversion snippet,
 *              the FP8 formats, the per-tensor scale (amax clamped at 1e-12, FP8 max over amax, times a
 *              margin) in the DelayedScale sketch and in Exercise 6 (to_fp8_e4m3, fp8_linear).
 *   [OLMO11]   "OLMo-core MoE, Section 11: MXFP8 Training": Figure 49's format table, Eq. 57 (33/32 bytes per
 *              value), Eq. 58 (q = E4M3(x/s), x_hat = s*q), Figure 50 (worked block example), Eq. 60 (operand
 *              orientations), Section 11.3.5 / Table 24 (rceil and floor scale rules).
 *
 * Readings where the pages are silent (the same list is kept with the design notes):
 *   - Conversions to E4M3/E5M2 round to nearest even and saturate at the largest finite value ([OLMO11]
 *     Figure 49 caption), also for infinities. A NaN input encodes to a NaN code.
 *   - An all-zero MX block gets scale byte 0 (2^-127): the smallest power of two that keeps the block
 *     maximum at or below 448. The scale exponent is clamped to [-127, 127], E8M0's finite range.
 *   - A block holding a NaN gets scale byte 0xFF (E8M0 NaN); its qdata are encoded as if the exponent were 127.
 *   - The per-tensor product x*s is rounded once to fp32 and then converted to FP8 (no bf16 intermediate).
 *   - Adam: the fp32 m_t and v_t computed this step feed this step's update; the stored E4M3/FP16 copies only
 *     feed the next step. Bias-correction scalars are computed in double and rounded once to float.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_E4M3 = 0, ORC_E5M2 = 1 };
enum { ORC_RCEIL = 0, ORC_FLOOR = 1 };
enum { ORC_PER_TENSOR = 0, ORC_MX_BLOCK32 = 1 };

int orc_version(void) { return 1; }

/* ------------------------------------------------------------------------------------------------------
 * Formats. Values are taken from the bit fields of each format ([OLMO11] Figure 49; [FP8-LM] and [LLMSB]
 * give the same maxima and minima). Decoding is exact in double.
 * ------------------------------------------------------------------------------------------------------ */

/* E4M3 (OCP E4M3FN): sign 1, exponent 4 (bias 7), mantissa 3, no infinities, S.1111.111 is NaN. */
double orc_e4m3_value(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return s ? -NAN : NAN;
    if (e == 0) v = ldexp((double)m, -9);            /* subnormal: m * 2^-9 */
    else v = ldexp(1.0 + m / 8.0, e - 7);            /* normal: (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* E5M2: sign 1, exponent 5 (bias 15), mantissa 2, IEEE-style infinities and NaNs. */
double orc_e5m2_value(uint8_t c)
{
    int s = c >> 7, e = (c >> 2) & 31, m = c & 3;
    double v;
    if (e == 31) v = (m == 0) ? INFINITY : NAN;
    else if (e == 0) v = ldexp((double)m, -16);      /* subnormal: m * 2^-16 */
    else v = ldexp(1.0 + m / 4.0, e - 15);           /* normal: (1 + m/4) * 2^(e-15) */
    return s ? -v : v;
}

/* IEEE binary16: sign 1, exponent 5 (bias 15), mantissa 10. */
double orc_f16_value(uint16_t c)
{
    int s = c >> 15, e = (c >> 10) & 31, m = c & 1023;
    double v;
    if (e == 31) v = (m == 0) ? INFINITY : NAN;
    else if (e == 0) v = ldexp((double)m, -24);
    else v = ldexp(1.0 + m / 1024.0, e - 15);
    return s ? -v : v;
}

float orc_bf16_to_f32(uint16_t h)
{
    uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, 4);
    return f;
}

/* fp32 -> bf16, round to nearest even on the 16 dropped bits, as in [LLMSB]'s conversion snippet (add a
 * rounding bias of 0x7FFF plus the kept LSB, then drop the low half). A NaN keeps its high bits and is made quiet. */
uint16_t orc_bf16_from_f32(float f)
{
    uint32_t b;
    memcpy(&b, &f, 4);
    if (isnan(f)) return (uint16_t)((b >> 16) | 0x0040);
    uint32_t bias = 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)((b + bias) >> 16);
}

/* Sorted tables of the non-negative finite values, indexed by code. */
static double tab_e4m3[0x7F];        /* codes 0x00..0x7E, max 448 */
static double tab_e5m2[0x7C];        /* codes 0x00..0x7B, max 57344 */
static double tab_f16[0x7C01];       /* codes 0x0000..0x7BFF, plus 0x7C00 standing for 2^16 (the overflow rung) */
static pthread_once_t tab_once = PTHREAD_ONCE_INIT;

static void build_tables(void)
{
    for (int c = 0; c <= 0x7E; ++c) tab_e4m3[c] = orc_e4m3_value((uint8_t)c);
    for (int c = 0; c <= 0x7B; ++c) tab_e5m2[c] = orc_e5m2_value((uint8_t)c);
    for (int c = 0; c <= 0x7BFF; ++c) tab_f16[c] = orc_f16_value((uint16_t)c);
    tab_f16[0x7C00] = 65536.0;
}

static void tables(void) { pthread_once(&tab_once, build_tables); }

/* Nearest entry of a sorted table to a (0 <= a < tab[maxc]); on an exact midpoint the even code wins. */
static int nearest_code(const double* tab, int maxc, double a)
{
    int lo = 0, hi = maxc;                 /* invariant: tab[lo] <= a < tab[hi] */
    while (hi - lo > 1) {
        int mid = lo + (hi - lo) / 2;
        if (tab[mid] <= a) lo = mid; else hi = mid;
    }
    if (tab[lo] == a) return lo;
    double midpoint = (tab[lo] + tab[hi]) / 2.0;   /* exact: adjacent dyadic values */
    if (a < midpoint) return lo;
    if (a > midpoint) return hi;
    return (lo & 1) ? hi : lo;
}

/* Encode a real value (held exactly in double) to E4M3 or E5M2: round to nearest even, saturate at the
 * largest finite value (infinities included), sign kept (so -0 and negatives rounding to zero give 0x80). */
uint8_t orc_fp8_encode(double v, int fmt)
{
    tables();
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    const double* tab = (fmt == ORC_E4M3) ? tab_e4m3 : tab_e5m2;
    int maxc = (fmt == ORC_E4M3) ? 0x7E : 0x7B;
    if (isnan(v)) return sign | ((fmt == ORC_E4M3) ? 0x7F : 0x7E);
    double a = fabs(v);
    if (a >= tab[maxc]) return sign | (uint8_t)maxc;
    return sign | (uint8_t)nearest_code(tab, maxc, a);
}

double orc_fp8_value(uint8_t c, int fmt) { return fmt == ORC_E4M3 ? orc_e4m3_value(c) : orc_e5m2_value(c); }

/* fp32 -> IEEE binary16, round to nearest even (subnormals kept); magnitudes from 65520 up become infinity. */
uint16_t orc_f16_from_f32(float f)
{
    tables();
    uint16_t sign = signbit(f) ? 0x8000 : 0x0000;
    if (isnan(f)) return sign | 0x7E00;
    double a = fabs((double)f);
    if (a >= 65536.0) return sign | 0x7C00;
    return sign | (uint16_t)nearest_code(tab_f16, 0x7C00, a);
}

/* ------------------------------------------------------------------------------------------------------
 * MXFP8 ([OLMO11] Section 11.2.1, Eq. 58; Section 11.3.5, Table 24).
 * ------------------------------------------------------------------------------------------------------ */

/* Scale exponent e (scale s = 2^e, E8M0 byte = e + 127) for a block with maximum magnitude amax.
 *   rceil: the smallest power of two keeping amax <= 448 * s (the E4M3 maximum), found by exact comparison.
 *   floor: the block maximum rounded down to a power of two, divided by 2^8 (E4M3's largest power of two).
 * Clamped to [-127, 127]. Returns 128 for a NaN amax (the block's byte is then 0xFF). */
int orc_mx_scale_exp(double amax, int rule)
{
    if (isnan(amax)) return 128;
    if (rule == ORC_RCEIL) {
        if (!(amax <= ldexp(448.0, 127))) return 127;        /* includes +inf: no admissible e, clamp */
        int lo = -127, hi = 127;                              /* the predicate holds at hi */
        while (lo < hi) {
            int mid = lo + (hi - lo) / 2;
            if (amax <= ldexp(448.0, mid)) hi = mid; else lo = mid + 1;
        }
        return lo;
    }
    if (amax == 0.0) return -127;
    if (isinf(amax)) return 127;
    int x;
    frexp(amax, &x);                 /* amax = f * 2^x with f in [0.5, 1): floor(log2 amax) = x - 1 */
    int e = (x - 1) - 8;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* Encode one 32-value block: src[i * stride], i < 32 -> q[i], returns the scale byte. */
static uint8_t mx_block(const uint16_t* src, int64_t stride, int rule, uint8_t* q)
{
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) {
        double a = fabs((double)orc_bf16_to_f32(src[i * stride]));
        if (isnan(a) || isnan(amax)) amax = NAN;
        else if (a > amax) amax = a;
    }
    int e = orc_mx_scale_exp(amax, rule);
    int eq = (e == 128) ? 127 : e;
    for (int i = 0; i < 32; ++i)
        q[i] = orc_fp8_encode(ldexp((double)orc_bf16_to_f32(src[i * stride]), -eq), ORC_E4M3);  /* x / s, exact */
    return (e == 128) ? 0xFF : (uint8_t)(e + 127);
}

/* The same block rule for fp32 values (the weight-cache refresh quantizes the fp32 master weight directly: one
 * rounding from fp32 to E4M3; [OLMO11] Section 11.3.2, Figure 55: caches derived from the FP32 main weight). */
static uint8_t mx_block_f32(const float* src, int64_t stride, int rule, uint8_t* q)
{
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) {
        double a = fabs((double)src[i * stride]);
        if (isnan(a) || isnan(amax)) amax = NAN;
        else if (a > amax) amax = a;
    }
    int e = orc_mx_scale_exp(amax, rule);
    int eq = (e == 128) ? 127 : e;
    for (int i = 0; i < 32; ++i)
        q[i] = orc_fp8_encode(ldexp((double)src[i * stride], -eq), ORC_E4M3);
    return (e == 128) ? 0xFF : (uint8_t)(e + 127);
}

typedef struct {
    const uint16_t* x; int64_t rows, cols; int rule;
    uint8_t *q_row, *s_row, *q_col, *s_col;
    int nthreads, tid;
    const float* xf;            /* fp32 input instead of x when not NULL */
} mxq_job;

static void* mx_worker(void* p)
{
    mxq_job* j = (mxq_job*)p;
    if (j->q_row) {
        for (int64_t r = j->tid; r < j->rows; r += j->nthreads)
            for (int64_t b = 0; b < j->cols / 32; ++b)
                j->s_row[r * (j->cols / 32) + b] = j->xf
                    ? mx_block_f32(j->xf + r * j->cols + 32 * b, 1, j->rule, j->q_row + r * j->cols + 32 * b)
                    : mx_block(j->x + r * j->cols + 32 * b, 1, j->rule, j->q_row + r * j->cols + 32 * b);
    }
    if (j->q_col) {
        for (int64_t c = j->tid; c < j->cols; c += j->nthreads)
            for (int64_t b = 0; b < j->rows / 32; ++b)
                j->s_col[c * (j->rows / 32) + b] = j->xf
                    ? mx_block_f32(j->xf + (32 * b) * j->cols + c, j->cols, j->rule, j->q_col + c * j->rows + 32 * b)
                    : mx_block(j->x + (32 * b) * j->cols + c, j->cols, j->rule, j->q_col + c * j->rows + 32 * b);
    }
    return NULL;
}

static int clamp_threads(int n) { return n < 1 ? 1 : (n > 256 ? 256 : n); }

/* Row orientation: blocks of 32 along each row -> q_row[rows][cols], s_row[rows][cols/32].
 * Column orientation: blocks of 32 down each column, stored transposed -> q_col[cols][rows], s_col[cols][rows/32].
 * Either output pair may be NULL. */
void orc_mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, int rule, uint8_t* q_row, uint8_t* s_row,
                     uint8_t* q_col, uint8_t* s_col, int nthreads)
{
    tables();
    nthreads = clamp_threads(nthreads);
    pthread_t th[256];
    mxq_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (mxq_job){x, rows, cols, rule, q_row, s_row, q_col, s_col, nthreads, t, NULL};
        pthread_create(&th[t], NULL, mx_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* MXFP8 quantize of an fp32 matrix (same layouts and rules as orc_mx_quantize). */
void orc_mx_quantize_f32(const float* x, int64_t rows, int64_t cols, int rule, uint8_t* q_row, uint8_t* s_row,
                         uint8_t* q_col, uint8_t* s_col, int nthreads)
{
    tables();
    nthreads = clamp_threads(nthreads);
    pthread_t th[256];
    mxq_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (mxq_job){NULL, rows, cols, rule, q_row, s_row, q_col, s_col, nthreads, t, x};
        pthread_create(&th[t], NULL, mx_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------------------------------------
 * Fused SwiGLU + MX row quantize ([OLMO11] Section 11.4.1: the hidden representation of the routed experts is
 * produced by a fused SwiGLU-plus-quantization step, straight into the down projection's MXFP8 operand).
 * Reading: the up/gate GEMM output C[rows][2F] holds the gate in columns [0, F) and up in [F, 2F);
 * h = silu(g) * u with silu(g) = g / (1 + exp(-g)), every operation one fp32 rounding, and h is quantized from fp32
 * (one rounding to E4M3) in 32-value blocks along each row.
 * exp is evaluated by a fixed fp32 sequence both implementations follow: Cody-Waite reduction x = k ln2 + r
 * (k = rint(x log2 e), ln2 split into a high part with few significant bits and a low part), the degree-6 Taylor
 * polynomial of e^r in Horner form, then the exact scaling by 2^k. Its error against the true exponential is a few
 * ulp; it is fixed so that both sides produce the same fp32 value.
 * ------------------------------------------------------------------------------------------------------ */
float orc_exp_f32(float x)
{
    if (x != x) return x;
    if (x > 88.75f) return INFINITY;
    if (x < -104.0f) return 0.0f;
    const float log2e = 1.44269504f;
    const float ln2_hi = 0.693145751953125f;          /* 0x3F317200: ln 2 to 16 significant bits */
    const float ln2_lo = 1.42860677e-06f;             /* ln 2 - ln2_hi */
    float t = x * log2e;
    float k = rintf(t);
    float a = k * ln2_hi;                             /* exact: k has at most 8 significant bits */
    float r = x - a;
    float b = k * ln2_lo;
    r = r - b;
    float p = 1.0f / 720.0f;
    p = p * r; p = p + 1.0f / 120.0f;
    p = p * r; p = p + 1.0f / 24.0f;
    p = p * r; p = p + 1.0f / 6.0f;
    p = p * r; p = p + 0.5f;
    p = p * r; p = p + 1.0f;
    p = p * r; p = p + 1.0f;
    return ldexpf(p, (int)k);
}

float orc_swiglu_f32(float g, float u)
{
    float e = orc_exp_f32(-g);
    float d = 1.0f + e;
    float silu = g / d;
    return silu * u;
}

void orc_swiglu_mx_quantize(const uint16_t* c, int64_t rows, int64_t F, int rule, uint8_t* q, uint8_t* s,
                            float* h_out)
{
    tables();
    float* h = (float*)malloc(sizeof(float) * (size_t)F);
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* row = c + r * 2 * F;
        for (int64_t j = 0; j < F; ++j) {
            h[j] = orc_swiglu_f32(orc_bf16_to_f32(row[j]), orc_bf16_to_f32(row[F + j]));
            if (h_out) h_out[r * F + j] = h[j];
        }
        for (int64_t b = 0; b < F / 32; ++b)
            s[r * (F / 32) + b] = mx_block_f32(h + 32 * b, 1, rule, q + r * F + 32 * b);
    }
    free(h);
}

/* ------------------------------------------------------------------------------------------------------
 * Routed-expert backward ([OLMO11] Section 11.4.1, backward of the routed experts; Section 11.4.4, Table 25).
 *
 * Combine backward: the route weight of each routed row multiplies that row's output gradient, and the product
 * is quantized straight to MXFP8 (the fused route-weighting + gradient Q of Table 25). Reading: the product is one
 * fp32 rounding of p * float(dy); both orientations follow the fp32 MX block rule (mx_block_f32), the row
 * orientation for the down projection's dgrad, the column orientation (blocks of 32 routed rows) for its Wgrad.
 * ------------------------------------------------------------------------------------------------------ */
void orc_route_weighted_mx_quantize(const uint16_t* dy, const float* p, int64_t rows, int64_t cols, int rule,
                                    uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, float* x_out,
                                    int nthreads)
{
    tables();
    float* x = x_out ? x_out : (float*)malloc(sizeof(float) * (size_t)(rows * cols));
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            float v = orc_bf16_to_f32(dy[r * cols + c]);
            x[r * cols + c] = p[r] * v;
        }
    orc_mx_quantize_f32(x, rows, cols, rule, q_row, s_row, q_col, s_col, nthreads);
    if (!x_out) free(x);
}

/* SwiGLU backward. Forward h = silu(g) u with silu(g) = g sigma(g), sigma(g) = 1 / (1 + e^-g). Its partial
 * derivatives: dh/du = silu(g); dh/dg = u silu'(g) with silu'(g) = sigma(g) (1 + g (1 - sigma(g))).
 * Given the incoming gradient dh: d_gate = (dh u) silu'(g), d_up = dh silu(g).
 * Reading (the pages fix only that SwiGLU feeds the down projection and that backward follows the forward's data
 * dependencies in reverse): every step is one fp32 operation in the order written below, with the forward's fixed
 * exponential and the forward's silu = g / (1 + e^-g), so the d_up factor equals the forward's silu bit for bit. */
void orc_swiglu_bwd_f32(float g, float u, float dh, float* d_gate, float* d_up)
{
    float e = orc_exp_f32(-g);
    float d = 1.0f + e;
    float silu = g / d;
    float sig = 1.0f / d;
    float one_m = 1.0f - sig;
    float t = g * one_m;
    t = 1.0f + t;
    float ds = sig * t;
    float du = dh * u;
    *d_gate = du * ds;
    *d_up = dh * silu;
}

/* The fused backward step between the down projection's dgrad and the up/gate projection's dgrad and Wgrad:
 * c[rows][2F] is the forward's up/gate output (gate in columns [0, F), up in [F, 2F)), dh[rows][F] the gradient
 * of h. dc[rows][2F] = (d_gate | d_up) is quantized in both orientations with the fp32 MX block rule: row blocks
 * along 2F feed the up/gate dgrad (K = 2F), column blocks of 32 routed rows feed its Wgrad (K = routed rows). */
void orc_swiglu_bwd_mx_quantize(const uint16_t* c, const uint16_t* dh, int64_t rows, int64_t F, int rule,
                                uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, float* dc_out,
                                int nthreads)
{
    tables();
    float* dc = dc_out ? dc_out : (float*)malloc(sizeof(float) * (size_t)(rows * 2 * F));
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < F; ++j) {
            float g = orc_bf16_to_f32(c[r * 2 * F + j]);
            float u = orc_bf16_to_f32(c[r * 2 * F + F + j]);
            float h = orc_bf16_to_f32(dh[r * F + j]);
            orc_swiglu_bwd_f32(g, u, h, &dc[r * 2 * F + j], &dc[r * 2 * F + F + j]);
        }
    orc_mx_quantize_f32(dc, rows, 2 * F, rule, q_row, s_row, q_col, s_col, nthreads);
    if (!dc_out) free(dc);
}

/* ------------------------------------------------------------------------------------------------------
 * FP8 gradient all-reduce, the parts one GPU runs ([FP8-LM] Section 3.4, automatic scaling (Eq. 3) and the shared
 * scaling factor of Eq. 4-6).
 * Auto-scaled cast: g' = mu * g (one fp32 rounding), q = FP8(g') with saturation; the tensor's scale is mu
 * (g ~ val(q) / mu). The overflow ratio is the fraction of codes at the format's maximum magnitude; if it exceeds
 * 0.001 % (ratio > 1e-5, evaluated in double) mu is halved for the next step, otherwise multiplied by 2^(1/1000)
 * (that factor rounded once to fp32; the product rounded in fp32).
 * Shared-scale requantize: s_g = the minimum of the gathered per-rank scales; each value is decoded, divided by its
 * own scale s_i, multiplied by s_g (each an fp32 rounding) and re-encoded; the sum of N such tensors carries the
 * scale N * s_g.
 * ------------------------------------------------------------------------------------------------------ */
void orc_autoscale_cast(const uint16_t* g, int64_t n, int fmt, float* mu, uint8_t* q, uint64_t* overflow,
                        float* scale_out)
{
    tables();
    const float m = *mu;
    const uint8_t maxcode = (fmt == ORC_E4M3) ? 0x7E : 0x7B;
    uint64_t count = 0;
    for (int64_t i = 0; i < n; ++i) {
        float p = m * orc_bf16_to_f32(g[i]);
        uint8_t c = orc_fp8_encode((double)p, fmt);
        q[i] = c;
        if ((c & 0x7F) == maxcode) ++count;
    }
    const float up = (float)exp2(1.0 / 1000.0);
    double ratio = (n > 0) ? (double)count / (double)n : 0.0;
    *overflow = count;
    if (scale_out) *scale_out = m;
    *mu = (ratio > 1e-5) ? m * 0.5f : m * up;
}

float orc_min_scale(const float* scales, int64_t N)
{
    float m = scales[0];
    for (int64_t i = 1; i < N; ++i) {
        if (isnan(scales[i]) || isnan(m)) m = NAN;
        else if (scales[i] < m) m = scales[i];
    }
    return m;
}

void orc_requantize_shared(const uint8_t* q_in, int64_t n, int fmt_in, float s_in, float s_g, int fmt_out,
                           uint8_t* q_out)
{
    tables();
    for (int64_t i = 0; i < n; ++i) {
        float v = (float)orc_fp8_value(q_in[i], fmt_in);        /* every FP8 value is exact in fp32 */
        float t = v / s_in;
        float u = s_g * t;
        q_out[i] = orc_fp8_encode((double)u, fmt_out);
    }
}

/* ------------------------------------------------------------------------------------------------------
 * Per-tensor current scaling ([FP8-LM] tensor scaling; [LLMSB] per-tensor scaling and Exercise 6).
 *   amax = max |x|;  s = (FMAX / max(amax, 1e-12)) * margin  (fp32);  q = FP8(fp32(x * s));  x ~ q / s.
 * With scale_in given (delayed scaling) s = *scale_in and amax is still reported.
 * ------------------------------------------------------------------------------------------------------ */
typedef struct {
    const uint16_t* x; int64_t rows, cols; int fmt; float s;
    uint8_t *q, *q_t; float amax; int pass; int nthreads, tid;
} pt_job;

static void* pt_worker(void* p)
{
    pt_job* j = (pt_job*)p;
    int64_t lo = j->rows * j->tid / j->nthreads, hi = j->rows * (j->tid + 1) / j->nthreads;
    if (j->pass == 1) {
        float amax = 0.0f;
        for (int64_t i = lo * j->cols; i < hi * j->cols; ++i) {
            float a = fabsf(orc_bf16_to_f32(j->x[i]));
            if (isnan(a) || isnan(amax)) amax = NAN;
            else if (a > amax) amax = a;
        }
        j->amax = amax;
        return NULL;
    }
    for (int64_t r = lo; r < hi; ++r)
        for (int64_t c = 0; c < j->cols; ++c) {
            float p = orc_bf16_to_f32(j->x[r * j->cols + c]) * j->s;     /* one fp32 rounding */
            uint8_t code = orc_fp8_encode((double)p, j->fmt);
            if (j->q) j->q[r * j->cols + c] = code;
            if (j->q_t) j->q_t[c * j->rows + r] = code;
        }
    return NULL;
}

void orc_pertensor_quantize(const uint16_t* x, int64_t rows, int64_t cols, int fmt, float margin,
                            const float* scale_in, float* amax_out, float* scale_out, uint8_t* q, uint8_t* q_t,
                            int nthreads)
{
    tables();
    nthreads = clamp_threads(nthreads);
    pthread_t th[256];
    pt_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (pt_job){x, rows, cols, fmt, 0.0f, q, q_t, 0.0f, 1, nthreads, t};
        pthread_create(&th[t], NULL, pt_worker, &jobs[t]);
    }
    float amax = 0.0f;
    for (int t = 0; t < nthreads; ++t) {
        pthread_join(th[t], NULL);
        float a = jobs[t].amax;
        if (isnan(a) || isnan(amax)) amax = NAN;
        else if (a > amax) amax = a;
    }
    float s;
    if (scale_in) {
        s = *scale_in;
    } else {
        float fmax = (fmt == ORC_E4M3) ? 448.0f : 57344.0f;
        float a = (amax < 1e-12f) ? 1e-12f : amax;            /* clamp_min keeps a NaN */
        s = fmax / a;
        s = s * margin;
    }
    if (amax_out) *amax_out = amax;
    if (scale_out) *scale_out = s;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].pass = 2;
        jobs[t].s = s;
        pthread_create(&th[t], NULL, pt_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------------------------------------
 * Delayed per-tensor scaling ([LLMSB] "Per-tensor scaling and the delayed-scaling recipe", the DelayedScale
 * sketch; [FP8-LM] Section 3.4, delayed scaling): a rolling history of the amax of past calls; this call's scale
 * is FMAX over the history's maximum (clamped below at 1e-12) times the margin; the tensor is cast with it; then
 * this call's own amax is written at the history's current position, which advances cyclically.
 * ------------------------------------------------------------------------------------------------------ */

/* max over the history (a NaN entry makes it NaN), clamped at 1e-12, FMAX / that, times margin; all fp32. */
float orc_delayed_scale(const float* history, int64_t H, int fmt, float margin)
{
    float m = 0.0f;
    for (int64_t i = 0; i < H; ++i) {
        float h = history[i];
        if (isnan(h) || isnan(m)) m = NAN;
        else if (h > m) m = h;
    }
    float fmax = (fmt == ORC_E4M3) ? 448.0f : 57344.0f;
    float a = (m < 1e-12f) ? 1e-12f : m;
    float s = fmax / a;
    return s * margin;
}

void orc_history_push(float* history, int64_t H, int32_t* pos, float amax)
{
    history[*pos] = amax;
    *pos = (int32_t)((*pos + 1) % H);
}

void orc_pertensor_quantize_delayed(const uint16_t* x, int64_t rows, int64_t cols, int fmt, float margin,
                                    float* history, int64_t H, int32_t* pos, float* amax_out, float* scale_out,
                                    uint8_t* q, uint8_t* q_t, int nthreads)
{
    float s = orc_delayed_scale(history, H, fmt, margin);
    float amax = 0.0f;
    orc_pertensor_quantize(x, rows, cols, fmt, margin, &s, &amax, scale_out, q, q_t, nthreads);
    if (amax_out) *amax_out = amax;
    orc_history_push(history, H, pos, amax);
}

/* ------------------------------------------------------------------------------------------------------
 * GEMM reference: C = A * B^T with A given as [M][K] qdata and B as [N][K] qdata (both K-contiguous).
 *   MX_BLOCK32: a_hat[i][k] = val(qa[i][k]) * 2^(sa[i][k/32] - 127), likewise b_hat; y = sum_k a_hat * b_hat.
 *   PER_TENSOR: y = (sum_k val(qa) * val(qb)) / (s_a * s_b)     ([LLMSB] Exercise 6: de-scale by 1/(s_x s_w)).
 * Every sum runs over k in ascending order in double. S = sum_k |a_hat * b_hat| (same scaling) is returned
 * beside y for the error bound. Computes the sub-block rows[0..nr) x cols[0..nc) into y[nr][nc], S[nr][nc].
 * ------------------------------------------------------------------------------------------------------ */
typedef struct {
    const double* arows;      /* [nr][K] dequantized A rows */
    const uint8_t *bq, *bs; int b_fmt; int scaling;
    int64_t K, nr, nc; const int64_t* cols; double post;
    double *y, *S;
    int nthreads, tid;
} gemm_job;

static void dequant_row(const uint8_t* q, const uint8_t* s, int fmt, int scaling, int64_t K, double* out)
{
    for (int64_t k = 0; k < K; ++k) {
        double v = orc_fp8_value(q[k], fmt);
        if (scaling == ORC_MX_BLOCK32) {
            uint8_t byte = s[k / 32];
            v = (byte == 0xFF) ? NAN : ldexp(v, (int)byte - 127);
        }
        out[k] = v;
    }
}

static void* gemm_worker(void* p)
{
    gemm_job* j = (gemm_job*)p;
    double* brow = (double*)malloc(sizeof(double) * (size_t)j->K);
    for (int64_t jj = j->tid; jj < j->nc; jj += j->nthreads) {
        int64_t col = j->cols[jj];
        dequant_row(j->bq + col * j->K, j->bs ? j->bs + col * (j->K / 32) : NULL, j->b_fmt, j->scaling, j->K, brow);
        for (int64_t i = 0; i < j->nr; ++i) {
            const double* a = j->arows + i * j->K;
            double acc = 0.0, sabs = 0.0;
            for (int64_t k = 0; k < j->K; ++k) {
                double prod = a[k] * brow[k];
                acc += prod;
                sabs += fabs(prod);
            }
            j->y[i * j->nc + jj] = acc * j->post;
            j->S[i * j->nc + jj] = sabs * j->post;
        }
    }
    free(brow);
    return NULL;
}

static void gemm_core(const double* arows, int64_t nr, const uint8_t* bq, const uint8_t* bs, int b_fmt, int scaling,
                      int64_t K, const int64_t* cols, int64_t nc, double post, double* y, double* S, int nthreads)
{
    nthreads = clamp_threads(nthreads);
    pthread_t th[256];
    gemm_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (gemm_job){arows, bq, bs, b_fmt, scaling, K, nr, nc, cols, post, y, S, nthreads, t};
        pthread_create(&th[t], NULL, gemm_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

void orc_gemm_ref(const uint8_t* aq, const void* a_scale, int a_fmt, const uint8_t* bq, const void* b_scale, int b_fmt,
                  int64_t M, int64_t N, int64_t K, int scaling, const int64_t* rows, int64_t nr, const int64_t* cols,
                  int64_t nc, double* y, double* S, int nthreads)
{
    tables();
    (void)M; (void)N;
    double* arows = (double*)malloc(sizeof(double) * (size_t)(nr * K));
    for (int64_t i = 0; i < nr; ++i)
        dequant_row(aq + rows[i] * K, scaling == ORC_MX_BLOCK32 ? (const uint8_t*)a_scale + rows[i] * (K / 32) : NULL,
                    a_fmt, scaling, K, arows + i * K);
    double post = 1.0;
    if (scaling == ORC_PER_TENSOR) post = 1.0 / ((double)*(const float*)a_scale * (double)*(const float*)b_scale);
    gemm_core(arows, nr, bq, scaling == ORC_MX_BLOCK32 ? (const uint8_t*)b_scale : NULL, b_fmt, scaling, K, cols, nc,
              post, y, S, nthreads);
    free(arows);
}

/* Grouped MX GEMM reference: row i of C, in group g (offsets[g] <= i < offsets[g+1]), is row i of A times B[g]^T.
 * B is [G][N][K] qdata with [G][N][K/32] scales. Rows are processed one at a time against their own group. */
void orc_grouped_gemm_ref(const uint8_t* aq, const uint8_t* as, const int64_t* offsets, int64_t G, const uint8_t* bq,
                          const uint8_t* bs, int64_t N, int64_t K, const int64_t* rows, int64_t nr, const int64_t* cols,
                          int64_t nc, double* y, double* S, int nthreads)
{
    tables();
    double* arow = (double*)malloc(sizeof(double) * (size_t)K);
    for (int64_t r = 0; r < nr; ++r) {
        int64_t i = rows[r];
        int64_t g = 0;
        while (g < G && !(offsets[g] <= i && i < offsets[g + 1])) ++g;
        if (g == G) {                      /* not inside any group: no output defined */
            for (int64_t c = 0; c < nc; ++c) { y[r * nc + c] = NAN; S[r * nc + c] = NAN; }
            continue;
        }
        dequant_row(aq + i * K, as + i * (K / 32), ORC_E4M3, ORC_MX_BLOCK32, K, arow);
        gemm_core(arow, 1, bq + g * N * K, bs + g * N * (K / 32), ORC_E4M3, ORC_MX_BLOCK32, K, cols, nc, 1.0,
                  y + r * nc, S + r * nc, nthreads);
    }
    free(arow);
}

/* Routed Wgrad as a contraction over tokens ([OLMO11] Section 11.4.1 and Section 11.4.4: the reduction dimension of
 * the routed Wgrad is the expert's token rows). A[M][Kt] and B[N][Kt] are column-orientation MX operands (blocks of 32
 * along the token dimension, scales [M][Kt/32] and [N][Kt/32]); expert g owns tokens [offsets[g], offsets[g+1]), each
 * offset a multiple of 32. y_g[m][n] = sum over those k, ascending, of a_hat[m][k] b_hat[n][k] in double, with
 * a_hat = val(q) 2^(byte - 127); S_g = the same sum of |products|. Computes the requested groups, rows and columns
 * into y[ng][nr][nc] and S[ng][nr][nc]. An empty group gives 0. */
void orc_grouped_wgrad_ref(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs,
                           const int64_t* offsets, int64_t Kt, const int64_t* groups, int64_t ng, const int64_t* rows,
                           int64_t nr, const int64_t* cols, int64_t nc, double* y, double* S)
{
    tables();
    for (int64_t gi = 0; gi < ng; ++gi) {
        int64_t g = groups[gi];
        int64_t k0 = offsets[g], Kg = offsets[g + 1] - offsets[g];
        size_t len = (size_t)(Kg > 0 ? Kg : 1);
        double* a = (double*)malloc(sizeof(double) * len * (size_t)nr);
        double* b = (double*)malloc(sizeof(double) * len * (size_t)nc);
        for (int64_t i = 0; i < nr; ++i)
            dequant_row(aq + rows[i] * Kt + k0, as + rows[i] * (Kt / 32) + k0 / 32, ORC_E4M3, ORC_MX_BLOCK32, Kg,
                        a + (size_t)i * len);
        for (int64_t j = 0; j < nc; ++j)
            dequant_row(bq + cols[j] * Kt + k0, bs + cols[j] * (Kt / 32) + k0 / 32, ORC_E4M3, ORC_MX_BLOCK32, Kg,
                        b + (size_t)j * len);
        for (int64_t i = 0; i < nr; ++i)
            for (int64_t j = 0; j < nc; ++j) {
                const double* ai = a + (size_t)i * len;
                const double* bj = b + (size_t)j * len;
                double acc = 0.0, sabs = 0.0;
                for (int64_t k = 0; k < Kg; ++k) {
                    double prod = ai[k] * bj[k];
                    acc += prod;
                    sabs += fabs(prod);
                }
                y[(gi * nr + i) * nc + j] = acc;
                S[(gi * nr + i) * nc + j] = sabs;
            }
        free(a);
        free(b);
    }
}

/* ------------------------------------------------------------------------------------------------------
 * Precision-decoupled FP8 AdamW step ([FP8-LM] AdamW update rule and Eq. 7-8): master weight fp32, first moment
 * m in E4M3 with one per-tensor scale s_m (m_q ~ m * s_m), second moment v in FP16, bf16 gradient, and a bf16
 * copy of the updated weight. The new m scale uses current scaling: s_m = 448 / max(amax(m_t), 1e-12).
 *   m_t = b1 m_{t-1} + (1-b1) g;   v_t = b2 v_{t-1} + (1-b2) g^2;
 *   theta_t = theta_{t-1} - lr * ( (m_t c1) / (sqrt(v_t c2) + eps) + wd theta_{t-1} ),  c1 = 1/(1-b1^t), c2 = 1/(1-b2^t).
 * ------------------------------------------------------------------------------------------------------ */
typedef struct { float lr, beta1, beta2, eps, weight_decay; int64_t step; } orc_adam_hp;

typedef struct {
    float b1, ob1, b2, ob2, c1, c2, lr, eps, wd, inv_s_old, s_new;
} adam_consts;

static adam_consts adam_setup(const orc_adam_hp* hp, float s_old)
{
    adam_consts k;
    double p1 = 1.0, p2 = 1.0;
    for (int64_t t = 0; t < hp->step; ++t) { p1 *= (double)hp->beta1; p2 *= (double)hp->beta2; }
    k.b1 = hp->beta1;
    k.ob1 = (float)(1.0 - (double)hp->beta1);
    k.b2 = hp->beta2;
    k.ob2 = (float)(1.0 - (double)hp->beta2);
    k.c1 = (float)(1.0 / (1.0 - p1));
    k.c2 = (float)(1.0 / (1.0 - p2));
    k.lr = hp->lr; k.eps = hp->eps; k.wd = hp->weight_decay;
    k.inv_s_old = 1.0f / s_old;
    k.s_new = 0.0f;
    return k;
}

static inline void adam_moments(const adam_consts* k, uint16_t g16, uint8_t mq, uint16_t v16, float* m, float* v)
{
    float g = orc_bf16_to_f32(g16);
    float m_old = (float)orc_e4m3_value(mq) * k->inv_s_old;
    float v_old = (float)orc_f16_value(v16);
    float t1 = k->b1 * m_old;
    float t2 = k->ob1 * g;
    *m = t1 + t2;
    float gg = g * g;
    float t3 = k->b2 * v_old;
    float t4 = k->ob2 * gg;
    *v = t3 + t4;
}

typedef struct {
    float* master; const uint16_t* g; uint8_t* m_q; uint16_t* v16; uint16_t* w; int64_t n;
    const adam_consts* k; float amax; int pass; int nthreads, tid;
} adam_job;

static void* adam_worker(void* p)
{
    adam_job* j = (adam_job*)p;
    const adam_consts* k = j->k;
    int64_t lo = j->n * j->tid / j->nthreads, hi = j->n * (j->tid + 1) / j->nthreads;
    if (j->pass == 1) {
        float amax = 0.0f;
        for (int64_t i = lo; i < hi; ++i) {
            float m, v;
            adam_moments(k, j->g[i], j->m_q[i], j->v16[i], &m, &v);
            float a = fabsf(m);
            if (isnan(a) || isnan(amax)) amax = NAN;
            else if (a > amax) amax = a;
        }
        j->amax = amax;
        return NULL;
    }
    for (int64_t i = lo; i < hi; ++i) {
        float m, v;
        adam_moments(k, j->g[i], j->m_q[i], j->v16[i], &m, &v);
        float theta = j->master[i];
        float mh = m * k->c1;
        float vh = v * k->c2;
        float den = sqrtf(vh) + k->eps;
        float u = mh / den;
        if (k->wd != 0.0f) {
            float dec = k->wd * theta;
            u = u + dec;
        }
        float step = k->lr * u;
        float theta_new = theta - step;
        float ms = m * k->s_new;
        j->master[i] = theta_new;
        j->m_q[i] = orc_fp8_encode((double)ms, ORC_E4M3);
        j->v16[i] = orc_f16_from_f32(v);
        if (j->w) j->w[i] = orc_bf16_from_f32(theta_new);
    }
    return NULL;
}

/* Returns the amax of m_t (pass 1). Updates master, m_q, m_scale[0], v16 in place and writes w_bf16 (may be NULL). */
float orc_adam_step(float* master, const uint16_t* grad_bf16, uint8_t* m_q, float* m_scale, uint16_t* v16,
                    uint16_t* w_bf16, int64_t n, const orc_adam_hp* hp, int nthreads)
{
    tables();
    nthreads = clamp_threads(nthreads);
    adam_consts k = adam_setup(hp, m_scale[0]);
    pthread_t th[256];
    adam_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (adam_job){master, grad_bf16, m_q, v16, w_bf16, n, &k, 0.0f, 1, nthreads, t};
        pthread_create(&th[t], NULL, adam_worker, &jobs[t]);
    }
    float amax = 0.0f;
    for (int t = 0; t < nthreads; ++t) {
        pthread_join(th[t], NULL);
        float a = jobs[t].amax;
        if (isnan(a) || isnan(amax)) amax = NAN;
        else if (a > amax) amax = a;
    }
    float a = (amax < 1e-12f) ? 1e-12f : amax;
    k.s_new = 448.0f / a;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].pass = 2;
        pthread_create(&th[t], NULL, adam_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    m_scale[0] = k.s_new;
    return amax;
}

/* Adam with a delayed first-moment scale: the scale that encodes this step's m_t is E4M3's 448 over the maximum of
 * the amax history of m from earlier steps (clamped at 1e-12); the amax of this step's m_t is then pushed into the
 * history. Every other operation is the one of orc_adam_step. Returns the amax of m_t. */
float orc_adam_step_delayed(float* master, const uint16_t* grad_bf16, uint8_t* m_q, float* m_scale, uint16_t* v16,
                            uint16_t* w_bf16, int64_t n, const orc_adam_hp* hp, float* history, int64_t H,
                            int32_t* pos, int nthreads)
{
    tables();
    nthreads = clamp_threads(nthreads);
    adam_consts k = adam_setup(hp, m_scale[0]);
    k.s_new = orc_delayed_scale(history, H, ORC_E4M3, 1.0f);
    pthread_t th[256];
    adam_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (adam_job){master, grad_bf16, m_q, v16, w_bf16, n, &k, 0.0f, 1, nthreads, t};
        pthread_create(&th[t], NULL, adam_worker, &jobs[t]);          /* amax of m_t, from the old state */
    }
    float amax = 0.0f;
    for (int t = 0; t < nthreads; ++t) {
        pthread_join(th[t], NULL);
        float a = jobs[t].amax;
        if (isnan(a) || isnan(amax)) amax = NAN;
        else if (a > amax) amax = a;
    }
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].pass = 2;
        pthread_create(&th[t], NULL, adam_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    m_scale[0] = k.s_new;
    orc_history_push(history, H, pos, amax);
    return amax;
}

/* The amax pass alone, over a sub-range [lo, hi) (for sampled checks at full size). */
float orc_adam_amax(const uint16_t* grad_bf16, const uint8_t* m_q, const uint16_t* v16, float m_scale_old, int64_t n,
                    const orc_adam_hp* hp, int nthreads)
{
    tables();
    nthreads = clamp_threads(nthreads);
    adam_consts k = adam_setup(hp, m_scale_old);
    pthread_t th[256];
    adam_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (adam_job){NULL, grad_bf16, (uint8_t*)m_q, (uint16_t*)v16, NULL, n, &k, 0.0f, 1, nthreads, t};
        pthread_create(&th[t], NULL, adam_worker, &jobs[t]);
    }
    float amax = 0.0f;
    for (int t = 0; t < nthreads; ++t) {
        pthread_join(th[t], NULL);
        float a = jobs[t].amax;
        if (isnan(a) || isnan(amax)) amax = NAN;
        else if (a > amax) amax = a;
    }
    return amax;
}

/* Pass 2 for a list of element indices, given the new scale (sampled checks at full size). Outputs are written
 * densely: out_master[i], out_mq[i], out_v16[i], out_w[i] for the i-th listed index. */
void orc_adam_elements(const float* master, const uint16_t* grad_bf16, const uint8_t* m_q, const uint16_t* v16,
                       float m_scale_old, float s_new, const int64_t* idx, int64_t count, const orc_adam_hp* hp,
                       float* out_master, uint8_t* out_mq, uint16_t* out_v16, uint16_t* out_w)
{
    tables();
    adam_consts k = adam_setup(hp, m_scale_old);
    k.s_new = s_new;
    for (int64_t r = 0; r < count; ++r) {
        int64_t i = idx[r];
        float th = master[i];
        uint8_t mq = m_q[i];
        uint16_t vv = v16[i];
        adam_job j = {&th, &grad_bf16[i], &mq, &vv, &out_w[r], 1, &k, 0.0f, 2, 1, 0};
        adam_worker(&j);
        out_master[r] = th;
        out_mq[r] = mq;
        out_v16[r] = vv;
    }
}

/* ------------------------------------------------------------------------------------------------------
 * Array forms of the codecs, for exhaustive checks from the test suite.
 * ------------------------------------------------------------------------------------------------------ */
void orc_fp8_encode_array(const double* v, int64_t n, int fmt, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_encode(v[i], fmt);
}

void orc_fp8_value_array(const uint8_t* c, int64_t n, int fmt, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_value(c[i], fmt);
}

void orc_bf16_from_f32_array(const float* f, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_f32(f[i]);
}

void orc_f16_from_f32_array(const float* f, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_from_f32(f[i]);
}

void orc_mx_scale_exp_array(const double* amax, int64_t n, int rule, int* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_mx_scale_exp(amax[i], rule);
}
