/*
 * Memory-safety driver for the oracle (test infrastructure only). Built together with mxq_oracle.c by the host gcc
 * with the address and undefined-behaviour sanitizers, it calls every routine of the oracle on small seeded inputs
 * whose buffers are allocated at exactly the sizes the routines document: ragged shapes, single blocks, empty
 * tensors, empty expert groups, several threads. A read or write past any buffer, a use after free or a leak ends
 * the run with a sanitizer report and a non-zero status. It checks no values (the pinned tests do that).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct { float lr, beta1, beta2, eps, weight_decay; int64_t step; } orc_adam_hp;

double orc_e4m3_value(uint8_t c);
double orc_e5m2_value(uint8_t c);
double orc_f16_value(uint16_t c);
float orc_bf16_to_f32(uint16_t h);
uint16_t orc_bf16_from_f32(float f);
uint8_t orc_fp8_encode(double v, int fmt);
uint16_t orc_f16_from_f32(float f);
int orc_mx_scale_exp(double amax, int rule);
void orc_mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, int rule, uint8_t* q_row, uint8_t* s_row,
                     uint8_t* q_col, uint8_t* s_col, int nthreads);
void orc_mx_quantize_f32(const float* x, int64_t rows, int64_t cols, int rule, uint8_t* q_row, uint8_t* s_row,
                         uint8_t* q_col, uint8_t* s_col, int nthreads);
float orc_exp_f32(float x);
float orc_swiglu_f32(float g, float u);
void orc_swiglu_mx_quantize(const uint16_t* c, int64_t rows, int64_t F, int rule, uint8_t* q, uint8_t* s, float* h);
void orc_route_weighted_mx_quantize(const uint16_t* dy, const float* p, int64_t rows, int64_t cols, int rule,
                                    uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, float* x_out,
                                    int nthreads);
void orc_swiglu_bwd_f32(float g, float u, float dh, float* d_gate, float* d_up);
void orc_swiglu_bwd_mx_quantize(const uint16_t* c, const uint16_t* dh, int64_t rows, int64_t F, int rule,
                                uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, float* dc_out,
                                int nthreads);
void orc_autoscale_cast(const uint16_t* g, int64_t n, int fmt, float* mu, uint8_t* q, uint64_t* overflow,
                        float* scale_out);
float orc_min_scale(const float* scales, int64_t N);
void orc_requantize_shared(const uint8_t* q_in, int64_t n, int fmt_in, float s_in, float s_g, int fmt_out,
                           uint8_t* q_out);
void orc_pertensor_quantize(const uint16_t* x, int64_t rows, int64_t cols, int fmt, float margin,
                            const float* scale_in, float* amax_out, float* scale_out, uint8_t* q, uint8_t* q_t,
                            int nthreads);
float orc_delayed_scale(const float* history, int64_t H, int fmt, float margin);
void orc_history_push(float* history, int64_t H, int32_t* pos, float amax);
void orc_pertensor_quantize_delayed(const uint16_t* x, int64_t rows, int64_t cols, int fmt, float margin,
                                    float* history, int64_t H, int32_t* pos, float* amax_out, float* scale_out,
                                    uint8_t* q, uint8_t* q_t, int nthreads);
void orc_gemm_ref(const uint8_t* aq, const void* a_scale, int a_fmt, const uint8_t* bq, const void* b_scale,
                  int b_fmt, int64_t M, int64_t N, int64_t K, int scaling, const int64_t* rows, int64_t nr,
                  const int64_t* cols, int64_t nc, double* y, double* S, int nthreads);
void orc_grouped_gemm_ref(const uint8_t* aq, const uint8_t* as, const int64_t* offsets, int64_t G, const uint8_t* bq,
                          const uint8_t* bs, int64_t N, int64_t K, const int64_t* rows, int64_t nr,
                          const int64_t* cols, int64_t nc, double* y, double* S, int nthreads);
void orc_grouped_wgrad_ref(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs,
                           const int64_t* offsets, int64_t Kt, const int64_t* groups, int64_t ng, const int64_t* rows,
                           int64_t nr, const int64_t* cols, int64_t nc, double* y, double* S);
float orc_adam_step(float* master, const uint16_t* grad_bf16, uint8_t* m_q, float* m_scale, uint16_t* v16,
                    uint16_t* w_bf16, int64_t n, const orc_adam_hp* hp, int nthreads);
float orc_adam_step_delayed(float* master, const uint16_t* grad_bf16, uint8_t* m_q, float* m_scale, uint16_t* v16,
                            uint16_t* w_bf16, int64_t n, const orc_adam_hp* hp, float* history, int64_t H,
                            int32_t* pos, int nthreads);
float orc_adam_amax(const uint16_t* grad_bf16, const uint8_t* m_q, const uint16_t* v16, float m_scale_old, int64_t n,
                    const orc_adam_hp* hp, int nthreads);
void orc_adam_elements(const float* master, const uint16_t* grad_bf16, const uint8_t* m_q, const uint16_t* v16,
                       float m_scale_old, float s_new, const int64_t* idx, int64_t count, const orc_adam_hp* hp,
                       float* out_master, uint8_t* out_mq, uint16_t* out_v16, uint16_t* out_w);

/* splitmix64: seeded input bits, no arithmetic of the method */
static uint64_t sm_state = 0x5EEDULL;
static uint64_t next64(void) {
    uint64_t z = (sm_state += 0x9E3779B97F4A7C15ULL);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}
/* a finite bf16 in roughly [-8, 8] (exponent field 100..130), or zero now and then */
static uint16_t rand_bf16(void) {
    uint64_t r = next64();
    if ((r & 31) == 0) return (uint16_t)((r >> 8) & 0x8000);
    return (uint16_t)(((r >> 8) & 0x8000) | ((100 + (r >> 16) % 31) << 7) | ((r >> 24) & 0x7F));
}
static uint16_t* bf16_buf(int64_t n) {
    uint16_t* p = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) p[i] = rand_bf16();
    return p;
}
static uint8_t* u8_buf(int64_t n, int fp8) {
    uint8_t* p = (uint8_t*)malloc((size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) {
        uint8_t c = (uint8_t)next64();
        if (fp8 && (c & 0x7F) == 0x7F) c = 0x30;           /* keep E4M3 codes finite */
        p[i] = c;
    }
    return p;
}
static uint8_t* scale_buf(int64_t n) {
    uint8_t* p = (uint8_t*)malloc((size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) p[i] = (uint8_t)(120 + next64() % 15);
    return p;
}
static float* f32_buf(int64_t n, float lo, float hi) {
    float* p = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * (float)((next64() >> 40) * (1.0 / 16777216.0));
    return p;
}
static int64_t* idx_buf(int64_t n, int64_t hi) {
    int64_t* p = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) p[i] = (int64_t)(next64() % (uint64_t)hi);
    return p;
}

static void mx_quantize_case(int64_t rows, int64_t cols, int rule, int nthreads) {
    uint16_t* x = bf16_buf(rows * cols);
    float* xf = f32_buf(rows * cols, -5.0f, 5.0f);
    uint8_t* qr = malloc((size_t)(rows * cols > 0 ? rows * cols : 1));
    uint8_t* sr = malloc((size_t)(rows * cols / 32 > 0 ? rows * cols / 32 : 1));
    uint8_t* qc = malloc((size_t)(rows * cols > 0 ? rows * cols : 1));
    uint8_t* sc = malloc((size_t)(rows * cols / 32 > 0 ? rows * cols / 32 : 1));
    orc_mx_quantize(x, rows, cols, rule, qr, sr, qc, sc, nthreads);
    orc_mx_quantize(x, rows, cols, rule, qr, sr, NULL, NULL, nthreads);
    orc_mx_quantize(x, rows, cols, rule, NULL, NULL, qc, sc, nthreads);
    orc_mx_quantize_f32(xf, rows, cols, rule, qr, sr, qc, sc, nthreads);
    free(x); free(xf); free(qr); free(sr); free(qc); free(sc);
}

static void pertensor_case(int64_t rows, int64_t cols, int fmt, int nthreads) {
    uint16_t* x = bf16_buf(rows * cols);
    uint8_t* q = malloc((size_t)(rows * cols > 0 ? rows * cols : 1));
    uint8_t* qt = malloc((size_t)(rows * cols > 0 ? rows * cols : 1));
    float amax, scale, sin = 3.5f;
    orc_pertensor_quantize(x, rows, cols, fmt, 1.0f, NULL, &amax, &scale, q, qt, nthreads);
    orc_pertensor_quantize(x, rows, cols, fmt, 2.0f, &sin, &amax, &scale, q, NULL, nthreads);
    float hist[5] = {1.0f, 0.5f, 0.0f, 4.0f, 2.0f};
    int32_t pos = 3;
    orc_pertensor_quantize_delayed(x, rows, cols, fmt, 1.0f, hist, 5, &pos, &amax, &scale, q, qt, nthreads);
    (void)orc_delayed_scale(hist, 5, fmt, 1.0f);
    orc_history_push(hist, 5, &pos, 7.0f);
    free(x); free(q); free(qt);
}

static void gemm_case(int64_t M, int64_t N, int64_t K, int nthreads) {
    uint8_t* aq = u8_buf(M * K, 1);
    uint8_t* bq = u8_buf(N * K, 1);
    uint8_t* as = scale_buf(M * K / 32);
    uint8_t* bs = scale_buf(N * K / 32);
    int64_t nr = M < 5 ? M : 5, nc = N < 7 ? N : 7;
    int64_t* rows = idx_buf(nr, M);
    int64_t* cols = idx_buf(nc, N);
    double* y = malloc(sizeof(double) * (size_t)(M * N));
    double* S = malloc(sizeof(double) * (size_t)(M * N));
    int64_t* all_r = idx_buf(M, M);
    int64_t* all_c = idx_buf(N, N);
    for (int64_t i = 0; i < M; ++i) all_r[i] = i;
    for (int64_t j = 0; j < N; ++j) all_c[j] = j;
    orc_gemm_ref(aq, as, 0, bq, bs, 0, M, N, K, 1, all_r, M, all_c, N, y, S, nthreads);
    orc_gemm_ref(aq, as, 0, bq, bs, 0, M, N, K, 1, rows, nr, cols, nc, y, S, nthreads);
    float sa = 2.0f, sb = 0.25f;
    orc_gemm_ref(aq, &sa, 1, bq, &sb, 0, M, N, K, 0, rows, nr, all_c, N, y, S, nthreads);
    free(aq); free(bq); free(as); free(bs); free(rows); free(cols); free(y); free(S); free(all_r); free(all_c);
}

static void grouped_case(int nthreads) {
    /* 4 groups of 32-row blocks, one empty; total 160 rows */
    const int64_t G = 4, N = 40, K = 96;
    int64_t off[5] = {0, 64, 64, 128, 160};
    uint8_t* aq = u8_buf(160 * K, 1);
    uint8_t* as = scale_buf(160 * K / 32);
    uint8_t* bq = u8_buf(G * N * K, 1);
    uint8_t* bs = scale_buf(G * N * K / 32);
    int64_t* rows = idx_buf(160, 160);
    int64_t* cols = idx_buf(N, N);
    for (int64_t i = 0; i < 160; ++i) rows[i] = i;
    for (int64_t j = 0; j < N; ++j) cols[j] = j;
    double* y = malloc(sizeof(double) * 160 * (size_t)N);
    double* S = malloc(sizeof(double) * 160 * (size_t)N);
    orc_grouped_gemm_ref(aq, as, off, G, bq, bs, N, K, rows, 160, cols, N, y, S, nthreads);
    free(aq); free(as); free(bq); free(bs); free(rows); free(cols); free(y); free(S);

    /* routed Wgrad: token ranges of 160 tokens, operands [M][Kt] and [N][Kt] */
    const int64_t M = 24, Nw = 16, Kt = 160;
    uint8_t* wa = u8_buf(M * Kt, 1);
    uint8_t* wsa = scale_buf(M * Kt / 32);
    uint8_t* wb = u8_buf(Nw * Kt, 1);
    uint8_t* wsb = scale_buf(Nw * Kt / 32);
    int64_t groups[4] = {0, 1, 2, 3};
    int64_t* r = idx_buf(M, M);
    int64_t* c = idx_buf(Nw, Nw);
    for (int64_t i = 0; i < M; ++i) r[i] = i;
    for (int64_t j = 0; j < Nw; ++j) c[j] = j;
    double* wy = malloc(sizeof(double) * 4 * (size_t)(M * Nw));
    double* wS = malloc(sizeof(double) * 4 * (size_t)(M * Nw));
    orc_grouped_wgrad_ref(wa, wsa, wb, wsb, off, Kt, groups, 4, r, M, c, Nw, wy, wS);
    free(wa); free(wsa); free(wb); free(wsb); free(r); free(c); free(wy); free(wS);
}

static void adam_case(int64_t n, int nthreads) {
    orc_adam_hp hp = {3e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 3};
    float* master = f32_buf(n, -0.05f, 0.05f);
    uint16_t* g = bf16_buf(n);
    uint8_t* mq = u8_buf(n, 1);
    uint16_t* v = malloc(sizeof(uint16_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) v[i] = (uint16_t)(next64() % 0x3C00);
    uint16_t* w = malloc(sizeof(uint16_t) * (size_t)(n > 0 ? n : 1));
    float ms = 100.0f;
    (void)orc_adam_amax(g, mq, v, ms, n, &hp, nthreads);
    int64_t cnt = n < 9 ? n : 9;
    int64_t* idx = idx_buf(cnt, n > 0 ? n : 1);
    float* om = malloc(sizeof(float) * (size_t)(cnt > 0 ? cnt : 1));
    uint8_t* oq = malloc((size_t)(cnt > 0 ? cnt : 1));
    uint16_t* ov = malloc(sizeof(uint16_t) * (size_t)(cnt > 0 ? cnt : 1));
    uint16_t* ow = malloc(sizeof(uint16_t) * (size_t)(cnt > 0 ? cnt : 1));
    orc_adam_elements(master, g, mq, v, ms, 200.0f, idx, cnt, &hp, om, oq, ov, ow);
    (void)orc_adam_step(master, g, mq, &ms, v, w, n, &hp, nthreads);
    (void)orc_adam_step(master, g, mq, &ms, v, NULL, n, &hp, nthreads);
    float hist[3] = {0.5f, 0.25f, 1.0f};
    int32_t pos = 2;
    (void)orc_adam_step_delayed(master, g, mq, &ms, v, w, n, &hp, hist, 3, &pos, nthreads);
    free(master); free(g); free(mq); free(v); free(w); free(idx); free(om); free(oq); free(ov); free(ow);
}

static void elementwise_case(int64_t rows, int64_t F, int nthreads) {
    uint16_t* c = bf16_buf(rows * 2 * F);
    uint16_t* dh = bf16_buf(rows * F);
    uint8_t* q = malloc((size_t)(rows * 2 * F > 0 ? rows * 2 * F : 1));
    uint8_t* s = malloc((size_t)(rows * 2 * F / 32 > 0 ? rows * 2 * F / 32 : 1));
    uint8_t* qc = malloc((size_t)(rows * 2 * F > 0 ? rows * 2 * F : 1));
    uint8_t* sc = malloc((size_t)(rows * 2 * F / 32 > 0 ? rows * 2 * F / 32 : 1));
    float* h = malloc(sizeof(float) * (size_t)(rows * 2 * F > 0 ? rows * 2 * F : 1));
    orc_swiglu_mx_quantize(c, rows, F, 0, q, s, h);
    orc_swiglu_bwd_mx_quantize(c, dh, rows, F, 1, q, s, qc, sc, h, nthreads);
    float* p = f32_buf(rows, 0.01f, 1.0f);
    orc_route_weighted_mx_quantize(dh, p, rows, F, 0, q, s, qc, sc, h, nthreads);
    float dg, du;
    orc_swiglu_bwd_f32(-1.25f, 0.5f, 2.0f, &dg, &du);
    (void)orc_swiglu_f32(3.0f, -2.0f);
    (void)orc_exp_f32(-87.0f);
    free(c); free(dh); free(q); free(s); free(qc); free(sc); free(h); free(p);
}

static void allreduce_case(int64_t n) {
    uint16_t* g = bf16_buf(n);
    uint8_t* q = malloc((size_t)(n > 0 ? n : 1));
    uint8_t* q2 = malloc((size_t)(n > 0 ? n : 1));
    float mu = 1024.0f, sc;
    uint64_t over = 0;
    orc_autoscale_cast(g, n, 0, &mu, q, &over, &sc);
    orc_autoscale_cast(g, n, 1, &mu, q, &over, &sc);
    float scales[3] = {2.0f, 0.5f, 8.0f};
    float sg = orc_min_scale(scales, 3);
    orc_requantize_shared(q, n, 1, sc, sg, 0, q2);
    free(g); free(q); free(q2);
}

int main(void) {
    for (int c = 0; c < 256; ++c) {
        (void)orc_e4m3_value((uint8_t)c);
        (void)orc_e5m2_value((uint8_t)c);
        (void)orc_fp8_encode(orc_e4m3_value((uint8_t)c), 0);
    }
    for (int h = 0; h < 65536; h += 97) {
        (void)orc_f16_value((uint16_t)h);
        (void)orc_bf16_from_f32(orc_bf16_to_f32((uint16_t)h));
        (void)orc_f16_from_f32(orc_bf16_to_f32((uint16_t)h));
    }
    (void)orc_mx_scale_exp(500.0, 0);
    (void)orc_mx_scale_exp(500.0, 1);
    const int64_t shapes[][2] = {{32, 32}, {96, 160}, {160, 96}, {64, 1024}, {0, 64}, {64, 0}};
    for (int i = 0; i < 6; ++i)
        for (int t = 1; t <= 3; t += 2) {
            mx_quantize_case(shapes[i][0], shapes[i][1], t == 1 ? 0 : 1, t);
            pertensor_case(shapes[i][0], shapes[i][1], t == 1 ? 0 : 1, t);
        }
    gemm_case(1, 1, 32, 1);
    gemm_case(33, 47, 224, 3);
    gemm_case(64, 40, 96, 4);
    grouped_case(2);
    adam_case(1, 1);
    adam_case(1003, 3);
    adam_case(0, 2);
    elementwise_case(64, 64, 3);
    elementwise_case(32, 32, 1);
    allreduce_case(1027);
    allreduce_case(0);
    printf("asan driver: ok\n");
    return 0;
}
