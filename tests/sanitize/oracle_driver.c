/*
 * Drives every function of the CPU oracle (oracle/moe_oracle.c) on small
 * seeded inputs, including the edge cases (empty batch, one expert, k = E,
 * capacity 1, uncapped, no re-route, NaN rows, E = 256 with top-8), for a
 * build under AddressSanitizer and UndefinedBehaviorSanitizer.  Exits 0 when
 * every call ran and the invariants checked here hold; a sanitizer report
 * aborts the run.  Test infrastructure, built and run by
 * tests/test_sanitizers.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_num_threads(void);
void oracle_set_num_threads(int n);
double oracle_fp8_e4m3_value(uint8_t b);
void oracle_fp8_e4m3_decode(int64_t n, const uint8_t *q, double *out);
void oracle_dequant_rows(int64_t rows, int64_t cols, const uint8_t *q, const float *scale, double *w);
double oracle_dynamic_capacity_factor(int64_t T);
int64_t oracle_capacity(int64_t T, int64_t k, int64_t E, double cf);
void oracle_router_logits(int T, int d, int E, int dt, const void *x, const void *wr, const float *bias, float *raw);
void oracle_router_logits_glu(int T, int d, int E, int H, int dt, const void *x, const void *w1, const void *w2,
                              const float *bias1, const float *bias, float *raw);
void oracle_scores(int T, int E, const float *raw, const float *load, float lambda, float *s);
void oracle_topk(int T, int E, int K, const float *s, int32_t *cand, float *cand_score);
void oracle_gap_swap(int T, int K, float delta, int32_t *cand, float *cand_score);
void oracle_dispatch(int T, int E, int k, int64_t C, int reroute, float aux_coef, double tau, const int32_t *cand,
                     const float *cand_score, int32_t *eid, int32_t *pos, uint8_t *flag, int32_t *row, float *gate,
                     double *gate64, int32_t *offsets, int32_t *token_of_row, int32_t *demand, int32_t *kept,
                     int32_t *totals, float *aux_loss);
void oracle_ffn_rows(int n, const int32_t *expert, const int32_t *src, int d, int d_ff, int dt, const void *x,
                     const void *w1, const void *w3, const void *w2, double *y, double *h_out);
void oracle_layer_tokens(int n, const int32_t *tokens, int k, int d, int d_ff, int dt, const void *x, const void *w1,
                         const void *w3, const void *w2, const int32_t *eid, const double *gate64, double *y);
void oracle_combine(int T, int k, int d, int dt, const int32_t *row, const float *gate, const void *y_rows, double *y);
void oracle_backward_tokens(int n, const int32_t *tokens, int d, int E, int k, int d_ff, int dt, double tau,
                            const void *x, const void *wr, const void *w1, const void *w3, const void *w2,
                            const int32_t *eid, const double *gate64, const double *dy, double *dlogits, double *dx);
void oracle_backward_expert_units(int e, int nf, const int32_t *fs, int nrows, const int32_t *tok, const double *g,
                                  int d, int d_ff, int dt, const void *x, const void *w1, const void *w3,
                                  const void *w2, const double *dy, double *dw1, double *dw3, double *dw2);
void oracle_router_wgrad(int T, int d, int E, int dt, const void *x, const double *dlogits, double *dwr,
                         double *dbias);
void oracle_load_window(int T, int E, int k, int K1, const int32_t *cand, int window, double alpha, float *load);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) /* SplitMix64, uniform in [-1, 1) */
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) / 4503599627370496.0 - 1.0;
}

static void *xalloc(size_t n) /* never zero bytes, so every pointer is valid */
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static uint16_t to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFF + ((u >> 16) & 1)) >> 16);
}

static int failures = 0;
#define CHECK(c)                                                                  \
    do {                                                                          \
        if (!(c)) {                                                               \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);     \
            failures++;                                                           \
        }                                                                         \
    } while (0)

/* one layer: route, dispatch, FFN, combine, backward */
static void run_layer(int T, int d, int E, int k, int d_ff, double cf, int reroute, int dt, float lambda, float gap,
                      double tau, int nan_row)
{
    const size_t es = dt == 0 ? 4 : 2;
    void *x = xalloc((size_t)T * d * es), *wr = xalloc((size_t)E * d * es);
    void *w1 = xalloc((size_t)E * d_ff * d * es), *w3 = xalloc((size_t)E * d_ff * d * es);
    void *w2 = xalloc((size_t)E * d * d_ff * es);
    void *arrs[5] = {x, wr, w1, w3, w2};
    size_t ns[5] = {(size_t)T * d, (size_t)E * d, (size_t)E * d_ff * d, (size_t)E * d_ff * d, (size_t)E * d * d_ff};
    for (int a = 0; a < 5; a++)
        for (size_t i = 0; i < ns[a]; i++) {
            float v = (float)(urand() * (a == 0 ? 2.0 : 0.3));
            if (dt == 0)
                ((float *)arrs[a])[i] = v;
            else
                ((uint16_t *)arrs[a])[i] = to_bf16(v);
        }
    if (nan_row && T > 0) {
        if (dt == 0)
            ((float *)x)[0] = NAN;
        else
            ((uint16_t *)x)[0] = 0x7FC0;
    }
    float *bias = (float *)xalloc(E * sizeof(float)), *load = (float *)xalloc(E * sizeof(float));
    for (int e = 0; e < E; e++) {
        bias[e] = (float)urand();
        load[e] = (float)((urand() + 1.0) / E);
    }
    const int K1 = k + 1;
    float *raw = (float *)xalloc((size_t)T * E * 4), *s = (float *)xalloc((size_t)T * E * 4);
    int32_t *cand = (int32_t *)xalloc((size_t)T * K1 * 4);
    float *cs = (float *)xalloc((size_t)T * K1 * 4);
    oracle_router_logits(T, d, E, dt, x, wr, bias, raw);
    oracle_scores(T, E, raw, lambda > 0 ? load : NULL, lambda, s);
    oracle_topk(T, E, K1, s, cand, cs);
    oracle_gap_swap(T, K1, gap, cand, cs);
    const int64_t C = oracle_capacity(T, k, E, cf);
    const int64_t R = (int64_t)T * k < (int64_t)E * C ? (int64_t)T * k : (int64_t)E * C;
    int32_t *eid = (int32_t *)xalloc((size_t)T * k * 4), *pos = (int32_t *)xalloc((size_t)T * k * 4);
    int32_t *row = (int32_t *)xalloc((size_t)T * k * 4);
    uint8_t *flag = (uint8_t *)xalloc((size_t)T * k);
    float *gate = (float *)xalloc((size_t)T * k * 4);
    double *gate64 = (double *)xalloc((size_t)T * k * 8);
    int32_t *offsets = (int32_t *)xalloc((size_t)(E + 1) * 4), *tor = (int32_t *)xalloc((size_t)R * 4);
    int32_t *demand = (int32_t *)xalloc((size_t)E * 4), *kept = (int32_t *)xalloc((size_t)E * 4), totals[3];
    float aux;
    oracle_dispatch(T, E, k, C, reroute, 0.01f, tau, cand, cs, eid, pos, flag, row, gate, gate64, offsets, tor,
                    demand, kept, totals, &aux);
    int64_t sk = 0, sd = 0;
    for (int e = 0; e < E; e++) {
        CHECK(kept[e] <= C);
        sk += kept[e];
        sd += demand[e];
    }
    CHECK(sk == totals[0] && offsets[E] == totals[0]);
    CHECK(sd == (int64_t)T * k);
    CHECK(totals[0] + totals[1] == T * k);
    /* FFN of every kept row, combine, layer tokens */
    const int rows = totals[0];
    int32_t *ex = (int32_t *)xalloc((size_t)rows * 4);
    for (int e = 0; e < E; e++)
        for (int r = offsets[e]; r < offsets[e + 1]; r++)
            ex[r] = e;
    double *yr = (double *)xalloc((size_t)rows * d * 8), *hr = (double *)xalloc((size_t)rows * d_ff * 8);
    oracle_ffn_rows(rows, ex, tor, d, d_ff, dt, x, w1, w3, w2, yr, hr);
    float *yrf = (float *)xalloc((size_t)rows * d * 4);
    for (size_t i = 0; i < (size_t)rows * d; i++)
        yrf[i] = (float)yr[i];
    double *y = (double *)xalloc((size_t)T * d * 8), *y2 = (double *)xalloc((size_t)T * d * 8);
    oracle_combine(T, k, d, 0, row, gate, yrf, y);
    int32_t *toks = (int32_t *)xalloc((size_t)T * 4);
    for (int t = 0; t < T; t++)
        toks[t] = t;
    oracle_layer_tokens(T, toks, k, d, d_ff, dt, x, w1, w3, w2, eid, gate64, y2);
    /* backward */
    double *dy = (double *)xalloc((size_t)T * d * 8);
    for (size_t i = 0; i < (size_t)T * d; i++)
        dy[i] = urand();
    double *dl = (double *)xalloc((size_t)T * E * 8), *dx = (double *)xalloc((size_t)T * d * 8);
    oracle_backward_tokens(T, toks, d, E, k, d_ff, dt, tau, x, wr, w1, w3, w2, eid, gate64, dy, dl, dx);
    double *dwr = (double *)xalloc((size_t)E * d * 8), *db = (double *)xalloc((size_t)E * 8);
    oracle_router_wgrad(T, d, E, dt, x, dl, dwr, db);
    int32_t *fs = (int32_t *)xalloc((size_t)d_ff * 4);
    for (int f = 0; f < d_ff; f++)
        fs[f] = f;
    double *dw1 = (double *)xalloc((size_t)d_ff * d * 8), *dw3 = (double *)xalloc((size_t)d_ff * d * 8);
    double *dw2 = (double *)xalloc((size_t)d * d_ff * 8);
    int32_t *tk = (int32_t *)xalloc((size_t)(rows + 1) * 4);
    double *gk = (double *)xalloc((size_t)(rows + 1) * 8);
    for (int e = 0; e < E; e++) {
        int n = 0;
        for (int t = 0; t < T; t++)
            for (int j = 0; j < k; j++)
                if (eid[(size_t)t * k + j] == e) {
                    tk[n] = t;
                    gk[n++] = gate64[(size_t)t * k + j];
                }
        oracle_backward_expert_units(e, d_ff, fs, n, tk, gk, d, d_ff, dt, x, w1, w3, w2, dy, dw1, dw3, dw2);
    }
    /* windowed load statistic */
    float *lw = (float *)xalloc((size_t)E * 4);
    for (int e = 0; e < E; e++)
        lw[e] = 1.0f / E;
    oracle_load_window(T, E, k, K1, cand, 7, 0.99, lw);
    oracle_load_window(T, E, k, K1, cand, 1, 0.5, lw);
    free(lw);
    /* two-layer router */
    const int H = 2 * E;
    void *g1 = xalloc((size_t)H * d * es), *g2 = xalloc((size_t)E * H * es);
    memset(g1, 0, (size_t)H * d * es);
    memset(g2, 0, (size_t)E * H * es);
    float *b1 = (float *)xalloc((size_t)H * sizeof(float));
    for (int j = 0; j < H; j++)
        b1[j] = (float)urand();
    oracle_router_logits_glu(T, d, E, H, dt, x, g1, g2, b1, bias, raw);
    free(b1);
    void *frees[] = {x, wr, w1, w3, w2, bias, load, raw, s, cand, cs, eid, pos, row, flag, gate, gate64, offsets,
                     tor, demand, kept, ex, yr, hr, yrf, y, y2, toks, dy, dl, dx, dwr, db, fs, dw1, dw3, dw2, tk, gk,
                     g1, g2};
    for (size_t i = 0; i < sizeof frees / sizeof frees[0]; i++)
        free(frees[i]);
}

int main(void)
{
    oracle_set_num_threads(1);
    CHECK(oracle_num_threads() >= 1);
    /* one-byte weights */
    uint8_t q[256];
    double v[256];
    for (int i = 0; i < 256; i++)
        q[i] = (uint8_t)i;
    oracle_fp8_e4m3_decode(256, q, v);
    CHECK(v[0x38] == 1.0 && isnan(v[0x7F]));
    CHECK(oracle_fp8_e4m3_value(0x7E) == 448.0);
    float sc[16];
    for (int r = 0; r < 16; r++)
        sc[r] = 0.5f;
    double w[256];
    oracle_dequant_rows(16, 16, q, sc, w);
    /* capacity, including huge and infinite factors */
    CHECK(oracle_capacity(32, 2, 64, 1.3) == 2);
    CHECK(oracle_capacity(4096, 2, 8, INFINITY) == 4096);
    CHECK(oracle_capacity(4096, 2, 8, 1e30) == 4096);
    CHECK(oracle_capacity(100, 2, 8, 0.0) == 100);
    CHECK(oracle_dynamic_capacity_factor(32) > 1.049 && oracle_dynamic_capacity_factor(0) == 1.0);
    /*        T   d   E  k d_ff   cf  rr dt  lambda gap  tau nan */
    run_layer(0, 16, 4, 2, 8, 1.0, 1, 0, 0.0f, 0.0f, 1.0, 0);  /* empty batch */
    run_layer(1, 16, 4, 2, 8, 1.0, 1, 1, 0.0f, 0.0f, 1.0, 0);  /* one token */
    run_layer(37, 16, 5, 2, 24, 0.6, 1, 0, 0.3f, 0.1f, 0.5, 1); /* capped, penalty, gap, NaN row */
    run_layer(40, 8, 3, 3, 8, 0.5, 1, 1, 0.0f, 0.0f, 2.0, 0);  /* k = E */
    run_layer(50, 8, 4, 2, 8, 1e-6, 1, 0, 0.0f, 0.0f, 1.0, 0); /* capacity 1 */
    run_layer(30, 8, 4, 2, 8, 0.0, 1, 0, 0.0f, 0.0f, 1.0, 0);  /* uncapped */
    run_layer(30, 8, 4, 2, 8, 0.5, 0, 1, 0.0f, 0.0f, 1.0, 0);  /* no re-route */
    run_layer(20, 8, 1, 1, 8, 0.0, 1, 0, 0.0f, 0.0f, 1.0, 0);  /* one expert */
    run_layer(64, 8, 256, 8, 8, 1.0, 1, 1, 0.0f, 0.0f, 1.0, 0); /* 256 experts, top-8 */
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle driver ok\n");
    return 0;
}
