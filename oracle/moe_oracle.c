/*
 * moe_oracle.c -- plain, slow CPU oracle of the sparse Mixture-of-Experts FFN
 * layer forward pass.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * helper with the HIP path (the package under sparse_mixture_experts_gemm_amd/).
 *
 * Precision: every dot product is accumulated in double; the penalised score
 * and the top-k order are taken in fp32 because the routing decision must be
 * reproduced bit for bit from the same fp32 router logits.
 *
 * Sources (the five web pages on MoE sparse activation):
 *   P1 "GPT-4稀疏激活真相：万亿参数模型的MoE工程落地实践"
 *   P2 "MoE架构揭秘：逐Token路由与活跃参数量的工程真相"
 *   P3 "MoE稀疏激活原理与工程实践：从2%激活率到高效推理"
 *   P5 the page at 2kiu.com whose body covers the router and expert capacity
 * Where the pages leave a step open, the reading taken is stated at the step.
 *
 * Element types: dt = 0 means fp32 elements, dt = 1 means bfloat16 bit
 * patterns (uint16), widened exactly to float, dt = 2 means double elements
 * (used for dequantised one-byte expert weights, which are exact in double).
 *
 * Parity status: every function below is pinned by a CPU test (worked values
 * printed on the pages, closed forms, brute force, or special cases that reduce
 * to a textbook routine).  None is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double elem(const void *p, size_t i, int dt)
{
    if (dt == 0)
        return (double)((const float *)p)[i];
    if (dt == 2)
        return ((const double *)p)[i];
    uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the OpenMP loops that follow (n >= 1); used to time the oracle
 * single-threaded.  No effect on any result. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * One-byte expert weights (P5 §5.1, expert-kernel quantisation; P3 §3.2 on
 * INT8 expert weights; P1 §2.1 counts FP8 at one byte per parameter).  Reading: the byte format is OCP 8-bit
 * floating point E4M3 ("FN": no infinities): bit 7 sign, bits 6..3 a biased
 * exponent (bias 7), bits 2..0 the fraction.  Exponent field 0 encodes the
 * subnormals f/8 * 2^-6; exponent 15 with fraction 7 is NaN; every other code
 * is (1 + f/8) * 2^(e - 7).  Largest finite value 448.
 */
double oracle_fp8_e4m3_value(uint8_t b)
{
    int sgn = b >> 7, e = (b >> 3) & 15, f = b & 7;
    double v;
    if (e == 15 && f == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)f / 8.0, -6);
    else
        v = ldexp(1.0 + (double)f / 8.0, e - 7);
    return sgn ? -v : v;
}

void oracle_fp8_e4m3_decode(int64_t n, const uint8_t *q, double *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_fp8_e4m3_value(q[i]);
}

/*
 * Dequantised weight rows: w[r][c] = scale[r] * value(q[r][c]), one fp32 scale
 * per output row (per output channel) of a weight matrix.  Reading: the pages
 * give no scale granularity; a per-row scale keeps every dot product of the
 * layer a plain scaled sum.  The product of an fp32 scale and an E4M3 value is
 * exact in double.
 */
void oracle_dequant_rows(int64_t rows, int64_t cols, const uint8_t *q, const float *scale, double *w)
{
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++)
            w[r * cols + c] = (double)scale[r] * oracle_fp8_e4m3_value(q[r * cols + c]);
}

/*
 * Dynamic capacity factor (P1 §5.4: the factor grows with the batch as
 * 1 + 0.01 * log2(batch size), 1.05 at 32).  Reading: the batch size is the
 * number of tokens T routed together; evaluated in double; T < 1 gives 1.
 */
/*
 * INT8 expert weights (P3 §3.2 quantises the experts' weights to INT8; P5
 * §5.1 to integer formats).  Reading: a code is a two's complement byte,
 * value -128..127, and w[r][c] = scale[r] * q[r][c] with one fp32 scale per
 * output row, as for the E4M3 codes above; exact in double.
 */
void oracle_dequant_rows_i8(int64_t rows, int64_t cols, const int8_t *q, const float *scale, double *w)
{
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++)
            w[r * cols + c] = (double)scale[r] * (double)q[r * cols + c];
}

/*
 * INT4 expert weights (P5 §5.1 quantises the weights of some experts to INT4;
 * P3 §5.4 lists INT4 expert weights as the remedy for a bandwidth-bound
 * dispatch).  Reading: a code is a two's complement nibble, value -8..7; a
 * weight row of `cols` elements (cols even) is held in cols / 2 bytes, byte j
 * carrying element 2j in its low nibble and element 2j + 1 in its high
 * nibble; w[r][c] = scale[r] * q[r][c] with one fp32 scale per output row, as
 * for the one-byte codes above; exact in double.
 */
static int nibble_value(uint8_t byte, int high)
{
    const int v = high ? (byte >> 4) & 15 : byte & 15;
    return v >= 8 ? v - 16 : v;
}

void oracle_dequant_rows_i4(int64_t rows, int64_t cols, const uint8_t *q, const float *scale, double *w)
{
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++)
            w[r * cols + c] = (double)scale[r] * (double)nibble_value(q[r * (cols / 2) + c / 2], (int)(c & 1));
}

double oracle_dynamic_capacity_factor(int64_t T)
{
    if (T < 1)
        return 1.0;
    return 1.0 + 0.01 * log2((double)T);
}

/*
 * Expert capacity.  Reading: C = ceil(T*k/E * cf) evaluated in double in that
 * order (the expert_capacity formula of P2 §5.2, which gives 2 for 64 experts,
 * top-2, batch 32 and factor 1.3).  cf <= 0 means uncapped.  C never exceeds T:
 * an expert can receive at most one request per token.
 */
int64_t oracle_capacity(int64_t T, int64_t k, int64_t E, double cf)
{
    if (cf <= 0.0)
        return T;
    double c = ceil((double)T * (double)k / (double)E * cf);
    /* the clamp to T comes before the conversion: a factor so large (or
     * infinite) that c does not fit an int64_t still gives C = T */
    if (!(c < (double)T))
        return T;
    int64_t C = (int64_t)c;
    if (C < 0)
        C = 0;
    return C;
}

/*
 * Router logits: raw[t][e] = fp32(sum_i x[t][i] * Wr[e][i]) + bias[e]
 * (P2 §3.1: z = h . W_router with one weight vector per expert; a per-expert
 * bias added to the gate, as in the router-bias discussion of the page at
 * adg.csdn.net §3.1).  Wr is stored [E][d].  bias may be NULL.
 */
void oracle_router_logits(int T, int d, int E, int dt, const void *x, const void *wr,
                          const float *bias, float *raw)
{
    for (int t = 0; t < T; t++)
        for (int e = 0; e < E; e++) {
            double acc = 0.0;
            for (int i = 0; i < d; i++)
                acc += elem(x, (size_t)t * d + i, dt) * elem(wr, (size_t)e * d + i, dt);
            float r = (float)acc;
            if (bias)
                r = r + bias[e];
            raw[(size_t)t * E + e] = r;
        }
}

/*
 * Two-layer router ("MoE稀疏激活原理与工程实践" §3.1, second step: a gated
 * linear unit W1 x -> silu -> W2 instead of one linear map; W1 is
 * d x (2E), W2 (2E) x E, and W2's outputs are the expert scores; the
 * router of the page's MoELayer code (§4.2) is Linear(d, 2E) -> SiLU ->
 * Linear(2E, E), both linear maps with a bias):
 *   a[t][j]   = silu(sum_i x[t][i] * W1[j][i] + bias1[j]),  j < H,
 *               silu(v) = v / (1 + e^-v)
 *   raw[t][e] = fp32(sum_j a[t][j] * W2[e][j]) + bias[e]
 * in double up to the one fp32 rounding.  W1 is stored [H][d], W2 [E][H],
 * both of element type dt (H is the hidden width, 2E on the page); bias1
 * [H] and bias [E] are fp32 or NULL.
 */
void oracle_router_logits_glu(int T, int d, int E, int H, int dt, const void *x, const void *w1,
                              const void *w2, const float *bias1, const float *bias, float *raw)
{
    double *a = (double *)malloc((size_t)H * sizeof(double));
    for (int t = 0; t < T; t++) {
        for (int j = 0; j < H; j++) {
            double acc = 0.0;
            for (int i = 0; i < d; i++)
                acc += elem(x, (size_t)t * d + i, dt) * elem(w1, (size_t)j * d + i, dt);
            if (bias1)
                acc += bias1[j];
            a[j] = acc / (1.0 + exp(-acc));
        }
        for (int e = 0; e < E; e++) {
            double acc = 0.0;
            for (int j = 0; j < H; j++)
                acc += a[j] * elem(w2, (size_t)e * H + j, dt);
            float r = (float)acc;
            if (bias)
                r = r + bias[e];
            raw[(size_t)t * E + e] = r;
        }
    }
    free(a);
}

/*
 * Load-aware penalty (P1 §2.3: score_i = raw_i - lambda * load_i).  Taken as
 * one fused multiply-add in fp32, fmaf(-lambda, load, raw), so that both sides
 * round once.  load == NULL means no penalty (s = raw).
 */
void oracle_scores(int T, int E, const float *raw, const float *load, float lambda, float *s)
{
    for (int t = 0; t < T; t++)
        for (int e = 0; e < E; e++) {
            size_t i = (size_t)t * E + e;
            s[i] = load ? fmaf(-lambda, load[e], raw[i]) : raw[i];
        }
}

/*
 * Ranked candidates (P2 §3.1: softmax, then the top-2 indices).  Softmax is
 * monotone, so ranking by the fp32 score s is the same order without the
 * rounding of exp; ties go to the lower expert index, and NaN scores come
 * after every number (lower index first among them).  K columns are produced
 * (k chosen experts plus the fallback candidate); ranks >= E are -1 with score
 * -inf.
 */
/* a ranks above b: the larger score; a NaN ranks below every number.  The
 * pages never meet a NaN score; this reading keeps the order total, so every
 * rank below E names an expert. */
static int ranks_above(float a, float b)
{
    if (isnan(b))
        return !isnan(a);
    return a > b;
}

void oracle_topk(int T, int E, int K, const float *s, int32_t *cand, float *cand_score)
{
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    for (int t = 0; t < T; t++) {
        const float *st = s + (size_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int r = 0; r < K; r++) {
            int best = -1;
            for (int e = 0; e < E; e++) {
                if (taken[e])
                    continue;
                if (best < 0 || ranks_above(st[e], st[best]))
                    best = e;
            }
            cand[(size_t)t * K + r] = best;
            cand_score[(size_t)t * K + r] = best >= 0 ? st[best] : -INFINITY;
            if (best >= 0)
                taken[best] = 1;
        }
    }
    free(taken);
}

/*
 * Top-2 gap threshold (the adg.csdn.net page, §3.1: when the best and the
 * second-best score differ by less than a threshold, the second choice is
 * replaced by the third-ranked expert, so that the two experts are clearly
 * distinct).  Readings: the gap is taken on the ranking scores s (the fp32
 * difference s[rank 0] - s[rank 1], compared in fp32); the replacement swaps
 * ranks 1 and 2, so the displaced expert becomes the fallback candidate and
 * the list stays a permutation of the top K.  It applies only with a third
 * candidate that names an expert (K >= 3, cand[2] >= 0), and delta <= 0 turns
 * it off.  A NaN gap is not below delta.
 */
void oracle_gap_swap(int T, int K, float delta, int32_t *cand, float *cand_score)
{
    if (!(delta > 0.0f) || K < 3)
        return;
    for (int t = 0; t < T; t++) {
        int32_t *c = cand + (size_t)t * K;
        float *cs = cand_score + (size_t)t * K;
        const float gap = cs[0] - cs[1];
        if (c[2] >= 0 && gap < delta) {
            const int32_t ce = c[1];
            const float sc = cs[1];
            c[1] = c[2];
            cs[1] = cs[2];
            c[2] = ce;
            cs[2] = sc;
        }
    }
}

/*
 * Capacity-capped dispatch.
 *
 * Queue semantics (P1 §2.3: an expert whose queue has reached the limit sends
 * the token to its third-ranked candidate; P5 §2: once an expert is full, later
 * tokens go to the next-best expert; P2 §3.3: overflow is dropped or
 * re-routed).  Readings taken where the pages are open:
 *   - arrival order is rank-major: every token's rank-0 choice in token order,
 *     then every rank-1 choice, ..., then one fallback round in token order;
 *   - a token with at least one overflowed slot sends its lowest-rank
 *     overflowed slot to its rank-k candidate (the third-ranked expert for
 *     top-2); any further overflowed slot is dropped;
 *   - rows are packed per expert in arrival order; offsets is the exclusive
 *     scan of the kept counts.
 * Gates: the softmax of the chosen scores renormalised over the kept slots
 * (P2 §3.1 uses softmax probabilities p1, p2); a dropped slot gets 0.  With a
 * temperature tau > 0 the softmax is taken of score / tau (P3 §3.1, third
 * step: dividing the scores by a temperature sharpens or flattens the
 * distribution; the ranking is unchanged, so only the gates depend on it).
 * Load-balancing loss: aux_coef * sum_e (demand[e] / T)^2 with demand the
 * pre-cap rank < k selections (the balance loss of the MoELayer example in P3
 * §4.2, whose usage is normalised by the token count).
 *
 * cand, cand_score: [T][k+1].  Outputs eid, pos, row: [T][k] (-1 when dropped);
 * flag [T][k]: 0 kept, 1 re-routed, 2 dropped; gate [T][k] (fp32) and gate64
 * (double, may be NULL); offsets [E+1]; token_of_row [min(T*k, E*C)] (-1 past
 * the last row); demand, kept [E]; totals = {rows, dropped, rerouted}.
 */
void oracle_dispatch(int T, int E, int k, int64_t C, int reroute, float aux_coef, double tau,
                     const int32_t *cand, const float *cand_score,
                     int32_t *eid, int32_t *pos, uint8_t *flag, int32_t *row, float *gate,
                     double *gate64, int32_t *offsets, int32_t *token_of_row,
                     int32_t *demand, int32_t *kept, int32_t *totals, float *aux_loss)
{
    const int K = k + 1;
    int64_t *fill = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    int *src_rank = (int *)malloc((size_t)T * k * sizeof(int));

    for (int e = 0; e < E; e++)
        demand[e] = 0;
    for (int t = 0; t < T; t++)
        for (int r = 0; r < k; r++)
            demand[cand[(size_t)t * K + r]]++;

    /* primary rounds */
    for (int r = 0; r < k; r++)
        for (int t = 0; t < T; t++) {
            size_t j = (size_t)t * k + r;
            int e = cand[(size_t)t * K + r];
            src_rank[j] = r;
            if (fill[e] < C) {
                eid[j] = e;
                pos[j] = (int32_t)fill[e]++;
                flag[j] = 0;
            } else {
                eid[j] = -1;
                pos[j] = -1;
                flag[j] = 2;
            }
        }

    /* fallback round */
    if (reroute && k < E)
        for (int t = 0; t < T; t++) {
            int rs = -1;
            for (int r = 0; r < k; r++)
                if (flag[(size_t)t * k + r] == 2) {
                    rs = r;
                    break;
                }
            if (rs < 0)
                continue;
            int f = cand[(size_t)t * K + k];
            if (fill[f] < C) {
                size_t j = (size_t)t * k + rs;
                eid[j] = f;
                pos[j] = (int32_t)fill[f]++;
                flag[j] = 1;
                src_rank[j] = k;
            }
        }

    /* packed rows */
    int64_t acc = 0;
    for (int e = 0; e < E; e++) {
        kept[e] = (int32_t)fill[e];
        offsets[e] = (int32_t)acc;
        acc += fill[e];
    }
    offsets[E] = (int32_t)acc;
    int64_t cap_rows = (int64_t)T * k;
    if ((int64_t)E * C < cap_rows)
        cap_rows = (int64_t)E * C;
    for (int64_t i = 0; i < cap_rows; i++)
        token_of_row[i] = -1;
    int rerouted = 0;
    for (int t = 0; t < T; t++)
        for (int r = 0; r < k; r++) {
            size_t j = (size_t)t * k + r;
            if (flag[j] == 2) {
                row[j] = -1;
                continue;
            }
            row[j] = offsets[eid[j]] + pos[j];
            token_of_row[row[j]] = t;
            if (flag[j] == 1)
                rerouted++;
        }

    /* gates: softmax over the kept slots' scores */
    for (int t = 0; t < T; t++) {
        double m = -INFINITY;
        for (int r = 0; r < k; r++) {
            size_t j = (size_t)t * k + r;
            if (flag[j] != 2) {
                double sv = cand_score[(size_t)t * K + src_rank[j]];
                if (sv > m)
                    m = sv;
            }
        }
        double z = 0.0;
        for (int r = 0; r < k; r++) {
            size_t j = (size_t)t * k + r;
            if (flag[j] != 2)
                z += exp(((double)cand_score[(size_t)t * K + src_rank[j]] - m) / tau);
        }
        for (int r = 0; r < k; r++) {
            size_t j = (size_t)t * k + r;
            double g = 0.0;
            if (flag[j] != 2)
                g = exp(((double)cand_score[(size_t)t * K + src_rank[j]] - m) / tau) / z;
            gate[j] = (float)g;
            if (gate64)
                gate64[j] = g;
        }
    }

    totals[0] = (int32_t)acc;
    totals[1] = (int32_t)((int64_t)T * k - acc);
    totals[2] = rerouted;

    double l = 0.0;
    for (int e = 0; e < E; e++) {
        double u = T > 0 ? (double)demand[e] / (double)T : 0.0; /* empty batch: no load */
        l += u * u;
    }
    *aux_loss = (float)((double)aux_coef * l);

    free(fill);
    free(src_rank);
}

/*
 * One expert FFN application (P1 §3.1: Linear -> SwiGLU -> Linear per expert;
 * P5 §1: each expert is the W1/W2/W3 matrices of an FFN).  Reading:
 * h = silu(x W1^T) * (x W3^T), y = h W2^T, silu(a) = a / (1 + exp(-a)), no
 * biases.  W1, W3: [E][d_ff][d]; W2: [E][d][d_ff].  xrow points at element
 * offset xo of x.  h (scratch, d_ff doubles) is left holding the SwiGLU
 * activations; ye receives the d outputs.
 */
static void ffn_one(int e, size_t xo, int d, int d_ff, int dt, const void *x, const void *w1,
                    const void *w3, const void *w2, double *h, double *ye)
{
    size_t wo = (size_t)e * d_ff * d;
    for (int j = 0; j < d_ff; j++) {
        double a = 0.0, b = 0.0;
        size_t ro = wo + (size_t)j * d;
        for (int q = 0; q < d; q++) {
            double xv = elem(x, xo + q, dt);
            a += xv * elem(w1, ro + q, dt);
            b += xv * elem(w3, ro + q, dt);
        }
        h[j] = a / (1.0 + exp(-a)) * b;
    }
    size_t w2o = (size_t)e * d * d_ff;
    for (int q = 0; q < d; q++) {
        double acc = 0.0;
        size_t ro = w2o + (size_t)q * d_ff;
        for (int j = 0; j < d_ff; j++)
            acc += h[j] * elem(w2, ro + j, dt);
        ye[q] = acc;
    }
}

/*
 * Expert FFN on a list of rows: row i applies expert[i] to input row
 * x[src[i]].  y [n][d] and h [n][d_ff] (h may be NULL) are double.
 */
void oracle_ffn_rows(int n, const int32_t *expert, const int32_t *src, int d, int d_ff, int dt,
                     const void *x, const void *w1, const void *w3, const void *w2,
                     double *y, double *h_out)
{
#pragma omp parallel
    {
        double *h = (double *)malloc((size_t)d_ff * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < n; i++) {
            ffn_one(expert[i], (size_t)src[i] * d, d, d_ff, dt, x, w1, w3, w2, h,
                    y + (size_t)i * d);
            if (h_out)
                memcpy(h_out + (size_t)i * d_ff, h, (size_t)d_ff * sizeof(double));
        }
        free(h);
    }
}

/*
 * Layer output for a list of tokens: y_t = sum over kept slots j of
 * gate[t][j] * FFN_{eid[t][j]}(x_t) (P5 §3, step 5: the experts' results are
 * put back in token order; P1 §4.3: weighted fusion of the experts' outputs).
 * A token with no kept slot gets a zero row.  gate64 and eid are [T][k];
 * y [n][d].
 */
void oracle_layer_tokens(int n, const int32_t *tokens, int k, int d, int d_ff, int dt,
                         const void *x, const void *w1, const void *w3, const void *w2,
                         const int32_t *eid, const double *gate64, double *y)
{
#pragma omp parallel
    {
        double *h = (double *)malloc((size_t)d_ff * sizeof(double));
        double *ye = (double *)malloc((size_t)d * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < n; i++) {
            int t = tokens[i];
            double *yt = y + (size_t)i * d;
            for (int q = 0; q < d; q++)
                yt[q] = 0.0;
            for (int r = 0; r < k; r++) {
                int e = eid[(size_t)t * k + r];
                if (e < 0)
                    continue;
                ffn_one(e, (size_t)t * d, d, d_ff, dt, x, w1, w3, w2, h, ye);
                double g = gate64[(size_t)t * k + r];
                for (int q = 0; q < d; q++)
                    yt[q] += g * ye[q];
            }
        }
        free(h);
        free(ye);
    }
}

/*
 * Combine from given per-row expert outputs: y[t] = sum over kept slots of
 * gate[t][j] * y_rows[row[t][j]] (row == -1: slot dropped).  y_rows has element
 * type dt; gate is fp32 as produced by dispatch; y [T][d] double.
 */
void oracle_combine(int T, int k, int d, int dt, const int32_t *row, const float *gate,
                    const void *y_rows, double *y)
{
    for (int t = 0; t < T; t++) {
        double *yt = y + (size_t)t * d;
        for (int q = 0; q < d; q++)
            yt[q] = 0.0;
        for (int r = 0; r < k; r++) {
            int rw = row[(size_t)t * k + r];
            if (rw < 0)
                continue;
            double g = gate[(size_t)t * k + r];
            for (int q = 0; q < d; q++)
                yt[q] += g * elem(y_rows, (size_t)rw * d + q, dt);
        }
    }
}

/*
 * ------------------------------------------------------------------------
 * Backward pass (training).  The pages train the router through the experts:
 * its gradient is what flows back from the experts' outputs (P2 §3.3, "the
 * router's gradient comes from the experts' gradients flowing back").
 * Readings:
 *   - the routing decisions (ranking, capacity, re-route, drop) are held
 *     fixed, as the forward pass took them: they are piecewise constant in
 *     the inputs, so the gradient flows through the gates of the kept slots
 *     and through the experts only (inference-style deterministic top-k; the
 *     Gumbel noise P2 §3.3 adds during training is not part of this layer);
 *   - the load-balancing loss of P3 §4.2 counts top-k picks under no_grad,
 *     so its gradient with respect to every input is zero and adds nothing;
 *   - the penalty load vector is an input without a gradient.
 * With do = g_j dy_t the upstream gradient of a kept slot's expert output
 * o_j = FFN_e(x_t) (y_t = sum_j g_j o_j, P5 §3 step 5), the chain rule gives
 *   u    = W2_e^T dy_t                    (d_ff)
 *   dh   = g_j u                          (gradient of h = silu(a) * b)
 *   da   = dh * b * silu'(a),  db = dh * silu(a),
 *          silu'(a) = s(a) (1 + a (1 - s(a))), s the logistic function
 *   dW2_e += do h^T,  dW1_e += da x_t^T,  dW3_e += db x_t^T
 *   dx_t  += W1_e^T da + W3_e^T db
 *   dg_j  = dy_t . o_j
 * and through the gate softmax over the kept slots K_t (scores s divided by
 * the temperature tau, P3 §3.1):
 *   ds_j  = g_j (dg_j - sum_{l in K_t} g_l dg_l) / tau   for j in K_t,
 * which is the gradient of the router logit raw[t][eid_j] (s = raw - lambda
 * load, and raw = x W_r^T + bias), so
 *   dlogits[t][eid_j] = ds_j (0 for every other expert),
 *   dx_t += sum_e dlogits[t][e] W_r[e],  dW_r = dlogits^T x,  dbias = sum_t dlogits[t].
 * dy is double; x and the weights have element type dt.
 * ------------------------------------------------------------------------
 */

static double logistic(double a) { return 1.0 / (1.0 + exp(-a)); }

/*
 * Per-token part for a list of tokens: the router-logit gradient
 * dlogits [n][E] and the input gradient dx [n][d] (expert and router terms).
 */
void oracle_backward_tokens(int n, const int32_t *tokens, int d, int E, int k, int d_ff, int dt, double tau,
                            const void *x, const void *wr, const void *w1, const void *w3, const void *w2,
                            const int32_t *eid, const double *gate64, const double *dy, double *dlogits,
                            double *dx)
{
#pragma omp parallel
    {
        double *a = (double *)malloc((size_t)d_ff * sizeof(double));
        double *b = (double *)malloc((size_t)d_ff * sizeof(double));
        double *u = (double *)malloc((size_t)d_ff * sizeof(double));
        double dg[64];
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < n; i++) {
            const int t = tokens[i];
            const double *dyt = dy + (size_t)t * d;
            double *dxt = dx + (size_t)i * d;
            double *dlt = dlogits + (size_t)i * E;
            for (int q = 0; q < d; q++)
                dxt[q] = 0.0;
            for (int e = 0; e < E; e++)
                dlt[e] = 0.0;
            for (int r = 0; r < k; r++) {
                const int e = eid[(size_t)t * k + r];
                dg[r] = 0.0;
                if (e < 0)
                    continue;
                const double g = gate64[(size_t)t * k + r];
                const size_t wo = (size_t)e * d_ff * d, w2o = (size_t)e * d * d_ff;
                /* pre-activations a = W1 x, b = W3 x and u = W2^T dy */
                for (int j = 0; j < d_ff; j++) {
                    double sa = 0.0, sb = 0.0, su = 0.0;
                    for (int q = 0; q < d; q++) {
                        const double xv = elem(x, (size_t)t * d + q, dt);
                        sa += xv * elem(w1, wo + (size_t)j * d + q, dt);
                        sb += xv * elem(w3, wo + (size_t)j * d + q, dt);
                        su += dyt[q] * elem(w2, w2o + (size_t)q * d_ff + j, dt);
                    }
                    a[j] = sa;
                    b[j] = sb;
                    u[j] = su;
                }
                /* dg = dy . o = dy . (W2 h) = u . h */
                double s = 0.0;
                for (int j = 0; j < d_ff; j++) {
                    const double sg = logistic(a[j]);
                    const double silu = a[j] * sg;
                    s += u[j] * silu * b[j];
                    /* input gradient through the expert: W1^T da + W3^T db */
                    const double dh = g * u[j];
                    const double da = dh * b[j] * sg * (1.0 + a[j] * (1.0 - sg));
                    const double db = dh * silu;
                    for (int q = 0; q < d; q++)
                        dxt[q] += da * elem(w1, wo + (size_t)j * d + q, dt) + db * elem(w3, wo + (size_t)j * d + q, dt);
                }
                dg[r] = s;
            }
            /* softmax over the kept slots: ds_j = g_j (dg_j - sum_l g_l dg_l) / tau */
            double mean = 0.0;
            for (int r = 0; r < k; r++)
                if (eid[(size_t)t * k + r] >= 0)
                    mean += gate64[(size_t)t * k + r] * dg[r];
            for (int r = 0; r < k; r++) {
                const int e = eid[(size_t)t * k + r];
                if (e >= 0)
                    dlt[e] = gate64[(size_t)t * k + r] * (dg[r] - mean) / tau;
            }
            /* router term of the input gradient */
            for (int e = 0; e < E; e++) {
                if (dlt[e] == 0.0)
                    continue;
                for (int q = 0; q < d; q++)
                    dxt[q] += dlt[e] * elem(wr, (size_t)e * d + q, dt);
            }
        }
        free(a);
        free(b);
        free(u);
    }
}

/*
 * Weight gradients of one expert e for a list of its intermediate units
 * fs[0..nf): rows dW1[e][f][:] and dW3[e][f][:] into dw1, dw3 [nf][d], and
 * columns dW2[e][:][f] into dw2 [d][nf].  The expert's kept slots are given
 * as (token, gate) pairs in row order: tok [nrows], g [nrows].
 */
void oracle_backward_expert_units(int e, int nf, const int32_t *fs, int nrows, const int32_t *tok,
                                  const double *g, int d, int d_ff, int dt, const void *x, const void *w1,
                                  const void *w3, const void *w2, const double *dy, double *dw1, double *dw3,
                                  double *dw2)
{
    const size_t wo = (size_t)e * d_ff * d, w2o = (size_t)e * d * d_ff;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < nf; i++) {
        const int f = fs[i];
        double *r1 = dw1 + (size_t)i * d, *r3 = dw3 + (size_t)i * d;
        for (int q = 0; q < d; q++) {
            r1[q] = 0.0;
            r3[q] = 0.0;
            dw2[(size_t)q * nf + i] = 0.0;
        }
        for (int rr = 0; rr < nrows; rr++) {
            const int t = tok[rr];
            const double *dyt = dy + (size_t)t * d;
            double a = 0.0, b = 0.0, u = 0.0;
            for (int q = 0; q < d; q++) {
                const double xv = elem(x, (size_t)t * d + q, dt);
                a += xv * elem(w1, wo + (size_t)f * d + q, dt);
                b += xv * elem(w3, wo + (size_t)f * d + q, dt);
                u += dyt[q] * elem(w2, w2o + (size_t)q * d_ff + f, dt);
            }
            const double sg = logistic(a), silu = a * sg;
            const double h = silu * b, dh = g[rr] * u;
            const double da = dh * b * sg * (1.0 + a * (1.0 - sg)), db = dh * silu;
            for (int q = 0; q < d; q++) {
                const double xv = elem(x, (size_t)t * d + q, dt);
                r1[q] += da * xv;
                r3[q] += db * xv;
                dw2[(size_t)q * nf + i] += g[rr] * dyt[q] * h;
            }
        }
    }
}

/*
 * Router weight and bias gradients: dW_r[e][:] = sum_t dlogits[t][e] x_t,
 * dbias[e] = sum_t dlogits[t][e] (raw = x W_r^T + bias).  dlogits [T][E]
 * double; dwr [E][d], dbias [E].
 */
void oracle_router_wgrad(int T, int d, int E, int dt, const void *x, const double *dlogits, double *dwr,
                         double *dbias)
{
#pragma omp parallel for schedule(static)
    for (int e = 0; e < E; e++) {
        double *we = dwr + (size_t)e * d;
        double sb = 0.0;
        for (int q = 0; q < d; q++)
            we[q] = 0.0;
        for (int t = 0; t < T; t++) {
            const double gl = dlogits[(size_t)t * E + e];
            if (gl == 0.0)
                continue;
            sb += gl;
            for (int q = 0; q < d; q++)
                we[q] += gl * elem(x, (size_t)t * d + q, dt);
        }
        dbias[e] = sb;
    }
}

/*
 * Windowed load statistic (P5 §2, first constraint: an expert's load is its
 * selection frequency over a sliding window of the most recent tokens, for
 * example 1024, with a decay factor alpha = 0.99 so that the statistic
 * follows the current load).  Reading: the T tokens of a batch fall, in
 * token order, into consecutive windows of W tokens (the last one may be
 * shorter); each window updates the statistic once,
 *   load[e] <- alpha * load[e] + (1 - alpha) * f[e],
 *   f[e] = (selections of e in the window) / (k * tokens in the window),
 * a selection being one of a token's ranks 0..k-1 in its candidate list
 * (the router's top-k choices, before the capacity cap); entries outside
 * [0, E) select nothing.  In double, windows in order; load is fp32 in and
 * out, rounded once at the end.  cand is [T][K1].
 */
void oracle_load_window(int T, int E, int k, int K1, const int32_t *cand, int window, double alpha, float *load)
{
    double *l = (double *)malloc((size_t)E * sizeof(double));
    long *cnt = (long *)malloc((size_t)E * sizeof(long));
    for (int e = 0; e < E; e++)
        l[e] = load[e];
    for (int t0 = 0; t0 < T; t0 += window) {
        const int n = T - t0 < window ? T - t0 : window;
        for (int e = 0; e < E; e++)
            cnt[e] = 0;
        for (int t = t0; t < t0 + n; t++)
            for (int r = 0; r < k; r++) {
                const int c = cand[(size_t)t * K1 + r];
                if (c >= 0 && c < E)
                    cnt[c]++;
            }
        for (int e = 0; e < E; e++)
            l[e] = alpha * l[e] + (1.0 - alpha) * ((double)cnt[e] / ((double)k * n));
    }
    for (int e = 0; e < E; e++)
        load[e] = (float)l[e];
    free(l);
    free(cnt);
}
