// Stage 2: capacity-capped dispatch, deterministic and atomics-free.
//
// What it computes ("GPT-4稀疏激活真相" §2.3: an expert whose queue has reached
// the limit sends the token to its third-ranked candidate; "MoE架构揭秘" §3.3:
// overflow is dropped or re-routed; "企业官网建设流程全解析" page §2: once an
// expert is full, later tokens go to the next-best expert):
//   arrival order is rank-major: all rank-0 choices in token order, then rank
//   1, ..., then one fallback round in token order.  A request is kept while
//   its expert holds fewer than C rows.  A token with an overflowed slot sends
//   its lowest overflowed slot to its rank-k candidate; further overflowed
//   slots are dropped.  Gates are the softmax of the kept slots' scores,
//   divided by the gate temperature ("MoE稀疏激活原理与工程实践" §3.1,
//   third step; 1 when the parameter is 0).
//
// Because a primary request's queue position depends only on how many earlier
// requests chose the same expert, positions are counting problems: per-block
// expert histograms, an exclusive prefix over blocks, and an in-block rank from
// wave ballots (one ballot per bit of the expert index, then mbcnt over the
// lanes holding the same expert).  The fallback round depends on the primary
// overflow, so it takes a second histogram pass.
// Kernels (one token per thread, 1024 tokens per block):
//   hist      per-block counts of each primary round
//   primary   queue positions of the primary rounds, fallback histograms
//   finalize  fallback positions, packed rows, gates, statistics, loss
//   gather    copy of each token's x row to its kept rows (x_perm)
// Each block recomputes the prefix it needs from the per-block histograms, so
// no grid-wide synchronisation or atomic is needed.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
static_assert(kThreads == kDispatchBlock, "one token per thread");

// Rank of this lane among the lanes of its wave holding the same key (keys
// < 0 are ignored), and the per-key lane counts of the wave, written to
// wave_cnt[key].  The lanes holding this lane's key are found bit by bit:
// one ballot per key bit (nbits = ceil(log2 E)), each narrowing the set to
// the lanes that agree on that bit, so the cost does not grow with the
// number of distinct keys in the wave.  The lowest lane of each key writes
// the count.
__device__ __forceinline__ int wave_rank_count(int key, int nbits, int *wave_cnt) {
    uint64_t same = ballot64(key >= 0);
    for (int b = 0; b < nbits; b++) {  // nbits is uniform
        const bool bit = (key >> b) & 1;
        const uint64_t m = ballot64(bit);
        same &= bit ? m : ~m;
    }
    const int rank = rank_below(same);
    if (key >= 0 && rank == 0) wave_cnt[key] = __popcll(same);
    return rank;
}

// A candidate id outside [0, E) (moe_route writes -1 for ranks past E; a
// caller's own routing may hold anything) is read as "no expert", so it is
// never used as an index.
__device__ __forceinline__ int valid_expert(int c, int E) { return (unsigned)c < (unsigned)E ? c : -1; }

// Bits of an expert index: ceil(log2 E), at least 1.
__device__ __forceinline__ int key_bits(int E) { return E > 1 ? 32 - __builtin_clz((unsigned)(E - 1)) : 1; }

// Sum of p[j * stride] over j < n (all) and over j < lim (below), read in
// batches of eight independent loads (clamped indices, no branch) so that
// their latencies overlap instead of adding up.  n >= 1.
__device__ __forceinline__ void strided_sums(const int32_t *p, size_t stride, int n, int lim, int &below,
                                             int &all) {
    below = 0;
    all = 0;
    for (int j0 = 0; j0 < n; j0 += 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; u++) v[u] = p[(size_t)min(j0 + u, n - 1) * stride];
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int x = j0 + u < n ? v[u] : 0;
            all += x;
            below += j0 + u < lim ? x : 0;
        }
    }
}

__device__ __forceinline__ void zero_lds(int *a, int n) {
    for (int i = threadIdx.x; i < n; i += kThreads) a[i] = 0;
}

__device__ __forceinline__ void hist_body(int b, const int32_t *__restrict__ cand, int T, int E, int k,
                                          int32_t *__restrict__ hist, int (&wcnt)[kWaves][kMaxExperts]) {
    const int K1 = k + 1;
    const int t = b * kThreads + threadIdx.x;
    const int wave = threadIdx.x >> 6;
    for (int r = 0; r < k; r++) {
        zero_lds(&wcnt[0][0], kWaves * kMaxExperts);
        __syncthreads();
        const int key = t < T ? valid_expert(cand[(size_t)t * K1 + r], E) : -1;
        wave_rank_count(key, key_bits(E), wcnt[wave]);
        __syncthreads();
        for (int e = threadIdx.x; e < E; e += kThreads) {
            int s = 0;
            for (int w = 0; w < kWaves; w++) s += wcnt[w][e];
            hist[((size_t)b * k + r) * E + e] = s;
        }
        __syncthreads();
    }
}

// claim (null or kClaimCounters ints): the expert GEMM's work-claim counters,
// zeroed here for the launch that follows the dispatch.
__device__ __forceinline__ void zero_claim(int32_t *claim) {
    if (claim && blockIdx.x == 0 && threadIdx.x < kClaimCounters) claim[threadIdx.x] = 0;
}

__global__ __launch_bounds__(kThreads) void dispatch_hist(const int32_t *__restrict__ cand, int T,
                                                          int E, int k, int32_t *__restrict__ hist,
                                                          int32_t *__restrict__ claim) {
    __shared__ int wcnt[kWaves][kMaxExperts];
    zero_claim(claim);
    hist_body(blockIdx.x, cand, T, E, k, hist, wcnt);
}

struct PrimaryLds {
    int base[kMaxTopK][kMaxExperts];
    int tot[kMaxTopK][kMaxExperts];
    int wcnt[kWaves][kMaxExperts];
};

__device__ __forceinline__ void primary_body(int b, const int32_t *__restrict__ cand, int T, int E, int k, int C,
                                             int nb, int use_fallback, const int32_t *__restrict__ hist,
                                             int32_t *__restrict__ fill_prim, int32_t *__restrict__ eid,
                                             int32_t *__restrict__ pos, uint8_t *__restrict__ flag,
                                             int32_t *__restrict__ fb_hist, PrimaryLds &sm) {
    auto &base = sm.base;
    auto &tot = sm.tot;
    auto &wcnt = sm.wcnt;
    const int K1 = k + 1;
    const int t = b * kThreads + threadIdx.x;
    const int wave = threadIdx.x >> 6;

    // requests before this block, and in total, per (round, expert)
    for (int i = threadIdx.x; i < k * E; i += kThreads) {
        const int r = i / E, e = i % E;
        int pre, all;
        strided_sums(hist + (size_t)r * E + e, (size_t)k * E, nb, b, pre, all);
        base[r][e] = pre;
        tot[r][e] = all;
    }
    __syncthreads();
    // queue fill before each round: fill_{r+1} = min(C, fill_r + requests_r)
    for (int e = threadIdx.x; e < E; e += kThreads) {
        int fill = 0;
        for (int r = 0; r < k; r++) {
            base[r][e] += fill;
            fill = min(C, fill + tot[r][e]);
        }
        if (b == 0) fill_prim[e] = fill;
    }

    int first_over = -1;
    for (int r = 0; r < k; r++) {
        zero_lds(&wcnt[0][0], kWaves * kMaxExperts);
        __syncthreads();
        const int key = t < T ? valid_expert(cand[(size_t)t * K1 + r], E) : -1;
        const int rank = wave_rank_count(key, key_bits(E), wcnt[wave]);
        __syncthreads();
        if (t < T) {
            int p = C;  // a candidate that names no expert is never kept
            if (key >= 0) {
                p = base[r][key] + rank;
                for (int w = 0; w < wave; w++) p += wcnt[w][key];
            }
            const size_t j = (size_t)t * k + r;
            if (p < C) {
                eid[j] = key;
                pos[j] = p;
                flag[j] = 0;
            } else {
                eid[j] = -1;
                pos[j] = -1;
                flag[j] = 2;
                if (first_over < 0) first_over = r;
            }
        }
        __syncthreads();
    }

    // fallback requests of this block, per expert
    zero_lds(&wcnt[0][0], kWaves * kMaxExperts);
    __syncthreads();
    const int fkey = (t < T && use_fallback && first_over >= 0) ? valid_expert(cand[(size_t)t * K1 + k], E) : -1;
    wave_rank_count(fkey, key_bits(E), wcnt[wave]);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kThreads) {
        int s = 0;
        for (int w = 0; w < kWaves; w++) s += wcnt[w][e];
        fb_hist[(size_t)b * E + e] = s;
    }
}

__global__ __launch_bounds__(kThreads) void dispatch_primary(
    const int32_t *__restrict__ cand, int T, int E, int k, int C, int nb, int use_fallback,
    const int32_t *__restrict__ hist, int32_t *__restrict__ fill_prim, int32_t *__restrict__ eid,
    int32_t *__restrict__ pos, uint8_t *__restrict__ flag, int32_t *__restrict__ fb_hist) {
    __shared__ PrimaryLds sm;
    primary_body(blockIdx.x, cand, T, E, k, C, nb, use_fallback, hist, fill_prim, eid, pos, flag, fb_hist, sm);
}

struct FinalizeLds {
    int fbase[kMaxExperts];
    int kcnt[kMaxExperts];
    int offs[kMaxExperts + 1];
    int scan_tmp[2][kMaxExperts];
    int wcnt[kWaves][kMaxExperts];
};

__device__ __forceinline__ void finalize_body(
    int b, const int32_t *__restrict__ cand, const float *__restrict__ cand_score, int T, int E, int k,
    int C, int nb, int use_fallback, float aux_coef, float tau, int cap_rows, const int32_t *__restrict__ hist,
    const int32_t *__restrict__ fill_prim, const int32_t *__restrict__ fb_hist,
    int32_t *__restrict__ eid, int32_t *__restrict__ pos, uint8_t *__restrict__ flag,
    int32_t *__restrict__ row, float *__restrict__ gate, int32_t *__restrict__ offsets,
    int32_t *__restrict__ token_of_row, int32_t *__restrict__ demand, int32_t *__restrict__ kept,
    int32_t *__restrict__ totals, float *__restrict__ aux_loss, float *__restrict__ gate_of_row, FinalizeLds &sm) {
    auto &fbase = sm.fbase;
    auto &kcnt = sm.kcnt;
    auto &offs = sm.offs;
    auto &scan_tmp = sm.scan_tmp;
    auto &wcnt = sm.wcnt;
    const int K1 = k + 1;
    const int t = b * kThreads + threadIdx.x;
    const int wave = threadIdx.x >> 6;

    for (int e = threadIdx.x; e < E; e += kThreads) {
        int pre, all;
        strided_sums(fb_hist + e, (size_t)E, nb, b, pre, all);
        const int fp = fill_prim[e];
        fbase[e] = fp + pre;
        const int kc = min(C, fp + all);
        kcnt[e] = kc;
        scan_tmp[0][e] = kc;
    }
    __syncthreads();
    // inclusive Hillis-Steele scan over the experts, then shift to exclusive
    int src = 0;
    for (int step = 1; step < E; step <<= 1) {
        for (int e = threadIdx.x; e < E; e += kThreads)
            scan_tmp[src ^ 1][e] = scan_tmp[src][e] + (e >= step ? scan_tmp[src][e - step] : 0);
        __syncthreads();
        src ^= 1;
    }
    for (int e = threadIdx.x; e < E; e += kThreads) offs[e + 1] = scan_tmp[src][e];
    if (threadIdx.x == 0) offs[0] = 0;

    // fallback positions
    zero_lds(&wcnt[0][0], kWaves * kMaxExperts);
    __syncthreads();
    int first_over = -1;
    if (t < T)
        for (int r = 0; r < k; r++)
            if (flag[(size_t)t * k + r] == 2) {
                first_over = r;
                break;
            }
    const int fkey = (t < T && use_fallback && first_over >= 0) ? valid_expert(cand[(size_t)t * K1 + k], E) : -1;
    const int rank = wave_rank_count(fkey, key_bits(E), wcnt[wave]);
    __syncthreads();
    if (fkey >= 0) {
        int p = fbase[fkey] + rank;
        for (int w = 0; w < wave; w++) p += wcnt[w][fkey];
        if (p < C) {
            const size_t j = (size_t)t * k + first_over;
            eid[j] = fkey;
            pos[j] = p;
            flag[j] = 1;
        }
    }

    // packed rows and gates
    if (t < T) {
        float sc[kMaxTopK];
        int e_s[kMaxTopK], p_s[kMaxTopK], f_s[kMaxTopK];
        float m = -INFINITY;
        for (int r = 0; r < k; r++) {
            const size_t j = (size_t)t * k + r;
            f_s[r] = flag[j];
            e_s[r] = eid[j];
            p_s[r] = pos[j];
            sc[r] = f_s[r] == 2 ? -INFINITY : cand_score[(size_t)t * K1 + (f_s[r] == 1 ? k : r)];
            if (f_s[r] != 2) m = fmaxf(m, sc[r]);
        }
        float z = 0.0f;
        for (int r = 0; r < k; r++)
            if (f_s[r] != 2) z += expf((sc[r] - m) / tau);
        for (int r = 0; r < k; r++) {
            const size_t j = (size_t)t * k + r;
            if (f_s[r] == 2) {
                row[j] = -1;
                gate[j] = 0.0f;
            } else {
                const int rw = offs[e_s[r]] + p_s[r];
                const float gv = expf((sc[r] - m) / tau) / z;
                row[j] = rw;
                token_of_row[rw] = t;
                gate[j] = gv;
                if (gate_of_row) gate_of_row[rw] = gv;  // the row's combine weight, for the down epilogue
            }
        }
    }

    // rows past the last kept row carry no token
    const int rows = offs[E];
    for (int i = rows + b * kThreads + threadIdx.x; i < cap_rows; i += nb * kThreads) token_of_row[i] = -1;

    if (b == 0) {
        for (int e = threadIdx.x; e <= E; e += kThreads) offsets[e] = offs[e];
        for (int e = threadIdx.x; e < E; e += kThreads) {
            int dem, unused;
            strided_sums(hist + e, (size_t)E, nb * k, 0, unused, dem);  // rows (block, round) of hist
            demand[e] = dem;
            kept[e] = kcnt[e];
            scan_tmp[0][e] = dem;  // reuse for the loss below
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            int rer = 0;
            double l = 0.0;
            for (int e = 0; e < E; e++) {
                rer += kcnt[e] - fill_prim[e];
                const double u = T > 0 ? (double)scan_tmp[0][e] / (double)T : 0.0;
                l += u * u;
            }
            totals[0] = rows;
            totals[1] = T * k - rows;
            totals[2] = rer;
            aux_loss[0] = (float)((double)aux_coef * l);
        }
    }
}

__global__ __launch_bounds__(kThreads) void dispatch_finalize(
    const int32_t *__restrict__ cand, const float *__restrict__ cand_score, int T, int E, int k,
    int C, int nb, int use_fallback, float aux_coef, float tau, int cap_rows, const int32_t *__restrict__ hist,
    const int32_t *__restrict__ fill_prim, const int32_t *__restrict__ fb_hist,
    int32_t *__restrict__ eid, int32_t *__restrict__ pos, uint8_t *__restrict__ flag,
    int32_t *__restrict__ row, float *__restrict__ gate, int32_t *__restrict__ offsets,
    int32_t *__restrict__ token_of_row, int32_t *__restrict__ demand, int32_t *__restrict__ kept,
    int32_t *__restrict__ totals, float *__restrict__ aux_loss, float *__restrict__ gate_of_row) {
    __shared__ FinalizeLds sm;
    finalize_body(blockIdx.x, cand, cand_score, T, E, k, C, nb, use_fallback, aux_coef, tau, cap_rows, hist, fill_prim,
                  fb_hist, eid, pos, flag, row, gate, offsets, token_of_row, demand, kept, totals, aux_loss,
                  gate_of_row, sm);
}

// T <= kThreads: one block runs the three phases back to back, saving two
// launches and their latency.  The histograms, fills and fallback counts
// pass through LDS; the slot arrays (eid, pos, flag) through global memory,
// as between the three kernels.  The block's barriers order the phases.
__global__ __launch_bounds__(kThreads) void dispatch_single(
    const int32_t *__restrict__ cand, const float *__restrict__ cand_score, int T, int E, int k, int C,
    int use_fallback, float aux_coef, float tau, int cap_rows, int32_t *__restrict__ hist, int32_t *__restrict__ fill_prim,
    int32_t *__restrict__ fb_hist, int32_t *__restrict__ eid, int32_t *__restrict__ pos,
    uint8_t *__restrict__ flag, int32_t *__restrict__ row, float *__restrict__ gate,
    int32_t *__restrict__ offsets, int32_t *__restrict__ token_of_row, int32_t *__restrict__ demand,
    int32_t *__restrict__ kept, int32_t *__restrict__ totals, float *__restrict__ aux_loss,
    float *__restrict__ gate_of_row, int32_t *__restrict__ claim) {
    __shared__ union {
        int wcnt[kWaves][kMaxExperts];
        PrimaryLds p;
        FinalizeLds f;
    } sm;
    zero_claim(claim);
    // the histograms and fills stay in LDS (the kernel arguments of the same
    // names are unused here)
    __shared__ int32_t hist_l[kMaxTopK * kMaxExperts], fill_l[kMaxExperts], fb_l[kMaxExperts];
    (void)hist;
    (void)fill_prim;
    (void)fb_hist;
    hist_body(0, cand, T, E, k, hist_l, sm.wcnt);
    __threadfence_block();
    __syncthreads();
    primary_body(0, cand, T, E, k, C, 1, use_fallback, hist_l, fill_l, eid, pos, flag, fb_l, sm.p);
    __threadfence_block();
    __syncthreads();
    finalize_body(0, cand, cand_score, T, E, k, C, 1, use_fallback, aux_coef, tau, cap_rows, hist_l, fill_l, fb_l, eid,
                  pos, flag, row, gate, offsets, token_of_row, demand, kept, totals, aux_loss, gate_of_row, sm.f);
}

// x_perm[row[t][j]] = x[t] for every kept slot: the token row is read once.
__global__ __launch_bounds__(256) void dispatch_gather(const uint4 *__restrict__ x,
                                                       const int32_t *__restrict__ row, int k,
                                                       int chunks, uint4 *__restrict__ x_perm) {
    const int t = blockIdx.x;
    int rws[kMaxTopK];
    for (int r = 0; r < k; r++) rws[r] = row[(size_t)t * k + r];
    for (int c = threadIdx.x; c < chunks; c += 256) {
        const uint4 v = x[(size_t)t * chunks + c];
        for (int r = 0; r < k; r++)
            if (rws[r] >= 0) x_perm[(size_t)rws[r] * chunks + c] = v;
    }
}

// Windowed load statistic ("企业官网建设流程全解析" page §2: an expert's
// selection frequency over a sliding window of recent tokens, with a decay
// factor).  Block w counts the top-k selections (ranks 0..k-1 of the
// candidate lists; entries outside [0, E) select nothing) of tokens
// [w W, min(T, (w+1) W)); integer LDS counts, so the result does not depend
// on the order of the adds.
__global__ __launch_bounds__(256) void load_window_counts(const int32_t *__restrict__ cand, int T, int E, int k,
                                                          int K1, int window, int32_t *__restrict__ counts) {
    __shared__ int c[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += 256) c[e] = 0;
    __syncthreads();
    const int64_t t0 = (int64_t)blockIdx.x * window, t1 = min((int64_t)T, t0 + window);
    for (int64_t i = t0 * k + threadIdx.x; i < t1 * k; i += 256) {
        const int64_t t = i / k;
        const int ex = valid_expert(cand[t * K1 + (i - t * k)], E);
        if (ex >= 0) atomicAdd(&c[ex], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) counts[(size_t)blockIdx.x * E + e] = c[e];
}

// load[e] <- alpha load[e] + (1 - alpha) f_w[e] for the windows in order, in
// double (f_w the window's selections over k x its tokens), one thread per
// expert, rounded to fp32 once.  No contraction into fused multiply-adds:
// each operation rounds as written.
__global__ __launch_bounds__(256) void load_window_update(const int32_t *__restrict__ counts, int nw, int T, int E,
                                                          int k, int window, double alpha, float *__restrict__ load) {
#pragma clang fp contract(off)
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= E) return;
    double l = load[e];
    for (int w = 0; w < nw; w++) {
        const int n = (int)min((int64_t)window, (int64_t)T - (int64_t)w * window);
        const double f = (double)counts[(size_t)w * E + e] / ((double)k * (double)n);
        l = alpha * l + (1.0 - alpha) * f;
    }
    load[e] = (float)l;
}

}  // namespace

hipError_t launch_load_window(const moe_params &p, const int32_t *cand, int window, float decay, float *load,
                              int32_t *counts, hipStream_t st) {
    if (p.T == 0) return hipSuccess;
    const int nw = (int)ceil_div(p.T, window);
    hipLaunchKernelGGL(load_window_counts, dim3(nw), dim3(256), 0, st, cand, p.T, p.E, p.k, p.k + 1, window, counts);
    hipLaunchKernelGGL(load_window_update, dim3((unsigned)ceil_div(p.E, 256)), dim3(256), 0, st, counts, nw, p.T,
                       p.E, p.k, window, (double)decay, load);
    return hipGetLastError();
}

hipError_t launch_dispatch(const moe_params &p, int64_t C, const void *x, const moe_routing &r,
                           void *x_perm, const DispatchScratch &ws, hipStream_t st) {
    const int T = p.T, E = p.E, k = p.k;
    const int nb = (int)ceil_div(T > 0 ? T : 1, kThreads);
    const int use_fb = (p.reroute && k < E) ? 1 : 0;
    const float tau = p.gate_temperature > 0.0f ? p.gate_temperature : 1.0f;  // 0: plain softmax
    int64_t cap_rows = (int64_t)T * k;
    if ((int64_t)E * C < cap_rows) cap_rows = (int64_t)E * C;
    if (nb == 1) {
        hipLaunchKernelGGL(dispatch_single, dim3(1), dim3(kThreads), 0, st, r.cand, r.cand_score, T, E, k,
                           (int)C, use_fb, p.aux_coef, tau, (int)cap_rows, ws.hist, ws.fill_prim, ws.fb_hist, r.eid,
                           r.pos, r.flag, r.row, r.gate, r.offsets, r.token_of_row, r.demand, r.kept, r.totals,
                           r.aux_loss, ws.gate_of_row, ws.claim);
    } else {
        hipLaunchKernelGGL(dispatch_hist, dim3(nb), dim3(kThreads), 0, st, r.cand, T, E, k, ws.hist, ws.claim);
        hipLaunchKernelGGL(dispatch_primary, dim3(nb), dim3(kThreads), 0, st, r.cand, T, E, k, (int)C,
                           nb, use_fb, ws.hist, ws.fill_prim, r.eid, r.pos, r.flag, ws.fb_hist);
        hipLaunchKernelGGL(dispatch_finalize, dim3(nb), dim3(kThreads), 0, st, r.cand, r.cand_score, T,
                           E, k, (int)C, nb, use_fb, p.aux_coef, tau, (int)cap_rows, ws.hist, ws.fill_prim,
                           ws.fb_hist, r.eid, r.pos, r.flag, r.row, r.gate, r.offsets, r.token_of_row,
                           r.demand, r.kept, r.totals, r.aux_loss, ws.gate_of_row);
    }
    if (T > 0 && x_perm) {
        const int esz = p.dtype == MOE_BF16 ? 2 : 4;
        const int chunks = p.d * esz / 16;
        hipLaunchKernelGGL(dispatch_gather, dim3(T), dim3(256), 0, st,
                           static_cast<const uint4 *>(x), r.row, k, chunks,
                           static_cast<uint4 *>(x_perm));
    }
    return hipGetLastError();
}

}  // namespace moe
