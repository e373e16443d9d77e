// Stage 1: router GEMM + bias + load penalty + top-(k+1) ranking, one kernel.
//
// What it computes ("MoE架构揭秘" §3.1; "GPT-4稀疏激活真相" §2.3):
//   raw[t][e] = sum_i x[t][i] * Wr[e][i] + bias[e]
//   s[t][e]   = fmaf(-lambda, load[e], raw[t][e])      (raw when load == NULL)
//   cand[t]   = the k+1 experts with the largest s, ties to the lower index;
//               with the top-2 gap threshold, ranks 1 and 2 swapped where
//               s[rank 0] - s[rank 1] < gap (the adg.csdn.net page, §3.1).
//
// Mapping on CDNA4.  The router is a skinny GEMM (N = E is 1..256) and one
// pass over x.  bf16 layers with E <= 64 run it on the matrix cores
// (route_mfma, below).  Otherwise (fp32 layers, more experts) it runs on the
// vector ALU: a wave owns TPW tokens and holds their x rows
// in registers, 16-byte chunks strided over the 64 lanes.  The gate vectors
// are staged in LDS in chunks of experts and read conflict-free (consecutive
// lanes read consecutive 16-byte chunks).  bf16 products are accumulated with
// v_dot2_f32_bf16.  Each lane ends with 32 partial sums (TPW tokens x EA
// experts); a butterfly reduce-scatter over the 64 lanes (DPP inside rows of
// 16, the gfx950 lane swaps across rows) leaves one full sum per lane pair, so the
// cross-lane cost is one shuffle per logit.  Ranking is k+1 wave max
// reductions of a 64-bit key (order-preserving score bits with NaN lowest,
// then the inverted expert index), also DPP / lane-swap butterflies.
//
// The penalty is an explicit fmaf and the file is built without fast-math, so
// the fp32 ranking is reproducible from the fp32 logits bit for bit.
#include <type_traits>

#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouteThreads = 512;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kRouteLdsW = 64 * 1024;  // bytes of gate vectors staged per chunk

template <typename TIn>
struct ChunkDot;

// 16-byte chunk = 8 bf16
template <>
struct ChunkDot<uint16_t> {
    static constexpr int kVec = 8;
    __device__ static __forceinline__ float dot(uint4 a, uint4 b, float acc) {
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x), __builtin_bit_cast(bf16x2_t, b.x), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y), __builtin_bit_cast(bf16x2_t, b.y), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z), __builtin_bit_cast(bf16x2_t, b.z), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w), __builtin_bit_cast(bf16x2_t, b.w), acc, false);
        return acc;
    }
    __device__ static __forceinline__ float widen(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
};

// 16-byte chunk = 4 fp32
template <>
struct ChunkDot<float> {
    static constexpr int kVec = 4;
    __device__ static __forceinline__ float widen(float v) { return v; }
    __device__ static __forceinline__ float dot(uint4 a, uint4 b, float acc) {
        acc = __builtin_fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
        acc = __builtin_fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
        acc = __builtin_fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
        acc = __builtin_fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
        return acc;
    }
};

// Exchange across 32 or 16 lanes with the gfx950 lane-swap instructions:
// for a pair (a, b) they leave a' = a and b' = b of the partner half, so
// that a' + b' is a reduce-scatter step (a lane whose STEP bit is clear
// gets a[l] + a[l ^ STEP], a lane whose bit is set b[l ^ STEP] + b[l]).
// VALU only, no LDS round trip.
template <int STEP>
__device__ __forceinline__ void swap_halves(uint32_t &a, uint32_t &b) {
    static_assert(STEP == 16 || STEP == 32, "lane-swap steps");
    if constexpr (STEP == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
        a = r[0];
        b = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
        a = r[0];
        b = r[1];
    }
}

// One butterfly reduce-scatter step: the lane keeps half of its V values
// (the upper half when its STEP bit is set) and adds the partner's copy.
template <int STEP, int V, int N>
__device__ __forceinline__ void rs_step(float (&v)[N], int lane) {
    if constexpr (STEP >= 16) {
#pragma unroll
        for (int i = 0; i < V / 2; i++) {
            uint32_t a = __float_as_uint(v[i]), b = __float_as_uint(v[i + V / 2]);
            swap_halves<STEP>(a, b);
            v[i] = __uint_as_float(a) + __uint_as_float(b);
        }
    } else {
        const bool upper = (lane & STEP) != 0;
#pragma unroll
        for (int i = 0; i < V / 2; i++) {
            float send = upper ? v[i] : v[i + V / 2];
            float keep = upper ? v[i + V / 2] : v[i];
            v[i] = keep + exch_f32<STEP>(send);
        }
    }
}

// Ranking key of (score, expert): a larger key ranks higher.  The high word
// is an order-preserving map of the fp32 score onto uint32, with -0 and +0
// merged (equal scores) and every NaN placed below -inf, so the order is total
// and every rank below E names an expert even when a row's logits are NaN.
// The low word is the inverted expert index, so among equal scores the lower
// index has the larger key.  Key 0 means "no expert".
__device__ __forceinline__ uint64_t rank_key(float s, int e) {
    const uint32_t u = s == 0.0f ? 0u : __float_as_uint(s);
    uint32_t k = (u >> 31) ? ~u : (u | 0x80000000u);
    k = s != s ? 0u : k;
    return ((uint64_t)k << 32) | (uint32_t)~e;
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int STEP>
__device__ __forceinline__ uint64_t max_step(uint64_t v) {
    if constexpr (STEP >= 16) {
        uint32_t lo0 = (uint32_t)v, lo1 = lo0, hi0 = (uint32_t)(v >> 32), hi1 = hi0;
        swap_halves<STEP>(lo0, lo1);  // (own half, partner half) in some order
        swap_halves<STEP>(hi0, hi1);
        return max_u64(((uint64_t)hi0 << 32) | lo0, ((uint64_t)hi1 << 32) | lo1);
    } else {
        const uint32_t lo = (uint32_t)exch_i32<STEP>((int)(uint32_t)v);
        const uint32_t hi = (uint32_t)exch_i32<STEP>((int)(uint32_t)(v >> 32));
        return max_u64(v, ((uint64_t)hi << 32) | lo);
    }
}

// Write-out of one token's ranked candidates with the top-2 gap threshold
// (the adg.csdn.net page, §3.1): ranks 0-2 are held until the third is known;
// where the best two scores differ by less than `gap` (their fp32
// difference) and the third candidate names an expert, ranks 1 and 2 trade
// places, so the second choice is the third-ranked expert and the displaced
// one becomes the fallback.  gap <= 0 leaves the ranking as it is.  All lanes
// hold the same values; only `writer` stores.
struct RankOut {
    int c0 = -1, c1 = -1, c2 = -1;
    float s0 = -INFINITY, s1 = -INFINITY, s2 = -INFINITY;
    __device__ __forceinline__ void put(int r, int c, float sc, int32_t *cand_t, float *cs_t, bool writer) {
        if (r == 0) {
            c0 = c;
            s0 = sc;
        } else if (r == 1) {
            c1 = c;
            s1 = sc;
        } else if (r == 2) {
            c2 = c;
            s2 = sc;
        } else if (writer) {
            cand_t[r] = c;
            cs_t[r] = sc;
        }
    }
    __device__ __forceinline__ void flush(int K1, float gap, int32_t *cand_t, float *cs_t, bool writer) {
        if (gap > 0.0f && K1 >= 3 && c2 >= 0 && s0 - s1 < gap) {
            const int c = c1;
            const float sc = s1;
            c1 = c2;
            s1 = s2;
            c2 = c;
            s2 = sc;
        }
        if (writer) {
            cand_t[0] = c0;
            cs_t[0] = s0;
            cand_t[1] = c1;  // K1 >= 2 (k >= 1)
            cs_t[1] = s1;
            if (K1 >= 3) {
                cand_t[2] = c2;
                cs_t[2] = s2;
            }
        }
    }
};

typedef __attribute__((address_space(3))) char lds_char_t;
typedef const __attribute__((address_space(1))) char gbl_char_t;

// Stage `bytes` of gate vectors (a contiguous range of W rows) into `dst`
// with direct global -> LDS loads: wave w moves the 1 KiB pieces w, w+8, ...
// (lanes past the end re-read the last 16 bytes; `dst` has room for whole
// pieces).  No registers are involved and nothing waits here.
__device__ __forceinline__ void stage_w(const char *src, int bytes, char *dst, int wave, int lane) {
    const int pieces = (bytes + 1023) >> 10;
    for (int i = wave; i < pieces; i += kRouteWaves) {
        const int off = min(i * 1024 + lane * 16, bytes - 16);
        __builtin_amdgcn_global_load_lds((gbl_char_t *)(src + off), (lds_char_t *)(dst + i * 1024), 16, 0, 0);
    }
}

// Butterfly reduce-scatter of V partial sums per lane over the 64 lanes: the
// value set halves at steps 32, 16, ... until one value is left, then plain
// butterfly adds finish the sum.  Lane l ends with the full sum of value
// (l >> (6 - log2 V)) & (V - 1).
template <int V>
__device__ __forceinline__ float reduce_scatter(float (&v)[V], int lane) {
    static_assert(V == 8 || V == 16 || V == 32, "8, 16 or 32 values per lane");
    rs_step<32, V>(v, lane);
    rs_step<16, V / 2>(v, lane);
    rs_step<8, V / 4>(v, lane);
    if constexpr (V >= 16) rs_step<4, V / 8>(v, lane);
    else v[0] += exch_f32<4>(v[0]);
    if constexpr (V >= 32) rs_step<2, 2>(v, lane);
    else v[0] += exch_f32<2>(v[0]);
    return v[0] + exch_f32<1>(v[0]);
}

// Logits of experts [e0, e0 + ec) for this wave's TPW tokens from the gate
// vectors staged at w_lds, written to lg[token][expert].  Per group of EA
// experts: all NX gate-vector chunks of one expert are read from LDS first,
// then used for the TPW tokens held in registers (no lane-dependent
// branches: x chunks past the row end are zero, so the gate-vector read is
// simply clamped).  The TPW x EA partial sums per lane then go through one
// butterfly reduce-scatter (EA is the smallest power of two that holds the
// experts, up to 32 / TPW, so no shuffle carries an empty slot).
template <typename TIn, int NX, int TPW, int EA>
__device__ __forceinline__ void route_chunk(const uint4 *w_lds, const uint4 (&xr)[TPW][NX], int nchunk, int e0,
                                            int ec, const float *__restrict__ bias, float *lg, int E, int lane) {
    constexpr int V = TPW * EA;
    constexpr int kShift = V == 32 ? 1 : V == 16 ? 2 : 3;
    for (int ea = 0; ea < ec; ea += EA) {
        float v[V];
#pragma unroll
        for (int i = 0; i < V; i++) v[i] = 0.0f;
#pragma unroll
        for (int q = 0; q < EA; q++) {
            if (ea + q < ec) {  // wave-uniform
                const uint4 *wrow = w_lds + (size_t)(ea + q) * nchunk;
                uint4 w[NX];
#pragma unroll
                for (int c = 0; c < NX; c++) w[c] = wrow[min(lane + 64 * c, nchunk - 1)];
#pragma unroll
                for (int c = 0; c < NX; c++)
#pragma unroll
                    for (int j = 0; j < TPW; j++) v[j * EA + q] = ChunkDot<TIn>::dot(xr[j][c], w[c], v[j * EA + q]);
            }
        }
        const float sum = reduce_scatter<V>(v, lane);
        const int idx = (lane >> kShift) & (V - 1);
        const int j = idx / EA, q = idx % EA;
        const int e = e0 + ea + q;
        if ((lane & ((1 << kShift) - 1)) == 0 && ea + q < ec) {
            float r = sum;
            if (bias) r = r + bias[e];
            lg[j * E + e] = r;
        }
    }
}

// NX: 16-byte chunks of one x row per lane; TPW: tokens per wave; NB: W
// buffers (1 when all E gate vectors fit one chunk, else 2: the next chunk
// streams in while the current one is used); EA: experts per reduce-scatter
// group; EMAX: bound on E that sizes the logit buffer (a small one leaves
// room for two blocks per CU) and the experts per lane of the ranking.
// H > 0: the two-layer router.  wr holds W1 [H][d] followed by W2 [E][H];
// bias (or NULL) holds the H first-layer biases, then the E second-layer
// ones.  The dot loop computes the H hidden pre-activations (as it computes
// the E logits of the linear router); silu and the second layer follow,
// with W2 staged transposed in LDS in chunks of hidden units (fp32, hidden
// units in ascending order).  H <= EMAX.
template <typename TIn, int NX, int TPW, int NB, int EA, int EMAX>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const TIn *__restrict__ x, const TIn *__restrict__ wr, const float *__restrict__ bias,
    const float *__restrict__ load, float neg_lambda, float gap, int T, int d, int E, int K1, int EC, int H,
    float *__restrict__ logits, int32_t *__restrict__ cand, float *__restrict__ cand_score) {
    constexpr int kVec = ChunkDot<TIn>::kVec;
    // two distinct objects, so the compiler sees that the loads into one
    // buffer never alias the reads of the other
    __shared__ __attribute__((aligned(1024))) char w_buf0[kRouteLdsW];
    __shared__ __attribute__((aligned(1024))) char w_buf1[NB == 2 ? kRouteLdsW : 1024];
    __shared__ float lg_all[kRouteWaves * TPW * EMAX];
    constexpr int PL = (EMAX + 63) / 64;  // experts per lane in the ranking
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nchunk = d / kVec;
    const int row_bytes = d * (int)sizeof(TIn);
    const int t0 = (blockIdx.x * kRouteWaves + wave) * TPW;
    const int NO = H > 0 ? H : E;         // outputs of the dot loop
    float *lg = lg_all + wave * TPW * EMAX;  // [TPW][NO], then [TPW][E]

    // this wave's x rows, 16-byte chunks lane + 64 c (zero past the row end)
    uint4 xr[TPW][NX];
#pragma unroll
    for (int j = 0; j < TPW; j++) {
        const int t = t0 + j;
#pragma unroll
        for (int c = 0; c < NX; c++) {
            const int ci = lane + 64 * c;
            if (t < T && ci < nchunk)
                xr[j][c] = reinterpret_cast<const uint4 *>(x + (size_t)t * d)[ci];
            else
                xr[j][c] = make_uint4(0, 0, 0, 0);
        }
    }

    const char *wsrc = reinterpret_cast<const char *>(wr);
    stage_w(wsrc, min(EC, NO) * row_bytes, w_buf0, wave, lane);
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __syncthreads();
    // chunks of EC experts (hidden units), alternating buffers (unrolled by
    // two so each use names a fixed buffer); the next chunk streams in
    // during the use
    for (int e0 = 0; e0 < NO; e0 += 2 * EC) {
        if (NB == 2 && e0 + EC < NO)
            stage_w(wsrc + (size_t)(e0 + EC) * row_bytes, min(EC, NO - e0 - EC) * row_bytes, w_buf1, wave, lane);
        route_chunk<TIn, NX, TPW, EA>(reinterpret_cast<const uint4 *>(w_buf0), xr, nchunk, e0, min(EC, NO - e0),
                                  bias, lg, NO, lane);
        __builtin_amdgcn_s_waitcnt(0x0070);
        __syncthreads();
        if (NB == 1 || e0 + EC >= NO) break;
        if (e0 + 2 * EC < NO)
            stage_w(wsrc + (size_t)(e0 + 2 * EC) * row_bytes, min(EC, NO - e0 - 2 * EC) * row_bytes, w_buf0,
                    wave, lane);
        route_chunk<TIn, NX, TPW, EA>(reinterpret_cast<const uint4 *>(w_buf1), xr, nchunk, e0 + EC,
                                  min(EC, NO - e0 - EC), bias, lg, NO, lane);
        __builtin_amdgcn_s_waitcnt(0x0070);
        __syncthreads();
    }

    if (H > 0) {
        // silu of this wave's hidden pre-activations, in place
        for (int i = lane; i < TPW * H; i += 64) {
            const float v = lg[i];
            lg[i] = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
        }
        // second layer: lane e (+ 64 i) of every token; W2 chunks of HC hidden
        // units staged transposed ([HC][E] fp32: the lanes read consecutive
        // words) by the whole block
        const TIn *w2 = wr + (size_t)H * d;
        float *w2t = reinterpret_cast<float *>(w_buf0);
        const int HC = kRouteLdsW / (E * (int)sizeof(float));  // >= 64 (E <= 256)
        float acc2[TPW][PL];
#pragma unroll
        for (int j = 0; j < TPW; j++)
#pragma unroll
            for (int i = 0; i < PL; i++) acc2[j][i] = 0.0f;
        for (int h0 = 0; h0 < H; h0 += HC) {
            const int hn = min(HC, H - h0);
            __syncthreads();  // the previous chunk has been read by every wave
            for (int i = threadIdx.x; i < hn * E; i += kRouteThreads) {
                const int hh = i / E, e = i - hh * E;
                w2t[i] = ChunkDot<TIn>::widen(w2[(size_t)e * H + h0 + hh]);
            }
            __syncthreads();
            for (int hh = 0; hh < hn; hh++) {
                float hv[TPW];
#pragma unroll
                for (int j = 0; j < TPW; j++) hv[j] = lg[j * H + h0 + hh];
#pragma unroll
                for (int i = 0; i < PL; i++) {
                    const int e = lane + 64 * i;
                    const float w = e < E ? w2t[hh * E + e] : 0.0f;
#pragma unroll
                    for (int j = 0; j < TPW; j++) acc2[j][i] = __builtin_fmaf(hv[j], w, acc2[j][i]);
                }
            }
        }
        // the logits, [TPW][E], over the hidden values (every read of them is done)
#pragma unroll
        for (int j = 0; j < TPW; j++)
#pragma unroll
            for (int i = 0; i < PL; i++) {
                const int e = lane + 64 * i;
                if (e < E) lg[j * E + e] = bias ? acc2[j][i] + bias[H + e] : acc2[j][i];
            }
    }

    // ranking: lanes hold experts e = lane + 64 * i; each round is one wave
    // max of the ranking keys, and the winner's key is cleared
    for (int j = 0; j < TPW; j++) {
        const int t = t0 + j;
        if (t >= T) break;  // wave-uniform
        float sc[PL];
        uint64_t key[PL];
#pragma unroll
        for (int i = 0; i < PL; i++) {
            const int e = lane + 64 * i;
            sc[i] = 0.0f;
            key[i] = 0;
            if (e < E) {
                const float raw = lg[j * E + e];
                logits[(size_t)t * E + e] = raw;
                sc[i] = load ? __builtin_fmaf(neg_lambda, load[e], raw) : raw;
                key[i] = rank_key(sc[i], e);
            }
        }
        RankOut ro;
        for (int r = 0; r < K1; r++) {
            uint64_t m = key[0];
#pragma unroll
            for (int i = 1; i < PL; i++) m = max_u64(m, key[i]);
            m = max_step<1>(m);
            m = max_step<2>(m);
            m = max_step<4>(m);
            m = max_step<8>(m);
            m = max_step<16>(m);
            m = max_step<32>(m);
            const bool none = m == 0;
            const int e = __builtin_amdgcn_readfirstlane((int)~(uint32_t)m);
            // the winner's own score (its sign of zero and NaN bits), from its lane
            float s = sc[0];
#pragma unroll
            for (int i = 1; i < PL; i++) s = (e >> 6) == i ? sc[i] : s;
            s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), e & 63));
            ro.put(r, none ? -1 : e, none ? -INFINITY : s, cand + (size_t)t * K1, cand_score + (size_t)t * K1,
                   lane == 0);
#pragma unroll
            for (int i = 0; i < PL; i++)
                if (!none && (e & 63) == lane && (e >> 6) == i) key[i] = 0;
        }
        ro.flush(K1, gap, cand + (size_t)t * K1, cand_score + (size_t)t * K1, lane == 0);
    }
}

template <typename TIn, int NX, int TPW, int EA, int EMAX>
hipError_t launch_k(const moe_params &p, const void *x, const void *wr, const float *bias, const float *load,
                    float *logits, int32_t *cand, float *cand_score, hipStream_t st) {
    const int row_bytes = p.d * (int)sizeof(TIn);
    const int NO = p.router_hidden > 0 ? p.router_hidden : p.E;  // outputs of the dot loop
    int ec = kRouteLdsW / row_bytes;  // experts (hidden units) staged per LDS chunk
    if (ec < 1) ec = 1;
    if (ec > NO) ec = NO;
    const int tokens_per_block = kRouteWaves * TPW;
    const int grid = (int)ceil_div(p.T, tokens_per_block);
#define MOE_ROUTE_LAUNCH(NB)                                                                                  \
    hipLaunchKernelGGL((route_kernel<TIn, NX, TPW, NB, EA, EMAX>), dim3(grid), dim3(kRouteThreads), 0, st,    \
                       static_cast<const TIn *>(x), static_cast<const TIn *>(wr), bias, load, -p.lambda,    \
                       p.top2_gap, p.T,                                                                      \
                       p.d, p.E, p.k + 1, ec, p.router_hidden, logits, cand, cand_score)
    if (ec >= NO) MOE_ROUTE_LAUNCH(1);
    else MOE_ROUTE_LAUNCH(2);
#undef MOE_ROUTE_LAUNCH
    return hipGetLastError();
}

// SPEC: instantiate the expert-count classes (E <= 8, 16, 32 with one token
// per wave; E <= 64); otherwise one variant that serves every E <= 256.
template <typename TIn, int NX, int TPW, bool SPEC>
hipError_t launch_t(const moe_params &p, const void *x, const void *wr, const float *bias,
                    const float *load, float *logits, int32_t *cand, float *cand_score,
                    hipStream_t st) {
    constexpr int kEA = 32 / TPW;
    // the two-layer router: the hidden units and the experts both fit 256
    if (p.router_hidden > 0)
        return launch_k<TIn, NX, TPW, kEA, kMaxExperts>(p, x, wr, bias, load, logits, cand, cand_score, st);
    if constexpr (SPEC) {
        if constexpr (TPW == 1) {  // the only tokens-per-wave count used for E <= 32
            if (p.E <= 8) return launch_k<TIn, NX, 1, 8, 32>(p, x, wr, bias, load, logits, cand, cand_score, st);
            if (p.E <= 16) return launch_k<TIn, NX, 1, 16, 32>(p, x, wr, bias, load, logits, cand, cand_score, st);
            if (p.E <= 32) return launch_k<TIn, NX, 1, 32, 32>(p, x, wr, bias, load, logits, cand, cand_score, st);
        }
        if (p.E <= 64) return launch_k<TIn, NX, TPW, kEA, 64>(p, x, wr, bias, load, logits, cand, cand_score, st);
    }
    return launch_k<TIn, NX, TPW, kEA, kMaxExperts>(p, x, wr, bias, load, logits, cand, cand_score, st);
}

// Tokens per wave.  Up to 32 experts, one: the logit buffer is then small,
// two blocks share a CU, and one block's loads overlap the other's dot
// products (measured faster at every T).  With more experts the dot loop is
// bound by the VALU and the LDS reads of the gate vectors, which TPW tokens
// share: up to 4, fewer when that would leave compute units without a block.
template <typename TIn, int NX>
hipError_t launch_nx(const moe_params &p, const void *x, const void *wr, const float *bias,
                     const float *load, float *logits, int32_t *cand, float *cand_score, hipStream_t st) {
    constexpr int kCUs = 256;
    constexpr bool kSpec = std::is_same<TIn, uint16_t>::value && (NX == 4 || NX == 8);
    if (kSpec && p.E <= 32) return launch_t<TIn, NX, 1, kSpec>(p, x, wr, bias, load, logits, cand, cand_score, st);
    if (p.T >= kCUs * kRouteWaves * 4)
        return launch_t<TIn, NX, 4, kSpec>(p, x, wr, bias, load, logits, cand, cand_score, st);
    if (p.T >= kCUs * kRouteWaves * 2)
        return launch_t<TIn, NX, 2, kSpec>(p, x, wr, bias, load, logits, cand, cand_score, st);
    return launch_t<TIn, NX, 1, kSpec>(p, x, wr, bias, load, logits, cand, cand_score, st);
}

// ------------------------------------------------------------ MFMA router --
// bf16 layers with E <= 64 run the router GEMM on the matrix cores (and so
// does the two-layer router, whose first layer has at most 64 outputs).  A block
// owns BT = 16 NT tokens and every expert; its 4 waves split the hidden
// dimension into 64-element slabs (one 128-byte line of a row), wave w taking
// slabs w, w + 4, ... in an order rotated per block (so that the blocks
// resident at one time read different columns of x and W, not all the same
// HBM channels and L2 lines).  Each wave streams its slabs through a private
// ring of P LDS slots with direct global -> LDS loads: one load moves eight
// whole 128-byte lines (x rows of the block, then W rows; rows past the block's
// tokens or past E read nothing and write zeros), so the accesses coalesce,
// which loads straight into the MFMA register layout (16 rows per load) do
// not.  No barrier is needed in the loop: a wave reads only what it loaded.
// MFMA 16x16x32 bf16 on fragments read from the slot through the XOR
// swizzle; in k step i of a slab, lane l takes row l % 16 and 16-byte chunk
// 4 i + l / 16 (x and W alike).  The four waves' fp32 partials are added in
// LDS in wave order, then the bias, the penalty and the top-(k+1) ranking,
// with 64 / G tokens ranked at once in groups of G lanes.
constexpr int kRmThreads = 256;
constexpr int kRmWaves = kRmThreads / 64;
constexpr int kSlabBytes = 128;


__device__ __forceinline__ void rt_buf2lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, char *dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_char_t *)dst, 16, voff, soff, 0, 0);
}

template <int NT, int NE, int P, int G>
__global__ __launch_bounds__(kRmThreads) void route_mfma(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr, const float *__restrict__ bias,
    const float *__restrict__ load, float neg_lambda, float gap, int T, int d, int E, int K1, int H,
    float *__restrict__ logits, int32_t *__restrict__ cand, float *__restrict__ cand_score) {
    // H > 0: two-layer router; wr holds W1 [H][d] followed by W2 [E][H], the
    // MFMA GEMM computes the H hidden pre-activations, the epilogue the rest
    constexpr int BT = 16 * NT, EP = 16 * NE, TPP = 64 / G;
    constexpr int kXG = BT / 8, kWG = EP / 8, L = kXG + kWG;  // 1 KiB loads per slab
    constexpr int kSlot = L * 1024;                           // one wave's slab
    static_assert(G == 8 || G == 16 || G == 32 || G == 64, "ranking group");
    static_assert(P >= 2 && P <= 8 && (P - 1) * L <= 63, "ring depth");
    static_assert(kRmWaves * BT * EP * 4 <= kRmWaves * kSlot, "partials fit the first slot");
    __shared__ __attribute__((aligned(1024))) char s0[kRmWaves * kSlot];
    __shared__ __attribute__((aligned(1024))) char s1[kRmWaves * kSlot];
    __shared__ __attribute__((aligned(1024))) char s2[P > 2 ? kRmWaves * kSlot : 16];
    __shared__ __attribute__((aligned(1024))) char s3[P > 3 ? kRmWaves * kSlot : 16];
    __shared__ __attribute__((aligned(1024))) char s4[P > 4 ? kRmWaves * kSlot : 16];
    __shared__ __attribute__((aligned(1024))) char s5[P > 5 ? kRmWaves * kSlot : 16];
    __shared__ __attribute__((aligned(1024))) char s6[P > 6 ? kRmWaves * kSlot : 16];
    __shared__ __attribute__((aligned(1024))) char s7[P > 7 ? kRmWaves * kSlot : 16];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    auto slot = [&](int sl) -> char * {
        char *b = sl == 0 ? s0 : sl == 1 ? s1 : sl == 2 ? s2 : sl == 3 ? s3 : sl == 4 ? s4 : sl == 5 ? s5 : sl == 6 ? s6 : s7;
        return b + wave * kSlot;
    };
    const int t0 = blockIdx.x * BT;
    const int nt = min(BT, T - t0);
    const uint32_t row_bytes = (uint32_t)d * 2;
    const auto xs = make_rsrc(x + (size_t)t0 * d, (uint32_t)nt * row_bytes);
    const int NO = H > 0 ? H : E;  // rows of the matrix the MFMAs multiply by
    const auto ws = make_rsrc(wr, (uint32_t)NO * row_bytes);
    // load group gi moves rows 8 gi .. 8 gi + 7 of the slot (x rows, then W
    // rows); lane l fetches chunk (l % 8) ^ swz(row) of row 8 gi + l / 8, so
    // LDS chunk c of a row holds the row's chunk c ^ swz(row)
    uint32_t voff[L];
#pragma unroll
    for (int gi = 0; gi < L; gi++) {
        const int row = 8 * (gi < kXG ? gi : gi - kXG) + (lane >> 3);
        const int lim = gi < kXG ? nt : NO;
        voff[gi] = row < lim ? row * row_bytes + (((lane & 7) ^ swz(8 * gi + (lane >> 3))) << 4) : kPastEnd;
    }

    const int nslab = d / 64;
    const int mine = (nslab - wave + kRmWaves - 1) / kRmWaves;  // slabs of this wave
    const int rot = mine > 0 ? (int)(((blockIdx.x >> 3) + (blockIdx.x & 7) * 2) % (unsigned)mine) : 0;
    // slab j of this wave (past its last slab every load is out of range and
    // writes zeros, so the compute needs no branch)
    auto issue = [&](int j, char *dst) {
        const bool v = j < mine;
        int jj = j + rot;
        jj = jj >= mine ? jj - mine : jj;
        const uint32_t so = v ? (uint32_t)(wave + kRmWaves * jj) * kSlabBytes : 0u;
#pragma unroll
        for (int gi = 0; gi < L; gi++)
            rt_buf2lds(gi < kXG ? xs : ws, v ? voff[gi] : kPastEnd, so, dst + gi * 1024);
    };
    const int r16 = lane & 15, q = lane >> 4;
    f32x4_t acc[NT][NE];
#pragma unroll
    for (int f = 0; f < NT; f++)
#pragma unroll
        for (int g = 0; g < NE; g++) acc[f][g] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    auto compute = [&](const char *src) {
#pragma unroll
        for (int i = 0; i < 2; i++) {
            uint4 a[NT], b[NE];
#pragma unroll
            for (int f = 0; f < NT; f++) {
                const int row = 16 * f + r16;
                a[f] = *reinterpret_cast<const uint4 *>(src + row * kSlabBytes + (((4 * i + q) ^ swz(row)) << 4));
            }
#pragma unroll
            for (int g = 0; g < NE; g++) {
                const int row = BT + 16 * g + r16;
                b[g] = *reinterpret_cast<const uint4 *>(src + row * kSlabBytes + (((4 * i + q) ^ swz(row)) << 4));
            }
#pragma unroll
            for (int f = 0; f < NT; f++)
#pragma unroll
                for (int g = 0; g < NE; g++)
                    acc[f][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[f]),
                                                                       __builtin_bit_cast(bf16x8_t, b[g]), acc[f][g],
                                                                       0, 0, 0);
        }
    };
#pragma unroll
    for (int sl = 0; sl < P; sl++) issue(sl, slot(sl));
    // P slabs per loop iteration (slab j sits in slot j % P; when it is
    // used, the P - 1 later slabs may still be in flight); slabs past the
    // wave's last one, at most P - 1, are zeros
    for (int j0 = 0; j0 < mine; j0 += P) {
#pragma unroll
        for (int u = 0; u < P; u++) {
            WAIT_VMCNT((P - 1) * L);
            compute(slot(u));
            __builtin_amdgcn_sched_barrier(0);
            issue(j0 + u + P, slot(u));
        }
    }
    WAIT_VMCNT(0);  // the ring is reused below; no load may still write it
    __syncthreads();

    // the lane holds expert 16 g + lane % 16 of tokens 16 f + 4 (lane / 16) + c
    float(*part)[BT][EP] = reinterpret_cast<float(*)[BT][EP]>(s0);
#pragma unroll
    for (int f = 0; f < NT; f++)
#pragma unroll
        for (int g = 0; g < NE; g++)
#pragma unroll
            for (int c = 0; c < 4; c++) part[wave][16 * f + 4 * q + c][16 * g + r16] = acc[f][g][c];
    __syncthreads();
    float(*sc)[EP] = part[0];  // the scores the ranking reads
    if (H == 0) {
        for (int i = threadIdx.x; i < nt * E; i += kRmThreads) {
            const int t = i / E, e = i - t * E;
            float raw = ((part[0][t][e] + part[1][t][e]) + part[2][t][e]) + part[3][t][e];
            if (bias) raw = raw + bias[e];
            logits[(size_t)(t0 + t) * E + e] = raw;
            part[0][t][e] = load ? __builtin_fmaf(neg_lambda, load[e], raw) : raw;
        }
    } else {
        // hidden activations silu(sum of the partials + first-layer bias)
        // into part[0]; W2 as fp32 into the (now idle) second ring slot.
        // bias holds the H first-layer biases, then the E second-layer ones.
        for (int i = threadIdx.x; i < nt * H; i += kRmThreads) {
            const int t = i / H, j = i - t * H;
            float v = ((part[0][t][j] + part[1][t][j]) + part[2][t][j]) + part[3][t][j];
            if (bias) v = v + bias[j];
            part[0][t][j] = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
        }
        // (stored transposed, [H][E]: the lanes of a wave take consecutive
        // experts, so they read consecutive words, not one bank H apart)
        float *w2l = reinterpret_cast<float *>(s1);
        const uint16_t *w2 = wr + (size_t)H * d;
        for (int i = threadIdx.x; i < E * H; i += kRmThreads) {
            const int j = i / E, e = i - j * E;
            w2l[i] = __uint_as_float((uint32_t)w2[(size_t)e * H + j] << 16);
        }
        __syncthreads();
        // raw = a . W2^T + bias, j ascending in fp32, into part[1]
        for (int i = threadIdx.x; i < nt * E; i += kRmThreads) {
            const int t = i / E, e = i - t * E;
            float acc = 0.0f;
            for (int j = 0; j < H; j++) acc = __builtin_fmaf(part[0][t][j], w2l[j * E + e], acc);
            if (bias) acc = acc + bias[H + e];
            logits[(size_t)(t0 + t) * E + e] = acc;
            part[1][t][e] = load ? __builtin_fmaf(neg_lambda, load[e], acc) : acc;
        }
        sc = part[1];
    }
    __syncthreads();

    // ranking: groups of G lanes, one token each; lane e of a group holds
    // expert e; each round is a group max of the ranking keys, and the
    // winner's key is cleared
    const int e = lane & (G - 1);
    for (int base = wave * TPP; base < nt; base += kRmWaves * TPP) {
        const int t = base + lane / G;  // < BT
        const bool ok = t < nt && e < E;
        uint64_t key = ok ? rank_key(sc[t][e], e) : 0;
        const size_t to = (size_t)(t0 + min(t, nt - 1)) * K1;  // this group's token's candidate row
        const bool writer = e == 0 && t < nt;
        RankOut ro;
        for (int r = 0; r < K1; r++) {
            uint64_t m = max_step<1>(key);
            m = max_step<2>(m);
            m = max_step<4>(m);
            if constexpr (G >= 16) m = max_step<8>(m);
            if constexpr (G >= 32) m = max_step<16>(m);
            if constexpr (G >= 64) m = max_step<32>(m);
            const bool none = m == 0;
            const int we = none ? 0 : (int)~(uint32_t)m;  // the group's winner
            const float sw = sc[t][we];                    // its own score bits
            ro.put(r, none ? -1 : we, none ? -INFINITY : sw, cand + to, cand_score + to, writer);
            if (!none && e == we) key = 0;
        }
        ro.flush(K1, gap, cand + to, cand_score + to, writer);
    }
}

template <int NT, int NE, int G>
hipError_t launch_mfma_g(const moe_params &p, const void *x, const void *wr, const float *bias, const float *load,
                         float *logits, int32_t *cand, float *cand_score, hipStream_t st) {
    // ring depth: as many slots as 144 KiB of LDS holds (4 waves, one slab
    // of BT x rows and 16 NE W rows each), at most 8
    constexpr int kSlotBlock = 4 * (2 * NT + 2 * NE) * 1024;
    constexpr int P = 144 * 1024 / kSlotBlock > 8 ? 8 : 144 * 1024 / kSlotBlock;
    const int grid = (int)ceil_div(p.T, 16 * NT);
    hipLaunchKernelGGL((route_mfma<NT, NE, P, G>), dim3(grid), dim3(kRmThreads), 0, st,
                       static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(wr), bias, load, -p.lambda,
                       p.top2_gap, p.T, p.d, p.E, p.k + 1, p.router_hidden, logits, cand, cand_score);
    return hipGetLastError();
}

template <int NT>
hipError_t launch_mfma_nt(const moe_params &p, const void *x, const void *wr, const float *bias, const float *load,
                          float *logits, int32_t *cand, float *cand_score, hipStream_t st) {
    if (p.router_hidden > 0) {  // two-layer router: up to 64 hidden units, 4 fragments
        if (p.E <= 8) return launch_mfma_g<NT, 4, 8>(p, x, wr, bias, load, logits, cand, cand_score, st);
        if (p.E <= 16) return launch_mfma_g<NT, 4, 16>(p, x, wr, bias, load, logits, cand, cand_score, st);
        if (p.E <= 32) return launch_mfma_g<NT, 4, 32>(p, x, wr, bias, load, logits, cand, cand_score, st);
        return launch_mfma_g<NT, 4, 64>(p, x, wr, bias, load, logits, cand, cand_score, st);
    }
    if (p.E <= 8) return launch_mfma_g<NT, 1, 8>(p, x, wr, bias, load, logits, cand, cand_score, st);
    if (p.E <= 16) return launch_mfma_g<NT, 1, 16>(p, x, wr, bias, load, logits, cand, cand_score, st);
    if (p.E <= 32) return launch_mfma_g<NT, 2, 32>(p, x, wr, bias, load, logits, cand, cand_score, st);
    if (p.E <= 48) return launch_mfma_g<NT, 3, 64>(p, x, wr, bias, load, logits, cand, cand_score, st);
    return launch_mfma_g<NT, 4, 64>(p, x, wr, bias, load, logits, cand, cand_score, st);
}

// 32 tokens per block once that still gives every compute unit a block
// (half the gate-vector reads per token), else 16.
hipError_t launch_mfma(const moe_params &p, const void *x, const void *wr, const float *bias, const float *load,
                       float *logits, int32_t *cand, float *cand_score, hipStream_t st) {
    if (p.T >= 256 * 32) return launch_mfma_nt<2>(p, x, wr, bias, load, logits, cand, cand_score, st);
    return launch_mfma_nt<1>(p, x, wr, bias, load, logits, cand, cand_score, st);
}

template <typename TIn>
hipError_t launch_dtype(const moe_params &p, const void *x, const void *wr, const float *bias,
                        const float *load, float *logits, int32_t *cand, float *cand_score,
                        hipStream_t st) {
    constexpr int kVec = ChunkDot<TIn>::kVec;
    const int nx = (int)ceil_div(p.d / kVec, 64);
    if (nx <= 1) return launch_nx<TIn, 1>(p, x, wr, bias, load, logits, cand, cand_score, st);
    if (nx <= 2) return launch_nx<TIn, 2>(p, x, wr, bias, load, logits, cand, cand_score, st);
    if (nx <= 4) return launch_nx<TIn, 4>(p, x, wr, bias, load, logits, cand, cand_score, st);
    if (nx <= 8) return launch_nx<TIn, 8>(p, x, wr, bias, load, logits, cand, cand_score, st);
    if (nx <= 16) return launch_t<TIn, 16, 2, false>(p, x, wr, bias, load, logits, cand, cand_score, st);
    if (nx <= 32) return launch_t<TIn, 32, 1, false>(p, x, wr, bias, load, logits, cand, cand_score, st);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_route(const moe_params &p, const void *x, const void *wr, const float *bias,
                        const float *load, float *logits, int32_t *cand, float *cand_score,
                        hipStream_t st) {
    if (p.T == 0) return hipSuccess;
    // matrix cores for bf16 layers with at most 64 experts (and, for the
    // two-layer router, at most 64 hidden units); the vector-ALU kernel
    // otherwise
    if (p.dtype == MOE_BF16 && p.E <= 64 && p.router_hidden <= 64)
        return launch_mfma(p, x, wr, bias, load, logits, cand, cand_score, st);
    if (p.dtype == MOE_BF16)
        return launch_dtype<uint16_t>(p, x, wr, bias, load, logits, cand, cand_score, st);
    return launch_dtype<float>(p, x, wr, bias, load, logits, cand, cand_score, st);
}

}  // namespace moe
