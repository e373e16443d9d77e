// Stage 4: gate-weighted combine back to token order.
//
// y[t] = sum over kept slots j of gate[t][j] * y_perm[row[t][j]], accumulated
// in fp32 and rounded once ("企业官网建设流程全解析" page §3, step 5: the
// experts' results are put back in token order; "GPT-4稀疏激活真相" §4.3:
// weighted fusion).  A token with no kept slot gets zeros.
//
// Two sources:
//   * y_perm [R][d] fp32 with the gates applied here (moe_combine, and the
//     fp32 layer's forward pass);
//   * gated rows: fp16 slices holding gate * (partial product of d_ff slice
//     s), written by the down projection's epilogue in a bf16 layer's
//     forward pass.  The combine is then a plain sum of the k rows' slices
//     (slot order, then slice order), read at half the bytes of fp32.  Either
//     every row has S slices ([S][R][d]), or the down projection's split
//     plan holds: slice 0 of every row in [R][d], and slices 1 .. S-1 only
//     for the split rows r >= row0, at rest + ((s - 1) srows + r - row0) d,
//     with {row0, S, srows} read from the plan the down projection stored.
// HBM-bound gather: 16-byte loads and stores, each source row read once.
#include <algorithm>

#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// Each thread produces 8 consecutive outputs and writes 8 bf16 (16 bytes)
// or 8 fp32 (32 bytes).
template <typename TE>
__device__ __forceinline__ void store8(TE *y, const float (&a)[8]);

template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t *y, const float (&a)[8]) {
    *reinterpret_cast<uint4 *>(y) = make_uint4(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                               pack_bf16x2(a[4], a[5]), pack_bf16x2(a[6], a[7]));
}

template <>
__device__ __forceinline__ void store8<float>(float *y, const float (&a)[8]) {
    reinterpret_cast<float4 *>(y)[0] = make_float4(a[0], a[1], a[2], a[3]);
    reinterpret_cast<float4 *>(y)[1] = make_float4(a[4], a[5], a[6], a[7]);
}

// 8 consecutive source elements of one row: fp32 (two 16-byte loads) or
// fp16 (one).
struct Src8f {
    float4 u, v;
};
struct Src8h {
    uint4 u;
};

__device__ __forceinline__ Src8f load8(const float *row, int c) {
    const float4 *p = reinterpret_cast<const float4 *>(row) + 2 * c;
    return Src8f{p[0], p[1]};
}
__device__ __forceinline__ Src8h load8(const uint16_t *row, int c) {
    return Src8h{reinterpret_cast<const uint4 *>(row)[c]};
}

__device__ __forceinline__ void widen8(const Src8f &s, float (&o)[8]) {
    o[0] = s.u.x; o[1] = s.u.y; o[2] = s.u.z; o[3] = s.u.w;
    o[4] = s.v.x; o[5] = s.v.y; o[6] = s.v.z; o[7] = s.v.w;
}
__device__ __forceinline__ void widen8(const Src8h &s, float (&o)[8]) {
    const uint32_t w[4] = {s.u.x, s.u.y, s.u.z, s.u.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        o[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFF));
        o[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
    }
}

template <typename TY>
struct SrcOf;
template <>
struct SrcOf<float> {
    typedef Src8f type;
};
template <>
struct SrcOf<uint16_t> {
    typedef Src8h type;
};

// Generic path (any k <= 8, any slice count): one token row per group of
// threads, the loads of one slot's slices issued together.  GATED: the
// sources are gated fp16 slices and no gate is applied here.
template <typename TE, typename TY, bool GATED>
__global__ __launch_bounds__(kThreads) void combine_kernel(const TY *__restrict__ src, const TY *__restrict__ rest,
                                                           const int32_t *__restrict__ plan,
                                                           const int32_t *__restrict__ row,
                                                           const float *__restrict__ gate, int T, int k, int d,
                                                           int tpb, int splits, size_t stride,
                                                           TE *__restrict__ y) {
    const int per_tok = kThreads / tpb;  // threads per token
    if (threadIdx.x / per_tok >= tpb) return;
    const int t = blockIdx.x * tpb + threadIdx.x / per_tok;
    const int lt = threadIdx.x % per_tok;
    if (t >= T) return;
    int rws[kMaxTopK];
    float gs[kMaxTopK];
    for (int r = 0; r < k; r++) {
        rws[r] = row[(size_t)t * k + r];
        gs[r] = GATED ? 1.0f : gate[(size_t)t * k + r];
    }
    const int row0 = plan ? plan[0] : 0, srows = plan ? plan[2] : 0;
    const int groups = d / 8;
    for (int c = lt; c < groups; c += per_tok) {
        float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int r = 0; r < k; r++) {
            if (rws[r] < 0) continue;
            float u[8];
            widen8(load8(src + (size_t)rws[r] * d, c), u);
            const int ns = !plan ? splits : (rws[r] >= row0 ? plan[1] : 1);
            for (int sl = 1; sl < ns; sl++) {
                float v[8];
                const TY *sp = plan ? rest + ((size_t)(sl - 1) * srows + (rws[r] - row0)) * d
                                    : src + sl * stride + (size_t)rws[r] * d;
                widen8(load8(sp, c), v);
#pragma unroll
                for (int i = 0; i < 8; i++) u[i] += v[i];
            }
#pragma unroll
            for (int i = 0; i < 8; i++) a[i] += GATED ? u[i] : gs[r] * u[i];
        }
        store8<TE>(y + (size_t)t * d + 8 * c, a);
    }
}

// The common shapes (k and the slice count known at compile time): each
// thread owns G groups of 8 outputs of one token and issues every load it
// needs (K rows x S slices x G groups) before the first add, so a wave keeps
// a whole token row's worth of reads in flight.  A dropped slot reads row 0
// and is discarded by a select, so no branch splits the batch and an
// uninitialised row can never leak a NaN into the sum (R >= 1 here).
// PLAN: slice 0 of every row is read first, then slices 1 .. S-1 of the
// split rows (a minority: the rows of the last round's m tiles).
template <typename TE, typename TY, bool GATED, int K, int S, int G, bool PLAN>
__global__ __launch_bounds__(kThreads) void combine_fixed(const TY *__restrict__ src, const TY *__restrict__ rest,
                                                          const int32_t *__restrict__ plan,
                                                          const int32_t *__restrict__ row,
                                                          const float *__restrict__ gate, int T, int d, size_t stride,
                                                          TE *__restrict__ y) {
    typedef typename SrcOf<TY>::type Src;
    const int per_tok = d / (8 * G);  // threads per token (divides kThreads)
    const int t = blockIdx.x * (kThreads / per_tok) + threadIdx.x / per_tok;
    const int lt = threadIdx.x % per_tok;
    if (t >= T) return;
    int rws[K];
    float gs[K];
#pragma unroll
    for (int r = 0; r < K; r++) {
        rws[r] = row[(size_t)t * K + r];
        gs[r] = GATED ? 1.0f : gate[(size_t)t * K + r];
    }
    Src u[G][K][S];
#pragma unroll
    for (int gi = 0; gi < G; gi++)
#pragma unroll
        for (int r = 0; r < K; r++)
#pragma unroll
            for (int sl = 0; sl < S; sl++)
                u[gi][r][sl] = load8(src + sl * stride + (size_t)max(rws[r], 0) * d, lt + gi * per_tok);
#pragma unroll
    for (int gi = 0; gi < G; gi++) {
        float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < K; r++) {
            float p[8];
            widen8(u[gi][r][0], p);
#pragma unroll
            for (int sl = 1; sl < S; sl++) {
                float q[8];
                widen8(u[gi][r][sl], q);
#pragma unroll
                for (int i = 0; i < 8; i++) p[i] += q[i];
            }
            if (PLAN && rws[r] >= plan[0]) {
                // a split row (rare): its further slices one at a time
                const TY *sp = rest + (size_t)(rws[r] - plan[0]) * d;
                const size_t sstride = (size_t)plan[2] * d;
                for (int sl = 1; sl < plan[1]; sl++) {
                    float q[8];
                    widen8(load8(sp + (sl - 1) * sstride, lt + gi * per_tok), q);
#pragma unroll
                    for (int i = 0; i < 8; i++) p[i] += q[i];
                }
            }
            const bool kept = rws[r] >= 0;
#pragma unroll
            for (int i = 0; i < 8; i++) a[i] += kept ? (GATED ? p[i] : gs[r] * p[i]) : 0.0f;
        }
        store8<TE>(y + (size_t)t * d + 8 * (lt + gi * per_tok), a);
    }
}

// Every output element zero (no permuted rows at all: nothing to read).
__global__ __launch_bounds__(kThreads) void zero_fill(uint4 *__restrict__ y, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += (size_t)gridDim.x * kThreads)
        y[i] = make_uint4(0, 0, 0, 0);
}

template <typename TE, typename TY, bool GATED, int K, int S, bool PLAN = false>
bool launch_fixed(const moe_params &p, size_t stride, const TY *src, const TY *rest, const int32_t *plan,
                  const int32_t *row, const float *gate, void *y, hipStream_t st) {
    // G = 2 groups per thread when a token row has at least 512 groups
    const int groups = p.d / 8;
    const int G = groups >= 2 * kThreads ? 2 : 1;
    const int per_tok = groups / G;
    if (per_tok > kThreads || kThreads % per_tok != 0) return false;
    const int tpb = kThreads / per_tok;
    const int grid = (int)ceil_div(p.T, tpb);
    if (G == 2)
        hipLaunchKernelGGL((combine_fixed<TE, TY, GATED, K, S, 2, PLAN>), dim3(grid), dim3(kThreads), 0, st, src, rest,
                           plan, row, gate, p.T, p.d, stride, static_cast<TE *>(y));
    else
        hipLaunchKernelGGL((combine_fixed<TE, TY, GATED, K, S, 1, PLAN>), dim3(grid), dim3(kThreads), 0, st, src, rest,
                           plan, row, gate, p.T, p.d, stride, static_cast<TE *>(y));
    return true;
}

// plan: null (every row has `splits` slices, `stride` elements apart), or
// the down projection's split plan (splits is then 1, see the header).
template <typename TE, typename TY, bool GATED>
hipError_t launch_any(const moe_params &p, int splits, size_t stride, const TY *src, const TY *rest,
                      const int32_t *plan, const int32_t *row, const float *gate, void *y, hipStream_t st) {
    bool fixed = false;
    if (plan) {
        if (p.k == 2) fixed = launch_fixed<TE, TY, GATED, 2, 1, true>(p, stride, src, rest, plan, row, gate, y, st);
        else if (p.k == 1) fixed = launch_fixed<TE, TY, GATED, 1, 1, true>(p, stride, src, rest, plan, row, gate, y, st);
    } else if (p.k == 2 && splits == 1) {
        fixed = launch_fixed<TE, TY, GATED, 2, 1>(p, stride, src, rest, plan, row, gate, y, st);
    } else if (p.k == 2 && splits == 2) {
        fixed = launch_fixed<TE, TY, GATED, 2, 2>(p, stride, src, rest, plan, row, gate, y, st);
    } else if (p.k == 2 && splits == 4) {
        fixed = launch_fixed<TE, TY, GATED, 2, 4>(p, stride, src, rest, plan, row, gate, y, st);
    } else if (p.k == 1 && splits == 1) {
        fixed = launch_fixed<TE, TY, GATED, 1, 1>(p, stride, src, rest, plan, row, gate, y, st);
    }
    if (fixed) return hipGetLastError();
    const int groups = p.d / 8;
    // tokens per block: enough threads per token to cover its row in one pass
    const int per_tok = groups < kThreads ? groups : kThreads;
    int tpb = kThreads / per_tok;
    if (tpb < 1) tpb = 1;
    const int grid = (int)ceil_div(p.T, tpb);
    hipLaunchKernelGGL((combine_kernel<TE, TY, GATED>), dim3(grid), dim3(kThreads), 0, st, src, rest, plan, row, gate,
                       p.T, p.k, p.d, tpb, splits, stride, static_cast<TE *>(y));
    return hipGetLastError();
}

hipError_t launch_zero(const moe_params &p, void *y, hipStream_t st) {
    const size_t n16 = (size_t)p.T * p.d * (p.dtype == MOE_BF16 ? 2 : 4) / 16;
    const int grid = (int)std::min<size_t>((n16 + kThreads - 1) / kThreads, 4096);
    hipLaunchKernelGGL(zero_fill, dim3(grid), dim3(kThreads), 0, st, static_cast<uint4 *>(y), n16);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const moe_params &p, int64_t max_rows, const float *y_perm, const int32_t *row,
                          const float *gate, void *y, hipStream_t st) {
    if (p.T == 0) return hipSuccess;
    if (max_rows <= 0) return launch_zero(p, y, st);
    if (p.dtype == MOE_BF16)
        return launch_any<uint16_t, float, false>(p, 1, 0, y_perm, y_perm, nullptr, row, gate, y, st);
    return launch_any<float, float, false>(p, 1, 0, y_perm, y_perm, nullptr, row, gate, y, st);
}

hipError_t launch_combine_gated(const moe_params &p, int64_t max_rows, int splits, const uint16_t *yg,
                                const uint16_t *yrest, const int32_t *plan, const int32_t *row, void *y,
                                hipStream_t st) {
    if (p.T == 0) return hipSuccess;
    if (max_rows <= 0) return launch_zero(p, y, st);
    const size_t stride = (size_t)max_rows * p.d;
    return launch_any<uint16_t, uint16_t, true>(p, plan ? 1 : splits, stride, yg, yrest, plan, row, nullptr, y, st);
}

}  // namespace moe
