// Stage 4: gate-weighted combine back to token order.
//
// y[t] = sum over kept slots j of gate[t][j] * y_perm[row[t][j]], accumulated
// in fp32 and rounded once ("企业官网建设流程全解析" page §3, step 5: the
// experts' results are put back in token order; "GPT-4稀疏激活真相" §4.3:
// weighted fusion).  A token with no kept slot gets zeros.
//
// y_perm is fp32 (the down GEMM's accumulator precision), so the bf16 output
// is rounded exactly once.  It may hold S partial products (slices of the
// d_ff reduction, split_stride apart), which are added in slice order.
// HBM-bound gather: 16-byte loads and stores, the k source rows read once
// each.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// Each thread produces 8 consecutive outputs: it reads two 16-byte fp32
// chunks from each kept y_perm row and writes 8 bf16 (16 bytes) or 8 fp32
// (32 bytes).
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

// Sum of gate * (slices of row) for 8 consecutive elements.  Generic path
// (any k <= 8 and any slice count): the loads of one row's slices are
// issued together, rows one after another.
template <typename TE>
__global__ __launch_bounds__(kThreads) void combine_kernel(const float *__restrict__ y_perm,
                                                           const int32_t *__restrict__ row,
                                                           const float *__restrict__ gate, int T,
                                                           int k, int d, int tpb, int splits,
                                                           size_t split_stride,
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
        gs[r] = gate[(size_t)t * k + r];
    }
    const int groups = d / 8;
    for (int c = lt; c < groups; c += per_tok) {
        float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int r = 0; r < k; r++) {
            if (rws[r] < 0) continue;
            const float4 *src = reinterpret_cast<const float4 *>(y_perm + (size_t)rws[r] * d) + 2 * c;
            float4 u = src[0], v = src[1];
            // the down projection's d_ff slices, added in slice order
            for (int sl = 1; sl < splits; sl++) {
                const float4 *ps = reinterpret_cast<const float4 *>(y_perm + sl * split_stride + (size_t)rws[r] * d) + 2 * c;
                const float4 pu = ps[0], pv = ps[1];
                u.x += pu.x; u.y += pu.y; u.z += pu.z; u.w += pu.w;
                v.x += pv.x; v.y += pv.y; v.z += pv.z; v.w += pv.w;
            }
            const float g = gs[r];
            a[0] += g * u.x;
            a[1] += g * u.y;
            a[2] += g * u.z;
            a[3] += g * u.w;
            a[4] += g * v.x;
            a[5] += g * v.y;
            a[6] += g * v.z;
            a[7] += g * v.w;
        }
        store8<TE>(y + (size_t)t * d + 8 * c, a);
    }
}

// The common shapes (k and the slice count known at compile time): each
// thread owns G groups of 8 outputs of one token and issues every load it
// needs (K rows x S slices x G groups x 32 bytes) before the first add, so
// a wave keeps a whole token row's worth of reads in flight.  A dropped
// slot reads row 0 and is discarded by a select, so no branch splits the
// batch and an uninitialised row can never leak a NaN into the sum.
template <typename TE, int K, int S, int G>
__global__ __launch_bounds__(kThreads) void combine_fixed(const float *__restrict__ y_perm,
                                                          const int32_t *__restrict__ row,
                                                          const float *__restrict__ gate, int T, int d,
                                                          size_t split_stride, TE *__restrict__ y) {
    const int per_tok = d / (8 * G);  // threads per token (divides kThreads)
    const int t = blockIdx.x * (kThreads / per_tok) + threadIdx.x / per_tok;
    const int lt = threadIdx.x % per_tok;
    if (t >= T) return;
    int rws[K];
    float gs[K];
#pragma unroll
    for (int r = 0; r < K; r++) {
        rws[r] = row[(size_t)t * K + r];
        gs[r] = gate[(size_t)t * K + r];
    }
    float4 u[G][K][S][2];
#pragma unroll
    for (int gi = 0; gi < G; gi++)
#pragma unroll
        for (int r = 0; r < K; r++)
#pragma unroll
            for (int sl = 0; sl < S; sl++) {
                const float4 *src = reinterpret_cast<const float4 *>(
                                        y_perm + sl * split_stride + (size_t)max(rws[r], 0) * d) +
                                    2 * (lt + gi * per_tok);
                u[gi][r][sl][0] = src[0];
                u[gi][r][sl][1] = src[1];
            }
#pragma unroll
    for (int gi = 0; gi < G; gi++) {
        float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < K; r++) {
            float4 p = u[gi][r][0][0], q = u[gi][r][0][1];
#pragma unroll
            for (int sl = 1; sl < S; sl++) {
                p.x += u[gi][r][sl][0].x; p.y += u[gi][r][sl][0].y; p.z += u[gi][r][sl][0].z; p.w += u[gi][r][sl][0].w;
                q.x += u[gi][r][sl][1].x; q.y += u[gi][r][sl][1].y; q.z += u[gi][r][sl][1].z; q.w += u[gi][r][sl][1].w;
            }
            const bool kept = rws[r] >= 0;
            const float g = gs[r];
            a[0] += kept ? g * p.x : 0.0f;
            a[1] += kept ? g * p.y : 0.0f;
            a[2] += kept ? g * p.z : 0.0f;
            a[3] += kept ? g * p.w : 0.0f;
            a[4] += kept ? g * q.x : 0.0f;
            a[5] += kept ? g * q.y : 0.0f;
            a[6] += kept ? g * q.z : 0.0f;
            a[7] += kept ? g * q.w : 0.0f;
        }
        store8<TE>(y + (size_t)t * d + 8 * (lt + gi * per_tok), a);
    }
}

template <typename TE, int K, int S>
bool launch_fixed(const moe_params &p, size_t split_stride, const void *y_perm, const int32_t *row,
                  const float *gate, void *y, hipStream_t st) {
    // G = 2 groups per thread when a token row has at least 512 groups
    const int groups = p.d / 8;
    const int G = groups >= 2 * kThreads ? 2 : 1;
    const int per_tok = groups / G;
    if (per_tok > kThreads || kThreads % per_tok != 0) return false;
    const int tpb = kThreads / per_tok;
    const int grid = (int)ceil_div(p.T, tpb);
    if (G == 2)
        hipLaunchKernelGGL((combine_fixed<TE, K, S, 2>), dim3(grid), dim3(kThreads), 0, st,
                           static_cast<const float *>(y_perm), row, gate, p.T, p.d, split_stride,
                           static_cast<TE *>(y));
    else
        hipLaunchKernelGGL((combine_fixed<TE, K, S, 1>), dim3(grid), dim3(kThreads), 0, st,
                           static_cast<const float *>(y_perm), row, gate, p.T, p.d, split_stride,
                           static_cast<TE *>(y));
    return true;
}

template <typename TE>
bool launch_fixed_any(const moe_params &p, int splits, size_t split_stride, const void *y_perm,
                      const int32_t *row, const float *gate, void *y, hipStream_t st) {
    if (p.k == 2 && splits == 1) return launch_fixed<TE, 2, 1>(p, split_stride, y_perm, row, gate, y, st);
    if (p.k == 2 && splits == 2) return launch_fixed<TE, 2, 2>(p, split_stride, y_perm, row, gate, y, st);
    if (p.k == 2 && splits == 4) return launch_fixed<TE, 2, 4>(p, split_stride, y_perm, row, gate, y, st);
    if (p.k == 1 && splits == 1) return launch_fixed<TE, 1, 1>(p, split_stride, y_perm, row, gate, y, st);
    return false;
}

}  // namespace

hipError_t launch_combine(const moe_params &p, int splits, size_t split_stride, const void *y_perm,
                          const int32_t *row, const float *gate, void *y, hipStream_t st) {
    if (p.T == 0) return hipSuccess;
    const bool fixed = p.dtype == MOE_BF16
                           ? launch_fixed_any<uint16_t>(p, splits, split_stride, y_perm, row, gate, y, st)
                           : launch_fixed_any<float>(p, splits, split_stride, y_perm, row, gate, y, st);
    if (fixed) return hipGetLastError();
    const int groups = p.d / 8;
    // tokens per block: enough threads per token to cover its row in one pass
    const int per_tok = groups < kThreads ? groups : kThreads;
    int tpb = kThreads / per_tok;
    if (tpb < 1) tpb = 1;
    const int grid = (int)ceil_div(p.T, tpb);
    if (p.dtype == MOE_BF16)
        hipLaunchKernelGGL(combine_kernel<uint16_t>, dim3(grid), dim3(kThreads), 0, st,
                           static_cast<const float *>(y_perm), row, gate, p.T, p.k, p.d, tpb,
                           splits, split_stride, static_cast<uint16_t *>(y));
    else
        hipLaunchKernelGGL(combine_kernel<float>, dim3(grid), dim3(kThreads), 0, st,
                           static_cast<const float *>(y_perm), row, gate, p.T, p.k, p.d, tpb,
                           splits, split_stride, static_cast<float *>(y));
    return hipGetLastError();
}

}  // namespace moe
