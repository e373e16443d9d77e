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

// grid.x = blocks of tpb tokens; each token's row is spread over the
// block's threads in groups of 8 elements.
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

}  // namespace

hipError_t launch_combine(const moe_params &p, int splits, size_t split_stride, const void *y_perm,
                          const int32_t *row, const float *gate, void *y, hipStream_t st) {
    if (p.T == 0) return hipSuccess;
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
