// Backward pass of the bf16 layer (training), the forward routing held fixed.
//
// The router is trained through the experts: its gradient is what flows back
// from the experts' outputs through the gates ("MoE架构揭秘" §3.3).  The
// balance loss of "MoE稀疏激活原理与工程实践" §4.2 counts top-k picks under
// no_grad and adds no gradient; the penalty's load vector has none either.
// With dy the upstream gradient of y and, for a kept row r of expert e
// (token t, gate g):
//   a = W1_e x_t, b = W3_e x_t              (recomputed: the gate-up GEMM)
//   u = W2_e^T dy_t                          (grouped GEMM, dy rows gathered)
//   h = silu(a) * b,  dg_r = u . h           (= dy_t . o_r, o_r the expert output)
//   da = g u b silu'(a),  db = g u silu(a),  hg = g h
//   ds_j = g_j (dg_j - sum_l g_l dg_l) / tau over the token's kept slots
//   dlogits[t][e_j] = ds_j
//   dx_t = sum_j (W1_e^T da + W3_e^T db)[row_j] + sum_j ds_j W_r[e_j]
//   dW1_e = sum_r da_r x_t^T,  dW3_e = sum_r db_r x_t^T,  dW2_e = sum_r dy_t hg_r^T
//   dW_r[e] = sum_r ds_r x_t,  dbias[e] = sum_r ds_r
// Every gradient is fp32.  The GEMMs run on MFMA (32x32x16) with fp32
// accumulation: u = W2^T dy on bf16 (both exact), the others on fp16.  da,
// db and hg are computed in fp32; a single bf16 rounding of them would put
// up to 2^-9 of the largest terms into the gradients, so they were kept as
// hi = bf16(v) and lo = bf16(v - hi) pairs (about 2^-17 relative, two MFMAs
// per product).  They now enter as one fp16 value each (2^-12 relative, an
// eighth of a bf16 rounding), hi + lo scaled by a power of 2 per expert that
// keeps the expert's largest |da|, |db| (or |hg|) inside fp16's range
// (grad_scale_exp); dy is scaled by its largest magnitude in the same way.
// x, W1 and W3 enter as fp16 (exact from 2^-14 up to 65504, fp16's subnormal
// steps of 2^-24 below; the forward's W2 has the same range).  The weight
// gradients' epilogue and input_grad undo the scales.  This halves the K of
// the dx and weight-gradient GEMMs.  All sums run in a fixed order and the
// maxima are atomic maxima (the same in any order): the results are the same
// on every run.
#include <algorithm>
#include <mutex>

#include "device_common.h"
#include "grouped_tiles.h"
#include "moe_internal.h"

namespace moe {
namespace {

// The grouped GEMMs take A K-contiguous.  The weights of u and dx enter as
// they are (grouped_gemm_bf16<kPlainBT> reads N-contiguous B tiles with the
// transposing LDS read); the weight gradients' operands, whose K axis is the
// kept row, are transposed once into the workspace by to_kmajor, through
// 64 x 64 LDS tiles, for grouped_gemm_wgrad.

// The kept rows of each expert, transposed into its K window (kwin_start):
//   dst[c][kwin_e + koff + j] = conv(src[src_row(offsets[e] + j)][col0 + c])
// for j < rows_e, zeros for rows_e <= j < Kp_e (Kp_e = rows_e rounded up to
// 64); koff = half * Kp_e, or both halves (dup).  src_row(r) = gather[r] or
// r; src rows hold src_ld elements.  conv: CONV 0 copies the 16-bit value;
// CONV 1 scales a bf16 value by 2^grad_scale_exp(amax[0]) (amax null: 1) and
// rounds it to fp16 (to nearest even); CONV 2 adds the bf16 hi value and its
// lo partner lo_off elements further, scales the sum by
// 2^grad_scale_exp(amax[e]) and rounds it to fp16, which it also stores
// untransposed at rm[r][c] (rows of ncols) when rm is given.  Blocks:
// (expert, 64 kept rows, 64 columns), found like the GEMM's tiles.
__device__ __forceinline__ uint32_t f16x2_bits(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

template <int CONV>
__global__ __launch_bounds__(256) void to_kmajor(const uint16_t *__restrict__ src, int64_t src_ld,
                                                 const int32_t *__restrict__ gather, int col0, int ncols,
                                                 const int32_t *__restrict__ offsets, int E,
                                                 uint16_t *__restrict__ dst, int64_t ldk, int half, int dup,
                                                 int64_t lo_off, const uint32_t *__restrict__ amax,
                                                 uint16_t *__restrict__ rm) {
    __shared__ uint16_t t[64][66];
    TileInfo ti;
    if (!find_tile(offsets, E, ncols / 64, 64, 1, blockIdx.x, nullptr, nullptr, ti)) return;
    const int rbeg = offsets[ti.e], rows = ti.mend - rbeg;
    const int kp = (rows + 63) & ~63;
    const int j0 = ti.m0 - rbeg, c0 = ti.nt * 64;
    const int tid = threadIdx.x, q = (tid & 7) * 8;
    const int kscale = CONV == 2 ? grad_scale_exp(amax[ti.e]) : (CONV == 1 && amax ? grad_scale_exp(amax[0]) : 0);
#pragma unroll
    for (int ps = 0; ps < 2; ps++) {
        const int rr = (tid >> 3) + 32 * ps, r = ti.m0 + rr;
        uint4 v = make_uint4(0, 0, 0, 0), lo = make_uint4(0, 0, 0, 0);
        if (r < ti.mend) {
            const int64_t sr = gather ? gather[r] : r;
            v = *reinterpret_cast<const uint4 *>(src + sr * src_ld + col0 + c0 + q);
            if (CONV == 2) lo = *reinterpret_cast<const uint4 *>(src + sr * src_ld + col0 + c0 + q + lo_off);
        }
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
        if (CONV != 0) {
            const uint32_t l[4] = {lo.x, lo.y, lo.z, lo.w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                float f0 = bf16_bits_to_f32(w[i] & 0xFFFF), f1 = bf16_bits_to_f32(w[i] >> 16);
                if (CONV == 2) {
                    f0 += bf16_bits_to_f32(l[i] & 0xFFFF);
                    f1 += bf16_bits_to_f32(l[i] >> 16);
                }
                f0 = ldexpf(f0, kscale);
                f1 = ldexpf(f1, kscale);
                w[i] = f16x2_bits(f0, f1);
            }
            if (CONV == 2 && rm && r < ti.mend)
                *reinterpret_cast<uint4 *>(rm + (size_t)r * ncols + c0 + q) = make_uint4(w[0], w[1], w[2], w[3]);
        }
#pragma unroll
        for (int i = 0; i < 4; i++) *reinterpret_cast<uint32_t *>(&t[rr][q + 2 * i]) = w[i];
    }
    __syncthreads();
    const int64_t kw = kwin_start(rbeg, ti.e) + j0 + q;
#pragma unroll
    for (int ps = 0; ps < 2; ps++) {
        const int cc = (tid >> 3) + 32 * ps;
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; i++) w[i] = (uint32_t)t[q + 2 * i][cc] | ((uint32_t)t[q + 2 * i + 1][cc] << 16);
        const uint4 v = make_uint4(w[0], w[1], w[2], w[3]);
        uint16_t *d = dst + (size_t)(c0 + cc) * ldk + kw;
        if (dup) {
            *reinterpret_cast<uint4 *>(d) = v;
            *reinterpret_cast<uint4 *>(d + kp) = v;
        } else {
            *reinterpret_cast<uint4 *>(d + (size_t)half * kp) = v;
        }
    }
}

// unit_offsets: e * m1 (e = 0..E), then e * m2: the uniform row ranges of
// the weight-gradient GEMMs' outputs.
// (and the 2 E + 1 maxima zeroed, for swiglu_backward and abs_max)
__global__ __launch_bounds__(256) void unit_offsets_kernel(int32_t *__restrict__ o, int E, int m1, int m2,
                                                           uint32_t *__restrict__ amax) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i > E) return;
    o[i] = i * m1;
    o[E + 1 + i] = i * m2;
    if (i < E) {
        amax[i] = 0u;
        amax[E + i] = 0u;
    } else {
        amax[2 * E] = 0u;
    }
}

// *out = max(*out, the largest |v| of n bf16 values), as fp32 bits (an
// atomic maximum, the same in any order).
__global__ __launch_bounds__(256) void abs_max(const uint16_t *__restrict__ v, size_t n, uint32_t *__restrict__ out) {
    __shared__ uint32_t part[256];
    uint32_t m = 0u;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        m = max(m, (uint32_t)(v[i] & 0x7FFF) << 16);
    part[threadIdx.x] = m;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (threadIdx.x < w) part[threadIdx.x] = max(part[threadIdx.x], part[threadIdx.x + w]);
        __syncthreads();
    }
    if (threadIdx.x == 0) atomicMax(out, part[0]);
}

__global__ __launch_bounds__(256) void fill_zero(float *__restrict__ p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0.0f;
}

// Two fp32 values as bf16 hi = bf16(v) at p and lo = bf16(v - hi) at p + lo_off.
__device__ __forceinline__ void store_hi_lo(uint16_t *p, size_t lo_off, const float (&v)[2]) {
    const uint32_t hi = pack_bf16x2(v[0], v[1]);
    const float r0 = v[0] - bf16_bits_to_f32(hi & 0xFFFF), r1 = v[1] - bf16_bits_to_f32(hi >> 16);
    *reinterpret_cast<uint32_t *>(p) = hi;
    *reinterpret_cast<uint32_t *>(p + lo_off) = pack_bf16x2(r0, r1);
}

// Each kept row's gate: gate_of_row[row[t][j]] = gate[t][j].
__global__ __launch_bounds__(256) void row_gates(const int32_t *__restrict__ row, const float *__restrict__ gate,
                                                 int Tk, float *__restrict__ gate_of_row) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= Tk) return;
    const int r = row[i];
    if (r >= 0) gate_of_row[r] = gate[i];
}

// Per kept row (one block): h = silu(a) b, dg = u . h (fixed-order block
// reduction), da = g u b silu'(a), db = g u silu(a), hg = g h, each as a
// bf16 hi/lo pair: acat row [da hi | db hi | da lo | db lo] (4 d_ff), hg row
// [hi | lo] (2 d_ff).  The row's largest |da|, |db| goes into amax[e] of its
// expert and its largest |g h| into amax[E + e] (atomic maxima of the fp32
// bits, which order non-negative values: the same result in any order).
__global__ __launch_bounds__(256) void swiglu_backward(const float *__restrict__ a, const float *__restrict__ b,
                                                       const float *__restrict__ u,
                                                       const float *__restrict__ gate_of_row,
                                                       const int32_t *__restrict__ offsets, int E, int dff,
                                                       uint16_t *__restrict__ acat, uint16_t *__restrict__ hg,
                                                       float *__restrict__ dg, uint32_t *__restrict__ amax) {
    __shared__ float part[256];
    __shared__ uint32_t pmax[256], pmaxh[256];
    const int r = blockIdx.x;
    if (r >= offsets[E]) return;
    const float g = gate_of_row[r];
    const size_t o = (size_t)r * dff;
    uint16_t *ar = acat + 4 * o, *hr = hg + 2 * o;
    float s = 0.0f;
    uint32_t mx = 0u, mh = 0u;
    for (int f = threadIdx.x * 2; f < dff; f += 512) {
        float dav[2], dbv[2], hv[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const float av = a[o + f + i], bv = b[o + f + i], uv = u[o + f + i];
            const float sg = 1.0f / (1.0f + expf(-av));
            const float silu = av * sg, h = silu * bv, dh = g * uv;
            s = fmaf(uv, h, s);
            dav[i] = dh * bv * sg * (1.0f + av * (1.0f - sg));
            dbv[i] = dh * silu;
            hv[i] = g * h;
            mx = max(mx, max(__float_as_uint(fabsf(dav[i])), __float_as_uint(fabsf(dbv[i]))));
            mh = max(mh, __float_as_uint(fabsf(hv[i])));
        }
        store_hi_lo(ar + f, 2 * (size_t)dff, dav);
        store_hi_lo(ar + dff + f, 2 * (size_t)dff, dbv);
        store_hi_lo(hr + f, (size_t)dff, hv);
    }
    part[threadIdx.x] = s;
    pmax[threadIdx.x] = mx;
    pmaxh[threadIdx.x] = mh;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (threadIdx.x < w) {
            part[threadIdx.x] += part[threadIdx.x + w];
            pmax[threadIdx.x] = max(pmax[threadIdx.x], pmax[threadIdx.x + w]);
            pmaxh[threadIdx.x] = max(pmaxh[threadIdx.x], pmaxh[threadIdx.x + w]);
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        dg[r] = part[0];
        // the row's expert: the last e with offsets[e] <= r
        int lo = 0, hi = E;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (offsets[mid] <= r) lo = mid;
            else hi = mid;
        }
        atomicMax(&amax[lo], pmax[0]);
        atomicMax(&amax[E + lo], pmaxh[0]);
    }
}

// Gate softmax backward, one thread per token: ds_j = g_j (dg_j - sum_l g_l
// dg_l) / tau over the kept slots; dlogits[t] is ds at the kept experts and
// 0 elsewhere; ds_of_row[row_j] = ds_j.
__global__ __launch_bounds__(256) void gate_backward(const int32_t *__restrict__ row, const int32_t *__restrict__ eid,
                                                     const float *__restrict__ gate, const float *__restrict__ dg,
                                                     int T, int E, int k, float inv_tau, float *__restrict__ dlogits,
                                                     float *__restrict__ ds_of_row) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    float dgs[kMaxTopK], mean = 0.0f;
    for (int j = 0; j < k; j++) {
        const int r = row[(size_t)t * k + j];
        dgs[j] = r >= 0 ? dg[r] : 0.0f;
        if (r >= 0) mean = fmaf(gate[(size_t)t * k + j], dgs[j], mean);
    }
    float *dl = dlogits + (size_t)t * E;
    for (int e = 0; e < E; e++) dl[e] = 0.0f;
    for (int j = 0; j < k; j++) {
        const int r = row[(size_t)t * k + j];
        if (r < 0) continue;
        const float ds = gate[(size_t)t * k + j] * (dgs[j] - mean) * inv_tau;
        dl[eid[(size_t)t * k + j]] = ds;
        ds_of_row[r] = ds;
    }
}

// dx[t] = sum over kept slots j of dx_perm[row_j] + ds_j W_r[e_j] (slot
// order), fp32; 8 columns per thread.
__global__ __launch_bounds__(256) void input_grad(const float *__restrict__ dx_perm, const float *__restrict__ rest,
                                                  int nrest, size_t stride, const uint16_t *__restrict__ wr,
                                                  const int32_t *__restrict__ row, const int32_t *__restrict__ eid,
                                                  const float *__restrict__ ds_of_row,
                                                  const uint32_t *__restrict__ amax, int k, int d,
                                                  float *__restrict__ dx) {
    const int t = blockIdx.x;
    int rws[kMaxTopK], es[kMaxTopK];
    float ds[kMaxTopK], sc[kMaxTopK];
    for (int j = 0; j < k; j++) {
        rws[j] = row[(size_t)t * k + j];
        es[j] = eid[(size_t)t * k + j];
        ds[j] = rws[j] >= 0 ? ds_of_row[rws[j]] : 0.0f;
        // dx_perm rows hold W1^T da + W3^T db scaled by their expert's 2^k
        sc[j] = rws[j] >= 0 ? ldexpf(1.0f, -grad_scale_exp(amax[es[j]])) : 0.0f;
    }
    for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int j = 0; j < k; j++) {
            if (rws[j] < 0) continue;
            const float4 *p = reinterpret_cast<const float4 *>(dx_perm + (size_t)rws[j] * d + c);
            float4 v0 = p[0], v1 = p[1];
            // the row's further K slices, added in slice order
            for (int sl = 0; sl < nrest; sl++) {
                const float4 *q = reinterpret_cast<const float4 *>(rest + sl * stride + (size_t)rws[j] * d + c);
                const float4 u0 = q[0], u1 = q[1];
                v0.x += u0.x; v0.y += u0.y; v0.z += u0.z; v0.w += u0.w;
                v1.x += u1.x; v1.y += u1.y; v1.z += u1.z; v1.w += u1.w;
            }
            const float s = sc[j];
            acc[0] += s * v0.x; acc[1] += s * v0.y; acc[2] += s * v0.z; acc[3] += s * v0.w;
            acc[4] += s * v1.x; acc[5] += s * v1.y; acc[6] += s * v1.z; acc[7] += s * v1.w;
        }
        for (int j = 0; j < k; j++) {
            if (rws[j] < 0) continue;
            const uint4 w = *reinterpret_cast<const uint4 *>(wr + (size_t)es[j] * d + c);
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                acc[2 * i] = fmaf(ds[j], bf16_bits_to_f32(ww[i] & 0xFFFF), acc[2 * i]);
                acc[2 * i + 1] = fmaf(ds[j], bf16_bits_to_f32(ww[i] >> 16), acc[2 * i + 1]);
            }
        }
        float4 *o = reinterpret_cast<float4 *>(dx + (size_t)t * d + c);
        o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
}

// dW_r[e][c] = sum over the kept rows r of expert e of ds_r x[tok_r][c] and
// dbias[e] = sum_r ds_r, from the kept rows' transposed x (xt in fp16, the
// expert's K window: rows_e values then zero padding).  Block (e, 64 columns), a wave
// per 16 columns: lane l accumulates window positions 8l .. 8l+7 of every
// 512 in order, then a fixed butterfly over the lanes adds the partial sums.
__global__ __launch_bounds__(256) void router_wgrad(const uint16_t *__restrict__ xt, int64_t ldk,
                                                    const float *__restrict__ ds_of_row,
                                                    const int32_t *__restrict__ offsets, int d,
                                                    float *__restrict__ dwr, float *__restrict__ dbias) {
    const int nc = d / 64;
    const int e = blockIdx.x / nc, c0 = (blockIdx.x % nc) * 64 + (threadIdx.x >> 6) * 16;
    const int lane = threadIdx.x & 63;
    const int rbeg = offsets[e], rows = offsets[e + 1] - rbeg;
    const int kp = (rows + 63) & ~63;
    const uint16_t *xw = xt + kwin_start(rbeg, e);
    float acc[16], sb = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; c++) acc[c] = 0.0f;
    for (int j0 = lane * 8; j0 < kp; j0 += 512) {
        float ds[8];
#pragma unroll
        for (int i = 0; i < 8; i++) ds[i] = j0 + i < rows ? ds_of_row[rbeg + j0 + i] : 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i++) sb += ds[i];
#pragma unroll
        for (int c = 0; c < 16; c++) {
            const uint4 v = *reinterpret_cast<const uint4 *>(xw + (size_t)(c0 + c) * ldk + j0);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                acc[c] = fmaf(ds[2 * i], (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFF)), acc[c]);
                acc[c] = fmaf(ds[2 * i + 1], (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16)), acc[c]);
            }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
#pragma unroll
        for (int c = 0; c < 16; c++) acc[c] += __shfl_xor(acc[c], off, 64);
        sb += __shfl_xor(sb, off, 64);
    }
    if (lane < 16) {
        float v = acc[0];
#pragma unroll
        for (int c = 1; c < 16; c++) v = lane == c ? acc[c] : v;
        dwr[(size_t)e * d + c0 + lane] = v;
    }
    if (blockIdx.x % nc == 0 && threadIdx.x == 0) dbias[e] = sb;
}

// The weight-gradient half of the backward (the transposes of x, dy and
// g h, the three weight-gradient GEMMs and the router gradients) and its
// input-gradient half (the dx GEMM and input_grad) read the same inputs and
// write disjoint buffers.  The weight-gradient half runs on a second stream
// of the device, forked from the caller's stream and joined back to it by
// two events, so that its memory-bound transposes and the weight gradients'
// fp32 stores overlap the dx GEMM's matrix work.  The stream (default
// priority) and events are made on first use per device and kept until the
// process ends; where that fails (e.g. inside a graph capture), both halves
// run in order on the caller's stream.  side_mu is held from the fork to the
// join, so calls from several host threads never swap each other's events.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxSideDevices = 64;
std::mutex side_mu;
SideStream side_streams[kMaxSideDevices];

// The current device's side stream, or null; side_mu held.
const SideStream *side_stream() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSideDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    SideStream &ss = side_streams[dev];
    if (!ss.s) {
        hipStream_t s = nullptr;
        hipEvent_t f = nullptr, j = nullptr;
        if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) == hipSuccess &&
            hipEventCreateWithFlags(&f, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&j, hipEventDisableTiming) == hipSuccess) {
            ss.fork = f;
            ss.join = j;
            ss.s = s;
        } else {
            if (j) (void)hipEventDestroy(j);
            if (f) (void)hipEventDestroy(f);
            if (s) (void)hipStreamDestroy(s);
            (void)hipGetLastError();
        }
    }
    return ss.s ? &ss : nullptr;
}

}  // namespace

hipError_t launch_backward(const moe_params &p, int64_t max_rows, int64_t cap, const BackwardArgs &a, hipStream_t st) {
    const int T = p.T, d = p.d, E = p.E, k = p.k, dff = p.d_ff;
    const int64_t R = max_rows;
    const uint16_t *x = static_cast<const uint16_t *>(a.x);
    const uint16_t *dy = static_cast<const uint16_t *>(a.dy);
    if (T == 0 || R == 0) {
        // no kept rows: every weight gradient is zero
        const size_t nw = (size_t)E * dff * d;
        const int grid = (int)std::min<int64_t>(ceil_div((int64_t)nw, 256), 8192);
        hipLaunchKernelGGL(fill_zero, dim3(grid), dim3(256), 0, st, a.dw1, nw);
        hipLaunchKernelGGL(fill_zero, dim3(grid), dim3(256), 0, st, a.dw3, nw);
        hipLaunchKernelGGL(fill_zero, dim3(grid), dim3(256), 0, st, a.dw2, nw);
        if (T > 0) {
            // tokens, none kept: dlogits and dx are zero too
            hipLaunchKernelGGL(fill_zero, dim3((unsigned)std::min<int64_t>(ceil_div((int64_t)T * E, 256), 8192)),
                               dim3(256), 0, st, a.dlogits, (size_t)T * E);
            hipLaunchKernelGGL(fill_zero, dim3((unsigned)std::min<int64_t>(ceil_div((int64_t)T * d, 256), 8192)),
                               dim3(256), 0, st, a.dx, (size_t)T * d);
        }
        hipLaunchKernelGGL(router_wgrad, dim3((unsigned)(E * (d / 64))), dim3(256), 0, st, a.xt, a.ldk,
                           a.ds_of_row, a.offsets, d, a.dw_router, a.dbias);
        return hipGetLastError();
    }
    const float inv_tau = 1.0f / (p.gate_temperature > 0.0f ? p.gate_temperature : 1.0f);
    const int64_t ldk = a.ldk;
    const int32_t *uo_f = a.unit_offsets, *uo_d = a.unit_offsets + E + 1;
    // bound on the 64-row tiles of the kept rows, for the transposes' grids
    const int64_t mt64 = std::min<int64_t>(R / 64 + E, (int64_t)E * ceil_div(cap, 64));
    auto kmajor = [&](auto kern, const uint16_t *src, int64_t src_ld, const int32_t *gather, int col0, int ncols,
                      uint16_t *dst, int half, int dup, int64_t lo_off, const uint32_t *amax, uint16_t *rm,
                      hipStream_t s) {
        hipLaunchKernelGGL(kern, dim3((unsigned)(mt64 * (ncols / 64))), dim3(256), 0, s, src, src_ld, gather, col0,
                           ncols, a.offsets, E, dst, ldk, half, dup, lo_off, amax, rm);
    };
    const uint32_t *amax_dab = a.amax, *amax_hg = a.amax + E, *amax_dy = a.amax + 2 * E;
    // 1. the rows' gates, the weight-gradient row ranges; a and b
    //    recomputed by the gate-up GEMM
    hipLaunchKernelGGL(row_gates, dim3((unsigned)ceil_div((int64_t)T * k, 256)), dim3(256), 0, st, a.row, a.gate,
                       T * k, a.gate_of_row);
    hipLaunchKernelGGL(unit_offsets_kernel, dim3((unsigned)ceil_div(E + 1, 256)), dim3(256), 0, st, a.unit_offsets,
                       E, dff, d, a.amax);
    hipLaunchKernelGGL(abs_max, dim3((unsigned)std::min<int64_t>(ceil_div((int64_t)T * d, 256 * 8), 1024)), dim3(256), 0,
                       st, dy, (size_t)T * d, a.amax + 2 * E);
    hipError_t e = launch_gate_up_raw(p, R, cap, a.x, a.token_of_row, a.offsets, a.w1, a.w3, a.a, a.b, st);
    if (e != hipSuccess) return e;
    // 2. u = W2_e^T dy_t for every kept row (dy rows gathered by token; W2
    //    [d][d_ff] read as it is, N-contiguous)
    const uint16_t *w1 = static_cast<const uint16_t *>(a.w1), *w3 = static_cast<const uint16_t *>(a.w3),
                   *w2 = static_cast<const uint16_t *>(a.w2);
    e = launch_plain_gemm(R, cap, E, dy, a.token_of_row, (int64_t)T * d * 2, a.offsets, w2, nullptr, true, dff, d, d,
                          1, a.u, nullptr, st);
    if (e != hipSuccess) return e;
    // 3. SwiGLU backward per row, 4. gate softmax backward per token
    hipLaunchKernelGGL(swiglu_backward, dim3((unsigned)R), dim3(256), 0, st, a.a, a.b, a.u, a.gate_of_row, a.offsets,
                       E, dff, a.acat, a.hg, a.dg, a.amax);
    hipLaunchKernelGGL(gate_backward, dim3((unsigned)ceil_div(T, 256)), dim3(256), 0, st, a.row, a.eid, a.gate, a.dg,
                       T, E, k, inv_tau, a.dlogits, a.ds_of_row);
    // 5. da and db as scaled fp16 from their hi/lo pairs, K-major in their
    //    experts' K windows (dat) and row-major (dab16)
    kmajor(to_kmajor<2>, a.acat, 4 * (int64_t)dff, nullptr, 0, 2 * dff, a.dat, 0, 0, 2 * (int64_t)dff, amax_dab,
           a.dab16, st);
    // fork: the weight-gradient half (7-9) on the side stream sw
    std::lock_guard<std::mutex> lock(side_mu);
    const SideStream *ss = side_stream();
    hipStream_t sw = st;
    if (ss) {
        if (hipEventRecord(ss->fork, st) == hipSuccess && hipStreamWaitEvent(ss->s, ss->fork, 0) == hipSuccess)
            sw = ss->s;
        else
            (void)hipGetLastError();
    }
    // (the side half is enqueued first, so that its transposes start at once
    // and its short weight-gradient tiles interleave with the dx GEMM's)
    // 7. the kept rows transposed into their experts' K windows, fp16: x,
    //    dy (scaled by 2^k_dy), g h (from its hi/lo pair, scaled per expert)
    kmajor(to_kmajor<1>, x, d, a.token_of_row, 0, d, a.xt, 0, 0, 0, nullptr, nullptr, sw);
    kmajor(to_kmajor<1>, dy, d, a.token_of_row, 0, d, a.dyt, 0, 0, 0, amax_dy, nullptr, sw);
    kmajor(to_kmajor<2>, a.hg, 2 * (int64_t)dff, nullptr, 0, dff, a.hgt, 0, 0, dff, amax_hg, nullptr, sw);
    // 8. dW1 = da^T x, dW3 = db^T x, dW2 = dy^T (g h), each expert over its
    //    rows, the scales undone in the epilogue
    hipError_t ew = launch_wgrad_gemm(E, a.dat, a.xt, a.offsets, uo_f, dff, d, (int)ldk, a.dw1, sw, amax_dab);
    if (ew == hipSuccess)
        ew = launch_wgrad_gemm(E, a.dat + (size_t)dff * ldk, a.xt, a.offsets, uo_f, dff, d, (int)ldk, a.dw3, sw,
                               amax_dab);
    if (ew == hipSuccess)
        ew = launch_wgrad_gemm(E, a.dyt, a.hgt, a.offsets, uo_d, d, dff, (int)ldk, a.dw2, sw, amax_hg, amax_dy);
    // 9. router weight and bias gradients
    if (ew == hipSuccess)
        hipLaunchKernelGGL(router_wgrad, dim3((unsigned)(E * (d / 64))), dim3(256), 0, sw, a.xt, ldk, a.ds_of_row,
                           a.offsets, d, a.dw_router, a.dbias);
    // 6. dx_perm = 2^k_e (da W1 + db W3): two K periods of d_ff over the
    //    dab16 row, W1 and W3 ([d_ff][d], N-contiguous, widened to fp16) in
    //    turn, at least one K slice per period; dx, the scale undone per slot
    //    (its K slices are left apart: input_grad adds a row's slices in
    //    order as it reads the row, which saves the fix-up's pass)
    e = launch_plain_gemm(R, cap, E, a.dab16, nullptr, 0, a.offsets, w1, w3, true, d, 2 * dff, dff, a.dx_splits,
                          a.dx_perm, a.dx_rest, st, true, false);
    if (e == hipSuccess)
        hipLaunchKernelGGL(input_grad, dim3((unsigned)T), dim3(256), 0, st, a.dx_perm, a.dx_rest, a.dx_splits - 1,
                           (size_t)R * d, static_cast<const uint16_t *>(a.w_router), a.row, a.eid, a.ds_of_row,
                           amax_dab, k, d, a.dx);
    // join: the caller's stream waits for the side stream's work, also after
    // an error, so that nothing of this call is left running unordered
    const hipError_t el = hipGetLastError();
    hipError_t ej = hipSuccess;
    if (sw != st) {
        ej = hipEventRecord(ss->join, sw);
        if (ej == hipSuccess) ej = hipStreamWaitEvent(st, ss->join, 0);
        if (ej != hipSuccess) ej = hipDeviceSynchronize() == hipSuccess ? hipSuccess : ej;
    }
    if (e != hipSuccess) return e;
    if (ew != hipSuccess) return ew;
    return el != hipSuccess ? el : ej;
}

}  // namespace moe
