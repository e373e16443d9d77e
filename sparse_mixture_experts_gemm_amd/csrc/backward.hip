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
// Every gradient is fp32.  The GEMMs run on bf16 MFMA (32x32x16) with fp32
// accumulation.  x, dy and the weights are exact bf16 operands; da, db and hg
// are computed in fp32 and kept as a pair of bf16 values, hi = bf16(v) and
// lo = bf16(v - hi) (v to about 2^-17 relative), whose two MFMAs against the
// same partner fragment accumulate into one result: a single bf16 rounding of
// these operands would put up to 2^-9 of the largest terms into the weight
// gradients.  All reductions run in a fixed order: the results are the same
// on every run.
#include <algorithm>

#include "device_common.h"
#include "grouped_tiles.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBt = 256;        // threads of a GEMM block (4 waves, 2 x 2)
constexpr int kTm = 128;        // tile rows (M)
constexpr int kTn = 128;        // tile columns (N)
constexpr int kTk = 32;         // K per step
constexpr int kRowB = 80;       // LDS bytes per tile row: 32 bf16 + 16 bytes of padding (conflict-free reads)
constexpr int kTileB = kTm * kRowB;

__device__ __forceinline__ f32x16_t mfma_bf16(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// An operand tile staged as 128 LDS rows of 32 K elements.
//   K-contiguous source (row-major [row][k]): a thread moves 16 bytes (8 K
//   elements) of one row per pass, two passes.
//   Row-contiguous source ([k][row], the tile's rows along the source row):
//   a thread reads 8 consecutive tile rows at two consecutive k and writes
//   them as 8 pairs, transposing into the K-contiguous layout.
// `valid` bounds the tile rows (rows past it, and K past kvalid, are zero).
struct KcontigSrc {
    const uint16_t *base;   // element (row, k) at base[src(row) * ld + k]
    const int32_t *gather;  // src(row) = gather[row0 + row] or row0 + row
    int64_t ld;
};
struct RowcontigSrc {
    const uint16_t *base;   // element (k, n) at base[src(k) * ld + n]
    const int32_t *gather;  // src(k) = gather[k] or k (k absolute)
    int64_t ld;
};

struct Regs2 {
    uint4 v[2];
};

__device__ __forceinline__ Regs2 load_kcontig(const KcontigSrc &s, int row0, int valid, int k0) {
    Regs2 r;
    const int t = threadIdx.x;
#pragma unroll
    for (int ps = 0; ps < 2; ps++) {
        const int row = ps * 64 + (t >> 2), kc = (t & 3) * 8;
        r.v[ps] = make_uint4(0, 0, 0, 0);
        if (row < valid) {
            const int64_t sr = s.gather ? s.gather[row0 + row] : row0 + row;
            r.v[ps] = *reinterpret_cast<const uint4 *>(s.base + sr * s.ld + k0 + kc);
        }
    }
    return r;
}

__device__ __forceinline__ void store_kcontig(char *tile, const Regs2 &r) {
    const int t = threadIdx.x;
#pragma unroll
    for (int ps = 0; ps < 2; ps++) {
        const int row = ps * 64 + (t >> 2), kc = (t & 3) * 8;
        *reinterpret_cast<uint4 *>(tile + row * kRowB + kc * 2) = r.v[ps];
    }
}

// k in [k0, k0 + 32) with k < kend valid; tile rows n0 + [0, 128) with n < nend.
__device__ __forceinline__ Regs2 load_rowcontig(const RowcontigSrc &s, int k0, int kend, int n0, int nend) {
    Regs2 r;
    const int t = threadIdx.x;
    const int kp = t >> 4, nc = (t & 15) * 8;
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int k = k0 + 2 * kp + h;
        r.v[h] = make_uint4(0, 0, 0, 0);
        if (k < kend && n0 + nc < nend) {
            const int64_t sr = s.gather ? s.gather[k] : k;
            r.v[h] = *reinterpret_cast<const uint4 *>(s.base + sr * s.ld + n0 + nc);
        }
    }
    return r;
}

__device__ __forceinline__ void store_rowcontig(char *tile, const Regs2 &r) {
    const int t = threadIdx.x;
    const int kp = t >> 4, nc = (t & 15) * 8;
    const uint32_t lo[4] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w};
    const uint32_t hi[4] = {r.v[1].x, r.v[1].y, r.v[1].z, r.v[1].w};
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const uint32_t a = (lo[j >> 1] >> ((j & 1) * 16)) & 0xFFFF, b = (hi[j >> 1] >> ((j & 1) * 16)) & 0xFFFF;
        *reinterpret_cast<uint32_t *>(tile + (nc + j) * kRowB + kp * 4) = a | (b << 16);
    }
}

// Which operand of a GEMM comes as a hi/lo pair of bf16 tiles.
enum { kSplitNone = 0, kSplitA = 1, kSplitB = 2 };

// MFMAs of one 32-wide K step: the wave's 64 x 64 block (2 x 2 blocks of
// 32).  tl is the lo tile of the split operand (SPLIT A or B): its products
// with the other operand go into the same accumulators.
template <int SPLIT>
__device__ __forceinline__ void tile_mfma(const char *ta, const char *tb, const char *tl, int wm, int wn, int lane,
                                          f32x16_t (&acc)[2][2]) {
    const int l5 = lane & 31, hk = (lane >> 5) * 16;
#pragma unroll
    for (int ss = 0; ss < 2; ss++) {
        uint4 a[2], b[2], lo[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            a[i] = *reinterpret_cast<const uint4 *>(ta + (wm * 64 + i * 32 + l5) * kRowB + ss * 32 + hk);
            if (SPLIT == kSplitA)
                lo[i] = *reinterpret_cast<const uint4 *>(tl + (wm * 64 + i * 32 + l5) * kRowB + ss * 32 + hk);
        }
#pragma unroll
        for (int j = 0; j < 2; j++) {
            b[j] = *reinterpret_cast<const uint4 *>(tb + (wn * 64 + j * 32 + l5) * kRowB + ss * 32 + hk);
            if (SPLIT == kSplitB)
                lo[j] = *reinterpret_cast<const uint4 *>(tl + (wn * 64 + j * 32 + l5) * kRowB + ss * 32 + hk);
        }
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) {
                acc[i][j] = mfma_bf16(a[i], b[j], acc[i][j]);
                if (SPLIT == kSplitA) acc[i][j] = mfma_bf16(lo[i], b[j], acc[i][j]);
                if (SPLIT == kSplitB) acc[i][j] = mfma_bf16(a[i], lo[j], acc[i][j]);
            }
    }
}

// fp32 tile store: element (row, col) at c[row * ldc + col], rows < mvalid,
// cols < nvalid (tile-relative).  The lane holds column l5 of each 32 x 32
// block, rows 8 (q / 4) + 4 (lane / 32) + q % 4.
__device__ __forceinline__ void store_acc(float *c, int64_t ldc, int mvalid, int nvalid, int wm, int wn, int lane,
                                          const f32x16_t (&acc)[2][2]) {
    const int l5 = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int q = 0; q < 16; q++) {
                const int row = wm * 64 + i * 32 + 8 * (q >> 2) + 4 * hi + (q & 3);
                const int col = wn * 64 + j * 32 + l5;
                if (row < mvalid && col < nvalid) c[(int64_t)row * ldc + col] = acc[i][j][q];
            }
}

// Grouped "NN" GEMM over the permuted rows: for the rows r of expert e,
//   C[r][n] = sum_k A[src(r)][k] B_e[k][n]  (+ sum_k A2[r][k] B2_e[k][n])
// A K-contiguous (rows gathered through a_rows, or the permuted rows), B_e
// row-major [K][N] (N-contiguous, transposed while staged).  C fp32 [R][N].
// SPLIT == kSplitA: A and A2 are hi/lo pairs, the lo part lo_off elements
// after the hi part.
template <int SPLIT>
__global__ __launch_bounds__(kBt) void grouped_nn(const uint16_t *__restrict__ A, const int32_t *__restrict__ a_rows,
                                                  const uint16_t *__restrict__ B, const uint16_t *__restrict__ A2,
                                                  const uint16_t *__restrict__ B2, size_t lo_off,
                                                  const int32_t *__restrict__ offsets, int E, int K, int N,
                                                  int ntiles_n, float *__restrict__ C) {
    __shared__ __attribute__((aligned(16))) char lds[2][3][kTileB];
    TileInfo ti;
    if (!find_tile(offsets, E, ntiles_n, kTm, 1, blockIdx.x, nullptr, nullptr, ti)) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
    const int n0 = ti.nt * kTn, valid = ti.mend - ti.m0;
    const int pairs = A2 ? 2 : 1;
    const int nk = K / kTk, steps = nk * pairs;
    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int q = 0; q < 16; q++) acc[i][j][q] = 0.0f;
    auto srcs = [&](int st, KcontigSrc &sa, RowcontigSrc &sb, int &k0) {
        const bool second = st >= nk;
        k0 = (second ? st - nk : st) * kTk;
        sa = KcontigSrc{second ? A2 : A, second ? nullptr : a_rows, K};
        sb = RowcontigSrc{(second ? B2 : B) + (size_t)ti.e * K * N, nullptr, N};
    };
    auto lo_of = [&](KcontigSrc a) {
        a.base += lo_off;
        return a;
    };
    KcontigSrc sa;
    RowcontigSrc sb;
    int k0;
    srcs(0, sa, sb, k0);
    Regs2 ra = load_kcontig(sa, ti.m0, valid, k0), rb = load_rowcontig(sb, k0, K, n0, N), rl;
    if (SPLIT == kSplitA) rl = load_kcontig(lo_of(sa), ti.m0, valid, k0);
    store_kcontig(lds[0][0], ra);
    store_rowcontig(lds[0][1], rb);
    if (SPLIT == kSplitA) store_kcontig(lds[0][2], rl);
    __syncthreads();
    for (int st = 0; st < steps; st++) {
        const int cur = st & 1;
        if (st + 1 < steps) {
            srcs(st + 1, sa, sb, k0);
            ra = load_kcontig(sa, ti.m0, valid, k0);
            rb = load_rowcontig(sb, k0, K, n0, N);
            if (SPLIT == kSplitA) rl = load_kcontig(lo_of(sa), ti.m0, valid, k0);
        }
        tile_mfma<SPLIT>(lds[cur][0], lds[cur][1], lds[cur][2], wm, wn, lane, acc);
        if (st + 1 < steps) {
            store_kcontig(lds[cur ^ 1][0], ra);
            store_rowcontig(lds[cur ^ 1][1], rb);
            if (SPLIT == kSplitA) store_kcontig(lds[cur ^ 1][2], rl);
        }
        __syncthreads();
    }
    store_acc(C + (size_t)ti.m0 * N + n0, N, valid, N - n0, wm, wn, lane, acc);
}

// Grouped-K "TN" GEMM, one output matrix per expert: for block (e, m, n),
//   C_e[m][n] = sum over the rows r of expert e of A[srcA(r)][m] B[srcB(r)][n]
// A and B row-major over the rows (M- and N-contiguous), transposed while
// staged.  C fp32 [E][M][N]; an expert without rows gets zeros.  SPLIT: A
// (kSplitA) or B (kSplitB) is a hi/lo pair, the lo part lo_off elements after
// the hi part.
template <int SPLIT>
__global__ __launch_bounds__(kBt) void grouped_tn(const uint16_t *__restrict__ A, const int32_t *__restrict__ a_rows,
                                                  int64_t lda, const uint16_t *__restrict__ B,
                                                  const int32_t *__restrict__ b_rows, int64_t ldb, size_t lo_off,
                                                  const int32_t *__restrict__ offsets, int M, int N, int mt, int nt,
                                                  float *__restrict__ C) {
    __shared__ __attribute__((aligned(16))) char lds[2][3][kTileB];
    const int e = blockIdx.x / (mt * nt), rem = blockIdx.x % (mt * nt);
    const int m0 = (rem / nt) * kTm, n0 = (rem % nt) * kTn;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
    const int rbeg = offsets[e], rend = offsets[e + 1];
    const RowcontigSrc sa{A, a_rows, lda}, sb{B, b_rows, ldb};
    // the lo part of the split operand (same rows, same layout)
    const RowcontigSrc sl = SPLIT == kSplitA ? RowcontigSrc{A + lo_off, a_rows, lda}
                                             : RowcontigSrc{B + lo_off, b_rows, ldb};
    const int l0 = SPLIT == kSplitA ? m0 : n0, lend = SPLIT == kSplitA ? M : N;
    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int q = 0; q < 16; q++) acc[i][j][q] = 0.0f;
    const int steps = (rend - rbeg + kTk - 1) / kTk;
    if (steps > 0) {
        Regs2 ra = load_rowcontig(sa, rbeg, rend, m0, M), rb = load_rowcontig(sb, rbeg, rend, n0, N), rl;
        if (SPLIT != kSplitNone) rl = load_rowcontig(sl, rbeg, rend, l0, lend);
        store_rowcontig(lds[0][0], ra);
        store_rowcontig(lds[0][1], rb);
        if (SPLIT != kSplitNone) store_rowcontig(lds[0][2], rl);
        __syncthreads();
        for (int st = 0; st < steps; st++) {
            const int cur = st & 1;
            if (st + 1 < steps) {
                const int k0 = rbeg + (st + 1) * kTk;
                ra = load_rowcontig(sa, k0, rend, m0, M);
                rb = load_rowcontig(sb, k0, rend, n0, N);
                if (SPLIT != kSplitNone) rl = load_rowcontig(sl, k0, rend, l0, lend);
            }
            tile_mfma<SPLIT>(lds[cur][0], lds[cur][1], lds[cur][2], wm, wn, lane, acc);
            if (st + 1 < steps) {
                store_rowcontig(lds[cur ^ 1][0], ra);
                store_rowcontig(lds[cur ^ 1][1], rb);
                if (SPLIT != kSplitNone) store_rowcontig(lds[cur ^ 1][2], rl);
            }
            __syncthreads();
        }
    }
    store_acc(C + ((size_t)e * M + m0) * N + n0, N, M - m0, N - n0, wm, wn, lane, acc);
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
// reduction), da = g u b silu'(a), db = g u silu(a), hg = g h, each stored as
// a bf16 hi/lo pair (lo at lo_off elements after hi).
__global__ __launch_bounds__(256) void swiglu_backward(const float *__restrict__ a, const float *__restrict__ b,
                                                       const float *__restrict__ u,
                                                       const float *__restrict__ gate_of_row,
                                                       const int32_t *__restrict__ offsets, int E, int dff,
                                                       size_t lo_off, uint16_t *__restrict__ da,
                                                       uint16_t *__restrict__ db, uint16_t *__restrict__ hg,
                                                       float *__restrict__ dg) {
    __shared__ float part[256];
    const int r = blockIdx.x;
    if (r >= offsets[E]) return;
    const float g = gate_of_row[r];
    const size_t o = (size_t)r * dff;
    float s = 0.0f;
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
        }
        store_hi_lo(da + o + f, lo_off, dav);
        store_hi_lo(db + o + f, lo_off, dbv);
        store_hi_lo(hg + o + f, lo_off, hv);
    }
    part[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) dg[r] = part[0];
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
__global__ __launch_bounds__(256) void input_grad(const float *__restrict__ dx_perm, const uint16_t *__restrict__ wr,
                                                  const int32_t *__restrict__ row, const int32_t *__restrict__ eid,
                                                  const float *__restrict__ ds_of_row, int k, int d,
                                                  float *__restrict__ dx) {
    const int t = blockIdx.x;
    int rws[kMaxTopK], es[kMaxTopK];
    float ds[kMaxTopK];
    for (int j = 0; j < k; j++) {
        rws[j] = row[(size_t)t * k + j];
        es[j] = eid[(size_t)t * k + j];
        ds[j] = rws[j] >= 0 ? ds_of_row[rws[j]] : 0.0f;
    }
    for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int j = 0; j < k; j++) {
            if (rws[j] < 0) continue;
            const float4 *p = reinterpret_cast<const float4 *>(dx_perm + (size_t)rws[j] * d + c);
            const float4 v0 = p[0], v1 = p[1];
            acc[0] += v0.x; acc[1] += v0.y; acc[2] += v0.z; acc[3] += v0.w;
            acc[4] += v1.x; acc[5] += v1.y; acc[6] += v1.z; acc[7] += v1.w;
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

// dW_r[e][c] = sum over the rows r of expert e of ds_r x[tok_r][c] (row
// order); block (e, column chunk of 256); dbias[e] = sum_r ds_r.
__global__ __launch_bounds__(256) void router_wgrad(const uint16_t *__restrict__ x,
                                                    const int32_t *__restrict__ token_of_row,
                                                    const float *__restrict__ ds_of_row,
                                                    const int32_t *__restrict__ offsets, int d, int nchunk,
                                                    float *__restrict__ dwr, float *__restrict__ dbias) {
    const int e = blockIdx.x / nchunk, c = (blockIdx.x % nchunk) * 256 + threadIdx.x;
    const int rb = offsets[e], re = offsets[e + 1];
    float acc = 0.0f, sb = 0.0f;
    for (int r = rb; r < re; r++) {
        const float ds = ds_of_row[r];
        sb += ds;
        if (c < d) acc = fmaf(ds, bf16_bits_to_f32(x[(size_t)token_of_row[r] * d + c]), acc);
    }
    if (c < d) dwr[(size_t)e * d + c] = acc;
    if (blockIdx.x % nchunk == 0 && threadIdx.x == 0) dbias[e] = sb;
}

}  // namespace

hipError_t launch_backward(const moe_params &p, int64_t max_rows, int64_t cap, const BackwardArgs &a, hipStream_t st) {
    const int T = p.T, d = p.d, E = p.E, k = p.k, dff = p.d_ff;
    const int64_t R = max_rows;
    const int mt1 = (int)ceil_div(dff, kTm), nt1 = (int)ceil_div(d, kTn);  // dW1, dW3: [d_ff][d]
    const int mt2 = (int)ceil_div(d, kTm), nt2 = (int)ceil_div(dff, kTn);  // dW2: [d][d_ff]
    if (T == 0) {
        // no tokens: every weight gradient is zero (no expert has rows)
        const uint16_t *none = nullptr;
        const int32_t *nrow = nullptr;
        hipLaunchKernelGGL(grouped_tn<kSplitNone>, dim3((unsigned)(E * mt1 * nt1)), dim3(kBt), 0, st, none, nrow,
                           (int64_t)0, none, nrow, (int64_t)0, (size_t)0, a.offsets, dff, d, mt1, nt1, a.dw1);
        hipLaunchKernelGGL(grouped_tn<kSplitNone>, dim3((unsigned)(E * mt1 * nt1)), dim3(kBt), 0, st, none, nrow,
                           (int64_t)0, none, nrow, (int64_t)0, (size_t)0, a.offsets, dff, d, mt1, nt1, a.dw3);
        hipLaunchKernelGGL(grouped_tn<kSplitNone>, dim3((unsigned)(E * mt2 * nt2)), dim3(kBt), 0, st, none, nrow,
                           (int64_t)0, none, nrow, (int64_t)0, (size_t)0, a.offsets, d, dff, mt2, nt2, a.dw2);
        hipLaunchKernelGGL(router_wgrad, dim3((unsigned)(E * ceil_div(d, 256))), dim3(256), 0, st,
                           static_cast<const uint16_t *>(a.x), a.token_of_row, a.ds_of_row, a.offsets, d,
                           (int)ceil_div(d, 256), a.dw_router, a.dbias);
        return hipGetLastError();
    }
    const float inv_tau = 1.0f / (p.gate_temperature > 0.0f ? p.gate_temperature : 1.0f);
    const uint16_t *x = static_cast<const uint16_t *>(a.x);
    const uint16_t *dy = static_cast<const uint16_t *>(a.dy);
    const size_t lo_off = (size_t)R * dff;  // lo parts of da, db, hg follow their hi parts
    const int64_t mt = std::min<int64_t>(R / kTm + E, (int64_t)E * ceil_div(cap, kTm));
    // 1. the rows' gates; a and b recomputed by the gate-up GEMM
    hipLaunchKernelGGL(row_gates, dim3((unsigned)ceil_div((int64_t)T * k, 256)), dim3(256), 0, st, a.row, a.gate,
                       T * k, a.gate_of_row);
    hipError_t e = launch_gate_up_raw(p, R, cap, a.x, a.token_of_row, a.offsets, a.w1, a.w3, a.a, a.b, st);
    if (e != hipSuccess) return e;
    // 2. u = W2_e^T dy_t for every kept row
    const int nt_u = (int)ceil_div(dff, kTn);
    hipLaunchKernelGGL(grouped_nn<kSplitNone>, dim3((unsigned)(mt * nt_u)), dim3(kBt), 0, st, dy, a.token_of_row,
                       static_cast<const uint16_t *>(a.w2), (const uint16_t *)nullptr, (const uint16_t *)nullptr,
                       (size_t)0, a.offsets, E, d, dff, nt_u, a.u);
    // 3. SwiGLU backward per row, 4. gate softmax backward per token
    hipLaunchKernelGGL(swiglu_backward, dim3((unsigned)R), dim3(256), 0, st, a.a, a.b, a.u, a.gate_of_row, a.offsets,
                       E, dff, lo_off, a.da, a.db, a.hg, a.dg);
    hipLaunchKernelGGL(gate_backward, dim3((unsigned)ceil_div(T, 256)), dim3(256), 0, st, a.row, a.eid, a.gate, a.dg,
                       T, E, k, inv_tau, a.dlogits, a.ds_of_row);
    // 5. dx_perm = W1_e^T da + W3_e^T db, 6. dx
    const int nt_x = (int)ceil_div(d, kTn);
    hipLaunchKernelGGL(grouped_nn<kSplitA>, dim3((unsigned)(mt * nt_x)), dim3(kBt), 0, st, (const uint16_t *)a.da,
                       (const int32_t *)nullptr, static_cast<const uint16_t *>(a.w1), (const uint16_t *)a.db,
                       static_cast<const uint16_t *>(a.w3), lo_off, a.offsets, E, dff, d, nt_x, a.dx_perm);
    hipLaunchKernelGGL(input_grad, dim3((unsigned)T), dim3(256), 0, st, a.dx_perm,
                       static_cast<const uint16_t *>(a.w_router), a.row, a.eid, a.ds_of_row, k, d, a.dx);
    // 7. dW1 = da^T x, dW3 = db^T x, dW2 = dy^T (g h)
    hipLaunchKernelGGL(grouped_tn<kSplitA>, dim3((unsigned)(E * mt1 * nt1)), dim3(kBt), 0, st, (const uint16_t *)a.da,
                       (const int32_t *)nullptr, (int64_t)dff, x, a.token_of_row, (int64_t)d, lo_off, a.offsets, dff,
                       d, mt1, nt1, a.dw1);
    hipLaunchKernelGGL(grouped_tn<kSplitA>, dim3((unsigned)(E * mt1 * nt1)), dim3(kBt), 0, st, (const uint16_t *)a.db,
                       (const int32_t *)nullptr, (int64_t)dff, x, a.token_of_row, (int64_t)d, lo_off, a.offsets, dff,
                       d, mt1, nt1, a.dw3);
    hipLaunchKernelGGL(grouped_tn<kSplitB>, dim3((unsigned)(E * mt2 * nt2)), dim3(kBt), 0, st, dy, a.token_of_row,
                       (int64_t)d, (const uint16_t *)a.hg, (const int32_t *)nullptr, (int64_t)dff, lo_off, a.offsets,
                       d, dff, mt2, nt2, a.dw2);
    // 8. router weight and bias gradients
    hipLaunchKernelGGL(router_wgrad, dim3((unsigned)(E * ceil_div(d, 256))), dim3(256), 0, st, x, a.token_of_row,
                       a.ds_of_row, a.offsets, d, (int)ceil_div(d, 256), a.dw_router, a.dbias);
    return hipGetLastError();
}

}  // namespace moe
