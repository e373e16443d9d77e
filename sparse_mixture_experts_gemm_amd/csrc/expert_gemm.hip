// Stage 3: expert SwiGLU FFN as two grouped GEMMs over the permuted rows.
//
// What it computes ("GPT-4稀疏激活真相" §3.1: each expert is
// Linear -> SwiGLU -> Linear; "企业官网建设流程全解析" page §1: the expert's
// W1/W2/W3 matrices), for the rows [offsets[e], offsets[e+1]) of expert e:
//   h      = silu(x_perm . W1[e]^T) * (x_perm . W3[e]^T)     gate-up GEMM
//   y_perm = h . W2[e]^T                                      down GEMM
// Precision of the bf16 layer: the gate-up GEMM is bf16 x bf16 on the matrix
// cores; h is stored as fp16 (ten mantissa bits, so its rounding error is an
// eighth of bf16's; saturated at +-65504); the down GEMM is fp16 x fp16, with
// W2 widened from bf16 to fp16 while it is staged into LDS (exact for weights
// of magnitude 2^-14..65504); y_perm is stored in fp32, so the layer output
// is rounded to bf16 once, in the combine.
// Both products are "NT": the activation rows and the weight rows are
// contiguous along K (nn.Linear layout), which is the natural operand layout
// of the matrix cores: a lane's MFMA fragment is 8 consecutive K elements.
//
// bf16 path (gfx950 MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   * 256 threads = 4 waves in a 2x2 grid; block tile 256 rows x 256 weight
//     rows, K step 64.  In the gate-up GEMM the 256 weight rows are 128 rows
//     of W1 and the same 128 rows of W3, so every wave holds the W1 and W3
//     accumulators of the same h elements and applies silu(a)*b in registers.
//   * A and B K-slices are staged in LDS, double-buffered (one barrier per K
//     step), with an XOR swizzle of the 16-byte chunks so the MFMA fragment
//     reads (16 lanes = 16 rows at one K chunk) hit distinct banks.
//   * The grid is one flat list of (expert, n-tile, m-tile) tiles sized by
//     the row bound; each block finds its tile from the device-side offsets,
//     blocks past the last tile exit.  m-tiles of one (expert, n-tile) are
//     adjacent so they share weight tiles, and the block index is remapped so
//     that adjacent tiles land on the same XCD (blocks are dealt round-robin
//     over the 8 XCDs) and share its L2.
//   * 32-row MFMA blocks that lie wholly past an expert's last row are
//     skipped, so ragged tails and small groups cost little matrix-core time.
// fp32 path (the tiny fp32 layer): a plain LDS-tiled VALU GEMM.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kGemmThreads = 256;
constexpr int kBM = 256;   // rows per tile
constexpr int kBN = 256;   // weight rows per tile (gate-up: 128 of W1 + 128 of W3)
constexpr int kBK = 64;    // K per stage
constexpr int kChunksPerRow = kBK / 8;  // 16-byte chunks per tile row
constexpr int kTileBytes = kBM * kBK * 2;  // one operand tile, bf16
constexpr int kStageBytes = 2 * kTileBytes;
constexpr int kLdsBytes = 2 * kStageBytes;  // double-buffered

enum { kGateUp = 0, kDown = 1 };

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// byte offset of chunk c of row r in a swizzled tile
__device__ __forceinline__ int tile_off(int r, int c) { return r * (kBK * 2) + ((c ^ swz(r)) << 4); }

// Flat tile index -> (expert, m range, n tile).  Returns false past the end.
struct TileInfo {
    int e, m0, mend, nt;
};

__device__ __forceinline__ bool find_tile(const int32_t *__restrict__ offsets, int E, int ntiles_n,
                                          int bm, int L, TileInfo &ti) {
    int base = 0;
    for (int e = 0; e < E; e++) {
        const int beg = offsets[e], end = offsets[e + 1];
        const int mt = (end - beg + bm - 1) / bm;
        const int cnt = mt * ntiles_n;
        if (L < base + cnt) {
            const int local = L - base;
            ti.e = e;
            ti.nt = local / mt;
            ti.m0 = beg + (local % mt) * bm;
            ti.mend = end;
            return true;
        }
        base += cnt;
    }
    return false;
}

// Round-robin XCD placement: block b runs on XCD b % 8.  Give each XCD a
// contiguous range of logical tiles.
__device__ __forceinline__ int xcd_remap(int b, int nblk) {
    const int q = nblk / 8, rem = nblk % 8;
    const int xcd = b % 8, local = b / 8;
    const int start = xcd * q + min(xcd, rem);
    return start + local;
}

__device__ __forceinline__ float silu_mul(float a, float b) {
    return a / (1.0f + __expf(-a)) * b;
}

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// two bf16 -> two fp16 (exact in fp16's normal range)
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t v) {
    const float lo = __uint_as_float(v << 16), hi = __uint_as_float(v & 0xFFFF0000u);
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 v) {
    return make_uint4(bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z),
                      bf16x2_to_f16x2(v.w));
}

__device__ __forceinline__ uint16_t f32_to_f16_sat(float v) {
    v = fminf(fmaxf(v, -65504.0f), 65504.0f);
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// One MFMA step on 8-element fragments held as raw 16-byte words.
template <bool F16>
__device__ __forceinline__ f32x16_t mfma32(uint4 a, uint4 b, f32x16_t c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// MODE kGateUp: A = x_perm (bf16), B = W1/W3 (bf16), writes h (fp16).
// MODE kDown:   A = h (fp16), B = W2 (bf16, widened to fp16 into LDS),
//               writes y_perm (fp32).
template <int MODE>
__global__ __launch_bounds__(kGemmThreads, 1) void grouped_gemm_bf16(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B0, const uint16_t *__restrict__ B1,
    const int32_t *__restrict__ offsets, int E, int N, int K, int ntiles_n,
    void *__restrict__ out_v) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    TileInfo ti;
    if (!find_tile(offsets, E, ntiles_n, kBM, xcd_remap(blockIdx.x, gridDim.x), ti)) return;

    // n0: first output column of the tile; weight rows of the tile
    const int n0 = MODE == kGateUp ? ti.nt * (kBN / 2) : ti.nt * kBN;
    const size_t wexp = (size_t)ti.e * N * K;

    // global source of the chunks this thread loads: 8 A chunks and 8 B chunks
    const int lrow = tid >> 3;  // 0..31, + 32*j
    const int lc = tid & 7;
    const uint16_t *a_src[8];
    const uint16_t *b_src[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const int r = lrow + 32 * j;
        int gm = ti.m0 + r;
        if (gm >= ti.mend) gm = ti.mend - 1;
        a_src[j] = A + (size_t)gm * K + lc * 8;
        int gn;
        const uint16_t *B;
        if (MODE == kGateUp) {
            B = r < kBN / 2 ? B0 : B1;
            gn = n0 + (r & (kBN / 2 - 1));
        } else {
            B = B0;
            gn = n0 + r;
        }
        if (gn >= N) gn = N - 1;
        b_src[j] = B + wexp + (size_t)gn * K + lc * 8;
    }
    int st_off[8];
#pragma unroll
    for (int j = 0; j < 8; j++) st_off[j] = tile_off(lrow + 32 * j, lc);

    // MFMA blocks of this wave: rows wm*128 + i*32, weight rows per jn
    bool act[4];
#pragma unroll
    for (int i = 0; i < 4; i++) act[i] = ti.m0 + wm * 128 + i * 32 < ti.mend;
    int brow[4];
#pragma unroll
    for (int jn = 0; jn < 4; jn++) {
        if (MODE == kGateUp)
            brow[jn] = (jn < 2 ? 0 : kBN / 2) + wn * 64 + (jn & 1) * 32;
        else
            brow[jn] = wn * 128 + jn * 32;
    }
    const int fr = lane & 31;   // fragment row within a 32-row block
    const int fk = lane >> 5;   // which 8-element half of a 16-wide K slice

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int jn = 0; jn < 4; jn++)
#pragma unroll
            for (int q = 0; q < 16; q++) acc[i][jn][q] = 0.0f;

    const int nk = K / kBK;
    uint4 ra[8], rb[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        ra[j] = *reinterpret_cast<const uint4 *>(a_src[j]);
        rb[j] = *reinterpret_cast<const uint4 *>(b_src[j]);
    }
    constexpr bool kF16 = MODE == kDown;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        *reinterpret_cast<uint4 *>(lds + st_off[j]) = ra[j];
        *reinterpret_cast<uint4 *>(lds + kTileBytes + st_off[j]) = kF16 ? bf16x8_to_f16x8(rb[j]) : rb[j];
    }
    __syncthreads();

    for (int kt = 0; kt < nk; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            const size_t ko = (size_t)(kt + 1) * kBK;
#pragma unroll
            for (int j = 0; j < 8; j++) {
                ra[j] = *reinterpret_cast<const uint4 *>(a_src[j] + ko);
                rb[j] = *reinterpret_cast<const uint4 *>(b_src[j] + ko);
            }
        }
        const char *sa = lds + cur * kStageBytes;
        const char *sb = sa + kTileBytes;
#pragma unroll
        for (int s = 0; s < kBK / 16; s++) {
            const int c = s * 2 + fk;
            uint4 af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; i++)
                af[i] = *reinterpret_cast<const uint4 *>(sa + tile_off(wm * 128 + i * 32 + fr, c));
#pragma unroll
            for (int jn = 0; jn < 4; jn++)
                bfr[jn] = *reinterpret_cast<const uint4 *>(sb + tile_off(brow[jn] + fr, c));
#pragma unroll
            for (int i = 0; i < 4; i++) {
                if (!act[i]) continue;
#pragma unroll
                for (int jn = 0; jn < 4; jn++) acc[i][jn] = mfma32<kF16>(af[i], bfr[jn], acc[i][jn]);
            }
        }
        if (kt + 1 < nk) {
            char *da = lds + (cur ^ 1) * kStageBytes;
#pragma unroll
            for (int j = 0; j < 8; j++) {
                *reinterpret_cast<uint4 *>(da + st_off[j]) = ra[j];
                *reinterpret_cast<uint4 *>(da + kTileBytes + st_off[j]) = kF16 ? bf16x8_to_f16x8(rb[j]) : rb[j];
            }
        }
        __syncthreads();
    }

    // epilogue: lane holds column fr of each 32x32 block, rows 8*(q/4) + 4*fk + q%4
    const int ldo = N;
    uint16_t *out_h = static_cast<uint16_t *>(out_v);
    float *out_y = static_cast<float *>(out_v);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        if (!act[i]) continue;
        const int rbase = ti.m0 + wm * 128 + i * 32 + 4 * fk;
        if (MODE == kGateUp) {
#pragma unroll
            for (int jn = 0; jn < 2; jn++) {
                const int col = n0 + wn * 64 + jn * 32 + fr;
                if (col >= N) continue;
#pragma unroll
                for (int q = 0; q < 16; q++) {
                    const int m = rbase + 8 * (q >> 2) + (q & 3);
                    if (m < ti.mend)
                        out_h[(size_t)m * ldo + col] = f32_to_f16_sat(silu_mul(acc[i][jn][q], acc[i][jn + 2][q]));
                }
            }
        } else {
#pragma unroll
            for (int jn = 0; jn < 4; jn++) {
                const int col = n0 + wn * 128 + jn * 32 + fr;
                if (col >= N) continue;
#pragma unroll
                for (int q = 0; q < 16; q++) {
                    const int m = rbase + 8 * (q >> 2) + (q & 3);
                    if (m < ti.mend) out_y[(size_t)m * ldo + col] = acc[i][jn][q];
                }
            }
        }
    }
}

// ---------------------------------------------------------------- fp32 ----
constexpr int kF32BM = 64, kF32BN = 64, kF32BK = 16;

template <int MODE>
__global__ __launch_bounds__(256) void grouped_gemm_f32(const float *__restrict__ A,
                                                        const float *__restrict__ B0,
                                                        const float *__restrict__ B1,
                                                        const int32_t *__restrict__ offsets, int E,
                                                        int N, int K, int ntiles_n,
                                                        float *__restrict__ out) {
    __shared__ float sa[kF32BK][kF32BM + 1];
    __shared__ float sb0[kF32BK][kF32BN + 1];
    __shared__ float sb1[kF32BK][kF32BN + 1];
    TileInfo ti;
    if (!find_tile(offsets, E, ntiles_n, kF32BM, blockIdx.x, ti)) return;
    const int n0 = ti.nt * kF32BN;
    const size_t wexp = (size_t)ti.e * N * K;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;  // 4x4 outputs each
    float c0[4][4] = {}, c1[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += kF32BK) {
        for (int i = threadIdx.x; i < kF32BM * kF32BK; i += 256) {
            const int r = i / kF32BK, kk = i % kF32BK;
            int gm = ti.m0 + r;
            if (gm >= ti.mend) gm = ti.mend - 1;
            sa[kk][r] = A[(size_t)gm * K + k0 + kk];
            int gn = n0 + r;
            if (gn >= N) gn = N - 1;
            sb0[kk][r] = B0[wexp + (size_t)gn * K + k0 + kk];
            if (MODE == kGateUp) sb1[kk][r] = B1[wexp + (size_t)gn * K + k0 + kk];
        }
        __syncthreads();
        for (int kk = 0; kk < kF32BK; kk++) {
            float av[4], bv0[4], bv1[4];
            for (int i = 0; i < 4; i++) av[i] = sa[kk][ty * 4 + i];
            for (int j = 0; j < 4; j++) {
                bv0[j] = sb0[kk][tx * 4 + j];
                if (MODE == kGateUp) bv1[j] = sb1[kk][tx * 4 + j];
            }
            for (int i = 0; i < 4; i++)
                for (int j = 0; j < 4; j++) {
                    c0[i][j] = __builtin_fmaf(av[i], bv0[j], c0[i][j]);
                    if (MODE == kGateUp) c1[i][j] = __builtin_fmaf(av[i], bv1[j], c1[i][j]);
                }
        }
        __syncthreads();
    }
    for (int i = 0; i < 4; i++) {
        const int m = ti.m0 + ty * 4 + i;
        if (m >= ti.mend) continue;
        for (int j = 0; j < 4; j++) {
            const int col = n0 + tx * 4 + j;
            if (col >= N) continue;
            out[(size_t)m * N + col] = MODE == kGateUp ? silu_mul(c0[i][j], c1[i][j]) : c0[i][j];
        }
    }
}

// Dynamic LDS above the default limit must be allowed per kernel.
hipError_t allow_lds(const void *kernel, int bytes) {
    return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

}  // namespace

hipError_t launch_expert_ffn(const moe_params &p, int64_t max_rows, const void *x_perm,
                             const int32_t *offsets, const void *w1, const void *w3,
                             const void *w2, void *h, void *y_perm, hipStream_t st) {
    if (max_rows <= 0) return hipSuccess;
    const int E = p.E, d = p.d, dff = p.d_ff;
    if (p.dtype == MOE_BF16) {
        const int64_t mt = max_rows / kBM + E;  // bound on sum_e ceil(rows_e / kBM)
        const int nt_up = (int)ceil_div(dff, kBN / 2);
        const int nt_dn = (int)ceil_div(d, kBN);
        hipError_t e = allow_lds(reinterpret_cast<const void *>(&grouped_gemm_bf16<kGateUp>), kLdsBytes);
        if (e != hipSuccess) return e;
        e = allow_lds(reinterpret_cast<const void *>(&grouped_gemm_bf16<kDown>), kLdsBytes);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(grouped_gemm_bf16<kGateUp>, dim3((unsigned)(mt * nt_up)), dim3(kGemmThreads),
                           kLdsBytes, st, static_cast<const uint16_t *>(x_perm),
                           static_cast<const uint16_t *>(w1), static_cast<const uint16_t *>(w3),
                           offsets, E, dff, d, nt_up, h);
        hipLaunchKernelGGL(grouped_gemm_bf16<kDown>, dim3((unsigned)(mt * nt_dn)), dim3(kGemmThreads),
                           kLdsBytes, st, static_cast<const uint16_t *>(h),
                           static_cast<const uint16_t *>(w2), static_cast<const uint16_t *>(w2),
                           offsets, E, d, dff, nt_dn, y_perm);
    } else {
        const int64_t mt = max_rows / kF32BM + E;
        const int nt_up = (int)ceil_div(dff, kF32BN);
        const int nt_dn = (int)ceil_div(d, kF32BN);
        hipLaunchKernelGGL(grouped_gemm_f32<kGateUp>, dim3((unsigned)(mt * nt_up)), dim3(256), 0, st,
                           static_cast<const float *>(x_perm), static_cast<const float *>(w1),
                           static_cast<const float *>(w3), offsets, E, dff, d, nt_up,
                           static_cast<float *>(h));
        hipLaunchKernelGGL(grouped_gemm_f32<kDown>, dim3((unsigned)(mt * nt_dn)), dim3(256), 0, st,
                           static_cast<const float *>(h), static_cast<const float *>(w2),
                           static_cast<const float *>(w2), offsets, E, d, dff, nt_dn,
                           static_cast<float *>(y_perm));
    }
    return hipGetLastError();
}

}  // namespace moe
