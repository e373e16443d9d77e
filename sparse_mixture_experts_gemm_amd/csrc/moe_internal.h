// Internal interface between the C ABI (moe_api.cpp) and the HIP kernels.
#pragma once

#include <math.h>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 8;
constexpr int kDispatchBlock = 1024;  // tokens per dispatch block

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// Dispatch scratch: per-block histograms of the primary rounds and of the
// fallback round, and the per-expert fill after the primary rounds.
struct DispatchScratch {
    int32_t *hist;       // [NB][k][E]
    int32_t *fb_hist;    // [NB][E]
    int32_t *fill_prim;  // [E]
    int32_t *claim = nullptr;  // [kClaimCounters] zeroed by the dispatch for the GEMM's work claims, or null
    float *gate_of_row = nullptr;  // [R] each kept row's gate (the down projection folds it in), or null
};

// Work-claim counters of the expert GEMM (one per XCD, gate-up then down).
constexpr int kClaimCounters = 16;
// The down projection's split plan (find_tile_planned): items per round
// (the chip's CUs) and the most K slices of a split tile.
constexpr int kPlanCUs = 256;
constexpr int kPlanMaxS = 8;

inline size_t dispatch_scratch_bytes(int T, int E, int k) {
    int64_t nb = ceil_div(T > 0 ? T : 1, kDispatchBlock);
    return align256(sizeof(int32_t) * nb * k * E) + align256(sizeof(int32_t) * nb * E) +
           align256(sizeof(int32_t) * E);
}

inline DispatchScratch carve_dispatch(void *ws, int T, int E, int k) {
    int64_t nb = ceil_div(T > 0 ? T : 1, kDispatchBlock);
    char *p = static_cast<char *>(ws);
    DispatchScratch s;
    s.hist = reinterpret_cast<int32_t *>(p);
    p += align256(sizeof(int32_t) * nb * k * E);
    s.fb_hist = reinterpret_cast<int32_t *>(p);
    p += align256(sizeof(int32_t) * nb * E);
    s.fill_prim = reinterpret_cast<int32_t *>(p);
    return s;
}

hipError_t launch_route(const moe_params &p, const void *x, const void *wr, const float *bias,
                        const float *load, float *logits, int32_t *cand, float *cand_score,
                        hipStream_t st);

// x_perm == nullptr: routing only, no copy of the token rows.
hipError_t launch_dispatch(const moe_params &p, int64_t C, const void *x, const moe_routing &r,
                           void *x_perm, const DispatchScratch &ws, hipStream_t st);

// Windowed load statistic: counts [ceil(T/window)][E] int32 scratch.
hipError_t launch_load_window(const moe_params &p, const int32_t *cand, int window, float decay, float *load,
                              int32_t *counts, hipStream_t st);

// Capacity C = min(T, ceil(T*k/E * cf)) evaluated in double, cf the
// capacity_factor, or 1 + 0.01 * log2(T) with dynamic_capacity; a
// capacity_factor <= 0 (without dynamic_capacity) means uncapped (C = T).
inline int64_t capacity_rows(const moe_params &p) {
    if (!p.dynamic_capacity && p.capacity_factor <= 0.0f) return p.T;
    const double cf = p.dynamic_capacity ? (p.T >= 1 ? 1.0 + 0.01 * log2((double)p.T) : 1.0)
                                         : (double)p.capacity_factor;
    const double c = ceil((double)p.T * (double)p.k / (double)p.E * cf);
    // clamp before the conversion: an infinite or huge factor gives C = T
    // (converting a double beyond the int64_t range is undefined)
    if (!(c < (double)p.T)) return p.T;
    int64_t C = (int64_t)c;
    if (C < 0) C = 0;
    return C;
}

// Number of d_ff slices the down projection is split into (each slice
// stores its partial product; the fix-up or the combine adds them in slice
// order).  1 for fp32 layers.
int ffn_splits(const moe_params &p, int64_t max_rows);

// Where the expert GEMM writes.  Gate-up: h at y0.  Down: the partial
// product of d_ff slice s goes to y0 (s = 0) or to y_rest + (s - 1) * stride
// elements; with row_gate null each partial is stored in fp32 (the layer's
// element type for fp32 layers), otherwise as the fp16 of row_gate[row] *
// partial (the combine weight folded in, saturated at +-65504; bf16 layers).
// With plan set (the 256-row down GEMM of moe_forward), the slices follow
// the device-side split plan of find_tile_planned instead: slice 0 of every
// row at y0, slice s >= 1 of a split row r at y_rest + ((s - 1) * srows +
// r - row0) * d elements, and plan[0..2] = {row0, S, srows} is stored for
// the combine.  At most plan_extra_elems(...) elements past y_rest are used.
struct GemmOut {
    void *y0;
    void *y_rest;
    size_t stride;
    const float *row_gate;
    int32_t *plan = nullptr;
    float scale = 1.0f;  // kPlainH (weight gradients on scaled fp16): the epilogue's factor
};

// Elements of the planned down projection's second slice buffer: (S - 1)
// split rows of d each, with S G ntn <= 256 and S <= plan_max_splits: at most
// 256 * 256 * 256 (d <= 256 ntn) and at most (plan_max_splits - 1) R d.
inline size_t plan_extra_elems(int64_t max_rows, int d, int d_ff) {
    const int64_t nk = d_ff / 64;
    const int64_t smax = nk / 8 < 1 ? 1 : (nk / 8 > 8 ? 8 : nk / 8);
    const int64_t a = (smax - 1) * max_rows * d, b = (int64_t)1 << 24;
    return (size_t)(a < b ? a : b);
}

// a_rows == nullptr: A is x_perm.  Otherwise A is the unpermuted x and packed
// row m is x row a_rows[m] (token_of_row); x must span less than 2 GiB.
// cap bounds the rows of any one expert (the capacity C).  claim: null, or
// kClaimCounters zeroed ints through which the 256-row GEMM's blocks claim
// their work items (an XCD whose range is done takes items of another).
// mid: null, or an event recorded between the gate-up and down launches.
// splits: the down projection's uniform slices (ignored with down.plan; the
// weight-streaming kernel's down projection honours it too).
hipError_t launch_expert_ffn(const moe_params &p, int64_t max_rows, int64_t cap, const void *x_perm,
                             const int32_t *a_rows, const int32_t *offsets, const void *w1,
                             const void *w3, const void *w2, void *h, const GemmOut &down, int32_t *claim,
                             hipEvent_t mid, hipStream_t st, int splits);

// y_perm[r] += rest[0][r] + ... + rest[nrest-1][r] (slices max_rows * d
// apart) for the rows below offsets[E]: a split down projection reduced in
// slice order.
hipError_t launch_ffn_fixup(const moe_params &p, int64_t max_rows, const int32_t *offsets, float *y_perm,
                            const float *rest, int nrest, hipStream_t st);

// One-byte (E4M3 or INT8) expert weights with fp32 row scales, bf16 layers:
// the weight-streaming kernel when every expert holds at most 32 rows (d and
// d_ff multiples of 128), else the 256 x 256 MFMA tile with the codes widened
// in registers, the down projection cut into `splits` K slices as for bf16
// weights (ffn_splits) and claim counters as for launch_expert_ffn.
// fp8_ffn_supported tells whether a layer qualifies.
bool fp8_ffn_supported(const moe_params &p);
// INT4 codes (two per byte): the weight-streaming kernel only, so every
// expert must hold at most 32 rows (d and d_ff multiples of 128)
bool q4_ffn_supported(const moe_params &p);
// weight code formats
enum { MOE_Q_E4M3 = 0, MOE_Q_INT8 = 1, MOE_Q_INT4 = 2 };
hipError_t launch_expert_ffn_fp8(const moe_params &p, int64_t max_rows, int64_t cap, const void *x_perm,
                                 const int32_t *a_rows, const int32_t *offsets, const uint8_t *w1, const float *s1,
                                 const uint8_t *w3, const float *s3, const uint8_t *w2, const float *s2, void *h,
                                 const GemmOut &down, int splits, int32_t *claim, hipEvent_t mid, int qfmt,
                                 hipStream_t st);

// The gate-up GEMM storing its two products a = x W1^T and b = x W3^T
// (fp32 [R][d_ff] each) for the kept rows; rows read from x through a_rows
// (token_of_row; x below 2 GiB).
hipError_t launch_gate_up_raw(const moe_params &p, int64_t max_rows, int64_t cap, const void *x,
                              const int32_t *a_rows, const int32_t *offsets, const void *w1, const void *w3,
                              float *a, float *b, hipStream_t st);

// C = A B_e^T over the kept rows of every expert, bf16 operands, fp32
// result (the backward pass's grouped GEMMs): A [rows][K] (the permuted
// rows, or rows of a matrix spanning a_span_bytes < 2 GiB through a_rows),
// C [max_rows][N].  B is [E][N][ldb] (K-contiguous), or with b_n_contig
// [E][ldb][N] (N-contiguous: C = A B_e) with B and B1 taken in turn by
// consecutive K periods of ldb.  K is cut into S slices (K / S a multiple
// of 64 that divides ldb); slice s reads B at K position (s K / S) mod ldb,
// so slices can share one B; slice s > 0 stores its partial product at
// rest + (s - 1) max_rows N, and a fix-up adds the slices into C in order.
// a_f16 (with b_n_contig): A holds fp16 values, and B is widened to fp16.
// fixup false: the slices are left apart for the caller to add in order.
int plain_gemm_splits(int64_t max_rows, int E, int N, int K, int ldb);
hipError_t launch_plain_gemm(int64_t max_rows, int64_t cap, int E, const uint16_t *A, const int32_t *a_rows,
                             int64_t a_span_bytes, const int32_t *offsets, const uint16_t *B, const uint16_t *B1,
                             bool b_n_contig, int N, int K, int ldb, int S, float *C, float *rest, hipStream_t st,
                             bool a_f16 = false, bool fixup = true);

// Per-expert K windows of the backward's transposed operands: the kept rows
// of expert e (rows_e of them, from offsets[e]) become K positions
// [kwin_start, kwin_start + 2 Kp_e) of a matrix with ldk columns, Kp_e =
// rows_e rounded up to 64: the rows and zero padding, then the same for the
// lo part of a hi/lo pair (or a second copy).  Windows of consecutive experts
// never overlap, and all fit in backward_ldk(max_rows, E) columns.
constexpr int kwin_start(int rbeg, int e) { return 2 * (((rbeg + 63) & ~63) + 64 * e); }
constexpr int64_t backward_ldk(int64_t max_rows, int E) { return 2 * (((max_rows + 63) & ~(int64_t)63) + 64 * (int64_t)E); }

// Weight gradients: C_e = A_e B_e^T over expert e's K window, A [M][ldk],
// B [N][ldk] bf16, C fp32 [E][M][N] (zeros for an expert without rows);
// unit_offsets[e] = e M (E + 1 ints).  256 rows of ldk elements must stay
// below 2 GiB.  With amax: A and B fp16 over the first half of each window
// only, one of them scaled by 2^grad_scale_exp(amax[e]) and, with gmax, the
// other by 2^grad_scale_exp(*gmax), which C undoes.
hipError_t launch_wgrad_gemm(int E, const uint16_t *A, const uint16_t *B, const int32_t *offsets,
                             const int32_t *unit_offsets, int M, int N, int ldk, float *C, hipStream_t st,
                             const uint32_t *amax = nullptr, const uint32_t *gmax = nullptr);

// Power-of-2 exponent k of a scaled fp16 gradient operand whose largest
// magnitude has the fp32 bits amax_bits: 2^k maps that magnitude into
// [2^14, 2^15), inside fp16's range with 2^28 of headroom below it for the
// smaller elements' normal numbers (fp16 keeps 11 significant bits there,
// against bf16's 8).  No scaling for a zero, subnormal, infinite or NaN
// maximum (which the fp16 values then carry as they are).
__host__ __device__ inline int grad_scale_exp(uint32_t amax_bits) {
    const int ex = (int)((amax_bits >> 23) & 0xFF);
    return (ex == 0 || ex == 255) ? 0 : 141 - ex;
}

// Backward pass of a bf16 layer: inputs, the forward's routing, gradients
// (fp32) and the workspace buffers.
struct BackwardArgs {
    const void *x, *w_router, *w1, *w3, *w2, *dy;
    const int32_t *eid, *row, *offsets, *token_of_row;
    const float *gate;
    float *dx, *dlogits, *dw_router, *dbias, *dw1, *dw3, *dw2;
    float *gate_of_row, *ds_of_row, *dg;  // [R]
    float *a, *b, *u;                     // [R][d_ff]
    uint16_t *acat;                       // [R][4 d_ff] bf16: da hi, db hi, da lo, db lo
    uint16_t *dab16;                      // [R][2 d_ff] fp16: da, db scaled by 2^k_e (over a, once free)
    uint16_t *hg;                         // [R][2 d_ff] bf16: (g h) hi, lo
    float *dx_perm;                       // [R][d]
    float *dx_rest;                       // [S - 1][R][d]: the dx GEMM's other K slices
    uint16_t *dat;                        // [2 d_ff][ldk]: da^T then db^T, fp16 scaled by 2^k_e (first half
                                          // of each expert's K window)
    uint16_t *xt;                         // [d][ldk]: x^T of the kept rows in fp16 (first half of each window)
    uint16_t *dyt;                        // [d][ldk]: dy^T of the kept rows in fp16 scaled by 2^k_dy (first half)
    uint32_t *amax;                       // [2 E + 1] fp32 bits: each expert's largest |da|, |db|; each
                                          // expert's largest |g h|; the largest |dy|
    uint16_t *hgt;                        // [d_ff][ldk]: (g h)^T in fp16 scaled by 2^k_e (first half)
    int32_t *unit_offsets;                // [2][E + 1]: e 2 d_ff, then e d
    int64_t ldk;
    int dx_splits;
};
hipError_t launch_backward(const moe_params &p, int64_t max_rows, int64_t cap, const BackwardArgs &a,
                           hipStream_t st);

// y[t] = sum over kept slots j of gate[t][j] * y_perm[row[t][j]], y_perm
// [R][d] fp32; zeros everywhere when max_rows is 0 (y_perm is then not read).
hipError_t launch_combine(const moe_params &p, int64_t max_rows, const float *y_perm, const int32_t *row,
                          const float *gate, void *y, hipStream_t st);

// bf16 layers: y[t] = sum over kept slots j and slices s of the gated fp16
// slices of row[t][j]: with plan null, yg[s][row] ([splits][max_rows][d],
// yrest = yg + max_rows d); otherwise the down projection's split plan
// (GemmOut): slice 0 in yg [max_rows][d], slices 1.. of the split rows at
// yrest.
hipError_t launch_combine_gated(const moe_params &p, int64_t max_rows, int splits, const uint16_t *yg,
                                const uint16_t *yrest, const int32_t *plan, const int32_t *row, void *y,
                                hipStream_t st);

// moe_forward's down projection (bf16 layers): the 256-row MFMA GEMM with
// the device-side split plan (planned), or S uniform slices (S = 1 for the
// weight-streaming kernel, groups of at most 32 rows).
struct DownSplit {
    bool planned;
    int S;
};
DownSplit forward_down_split(const moe_params &p, int64_t max_rows);

}  // namespace moe
