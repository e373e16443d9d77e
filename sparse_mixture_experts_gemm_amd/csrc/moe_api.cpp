// C ABI of the MoE layer: argument checks, capacity, workspace carving and
// kernel launches on the caller's stream.  No allocation, no synchronisation.
#include <math.h>
#include <string.h>

#include <mutex>

#include "moe_internal.h"

using namespace moe;

// Scratch of moe_forward_noalloc: a file-scope device array, one copy per
// GPU, held until the process ends.  Host code never passes `scratch`
// itself to a kernel (in host code the name is a host-side stand-in); it
// uses the device address hipGetSymbolAddress returns for the current GPU.
static __device__ __align__(256) char scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

// The device address of `scratch` on the current GPU, looked up once per
// device (with that device current) and kept; null if the lookup fails.
void *scratch_ptr() {
    static std::mutex mu;
    static void *ptr[kMaxDevices] = {};
    static bool done[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!done[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        ptr[dev] = p;
        done[dev] = true;
    }
    return ptr[dev];
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Shape checks shared by every entry point.
int check_params(const moe_params *p) {
    if (!p) return MOE_ERR_INVALID_ARG;
    if (p->T < 0 || p->T > (1 << 20)) return MOE_ERR_INVALID_ARG;
    if (p->E < 1 || p->E > kMaxExperts) return MOE_ERR_INVALID_ARG;
    if (p->k < 1 || p->k > kMaxTopK || p->k > p->E) return MOE_ERR_INVALID_ARG;
    if (p->d < 1 || p->d_ff < 1) return MOE_ERR_INVALID_ARG;
    if (p->dtype != MOE_F32 && p->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (p->d % 64 != 0 || p->d_ff % 64 != 0) return MOE_ERR_UNSUPPORTED;
    if (p->d > (p->dtype == MOE_BF16 ? 16384 : 8192)) return MOE_ERR_UNSUPPORTED;
    // one expert's weight matrix is addressed with 32-bit byte offsets
    if ((int64_t)p->d * p->d_ff * (p->dtype == MOE_BF16 ? 2 : 4) >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
    // a 256-row tile of h (the down projection's A operand) is addressed with
    // byte offsets below 2 GiB (an offset of 2 GiB marks a load past the end)
    if ((int64_t)256 * p->d_ff * 2 >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    if (!(p->lambda == p->lambda) || !(p->capacity_factor == p->capacity_factor)) return MOE_ERR_INVALID_ARG;
    if (!(p->gate_temperature >= 0.0f) || isinf(p->gate_temperature)) return MOE_ERR_INVALID_ARG;
    if (!(p->top2_gap >= 0.0f) || isinf(p->top2_gap)) return MOE_ERR_INVALID_ARG;
    if (p->router_hidden < 0) return MOE_ERR_INVALID_ARG;
    if (p->dynamic_capacity != 0 && p->dynamic_capacity != 1) return MOE_ERR_INVALID_ARG;
    if (p->router_hidden > kMaxExperts) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int64_t capacity_of(const moe_params &p) { return capacity_rows(p); }

int64_t max_rows_of(const moe_params &p) {
    const int64_t C = capacity_of(p);
    const int64_t a = (int64_t)p.T * p.k, b = (int64_t)p.E * C;
    return a < b ? a : b;
}

size_t esize(const moe_params &p) { return p.dtype == MOE_BF16 ? 2 : 4; }

// Per-token arrays may be NULL for an empty batch, token_of_row when R = 0.
int routing_ok(const moe_routing *r, const moe_params &p) {
    if (!r) return 0;
    if (!(r->offsets && r->demand && r->kept && r->totals && r->aux_loss)) return 0;
    if (p.T > 0 && !(r->cand && r->cand_score && r->eid && r->pos && r->row && r->flag && r->gate))
        return 0;
    if (max_rows_of(p) > 0 && !r->token_of_row) return 0;
    return 1;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

// Expert weights of a forward pass: matrices of the layer's dtype, or codes
// (E4M3, INT8 or INT4, qfmt) with fp32 row scales (s1 non-null).
struct FfnWeights {
    const void *w1, *w3, *w2;
    const float *s1, *s3, *s2;
    int qfmt = MOE_Q_E4M3;
};

int fp8_weights_ok(const moe_params &p, const FfnWeights &w) {
    if (!w.w1 || !w.w3 || !w.w2 || !w.s1 || !w.s3 || !w.s2) return MOE_ERR_INVALID_ARG;
    if (w.qfmt == MOE_Q_INT4 ? !q4_ffn_supported(p) : !fp8_ffn_supported(p)) return MOE_ERR_UNSUPPORTED;
    if (!aligned16(w.w1) || !aligned16(w.w3) || !aligned16(w.w2) || !aligned4(w.s1) || !aligned4(w.s3) ||
        !aligned4(w.s2))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// splits: the down projection's uniform K slices (moe_forward: its down
// split, as the combine expects; the staged one-byte entry points: 1).
hipError_t launch_ffn(const moe_params &p, int64_t R, int64_t C, const void *a, const int32_t *a_rows,
                      const int32_t *offsets, const FfnWeights &w, void *h, const GemmOut &down, int32_t *claim,
                      hipEvent_t mid, hipStream_t st, int splits = 1) {
    if (w.s1)
        return launch_expert_ffn_fp8(p, R, C, a, a_rows, offsets, static_cast<const uint8_t *>(w.w1), w.s1,
                                     static_cast<const uint8_t *>(w.w3), w.s3,
                                     static_cast<const uint8_t *>(w.w2), w.s2, h, down, splits, claim, mid, w.qfmt,
                                     st);
    return launch_expert_ffn(p, R, C, a, a_rows, offsets, w.w1, w.w3, w.w2, h, down, claim, mid, st, splits);
}

// moe_forward folds the dispatch gather into the gate-up GEMM (A rows read
// from x through token_of_row) whenever x spans less than 2 GiB (the GEMM
// reads A through a buffer extent kept below 2 GiB, so that an offset of
// 2 GiB marks a load that fetches nothing); x_perm is then never materialised.
bool gather_in_gemm(const moe_params &p) { return (int64_t)p.T * p.d * (int64_t)esize(p) < ((int64_t)1 << 31); }

int splits_of(const moe_params &p) { return ffn_splits(p, max_rows_of(p)); }

// moe_expert_ffn's scratch: the partial products of d_ff slices 1..S-1
// (slice 0 goes straight to y_perm; the fix-up adds the others).
size_t ffn_ws_bytes(const moe_params &p) {
    const size_t R = (size_t)max_rows_of(p);
    const int S = splits_of(p);
    return S > 1 ? align256((size_t)(S - 1) * R * p.d * sizeof(float)) : 0;
}

// Workspace layout of moe_forward.
struct ForwardWs {
    void *dispatch, *x_perm, *h;  // x_perm null when the GEMM gathers
    void *y;                      // bf16: gated fp16 slice 0 [R][d], then the split rows' further
                                  // slices (split plan); fp32: y_perm [R][d]
    float *gate_of_row;           // bf16: [R] each row's gate, for the down epilogue; fp32: null
    int32_t *claim;               // the expert GEMM's work-claim counters, then the split plan (4 ints)
};

size_t forward_y_bytes(const moe_params &p) {
    const size_t R = (size_t)max_rows_of(p);
    if (p.dtype != MOE_BF16) return R * p.d * sizeof(float);
    // slices past the first: the split plan's (or S - 1 uniform ones of R x d
    // each, which the same bound covers: (S - 1) R <= (S - 1) G 256 <= 256^3 / d
    // and S <= plan_max_splits)
    const DownSplit ds = forward_down_split(p, (int64_t)R);
    const size_t extra = ds.planned || ds.S > 1 ? plan_extra_elems((int64_t)R, p.d, p.d_ff) : 0;
    return (R * p.d + extra) * 2;
}

size_t forward_ws_bytes(const moe_params &p) {
    const size_t R = (size_t)max_rows_of(p);
    const size_t xp = gather_in_gemm(p) ? 0 : align256(R * p.d * esize(p));
    const size_t gr = p.dtype == MOE_BF16 ? align256(R * sizeof(float)) : 0;
    return align256(dispatch_scratch_bytes(p.T, p.E, p.k)) + xp + align256(R * p.d_ff * esize(p)) +
           align256(forward_y_bytes(p)) + gr + align256(sizeof(int32_t) * (kClaimCounters + 4));
}

ForwardWs carve_forward(void *ws, const moe_params &p) {
    const size_t R = (size_t)max_rows_of(p);
    char *c = static_cast<char *>(ws);
    ForwardWs f;
    f.dispatch = c;
    c += align256(dispatch_scratch_bytes(p.T, p.E, p.k));
    f.x_perm = nullptr;
    if (!gather_in_gemm(p)) {
        f.x_perm = c;
        c += align256(R * p.d * esize(p));
    }
    f.h = c;
    c += align256(R * p.d_ff * esize(p));
    f.y = c;
    c += align256(forward_y_bytes(p));
    f.gate_of_row = nullptr;
    if (p.dtype == MOE_BF16) {
        f.gate_of_row = reinterpret_cast<float *>(c);
        c += align256(R * sizeof(float));
    }
    f.claim = reinterpret_cast<int32_t *>(c);
    return f;
}

// Workspace layout of moe_backward (sizes in bytes, each 256-aligned):
// gate_of_row, ds_of_row, dg [R] fp32; a, b, u [R][d_ff] fp32 (a's bytes
// then hold the scaled fp16 da, db [R][2 d_ff]); acat [R][4 d_ff] and hg
// [R][2 d_ff] bf16; dx_perm [S][R][d] fp32 (S K slices
// of the dx GEMM, at least one per d_ff period of its K); the K-major
// copies of the kept rows, [2 d_ff], [d], [d] and [d_ff] rows of ldk 16-bit
// values (da, db, x, dy and g h in fp16); two sets of E + 1 unit offsets;
// the largest magnitudes that set the fp16 scales [2 E + 1].
struct BackwardSizes {
    size_t R, F, D, E, ldk;
    int S;
};

BackwardSizes backward_sizes(const moe_params &p) {
    BackwardSizes z;
    z.R = (size_t)max_rows_of(p);
    z.F = (size_t)p.d_ff;
    z.D = (size_t)p.d;
    z.E = (size_t)p.E;
    z.ldk = (size_t)backward_ldk((int64_t)z.R, p.E);
    z.S = plain_gemm_splits((int64_t)z.R, p.E, p.d, 2 * p.d_ff, p.d_ff);
    return z;
}

size_t backward_ws_bytes(const moe_params &p) {
    const BackwardSizes z = backward_sizes(p);
    return 3 * align256(z.R * 4) + 3 * align256(z.R * z.F * 4) + align256(z.R * 4 * z.F * 2) +
           align256(z.R * 2 * z.F * 2) + align256((size_t)z.S * z.R * z.D * 4) + align256(2 * z.F * z.ldk * 2) +
           2 * align256(z.D * z.ldk * 2) +
           align256(z.F * z.ldk * 2) + align256(2 * (z.E + 1) * 4) + align256((2 * z.E + 1) * 4);
}

void carve_backward(void *ws, const moe_params &p, BackwardArgs &a) {
    const BackwardSizes z = backward_sizes(p);
    char *c = static_cast<char *>(ws);
    auto take = [&c](size_t n) {
        char *q = c;
        c += align256(n);
        return q;
    };
    a.gate_of_row = reinterpret_cast<float *>(take(z.R * 4));
    a.ds_of_row = reinterpret_cast<float *>(take(z.R * 4));
    a.dg = reinterpret_cast<float *>(take(z.R * 4));
    a.a = reinterpret_cast<float *>(take(z.R * z.F * 4));
    a.b = reinterpret_cast<float *>(take(z.R * z.F * 4));
    a.u = reinterpret_cast<float *>(take(z.R * z.F * 4));
    a.acat = reinterpret_cast<uint16_t *>(take(z.R * 4 * z.F * 2));
    a.dab16 = reinterpret_cast<uint16_t *>(a.a);  // a is read only by swiglu_backward, before
    a.hg = reinterpret_cast<uint16_t *>(take(z.R * 2 * z.F * 2));
    a.dx_perm = reinterpret_cast<float *>(take((size_t)z.S * z.R * z.D * 4));
    a.dx_rest = a.dx_perm + z.R * z.D;
    a.dat = reinterpret_cast<uint16_t *>(take(2 * z.F * z.ldk * 2));
    a.xt = reinterpret_cast<uint16_t *>(take(z.D * z.ldk * 2));
    a.dyt = reinterpret_cast<uint16_t *>(take(z.D * z.ldk * 2));
    a.hgt = reinterpret_cast<uint16_t *>(take(z.F * z.ldk * 2));
    a.unit_offsets = reinterpret_cast<int32_t *>(take(2 * (z.E + 1) * 4));
    a.amax = reinterpret_cast<uint32_t *>(take((2 * z.E + 1) * 4));
    a.ldk = (int64_t)z.ldk;
    a.dx_splits = z.S;
}

}  // namespace

extern "C" {

size_t moe_load_window_workspace_bytes(const moe_params *p, int32_t window) {
    if (check_params(p) != MOE_OK || window < 1) return 0;
    return align256(sizeof(int32_t) * (size_t)ceil_div(p->T > 0 ? p->T : 1, window) * p->E);
}

int moe_load_window(const moe_params *p, const int32_t *cand, int32_t window, float decay, float *load,
                    void *workspace, size_t ws_bytes, void *stream) {
    int rc = check_params(p);
    if (rc != MOE_OK) return rc;
    if (window < 1 || !(decay >= 0.0f && decay <= 1.0f) || !load || !workspace || (p->T > 0 && !cand))
        return MOE_ERR_INVALID_ARG;
    if (ws_bytes < moe_load_window_workspace_bytes(p, window)) return MOE_ERR_INVALID_ARG;
    if (!aligned4(load) || !aligned16(workspace)) return MOE_ERR_UNSUPPORTED;
    return hip_status(launch_load_window(*p, cand, window, decay, load, static_cast<int32_t *>(workspace),
                                         static_cast<hipStream_t>(stream)));
}

size_t moe_backward_workspace_bytes(const moe_params *p) {
    if (check_params(p) != MOE_OK) return 0;
    return backward_ws_bytes(*p);
}

int moe_backward(const moe_params *p, const void *x, const void *w_router, const void *w1, const void *w3,
                 const void *w2, const moe_routing *r, const void *dy, float *dx, float *dlogits,
                 float *dw_router, float *dbias, float *dw1, float *dw3, float *dw2, void *workspace,
                 size_t ws_bytes, void *stream) {
    int rc = check_params(p);
    if (rc != MOE_OK) return rc;
    if (p->dtype != MOE_BF16 || p->router_hidden != 0 || (int64_t)p->T * p->d * 2 >= ((int64_t)1 << 31))
        return MOE_ERR_UNSUPPORTED;
    const int64_t R = max_rows_of(*p);
    // the transposed kept rows: 256 rows of their K axis below 2 GiB
    if (256 * backward_ldk(R, p->E) * 2 >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    if (!r || !r->offsets || !w_router || !w1 || !w3 || !w2 || !dw_router || !dbias || !dw1 || !dw3 || !dw2 ||
        !workspace)
        return MOE_ERR_INVALID_ARG;
    if (p->T > 0 && (!x || !dy || !dx || !dlogits || !r->eid || !r->row || !r->gate || !r->token_of_row))
        return MOE_ERR_INVALID_ARG;
    if (ws_bytes < backward_ws_bytes(*p)) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(w1) || !aligned16(w3) || !aligned16(w2) ||
        !aligned16(dy) || !aligned16(dx) || !aligned16(workspace))
        return MOE_ERR_UNSUPPORTED;
    BackwardArgs a{};
    a.x = x;
    a.w_router = w_router;
    a.w1 = w1;
    a.w3 = w3;
    a.w2 = w2;
    a.dy = dy;
    a.eid = r->eid;
    a.row = r->row;
    a.offsets = r->offsets;
    a.token_of_row = r->token_of_row;
    a.gate = r->gate;
    a.dx = dx;
    a.dlogits = dlogits;
    a.dw_router = dw_router;
    a.dbias = dbias;
    a.dw1 = dw1;
    a.dw3 = dw3;
    a.dw2 = dw2;
    carve_backward(workspace, *p, a);
    return hip_status(launch_backward(*p, R, capacity_of(*p), a, static_cast<hipStream_t>(stream)));
}

int64_t moe_capacity(const moe_params *p) {
    if (check_params(p) != MOE_OK) return -1;
    return capacity_of(*p);
}

int64_t moe_max_rows(const moe_params *p) {
    if (check_params(p) != MOE_OK) return -1;
    return max_rows_of(*p);
}

size_t moe_dispatch_workspace_bytes(const moe_params *p) {
    if (check_params(p) != MOE_OK) return 0;
    return dispatch_scratch_bytes(p->T, p->E, p->k);
}

size_t moe_ffn_workspace_bytes(const moe_params *p) {
    if (check_params(p) != MOE_OK) return 0;
    return ffn_ws_bytes(*p);
}

size_t moe_workspace_bytes(const moe_params *p) {
    if (check_params(p) != MOE_OK) return 0;
    return forward_ws_bytes(*p);
}

int moe_route(const moe_params *p, const void *x, const void *w_router, const float *bias,
              const float *load, float *logits, moe_routing *r, void *stream) {
    int rc = check_params(p);
    if (rc != MOE_OK) return rc;
    if (!routing_ok(r, *p) || (p->T > 0 && (!x || !logits)) || !w_router) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_UNSUPPORTED;
    return hip_status(launch_route(*p, x, w_router, bias, load, logits, r->cand, r->cand_score,
                                   static_cast<hipStream_t>(stream)));
}

int moe_dispatch(const moe_params *p, const void *x, moe_routing *r, void *x_perm,
                 void *workspace, size_t ws_bytes, void *stream) {
    int rc = check_params(p);
    if (rc != MOE_OK) return rc;
    if (!routing_ok(r, *p) || !workspace || (p->T > 0 && (!x || !x_perm))) return MOE_ERR_INVALID_ARG;
    if (ws_bytes < dispatch_scratch_bytes(p->T, p->E, p->k)) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(x_perm) || !aligned16(workspace)) return MOE_ERR_UNSUPPORTED;
    const DispatchScratch s = carve_dispatch(workspace, p->T, p->E, p->k);
    return hip_status(launch_dispatch(*p, capacity_of(*p), x, *r, x_perm, s,
                                      static_cast<hipStream_t>(stream)));
}

int moe_expert_ffn(const moe_params *p, const void *x_perm, const int32_t *offsets,
                   const void *w1, const void *w3, const void *w2, void *h, void *y_perm,
                   void *workspace, size_t ws_bytes, void *stream) {
    int rc = check_params(p);
    if (rc != MOE_OK) return rc;
    const int64_t R = max_rows_of(*p);
    const size_t need = ffn_ws_bytes(*p);
    if (!offsets || !w1 || !w3 || !w2) return MOE_ERR_INVALID_ARG;
    if (R > 0 && (!x_perm || !h || !y_perm)) return MOE_ERR_INVALID_ARG;
    if (need > 0 && (!workspace || ws_bytes < need)) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x_perm) || !aligned16(w1) || !aligned16(w3) || !aligned16(w2) || !aligned16(h) ||
        !aligned16(y_perm) || !aligned16(workspace))
        return MOE_ERR_UNSUPPORTED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int S = splits_of(*p);
    const GemmOut down{y_perm, workspace, (size_t)R * p->d, nullptr};
    hipError_t e = launch_expert_ffn(*p, R, capacity_of(*p), x_perm, nullptr, offsets, w1, w3, w2, h, down,
                                     nullptr, nullptr, st, S);
    if (e != hipSuccess) return MOE_ERR_HIP;
    return hip_status(launch_ffn_fixup(*p, R, offsets, static_cast<float *>(y_perm),
                                       static_cast<const float *>(workspace), S - 1, st));
}

}  // extern "C"

namespace {

int expert_ffn_q8(const moe_params *p, const void *x_perm, const int32_t *offsets, const FfnWeights &w, void *h,
                  void *y_perm, void *stream) {
    int rc = check_params(p);
    if (rc != MOE_OK) return rc;
    const int64_t R = max_rows_of(*p);
    if (!offsets) return MOE_ERR_INVALID_ARG;
    if ((rc = fp8_weights_ok(*p, w)) != MOE_OK) return rc;
    if (R > 0 && (!x_perm || !h || !y_perm)) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x_perm) || !aligned16(h) || !aligned16(y_perm)) return MOE_ERR_UNSUPPORTED;
    const GemmOut down{y_perm, nullptr, 0, nullptr};
    return hip_status(launch_ffn(*p, R, capacity_of(*p), x_perm, nullptr, offsets, w, h, down, nullptr, nullptr,
                                 static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int moe_expert_ffn_fp8(const moe_params *p, const void *x_perm, const int32_t *offsets,
                       const uint8_t *w1, const float *s1, const uint8_t *w3, const float *s3,
                       const uint8_t *w2, const float *s2, void *h, void *y_perm, void *stream) {
    return expert_ffn_q8(p, x_perm, offsets, FfnWeights{w1, w3, w2, s1, s3, s2, MOE_Q_E4M3}, h, y_perm, stream);
}

int moe_expert_ffn_i8(const moe_params *p, const void *x_perm, const int32_t *offsets,
                      const int8_t *w1, const float *s1, const int8_t *w3, const float *s3,
                      const int8_t *w2, const float *s2, void *h, void *y_perm, void *stream) {
    return expert_ffn_q8(p, x_perm, offsets, FfnWeights{w1, w3, w2, s1, s3, s2, MOE_Q_INT8}, h, y_perm, stream);
}

int moe_expert_ffn_i4(const moe_params *p, const void *x_perm, const int32_t *offsets,
                      const uint8_t *w1, const float *s1, const uint8_t *w3, const float *s3,
                      const uint8_t *w2, const float *s2, void *h, void *y_perm, void *stream) {
    return expert_ffn_q8(p, x_perm, offsets, FfnWeights{w1, w3, w2, s1, s3, s2, MOE_Q_INT4}, h, y_perm, stream);
}

int moe_combine(const moe_params *p, const void *y_perm, const int32_t *row, const float *gate,
                void *y, void *stream) {
    int rc = check_params(p);
    if (rc != MOE_OK) return rc;
    const int64_t R = max_rows_of(*p);
    if (p->T > 0 && (!row || !gate || !y || (R > 0 && !y_perm))) return MOE_ERR_INVALID_ARG;
    if (!aligned16(y_perm) || !aligned16(y)) return MOE_ERR_UNSUPPORTED;
    return hip_status(launch_combine(*p, R, static_cast<const float *>(y_perm), row, gate, y,
                                     static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// events: null, or 6 hipEvent_t (null entries skipped) recorded before route,
// dispatch, the gate-up GEMM, the down GEMM and the combine, and after the
// combine.
int forward_impl(const moe_params *p, const void *x, const void *w_router, const float *bias,
                 const float *load, const FfnWeights &w, void *y, float *logits, moe_routing *r,
                 void *workspace, size_t ws_bytes, void *stream, void *const *events) {
    int rc = check_params(p);
    if (rc != MOE_OK) return rc;
    if (!routing_ok(r, *p) || !w_router || !w.w1 || !w.w3 || !w.w2 || !workspace ||
        (p->T > 0 && (!x || !y || !logits)))
        return MOE_ERR_INVALID_ARG;
    if (w.s1 && (rc = fp8_weights_ok(*p, w)) != MOE_OK) return rc;
    if (ws_bytes < forward_ws_bytes(*p)) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(w.w1) || !aligned16(w.w3) ||
        !aligned16(w.w2) || !aligned16(y) || !aligned16(workspace))
        return MOE_ERR_UNSUPPORTED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto mark = [&](int i) {
        return !(events && events[i]) || hipEventRecord(static_cast<hipEvent_t>(events[i]), st) == hipSuccess;
    };
    const ForwardWs f = carve_forward(workspace, *p);
    const int64_t C = capacity_of(*p);
    const int64_t R = max_rows_of(*p);
    // down-projection slices: uniform, or chosen on the device by the split
    // plan (the weight-streaming kernel and fp32 layers: one)
    const DownSplit dsp = forward_down_split(*p, R);
    const int S = dsp.planned ? 1 : dsp.S;
    if (!mark(0)) return MOE_ERR_HIP;
    hipError_t e = launch_route(*p, x, w_router, bias, load, logits, r->cand, r->cand_score, st);
    if (e != hipSuccess) return MOE_ERR_HIP;
    if (!mark(1)) return MOE_ERR_HIP;
    DispatchScratch ds = carve_dispatch(f.dispatch, p->T, p->E, p->k);
    ds.claim = f.claim;  // zeroed by the dispatch, used by the expert GEMM
    ds.gate_of_row = f.gate_of_row;
    e = launch_dispatch(*p, C, x, *r, f.x_perm, ds, st);
    if (e != hipSuccess) return MOE_ERR_HIP;
    if (!mark(2)) return MOE_ERR_HIP;
    // bf16: the down projection folds each row's gate in and stores fp16
    // slices (the 256-row GEMM after its device-side split plan, the
    // weight-streaming kernel as one slice); fp32: y_perm [R][d] in fp32,
    // gates applied by the combine
    const size_t stride = (size_t)R * p->d;
    int32_t *plan = dsp.planned ? f.claim + kClaimCounters : nullptr;
    uint16_t *yrest = static_cast<uint16_t *>(f.y) + stride;
    const GemmOut down = p->dtype == MOE_BF16 ? GemmOut{f.y, yrest, stride, f.gate_of_row, plan}
                                              : GemmOut{f.y, nullptr, stride, nullptr};
    hipEvent_t mid = events ? static_cast<hipEvent_t>(events[3]) : nullptr;
    if (f.x_perm)
        e = launch_ffn(*p, R, C, f.x_perm, nullptr, r->offsets, w, f.h, down, f.claim, mid, st, S);
    else
        e = launch_ffn(*p, R, C, x, r->token_of_row, r->offsets, w, f.h, down, f.claim, mid, st, S);
    if (e != hipSuccess) return MOE_ERR_HIP;
    if (!mark(4)) return MOE_ERR_HIP;
    if (p->dtype == MOE_BF16)
        e = launch_combine_gated(*p, R, S, static_cast<const uint16_t *>(f.y), yrest, plan, r->row, y, st);
    else
        e = launch_combine(*p, R, static_cast<const float *>(f.y), r->row, r->gate, y, st);
    if (e != hipSuccess) return MOE_ERR_HIP;
    if (!mark(5)) return MOE_ERR_HIP;
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward(const moe_params *p, const void *x, const void *w_router, const float *bias,
                const float *load, const void *w1, const void *w3, const void *w2, void *y,
                float *logits, moe_routing *r, void *workspace, size_t ws_bytes, void *stream) {
    return forward_impl(p, x, w_router, bias, load, FfnWeights{w1, w3, w2, nullptr, nullptr, nullptr}, y,
                        logits, r, workspace, ws_bytes, stream, nullptr);
}

int moe_forward_events(const moe_params *p, const void *x, const void *w_router, const float *bias,
                       const float *load, const void *w1, const void *w3, const void *w2, void *y,
                       float *logits, moe_routing *r, void *workspace, size_t ws_bytes, void *stream,
                       void *const *events) {
    return forward_impl(p, x, w_router, bias, load, FfnWeights{w1, w3, w2, nullptr, nullptr, nullptr}, y,
                        logits, r, workspace, ws_bytes, stream, events);
}

int moe_forward_noalloc(const moe_params *p, const void *x, const void *w_router, const float *bias,
                        const float *load, const void *w1, const void *w3, const void *w2, void *y,
                        float *logits, moe_routing *r, void *stream) {
    int rc = check_params(p);
    if (rc != MOE_OK) return rc;
    if (forward_ws_bytes(*p) > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_TOO_LARGE;
    void *ws = scratch_ptr();
    if (!ws) return MOE_ERR_HIP;
    return forward_impl(p, x, w_router, bias, load, FfnWeights{w1, w3, w2, nullptr, nullptr, nullptr}, y,
                        logits, r, ws, (size_t)MOE_STATIC_SCRATCH_BYTES, stream, nullptr);
}

int moe_forward_fp8(const moe_params *p, const void *x, const void *w_router, const float *bias,
                    const float *load, const uint8_t *w1, const float *s1, const uint8_t *w3,
                    const float *s3, const uint8_t *w2, const float *s2, void *y, float *logits,
                    moe_routing *r, void *workspace, size_t ws_bytes, void *stream) {
    if (!s1 || !s3 || !s2) return MOE_ERR_INVALID_ARG;
    return forward_impl(p, x, w_router, bias, load, FfnWeights{w1, w3, w2, s1, s3, s2, MOE_Q_E4M3}, y, logits, r,
                        workspace, ws_bytes, stream, nullptr);
}

int moe_forward_i8(const moe_params *p, const void *x, const void *w_router, const float *bias,
                   const float *load, const int8_t *w1, const float *s1, const int8_t *w3,
                   const float *s3, const int8_t *w2, const float *s2, void *y, float *logits,
                   moe_routing *r, void *workspace, size_t ws_bytes, void *stream) {
    if (!s1 || !s3 || !s2) return MOE_ERR_INVALID_ARG;
    return forward_impl(p, x, w_router, bias, load, FfnWeights{w1, w3, w2, s1, s3, s2, MOE_Q_INT8}, y, logits, r,
                        workspace, ws_bytes, stream, nullptr);
}

int moe_forward_i4(const moe_params *p, const void *x, const void *w_router, const float *bias,
                   const float *load, const uint8_t *w1, const float *s1, const uint8_t *w3,
                   const float *s3, const uint8_t *w2, const float *s2, void *y, float *logits,
                   moe_routing *r, void *workspace, size_t ws_bytes, void *stream) {
    if (!s1 || !s3 || !s2) return MOE_ERR_INVALID_ARG;
    return forward_impl(p, x, w_router, bias, load, FfnWeights{w1, w3, w2, s1, s3, s2, MOE_Q_INT4}, y, logits, r,
                        workspace, ws_bytes, stream, nullptr);
}

const char *moe_strerror(int code) {
    switch (code) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument (null pointer, size out of range or workspace too small)";
        case MOE_ERR_UNSUPPORTED: return "unsupported dtype, alignment or dimension";
        case MOE_ERR_HIP: return "HIP kernel launch failed";
        case MOE_ERR_TOO_LARGE: return "layer needs more scratch than the static scratch array holds";
        default: return "unknown error code";
    }
}

}  // extern "C"
