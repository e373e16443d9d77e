// Drives the C ABI's host-side logic (argument checks, capacity, row bounds,
// workspace sizing) over valid, invalid and extreme parameters, for a build
// of the library's host code under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Only calls that return before any kernel
// launch are made, so no device is touched.  Exits 0 when every check holds.
// Test infrastructure, built and run by tests/test_sanitizers.py.
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/moe.h"

static int failures = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            failures++;                                                       \
        }                                                                     \
    } while (0)

static moe_params P(int T, int d, int E, int k, int dff, float cf, int dtype) {
    moe_params p = {};
    p.T = T;
    p.d = d;
    p.E = E;
    p.k = k;
    p.d_ff = dff;
    p.capacity_factor = cf;
    p.reroute = 1;
    p.aux_coef = 0.01f;
    p.dtype = dtype;
    return p;
}

int main() {
    const int Ts[] = {0, 1, 7, 64, 4096, 8192, 1 << 18, 1 << 20, (1 << 20) + 1, -1};
    const int ds[] = {64, 128, 4096, 8192, 16384, 16448, 100, 0};
    const int Es[] = {1, 2, 8, 64, 256, 257, 0};
    const int ks[] = {1, 2, 8, 9, 0};
    const int dffs[] = {64, 14336, (1 << 22) - 64, 1 << 22, 96, 0};
    const float cfs[] = {1.0f, 1.25f, 0.0f, -1.0f, 1e-6f, 1e30f, INFINITY, NAN};
    int valid = 0;
    for (int T : Ts)
        for (int d : ds)
            for (int E : Es)
                for (int k : ks)
                    for (int dff : dffs)
                        for (float cf : cfs)
                            for (int dt = 0; dt < 3; dt++) {
                                moe_params p = P(T, d, E, k, dff, cf, dt);
                                const int64_t C = moe_capacity(&p), R = moe_max_rows(&p);
                                const size_t wf = moe_workspace_bytes(&p), wd = moe_dispatch_workspace_bytes(&p);
                                const size_t wn = moe_ffn_workspace_bytes(&p), wb = moe_backward_workspace_bytes(&p);
                                if (C < 0) {
                                    CHECK(R == -1 && wf == 0 && wd == 0 && wn == 0 && wb == 0);
                                    continue;
                                }
                                valid++;
                                CHECK(C >= (T > 0 ? 1 : 0) && C <= T);
                                CHECK(R >= 0 && R <= (int64_t)T * k && R <= (int64_t)E * C);
                                CHECK(wf >= wd && wd > 0);
                                CHECK(wf >= (size_t)R * dff * (dt == MOE_BF16 ? 2 : 4));
                                CHECK(wb >= (size_t)R * dff * 3 * 4);
                                // the rejected argument combinations return before any launch
                                moe_routing r = {};
                                CHECK(moe_route(&p, nullptr, nullptr, nullptr, nullptr, nullptr, &r, nullptr) ==
                                      MOE_ERR_INVALID_ARG);
                                CHECK(moe_forward(&p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                                  nullptr, nullptr, &r, nullptr, 0, nullptr) == MOE_ERR_INVALID_ARG);
                                // the backward takes bf16 layers whose x and 256 rows of the kept
                                // rows' transposed K axis (2 (R rounded up to 64 + 64 E) elements)
                                // fit its buffer extents
                                const int64_t ldk = 2 * (((R + 63) / 64) * 64 + 64 * (int64_t)E);
                                const bool bwd_ok = dt == MOE_BF16 && (int64_t)T * d * 2 < ((int64_t)1 << 31) &&
                                                    256 * ldk * 2 < ((int64_t)1 << 31);
                                CHECK(moe_backward(&p, nullptr, nullptr, nullptr, nullptr, nullptr, &r, nullptr,
                                                   nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                                   nullptr, 0, nullptr) ==
                                      (bwd_ok ? MOE_ERR_INVALID_ARG : MOE_ERR_UNSUPPORTED));
                                CHECK(moe_combine(&p, nullptr, nullptr, nullptr, nullptr, nullptr) ==
                                      (T > 0 ? MOE_ERR_INVALID_ARG : MOE_OK));
                                // a workspace one byte short is refused
                                moe_routing rf = {};
                                int32_t *fake = reinterpret_cast<int32_t *>(4096);
                                rf.cand = rf.eid = rf.pos = rf.row = rf.offsets = rf.token_of_row = rf.demand =
                                    rf.kept = rf.totals = fake;
                                rf.cand_score = rf.gate = rf.aux_loss = reinterpret_cast<float *>(4096);
                                rf.flag = reinterpret_cast<uint8_t *>(4096);
                                void *fp = reinterpret_cast<void *>(4096);
                                CHECK(moe_forward(&p, fp, fp, nullptr, nullptr, fp, fp, fp, fp,
                                                  reinterpret_cast<float *>(4096), &rf, fp, wf - 1,
                                                  nullptr) == MOE_ERR_INVALID_ARG);
                                CHECK(moe_dispatch(&p, fp, &rf, fp, fp, wd - 1, nullptr) == MOE_ERR_INVALID_ARG);
                            }
    // one-byte weights: bf16 layers only
    moe_params big = P(4096, 4096, 8, 2, 14336, 1.25f, MOE_F32);
    void *fp = reinterpret_cast<void *>(4096);
    const uint8_t *q = reinterpret_cast<const uint8_t *>(4096);
    const float *s = reinterpret_cast<const float *>(4096);
    CHECK(moe_expert_ffn_fp8(&big, fp, reinterpret_cast<const int32_t *>(4096), q, s, q, s, q, s, fp, fp,
                             nullptr) == MOE_ERR_UNSUPPORTED);
    // the static scratch refuses layers that need more
    moe_routing rr = {};
    int32_t *fi = reinterpret_cast<int32_t *>(4096);
    rr.cand = rr.eid = rr.pos = rr.row = rr.offsets = rr.token_of_row = rr.demand = rr.kept = rr.totals = fi;
    rr.cand_score = rr.gate = rr.aux_loss = reinterpret_cast<float *>(4096);
    rr.flag = reinterpret_cast<uint8_t *>(4096);
    CHECK(moe_forward_noalloc(&big, fp, fp, nullptr, nullptr, fp, fp, fp, fp, reinterpret_cast<float *>(4096), &rr,
                              nullptr) == MOE_ERR_TOO_LARGE);
    for (int c = -5; c <= 1; c++) CHECK(moe_strerror(c) != nullptr);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("abi host driver ok: %d valid parameter sets\n", valid);
    return 0;
}
