// Work items of the grouped GEMMs over the permuted rows: each expert's
// rows [offsets[e], offsets[e+1]) are cut into m tiles, and every launch
// finds its block's item from the device-side offsets.
#pragma once

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

// Flat work index -> (expert, m range, n tile, K split).  Work items are
// ordered expert, split, n tile, m tile (m fastest), so the m tiles that
// share a weight tile are adjacent.
struct TileInfo {
    int e, m0, mend, nt, split;
    int row0, srows;  // planned split (find_tile_planned): first split row, split rows
};

// First row (relative to the expert's first row) of m tile t when an
// expert's n rows are cut into mt = ceil(n / bm) balanced tiles (bm = 256):
// the nb = ceil(n / 32) blocks of 32 rows (the MFMA row block) are dealt
// out evenly, the first nb % mt tiles taking nb / mt + 1 blocks and the
// others nb / mt, and the last tile ends at row n.  No tile exceeds bm rows,
// none is a sliver, and the tiles hold nb row blocks in all, as many as
// tiles of bm rows would.  (Tiles of bm rows and a short last one cost
// nearly a full tile for the last: its weight tile streams whole.)
__host__ __device__ __forceinline__ int balanced_start(int n, int mt, int t) {
    const int nb = (n + 31) >> 5, q = nb / mt, r = nb % mt;
    const int row = 32 * (t * q + (t < r ? t : r));
    return row < n ? row : n;
}

// Blocks are dealt round-robin over the 8 XCDs (block b runs on XCD b % 8).
// The grid is sized by a bound on the work count; the real count comes from
// the device-side offsets.  Each XCD is given an equal, contiguous range of
// the real work items, so its L2 serves tiles that share operands and no
// XCD is left with the empty tail of the grid.  Without claim counters the
// block takes item (XCD b % 8, position b / 8).  With them (8 zeroed ints)
// thread 0 claims the next item of its XCD's range with an atomic add, and
// once that range is used up, the next item of another XCD's range: the
// XCDs run at different speeds, and the ones that finish early take over
// the others' last items.  Each item is claimed exactly once (the adds
// return distinct values), and a block that finds every range used up has
// nothing to do; the grid (at least the item count) always suffices.  The
// claimed index passes through `slot` (one int of LDS that nothing else uses
// until the second barrier).  Wave-parallel: lane l owns experts
// 4l .. 4l+3 (E <= 256).  Returns false for blocks with no work (uniformly
// over the block).  balanced: the expert's rows are cut into balanced m
// tiles (balanced_start) and ti.mend is the tile's end; otherwise tile t
// starts at row t bm and ti.mend is the expert's end.
__device__ __forceinline__ bool find_tile(const int32_t *__restrict__ offsets, int E, int ntiles_n,
                                          int bm, int splits, int blk, int32_t *claim, int *slot,
                                          TileInfo &ti, bool balanced = false) {
    const int lane = lane_id();
    const int e0 = lane * 4;
    const int xcd = blk & 7, local = blk >> 3;
    // The claim of this XCD's next item is issued first, so that its round
    // trip overlaps the reads of the offsets (whether it is in range is
    // known only once the item count is).  The counter's address goes
    // through an opaque zero held in a VGPR: for an address it knows to be
    // uniform the compiler combines the lanes' adds and waits for the result
    // on the spot, which would serialise the two round trips again.
    int first = 0;
    if (claim && threadIdx.x == 0) {
        int vzero;
        asm volatile("v_mov_b32 %0, 0" : "=v"(vzero));
        first = atomicAdd(claim + xcd + vzero, 1);
    }
    // offsets[e0 .. e0 + 4], clamped to offsets[E]: five independent loads
    // in flight together (a load per expert under a branch each would wait
    // for each one in turn)
    int ofs[5];
#pragma unroll
    for (int j = 0; j < 5; j++) ofs[j] = offsets[min(e0 + j, E)];
    int mts[4], c = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        mts[j] = (ofs[j + 1] - ofs[j] + bm - 1) / bm;  // 0 past E (both ends clamp to E)
        c += mts[j];
    }
    int incl = c;  // inclusive prefix of m tiles over lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
    }
    const int per = ntiles_n * splits;  // work items per m tile
    const int total = __builtin_amdgcn_readlane(incl, 63) * per;
    const int q = total >> 3, r = total & 7;
    int L;
    if (claim) {
        if (threadIdx.x == 0) {
            int item = -1;
            for (int s = 0; s < 8; s++) {
                const int y = (xcd + s) & 7;
                const int i = s == 0 ? first : atomicAdd(&claim[y], 1);
                if (i < q + (y < r ? 1 : 0)) {
                    item = y * q + min(y, r) + i;
                    break;
                }
            }
            *slot = item;
        }
        __syncthreads();
        L = __builtin_amdgcn_readfirstlane(*slot);
        __syncthreads();  // every wave has read the slot before its LDS is reused
        if (L < 0) return false;
    } else {
        if (local >= q + (xcd < r ? 1 : 0)) return false;
        L = xcd * q + min(xcd, r) + local;
    }
    const int lo = (incl - c) * per, hi = incl * per;
    const bool mine = L >= lo && L < hi;
    int e_sel = 0, base_sel = 0;
    if (mine) {
        int b = lo;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int cnt = mts[j] * per;
            if (L >= b && L < b + cnt) {
                e_sel = e0 + j;
                base_sel = b;
            }
            b += cnt;
        }
    }
    const int owner = __builtin_ctzll(ballot64(mine));
    const int e = __builtin_amdgcn_readlane(e_sel, owner);
    const int base = __builtin_amdgcn_readlane(base_sel, owner);
    const int beg = offsets[e], end = offsets[e + 1];
    const int mt = (end - beg + bm - 1) / bm;
    const int local_e = L - base;
    const int per_split = mt * ntiles_n;
    ti.e = e;
    ti.split = local_e / per_split;
    const int rem = local_e % per_split;
    ti.nt = rem / mt;
    if (balanced) {
        const int t = rem % mt;
        ti.m0 = beg + balanced_start(end - beg, mt, t);
        ti.mend = beg + balanced_start(end - beg, mt, t + 1);
    } else {
        ti.m0 = beg + (rem % mt) * bm;
        ti.mend = end;
    }
    ti.row0 = 0;
    ti.srows = 0;
    return true;
}

// Split plan of a K-split GEMM over M m tiles of ntn n tiles (the down
// projection of moe_forward).  One unsplit work item per tile would leave
// the chip's last round of kPlanCUs items partly empty, and splitting every
// tile in K multiplies the partial outputs that the combine must read.  So
// the m tiles that fill whole rounds run unsplit, and only the last G m
// tiles (the partial last round, rounded up to whole m tiles) are split into
// S slices of the K steps, as many as still fit in one round (S G ntn <=
// kPlanCUs), at most kPlanMaxS and at most nk / 8 (nk: K steps).  No split
// (G = 0, S = 1) when the tiles fill whole rounds or a split would not fit.
__host__ __device__ inline int plan_max_splits(int nk) {
    const int s = nk / 8;
    return s < 1 ? 1 : (s > kPlanMaxS ? kPlanMaxS : s);
}
__host__ __device__ inline void split_plan(int M, int ntn, int nk, int &G, int &S) {
    const int rem = (M * ntn) % kPlanCUs;
    G = rem == 0 ? 0 : (M < (rem + ntn - 1) / ntn ? M : (rem + ntn - 1) / ntn);
    S = 1;
    if (G > 0) {
        const int fit = kPlanCUs / (G * ntn), smax = plan_max_splits(nk);
        S = fit < smax ? fit : smax;
    }
    if (S <= 1) {
        S = 1;
        G = 0;
    }
}

// find_tile for the split plan: bulk items (one per tile of the first M - G
// m tiles, ordered expert, n tile, m tile) and split items (S per tile of
// the last G m tiles, ordered expert, split, n tile, m tile).  Each XCD's
// range holds an equal share of the bulk items followed by an equal share
// of the split items, so the short split items run last everywhere (an XCD
// that finishes early takes over another's remaining items, as in
// find_tile).  The split items of one tile cover K steps [s nk / S, (s + 1)
// nk / S); the bulk items all nk.  The rows of the split m tiles are the
// last ones, [row0, offsets[E]): slice 0 of every row goes to the output's
// first buffer, slices 1.. of the split rows to the second (see GemmOut).
// Block 0 stores {row0, S, split rows} in plan_out for the combine.
__device__ __forceinline__ bool find_tile_planned(const int32_t *__restrict__ offsets, int E, int ntn, int bm,
                                                  int nk, int blk, int32_t *claim, int *slot, int32_t *plan_out,
                                                  TileInfo &ti, int &k0s, int &nks) {
    const int lane = lane_id();
    const int e0 = lane * 4;
    const int xcd = blk & 7, local = blk >> 3;
    int first = 0;
    if (claim && threadIdx.x == 0) {
        int vzero;
        asm volatile("v_mov_b32 %0, 0" : "=v"(vzero));
        first = atomicAdd(claim + xcd + vzero, 1);
    }
    int ofs[5];
#pragma unroll
    for (int j = 0; j < 5; j++) ofs[j] = offsets[min(e0 + j, E)];
    int mts[4], c = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        mts[j] = (ofs[j + 1] - ofs[j] + bm - 1) / bm;
        c += mts[j];
    }
    int incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
    }
    const int M = __builtin_amdgcn_readlane(incl, 63);
    int G, S;
    split_plan(M, ntn, nk, G, S);
    // per expert: its bulk m tiles (those before global m tile M - G) and
    // split m tiles; the bulk m tiles being the first ones, the lanes'
    // prefixes of each kind follow from incl
    const int Mb = M - G;
    int pre = incl - c, mb[4], ml[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        mb[j] = min(max(Mb - pre, 0), mts[j]);
        ml[j] = mts[j] - mb[j];
        pre += mts[j];
    }
    const int ib = min(incl, Mb), it = incl - ib;                     // inclusive prefixes
    const int cb = ib - min(incl - c, Mb), ct = c - cb;               // this lane's counts
    const int nbulk = Mb * ntn;
    const int nsplit = G * ntn * S;
    // first split row: in the first expert that has split m tiles, after its
    // bulk ones (offsets[E] when nothing is split); m tiles are balanced
    int r0 = 0x7fffffff;
#pragma unroll
    for (int j = 3; j >= 0; j--)
        if (ml[j] > 0) r0 = ofs[j] + balanced_start(ofs[j + 1] - ofs[j], mts[j], mb[j]);
    const uint64_t has = ballot64(ct > 0);
    const int rows_end = __builtin_amdgcn_readlane(ofs[4], 63);  // offsets[E] (lane 63's experts lie past E)
    const int row0 = has ? __builtin_amdgcn_readlane(r0, __builtin_ctzll(has)) : rows_end;
    if (plan_out && blk == 0 && threadIdx.x == 0) {
        plan_out[0] = row0;
        plan_out[1] = S;
        plan_out[2] = rows_end - row0;
    }
    // XCD y's range: its share of the bulk items, then its share of the
    // split items; index i of the range -> flat item (bulk, then split)
    const int qb = nbulk >> 3, rb = nbulk & 7, qs = nsplit >> 3, rs = nsplit & 7;
    auto count = [&](int y) { return qb + (y < rb ? 1 : 0) + qs + (y < rs ? 1 : 0); };
    auto flat = [&](int y, int i) {
        const int nb = qb + (y < rb ? 1 : 0);
        return i < nb ? y * qb + min(y, rb) + i : nbulk + y * qs + min(y, rs) + (i - nb);
    };
    int L;
    if (claim) {
        if (threadIdx.x == 0) {
            int item = -1;
            for (int s = 0; s < 8; s++) {
                const int y = (xcd + s) & 7;
                const int i = s == 0 ? first : atomicAdd(&claim[y], 1);
                if (i < count(y)) {
                    item = flat(y, i);
                    break;
                }
            }
            *slot = item;
        }
        __syncthreads();
        L = __builtin_amdgcn_readfirstlane(*slot);
        __syncthreads();
        if (L < 0) return false;
    } else {
        if (local >= count(xcd)) return false;
        L = flat(xcd, local);
    }
    const bool split = L >= nbulk;
    const int Li = split ? L - nbulk : L;
    const int per_m = split ? ntn * S : ntn;  // items per m tile
    const int lo = (split ? it - ct : ib - cb) * per_m, hi = (split ? it : ib) * per_m;
    const bool mine = Li >= lo && Li < hi;
    int e_sel = 0, m0_sel = 0, mend_sel = 0, nt_sel = 0, sp_sel = 0;
    if (mine) {
        int b = lo;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int cm = split ? ml[j] : mb[j];  // this expert's m tiles of the kind
            const int cnt = cm * per_m;
            if (Li >= b && Li < b + cnt) {
                const int rem = Li - b;
                const int r2 = rem % (cm * ntn);
                sp_sel = rem / (cm * ntn);
                nt_sel = r2 / cm;
                const int t = (split ? mb[j] : 0) + r2 % cm;
                m0_sel = ofs[j] + balanced_start(ofs[j + 1] - ofs[j], mts[j], t);
                mend_sel = ofs[j] + balanced_start(ofs[j + 1] - ofs[j], mts[j], t + 1);
                e_sel = e0 + j;
            }
            b += cnt;
        }
    }
    const int owner = __builtin_ctzll(ballot64(mine));
    ti.e = __builtin_amdgcn_readlane(e_sel, owner);
    ti.m0 = __builtin_amdgcn_readlane(m0_sel, owner);
    ti.mend = __builtin_amdgcn_readlane(mend_sel, owner);
    ti.nt = __builtin_amdgcn_readlane(nt_sel, owner);
    ti.split = __builtin_amdgcn_readlane(sp_sel, owner);
    ti.row0 = row0;
    ti.srows = rows_end - row0;
    k0s = split ? (ti.split * nk) / S : 0;
    nks = split ? ((ti.split + 1) * nk) / S - k0s : nk;
    return true;
}

}  // namespace moe
