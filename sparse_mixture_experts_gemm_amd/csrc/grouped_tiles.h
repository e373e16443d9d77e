// Work items of the grouped GEMMs over the permuted rows: each expert's
// rows [offsets[e], offsets[e+1]) are cut into m tiles, and every launch
// finds its block's item from the device-side offsets.
#pragma once

#include "device_common.h"

namespace moe {

// Flat work index -> (expert, m range, n tile, K split).  Work items are
// ordered expert, split, n tile, m tile (m fastest), so the m tiles that
// share a weight tile are adjacent.
struct TileInfo {
    int e, m0, mend, nt, split;
};

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
// over the block).
__device__ __forceinline__ bool find_tile(const int32_t *__restrict__ offsets, int E, int ntiles_n,
                                          int bm, int splits, int blk, int32_t *claim, int *slot,
                                          TileInfo &ti) {
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
    ti.m0 = beg + (rem % mt) * bm;
    ti.mend = end;
    return true;
}

}  // namespace moe
