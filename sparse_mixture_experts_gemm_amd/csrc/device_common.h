// Device helpers shared by the gfx950 kernels: bf16 conversion, wave-level
// shuffles (DPP inside a row of 16 lanes, ds_bpermute across rows) and ballots.
#pragma once

#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __hip_bfloat16 b = __float2bfloat16(f);
    return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// DPP controls (gfx9 encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Partner exchange for butterfly steps.  For steps 1, 2, 4, 8 the partner is
// a DPP lane permutation inside a row of 16 (xor for 1 and 2, mirrors for 4
// and 8: the mirror partner lies in the other half of the same group, which
// is all a reduction needs); 16 and 32 cross rows through ds_bpermute.
template <int STEP>
__device__ __forceinline__ float exch_f32(float v) {
    if constexpr (STEP == 1) return dpp_f32<kDppQuadXor1>(v);
    else if constexpr (STEP == 2) return dpp_f32<kDppQuadXor2>(v);
    else if constexpr (STEP == 4) return dpp_f32<kDppRowHalfMirror>(v);
    else if constexpr (STEP == 8) return dpp_f32<kDppRowMirror>(v);
    else return __shfl_xor(v, STEP, 64);
}
template <int STEP>
__device__ __forceinline__ int exch_i32(int v) {
    if constexpr (STEP == 1) return dpp_i32<kDppQuadXor1>(v);
    else if constexpr (STEP == 2) return dpp_i32<kDppQuadXor2>(v);
    else if constexpr (STEP == 4) return dpp_i32<kDppRowHalfMirror>(v);
    else if constexpr (STEP == 8) return dpp_i32<kDppRowMirror>(v);
    else return __shfl_xor(v, STEP, 64);
}

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

// number of lanes below this one whose bit is set in m
__device__ __forceinline__ int rank_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0)); }

// Buffer resource over [base, base + bytes): base and extent are made
// wave-uniform explicitly, so the descriptor is built in scalar registers and
// every load takes it from there.  A load whose lane offset is at or past the
// extent reads nothing and returns zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>((hi << 32) | lo), (short)0,
                                             __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}
// A lane offset past every extent used with it (each is below 2 GiB): such a
// load fetches nothing.
constexpr uint32_t kPastEnd = 0x80000000u;

// XOR swizzle of the eight 16-byte chunks of a 128-byte LDS row.  Fragment
// reads touch one chunk of 16 (or 8) consecutive rows per LDS cycle; with
// this swizzle those rows hit distinct banks whether the LDS serves 16 lanes
// over 64 banks or 8 lanes over 32 banks per cycle.
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// s_waitcnt with only the vector-memory counter: at most n loads in flight.
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))

}  // namespace moe
