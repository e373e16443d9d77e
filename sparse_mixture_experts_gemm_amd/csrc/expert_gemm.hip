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
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "grouped_tiles.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kGemmThreads = 256;
constexpr int kBM = 256;   // rows per tile
constexpr int kBN = 256;   // weight rows per tile (gate-up: 128 of W1 + 128 of W3)
constexpr int kWgradGroupM = 8;  // m tiles per group in the weight-gradient tile order
constexpr int kBK = 64;    // K per pipeline step: 128-byte row segments (one cache line)
constexpr int kRowBytes = kBK * 2;           // one tile row in LDS
constexpr int kTileBytes = kBM * kRowBytes;  // one operand tile (32 KiB)
constexpr int kLoadsPerOperand = kTileBytes / 1024 / 4;  // 1 KiB wave loads per wave (8)
constexpr int kRowsPerLoad = 1024 / kRowBytes;           // rows per wave load (8)

// kGateUpRaw: the gate-up GEMM storing its two products a = x W1^T and
// b = x W3^T in fp32 instead of silu(a) * b (the backward pass needs them).
// kPlain: one bf16 x bf16 product C = A B^T stored in fp32 (the backward
// pass's GEMMs, K-split like the down projection).
// kGateUpE4M3 / kDownE4M3, kGateUpI8 / kDownI8: kGateUp / kDown with
// one-byte weight codes (OCP E4M3 or INT8) and one fp32 scale per weight
// row: the B tile holds the codes (64-byte rows), the fragments are widened
// exactly in registers, and the row scales multiply the fp32 accumulators
// in the epilogue (a weight row's scale factors out of its dot products).
// kPlainBT: kPlain with B given N-contiguous ([K][N] row-major per expert,
// the natural layout of W2 for u = dy W2 and of W1 / W3 for the input
// gradient): a B stage holds 64 K rows of the tile's 256 columns and the
// fragments are read with the transposing LDS read (ds_read_b64_tr_b16).
// kPlainH: kPlain on fp16 operands (the weight gradients dW1 and dW3: the
// scaled fp16 da or db against fp16 x), its fp32 result multiplied by
// GemmOut::scale in the epilogue.
// kPlainBTH: kPlainBT with A in fp16 (the input gradient: the scaled fp16 da
// and db against W1 and W3), B widened to fp16 after the transposing read.
enum { kGateUp = 0, kDown = 1, kGateUpRaw = 2, kPlain = 3, kGateUpE4M3 = 4, kDownE4M3 = 5, kGateUpI8 = 6,
       kDownI8 = 7, kPlainBT = 8, kPlainH = 9, kPlainBTH = 10 };

// one-byte weight codes: OCP E4M3 or INT8
enum { kQE4M3 = 0, kQInt8 = 1 };

template <int MODE>
__device__ __forceinline__ constexpr bool q_mode() { return MODE >= kGateUpE4M3 && MODE <= kDownI8; }
template <int MODE>
__device__ __forceinline__ constexpr int q_fmt() { return MODE >= kGateUpI8 ? kQInt8 : kQE4M3; }
template <int MODE>
__device__ __forceinline__ constexpr bool b_trans() { return MODE == kPlainBT || MODE == kPlainBTH; }
// The SwiGLU epilogue (h = silu(a) * b, fp16)
template <int MODE>
__device__ __forceinline__ constexpr bool gate_up() { return MODE == kGateUp || MODE == kGateUpE4M3 || MODE == kGateUpI8; }
// The B tile is 128 rows of W1 and the same 128 rows of W3 (gate-up modes),
// or 256 rows of one matrix.
template <int MODE>
__device__ __forceinline__ constexpr bool two_b() { return gate_up<MODE>() || MODE == kGateUpRaw; }
// The down projection: A = h (fp16), fp16 matrix cores
template <int MODE>
__device__ __forceinline__ constexpr bool down_mode() { return MODE == kDown || MODE == kDownE4M3 || MODE == kDownI8; }
// Bytes of one B tile row (64 K elements) in LDS, and this wave's B loads
// of 1 KiB per K step
template <int MODE>
__device__ __forceinline__ constexpr int b_row_bytes() { return q_mode<MODE>() ? 64 : 128; }
template <int MODE>
__device__ __forceinline__ constexpr int b_loads() { return q_mode<MODE>() ? 4 : 8; }
// Chunk swizzle of a 64-byte B row of codes (four 16-byte chunks): a
// fragment read takes 8 bytes of one chunk from 32 consecutive rows, which
// this spreads over 16 of the four chunk positions x four rows' bank
// groups (two lanes per bank pair)
__device__ __forceinline__ int swz4(int row) { return (row >> 2) & 3; }


template <typename T>
__device__ __forceinline__ T *slice_ptr(const GemmOut &o, int split) {
    return split == 0 ? static_cast<T *>(o.y0) : static_cast<T *>(o.y_rest) + (size_t)(split - 1) * o.stride;
}

// Row m of the tile's slice (GemmOut): the uniform layout, or (PLAN) the
// split plan's, whose slices 1.. hold only the split rows.
template <typename T, bool PLAN>
__device__ __forceinline__ T *slice_row(const GemmOut &o, const TileInfo &ti, int m, int N) {
    if (!PLAN) return slice_ptr<T>(o, ti.split) + (size_t)m * N;
    if (ti.split == 0) return static_cast<T *>(o.y0) + (size_t)m * N;
    return static_cast<T *>(o.y_rest) + ((size_t)(ti.split - 1) * ti.srows + (m - ti.row0)) * N;
}

// silu(a) * b with the hardware exp and reciprocal (about 1 ulp each in
// fp32, far below the fp16 / fp32 rounding of the stored result).  Large
// negative a gives exp -> inf, rcp -> 0, so silu -> -0.
__device__ __forceinline__ float silu_mul(float a, float b) {
    return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)) * b;
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

// eight INT8 values (two's complement) -> eight bf16 (gate-up) or fp16
// (down), element i from byte i: sign-extended, converted to fp32 and packed.
// Every value in [-128, 127] is exact in both types; for bf16 the fp32 bits
// of such an integer end in 16 zero bits, so the upper halves are packed.
template <bool F16>
__device__ __forceinline__ uint32_t i8x2_widen(uint32_t w, int byte0) {
    const float a = (float)(int32_t)__builtin_amdgcn_sbfe(w, 8 * byte0, 8),
                b = (float)(int32_t)__builtin_amdgcn_sbfe(w, 8 * byte0 + 8, 8);
    if constexpr (F16) return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
    else return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// eight one-byte codes -> eight bf16 (gate-up) or fp16 (down), element i
// from byte i
template <bool F16, int FMT = kQE4M3>
__device__ __forceinline__ uint4 fp8x8_widen(uint2 q) {
    if constexpr (FMT == kQInt8) {
        return make_uint4(i8x2_widen<F16>(q.x, 0), i8x2_widen<F16>(q.x, 2), i8x2_widen<F16>(q.y, 0),
                          i8x2_widen<F16>(q.y, 2));
    } else if constexpr (F16) {
        return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(q.x, 1.0f, false)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(q.x, 1.0f, true)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(q.y, 1.0f, false)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(q.y, 1.0f, true)));
    } else {
        return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, false)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, true)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, false)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, true)));
    }
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

typedef __attribute__((address_space(3))) char lds_char_t;
typedef const __attribute__((address_space(1))) char gbl_char_t;

// 16 bytes per lane straight from global memory into LDS: the 64 lanes of
// the wave fill the 1 KiB starting at the wave-uniform address `dst`.
__device__ __forceinline__ void g2lds16(const char *src, char *dst) {
    __builtin_amdgcn_global_load_lds((gbl_char_t *)src, (lds_char_t *)dst, 16, 0, 0);
}

// Loads through a buffer resource (make_rsrc, kPastEnd): the base and extent
// are in scalar registers, the lane's byte offset in `voff` and a
// wave-uniform offset (the K step) in `soff`, so no 64-bit address is kept
// per load; reads at or past the extent return zeros.
__device__ __forceinline__ void buf2lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, char *dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_char_t *)dst, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ uint4 lds_read16(const char *p) { return *reinterpret_cast<const uint4 *>(p); }

// gfx950's transposing LDS read of 16-bit elements: within each group of 16
// lanes, lane 4a + b receives element b of the four-element rows addressed
// by lanes a, a + 4, a + 8 and a + 12 (as elements 0..3).
typedef short u16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u16x4_t ds_read_tr16(const char *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) u16x4_t *)(p));
}

// LDS read issued as inline assembly, for the weight-streaming kernels: the
// compiler's wait-count pass then does not take it for a read of a buffer
// that a stage load in flight may still write, and adds no wait for all loads
// at the head of the K loop (the explicit vmcnt wait and the barrier before
// the read order the stage being read).  Ready only after the lgkmcnt wait
// that names it.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4_t lds_read16_async(const char *p) {
    u32x4_t v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"((uint32_t)(uintptr_t)(const lds_char_t *)p) : "memory");
    return v;
}

// Scheduling hints: interleave one group of `n` instructions of a class.
#define SCHED_MFMA(n) __builtin_amdgcn_sched_group_barrier(0x008, n, 0)
#define SCHED_DSR(n) __builtin_amdgcn_sched_group_barrier(0x100, n, 0)
#define SCHED_VMEM(n) __builtin_amdgcn_sched_group_barrier(0x020, n, 0)
#define SCHED_VALU(n) __builtin_amdgcn_sched_group_barrier(0x002, n, 0)

// Per-thread state of the MFMA grouped GEMM.
struct GemmThread {
    uint32_t a_off[kLoadsPerOperand], b_off[kLoadsPerOperand];  // byte offsets from the bases (16 B per lane)
    __amdgpu_buffer_rsrc_t a_rsrc;  // A rows: the tile's first row, or the unpermuted x
    __amdgpu_buffer_rsrc_t b_rsrc;  // this wave's weight rows: W1 / W3 (gate-up) or W2
    int a_valid;                          // valid rows of the tile (uniform)
    uint32_t fa[2][4], fb[2][4];  // LDS byte offsets of fragments [block parity][sub-step]
                                  // (kPlainBT: fb[0][jn] is block jn's base, see load_frags)
    uint32_t b_kstep;             // kPlainBT: bytes between the B rows of consecutive K steps
    int wave;
};

template <int MODE>
__device__ __forceinline__ int b_imm(int jn) {
    if (two_b<MODE>()) return ((jn < 2 ? 0 : kBN / 2) + (jn & 1) * 32) * b_row_bytes<MODE>();
    return jn * 32 * b_row_bytes<MODE>();
}

// Issue this wave's global -> LDS loads of one operand (HALF 0: A, 1: B) of
// one K step into that operand's LDS buffer `buf`.  Rows past the tile's last
// valid row in a partly valid 8-row group re-read that row (clamped offsets);
// groups wholly past it carry an offset beyond the buffer extent, so their
// loads fetch nothing and write zeros (those LDS rows feed only discarded
// outputs), with no branch in the loop.
template <int MODE, int HALF, int J0 = 0, int J1 = kLoadsPerOperand>
__device__ __forceinline__ void issue_loads(const GemmThread &g, char *buf, uint32_t kb) {
    if (HALF == 0 || !q_mode<MODE>()) {
        // kPlainBT: the K step advances 64 B rows, not 128 bytes along a row
        const uint32_t kbb = b_trans<MODE>() ? (kb / kRowBytes) * g.b_kstep : kb;
#pragma unroll
        for (int j = J0; j < J1; j++) {
            const int grp = g.wave * kLoadsPerOperand + j;  // 8-row group (kPlainBT: 2 K rows)
            if (HALF == 0) buf2lds16(g.a_rsrc, g.a_off[j], kb, buf + grp * 1024);
            else buf2lds16(g.b_rsrc, g.b_off[j], kbb, buf + grp * 1024);
        }
    } else {
        // one-byte codes: 16-row groups of 64-byte rows, the K step is 64 bytes
#pragma unroll
        for (int j = J0; j < (J1 < b_loads<MODE>() ? J1 : b_loads<MODE>()); j++) {
            const int grp = g.wave * b_loads<MODE>() + j;
            buf2lds16(g.b_rsrc, g.b_off[j], kb >> 1, buf + grp * 1024);
        }
    }
}

// Fragments of one 16-wide K sub-step: A of the wave's four 32-row blocks,
// B of its four 32-column blocks.
struct Frags {
    uint4 a[4], b[4];
};

template <int MODE>
__device__ __forceinline__ void load_frags(const GemmThread &g, const char *abuf, const char *bbuf, int ss,
                                           Frags &f) {
#pragma unroll
    for (int i = 0; i < 4; i++) f.a[i] = lds_read16(abuf + g.fa[i & 1][ss] + i * 32 * kRowBytes);
#pragma unroll
    for (int jn = 0; jn < 4; jn++) {
        if constexpr (b_trans<MODE>()) {
            // two transposing reads: K rows 16 ss + 8 (lane / 32) + 0..3, then
            // + 4..7 (2 KiB further), of the lane's column
            const char *p = bbuf + g.fb[0][jn] + ss * 16 * 512;
            const u16x4_t v0 = ds_read_tr16(p), v1 = ds_read_tr16(p + 4 * 512);
            const uint2 w0 = __builtin_bit_cast(uint2, v0), w1 = __builtin_bit_cast(uint2, v1);
            f.b[jn] = make_uint4(w0.x, w0.y, w1.x, w1.y);
        } else if constexpr (q_mode<MODE>()) {
            // eight codes, widened after the read has landed (widen_b)
            const uint2 v = *reinterpret_cast<const uint2 *>(bbuf + g.fb[jn & 1][ss] + b_imm<MODE>(jn));
            f.b[jn] = make_uint4(v.x, v.y, 0u, 0u);
        } else {
            f.b[jn] = lds_read16(bbuf + g.fb[jn & 1][ss] + b_imm<MODE>(jn));
        }
    }
}

// Down GEMM: W2 fragments (bf16) widened to fp16 for the fp16 MFMA; one-byte
// codes widened exactly to bf16 (gate-up) or fp16 (down).
template <int MODE>
__device__ __forceinline__ void widen_b(Frags &f) {
    if constexpr (MODE == kDown || MODE == kPlainBTH) {
#pragma unroll
        for (int jn = 0; jn < 4; jn++) f.b[jn] = bf16x8_to_f16x8(f.b[jn]);
    } else if constexpr (q_mode<MODE>()) {
#pragma unroll
        for (int jn = 0; jn < 4; jn++)
            f.b[jn] = fp8x8_widen<down_mode<MODE>(), q_fmt<MODE>()>(make_uint2(f.b[jn].x, f.b[jn].y));
    }
}

// A padding step (past an odd step count) must add zero: its A fragments
// are replaced by zeros with selects, not branches.
__device__ __forceinline__ void zero_a_if(bool pad, Frags &f) {
#pragma unroll
    for (int i = 0; i < 4; i++) f.a[i] = pad ? make_uint4(0, 0, 0, 0) : f.a[i];
}

// MFMAs of one 16-wide K sub-step on 32-row blocks [I0, min(I1, NACT)) of
// the wave (a partial tile's blocks past the expert's last row do no
// matrix-core work).  NACT is a template parameter so every variant is
// straight-line.
template <int MODE, int NACT, int I0, int I1>
__device__ __forceinline__ void mfma_blocks(const Frags &f, f32x16_t (&acc)[4][4]) {
    constexpr bool kF16 = down_mode<MODE>() || MODE == kPlainH || MODE == kPlainBTH;
#pragma unroll
    for (int i = I0; i < (I1 < NACT ? I1 : NACT); i++) {
#pragma unroll
        for (int jn = 0; jn < 4; jn++) acc[i][jn] = mfma32<kF16>(f.a[i], f.b[jn], acc[i][jn]);
    }
}

// s_waitcnt vmcnt(n) lgkmcnt(0): at most n loads in flight, no LDS access
#define WAIT_VMCNT_LGKM0(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4))
// s_waitcnt vmcnt(0) lgkmcnt(0)
#define WAIT_VM_LGKM0() __builtin_amdgcn_s_waitcnt(0x0070)

// Workgroup barrier without an implied wait on every outstanding memory
// operation (the waits the pipeline needs are explicit); the memory clobber
// keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void block_sync() { asm volatile("s_barrier" ::: "memory"); }

// One sub-step in two scheduling regions.  First half: the MFMAs of blocks
// 0-1 with the LDS reads of the next fragments between them.  Second half:
// the MFMAs of blocks 2-3 with the global loads (if any) and, for the down
// GEMM, the fp16 widening of the fragments just read (by then the reads
// have landed, so the widening does not wait on the LDS latency).
template <int MODE, int NACT, int HALF, bool LOADS, int NV = 8>
__device__ __forceinline__ void sched_half() {
    constexpr int kLo = NACT < 2 ? NACT : 2;
    constexpr int kM = 4 * (HALF == 0 ? kLo : NACT - kLo);  // MFMAs in this half
    if (kM >= 4) {
#pragma unroll
        for (int q = 0; q < 8; q++) {
            if (q < kM) SCHED_MFMA(1);
            if (HALF == 0) SCHED_DSR(1);
            if (HALF == 0 && LOADS && (q * NV) / 8 != ((q + 1) * NV) / 8) SCHED_VMEM(1);
            if (HALF == 1 && LOADS && (q * NV) / 8 != ((q + 1) * NV) / 8) SCHED_VMEM(1);
            if (HALF == 1 && (MODE == kDown || MODE == kPlainBTH)) SCHED_VALU(6);
            if (HALF == 1 && q_mode<MODE>()) SCHED_VALU(q_fmt<MODE>() == kQInt8 ? 6 : 2);
        }
    }
}

template <int MODE, int NACT, bool LOADS_HALF1, int J0 = 0, int J1 = kLoadsPerOperand, int AJ0 = 0,
          int AJ1 = 0>
__device__ __forceinline__ void substep(const GemmThread &g, const char *rd_a, const char *rd_b, int rd_ss,
                                        Frags &nextf, const Frags &f, char *ld_buf, uint32_t kb, int ld_operand,
                                        f32x16_t (&acc)[4][4], char *a_buf = nullptr, uint32_t a_kb = 0) {
    // first half: optionally A loads AJ0 .. AJ1 - 1 into a_buf
    if (AJ1 > AJ0) issue_loads<MODE, 0, AJ0, AJ1>(g, a_buf, a_kb);
    load_frags<MODE>(g, rd_a, rd_b, rd_ss, nextf);
    mfma_blocks<MODE, NACT, 0, 2>(f, acc);
    sched_half<MODE, NACT, 0, (AJ1 > AJ0), AJ1 - AJ0>();
    __builtin_amdgcn_sched_barrier(0);
    if (LOADS_HALF1) {
        if (ld_operand == 0) issue_loads<MODE, 0, J0, J1>(g, ld_buf, kb);
        else issue_loads<MODE, 1, J0, J1>(g, ld_buf, kb);
    }
    widen_b<MODE>(nextf);
    mfma_blocks<MODE, NACT, 2, 4>(f, acc);
    sched_half<MODE, NACT, 1, LOADS_HALF1, J1 - J0>();
    __builtin_amdgcn_sched_barrier(0);
}

// Loads spread over the sub-steps (bf16 gate-up and down GEMMs): a wave
// issues its weight-tile loads in three parts, 0-2 in sub-step 1, 3-5 in
// sub-step 2 and 6-7 in sub-step 3, and its A-tile loads in two, 0-3 after
// the barrier that frees the buffer (the last sub-step of the step) and 4-7
// in the first half of the next step's sub-step 1.  Eight 1 KiB loads per
// wave in one half sub-step (64 per CU) queue at the texture path and hold
// up the in-order issue of the MFMAs behind them; spread, they cost the
// Mixtral-shape layer 2.70 -> 2.52-2.58 ms (gate-up launch -5%, down -8%).
template <int MODE>
__device__ __forceinline__ constexpr bool split_b_loads() { return true; }
constexpr int kA1 = 4;
// weight-tile parts: loads [0, b_part<1>), [b_part<1>, b_part<2>), [b_part<2>, b_loads)
template <int MODE, int P>
__device__ __forceinline__ constexpr int b_part() { return q_mode<MODE>() ? 2 * P : 3 * P; }

// B buffers of each GEMM: three (the third lets a weight tile start almost
// two K steps before its use; measured 1.6% on the Mixtral-shape down
// projection), two for the one-byte down projections, whose widening leaves
// no registers for the addresses of a third.
template <int MODE>
__device__ __forceinline__ constexpr int b_buffers() { return (MODE == kDownE4M3 || MODE == kDownI8) ? 2 : 3; }

// One K step (4 sub-steps of 16) on the A buffer `ca` and B buffer `cb`.
// LDS holds two A buffers and NB B buffers (distinct objects, so the compiler
// can see that reading one never waits on loads into another).  Entry:
// sub-step 0's fragments are in f0; the A tile of the next step (into `na`)
// is already streaming, and with NB = 3 its B tile (into `nb`) too.
// Sub-step 0 starts a B tile: with NB = 3 that of the step after next, into
// the free third buffer `fb`; with NB = 2 that of the next step, into `nb`
// (the bf16 gate-up and down GEMMs spread it over sub-steps 0-2 and finish
// the next step's A tile in sub-step 0's first half, see kB1).
// After sub-step 2 every wave waits for its loads (but the eight B loads of
// this step, with NB = 3) and its LDS reads and meets the others at a
// barrier: the next step's tiles are then complete and no wave reads `ca` or
// `cb` any more, so sub-step 3 (whose fragments are already in registers)
// overlaps the first LDS reads of the next step and the A loads of the step
// after next into `ca`.  Fences between the halves of the sub-steps keep the
// compiler from chaining dependent MFMAs on one accumulator.
// MAYBE_PAD: the step may be the padding step past an odd step count
// (two B buffers only), which must add zero.
template <int MODE, int NACT, bool MAYBE_PAD>
__device__ __forceinline__ void kstep(const GemmThread &g, char *ca, char *cb, char *na, char *nb, char *fb,
                                      uint32_t kb1, uint32_t kb2, bool pad, Frags &f0, f32x16_t (&acc)[4][4]) {
    constexpr bool kRing = b_buffers<MODE>() == 3;
    Frags f1;
    if (MAYBE_PAD) zero_a_if(pad, f0);
    __builtin_amdgcn_sched_barrier(0);
    constexpr bool kSplit = kRing && split_b_loads<MODE>();
    constexpr int kB1 = b_part<MODE, 1>(), kB2 = b_part<MODE, 2>(), kBL = b_loads<MODE>();
    constexpr int kE1 = kSplit ? kB1 : kLoadsPerOperand;
    constexpr int kAE = kSplit ? kA1 : kLoadsPerOperand;  // A loads issued after the barrier
    substep<MODE, NACT, true, 0, kE1, kAE, kLoadsPerOperand>(g, ca, cb, 1, f1, f0, kRing ? fb : nb,
                                                             kRing ? kb2 : kb1, 1, acc, na, kb1);
    if (MAYBE_PAD) zero_a_if(pad, f1);
    substep<MODE, NACT, (kSplit && kB2 > kB1), kB1, kB2>(g, ca, cb, 2, f0, f1, fb, kb2, 1, acc);
    if (MAYBE_PAD) zero_a_if(pad, f0);
    substep<MODE, NACT, (kSplit && kB2 < kBL), kB2, kBL>(g, ca, cb, 3, f1, f0, fb, kb2, 1, acc);
    WAIT_VMCNT_LGKM0(kRing ? b_loads<MODE>() : 0);
    block_sync();
    __builtin_amdgcn_sched_barrier(0);
    if (MAYBE_PAD) zero_a_if(pad, f1);
    substep<MODE, NACT, true, 0, kAE>(g, na, nb, 0, f0, f1, ca, kb2, 0, acc);
}

// Step I of a buffer rotation: A alternates over two buffers, B rotates over
// NB.  The indices are constants, so every step names fixed buffers.
template <int MODE, int NACT, int I, bool MAYBE_PAD = false>
__device__ __forceinline__ void kstep_at(const GemmThread &g, char *a0, char *a1, char *b0, char *b1, char *b2,
                                         uint32_t kb1, uint32_t kb2, bool pad, Frags &f0,
                                         f32x16_t (&acc)[4][4]) {
    constexpr int NB = b_buffers<MODE>();
    char *const A[2] = {a0, a1};
    char *const B[3] = {b0, b1, b2};
    kstep<MODE, NACT, MAYBE_PAD>(g, A[I % 2], B[I % NB], A[(I + 1) % 2], B[(I + 1) % NB], B[(I + 2) % NB], kb1,
                                 kb2, pad, f0, acc);
}

// The K loop, unrolled over one period of the buffer rotation.  Three B
// buffers: 6 steps, then the remaining steps.  Two: pairs of steps, and with
// an odd step count (ODD) the last pair's second step is padding that adds
// zero (a separate last step would cost the down GEMM registers it does not
// have).  Loads past the last step re-read the last tile.
template <int MODE, int NACT, bool ODD>
__device__ __forceinline__ void main_loop(const GemmThread &g, char *a0, char *a1, char *b0, char *b1, char *b2,
                                          int nk, f32x16_t (&acc)[4][4]) {
    constexpr int NB = b_buffers<MODE>();
    auto kb = [nk](int k) -> uint32_t { return (uint32_t)min(k, nk - 1) * kRowBytes; };
    issue_loads<MODE, 0>(g, a0, kb(0));
    issue_loads<MODE, 1>(g, b0, kb(0));
    if (NB == 3) issue_loads<MODE, 1>(g, b1, kb(1));
    WAIT_VMCNT(NB == 3 ? b_loads<MODE>() : 0);
    block_sync();
    Frags f0;
    load_frags<MODE>(g, a0, b0, 0, f0);
    widen_b<MODE>(f0);
    // A(1): the loads the first step's sub-step 1 does not issue
    issue_loads<MODE, 0, 0, (b_buffers<MODE>() == 3 && split_b_loads<MODE>()) ? kA1 : kLoadsPerOperand>(g, a1,
                                                                                                         kb(1));
#define MOE_KSTEP(I, K) kstep_at<MODE, NACT, I>(g, a0, a1, b0, b1, b2, kb((K) + 1), kb((K) + 2), false, f0, acc)
    if constexpr (NB == 3) {
        const int nk6 = nk - nk % 6;
        for (int k = 0; k < nk6; k += 6) {
            MOE_KSTEP(0, k);
            MOE_KSTEP(1, k + 1);
            MOE_KSTEP(2, k + 2);
            MOE_KSTEP(3, k + 3);
            MOE_KSTEP(4, k + 4);
            MOE_KSTEP(5, k + 5);
        }
        // the last nk % 6 steps, in the same rotation.  Nested, so that each
        // step is reached from the previous one only: the compiler then still
        // tells the LDS buffers apart when it places its waits (a join of
        // paths with different loads in flight would make it wait for all).
        const int r = nk - nk6;
        if (r > 0) {
            MOE_KSTEP(0, nk6);
            if (r > 1) {
                MOE_KSTEP(1, nk6 + 1);
                if (r > 2) {
                    MOE_KSTEP(2, nk6 + 2);
                    if (r > 3) {
                        MOE_KSTEP(3, nk6 + 3);
                        if (r > 4) MOE_KSTEP(4, nk6 + 4);
                    }
                }
            }
        }
    } else {
        for (int k = 0; k < nk; k += 2) {
            MOE_KSTEP(0, k);
            kstep_at<MODE, NACT, 1, ODD>(g, a0, a1, b0, b1, b2, kb(k + 2), kb(k + 3), k + 1 >= nk, f0, acc);
        }
    }
#undef MOE_KSTEP
}

// Epilogue.  MFMA output layout: the lane holds column l5 of each 32x32
// block, rows 8*(q/4) + 4*hi + q%4.
// Gate-up: h = silu(W1 part) * (W3 part) in fp16.  Two-byte stores straight
// from that layout would take 128 store instructions per wave, so each wave
// stages its 128 x 64 block of h in LDS (row stride 128 B, the 16-byte
// chunks of a row XOR-swizzled by row % 8 so the two half-waves write
// disjoint banks) and writes it back with 16-byte stores, eight lanes per
// 128-byte row segment.  Only the wave's own LDS region is touched, so no
// barrier is needed between the LDS writes and reads.
// Down: fp32 partial products, 32 lanes store one 128-byte row segment.
// One-byte weights: the accumulators of weight row n are multiplied by its
// scale (sc0 for W1 or W2 rows, sc1 for W3 rows; [E][N]) first.
template <int MODE, int NACT, bool PLAN = false>
__device__ __forceinline__ void store_tile(const TileInfo &ti, int n0, int N, int wm, int wn, int lane,
                                           const GemmOut &out, const float *sc0, const float *sc1,
                                           const f32x16_t (&acc)[4][4], char *w) {
    const int l5 = lane & 31, hi = lane >> 5;
    if (gate_up<MODE>()) {
        uint16_t *out_h = static_cast<uint16_t *>(out.y0);
        // the scales of this lane's two h columns (W1 rows and W3 rows)
        float s1c[2] = {1.0f, 1.0f}, s3c[2] = {1.0f, 1.0f};
        if constexpr (q_mode<MODE>()) {
#pragma unroll
            for (int jn = 0; jn < 2; jn++) {
                const size_t col = (size_t)ti.e * N + min(n0 + wn * 64 + jn * 32 + l5, N - 1);
                s1c[jn] = sc0[col];
                s3c[jn] = sc1[col];
            }
        }
#pragma unroll
        for (int i = 0; i < NACT; i++)
#pragma unroll
            for (int jn = 0; jn < 2; jn++)
#pragma unroll
                for (int q = 0; q < 16; q++) {
                    const int row = i * 32 + 8 * (q >> 2) + 4 * hi + (q & 3);
                    const int col = jn * 32 + l5;
                    const int chunk = (col >> 3) ^ (row & 7);
                    const float av = q_mode<MODE>() ? acc[i][jn][q] * s1c[jn] : acc[i][jn][q];
                    const float bv = q_mode<MODE>() ? acc[i][jn + 2][q] * s3c[jn] : acc[i][jn + 2][q];
                    *reinterpret_cast<uint16_t *>(w + row * kRowBytes + chunk * 16 + (col & 7) * 2) =
                        f32_to_f16_sat(silu_mul(av, bv));
                    // one 16-value block at a time keeps the live register set small
                    if (q == 15) __builtin_amdgcn_sched_barrier(0);
                }
        const int cb = n0 + wn * 64;  // first column of this wave's block (N is a multiple of 64)
        if (cb >= N) return;
#pragma unroll
        for (int rd = 0; rd < NACT * 4; rd++) {
            const int row = rd * 8 + (lane >> 3), pc = lane & 7;
            const uint4 v = lds_read16(w + row * kRowBytes + pc * 16);
            const int m = ti.m0 + wm * 128 + row;
            if (m < ti.mend)
                *reinterpret_cast<uint4 *>(out_h + (size_t)m * N + cb + ((pc ^ (row & 7)) << 3)) = v;
        }
    } else if (MODE == kGateUpRaw) {
        // a (W1 part, blocks jn 0-1) and b (W3 part, jn 2-3) of the wave's 64
        // columns, staged per 32-row block as 128 fp32 columns (a, then b)
        // like the down projection's partials, then 16-byte stores to y0 (a)
        // and y_rest (b), both [rows][N]
        const int cb = n0 + wn * 64;
#pragma unroll
        for (int i = 0; i < NACT; i++) {
#pragma unroll
            for (int jn = 0; jn < 4; jn++)
#pragma unroll
                for (int q = 0; q < 16; q++) {
                    const int row = 8 * (q >> 2) + 4 * hi + (q & 3);
                    const int col = jn * 32 + l5;
                    const int chunk = (col >> 2) ^ (((row >> 2) & 1) << 3);
                    *reinterpret_cast<float *>(w + row * 512 + chunk * 16 + (col & 3) * 4) = acc[i][jn][q];
                }
#pragma unroll
            for (int rd = 0; rd < 16; rd++) {
                const int row = rd * 2 + (lane >> 5), pc = lane & 31;
                const uint4 v = lds_read16(w + row * 512 + pc * 16);
                const int m = ti.m0 + wm * 128 + i * 32 + row;
                const int lc = (pc ^ (((row >> 2) & 1) << 3)) << 2;  // logical column 0..127
                const int col = cb + (lc & 63);
                float *dst = static_cast<float *>(lc < 64 ? out.y0 : out.y_rest);
                if (m < ti.mend && col < N) *reinterpret_cast<uint4 *>(dst + (size_t)m * N + col) = v;
            }
        }
    } else {
        // one 32 x 128 fp32 block per pass through the wave's 16 KiB of LDS
        // (512-byte rows; the 16-byte chunks of rows 4..7 mod 8 XOR-swizzled by
        // 8 so the two half-waves, four rows apart, write disjoint banks), then
        // 32 lanes per 512-byte row segment: 16-byte stores of fp32, or, with
        // row gates, 8-byte stores of the fp16 gated values
        const int cb = n0 + wn * 128;  // first column of this wave's block (N is a multiple of 64)
        const bool gated = out.row_gate != nullptr;
        // one-byte weights: the scales of this lane's four output columns
        float s2c[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        if constexpr (q_mode<MODE>()) {
#pragma unroll
            for (int jn = 0; jn < 4; jn++) s2c[jn] = sc0[(size_t)ti.e * N + min(cb + jn * 32 + l5, N - 1)];
        }
        // gates of the wave's 128 rows: row l of the wave in g_lo of lane l,
        // row 64 + l in g_hi (rows past the expert's end read its last row)
        float g_lo = 0.0f, g_hi = 0.0f;
        if (gated) {
            const int r0 = ti.m0 + wm * 128;
            g_lo = out.row_gate[min(r0 + lane, ti.mend - 1)];
            g_hi = out.row_gate[min(r0 + 64 + lane, ti.mend - 1)];
        }
#pragma unroll
        for (int i = 0; i < NACT; i++) {
#pragma unroll
            for (int jn = 0; jn < 4; jn++)
#pragma unroll
                for (int q = 0; q < 16; q++) {
                    const int row = 8 * (q >> 2) + 4 * hi + (q & 3);
                    const int col = jn * 32 + l5;
                    const int chunk = (col >> 2) ^ (((row >> 2) & 1) << 3);
                    *reinterpret_cast<float *>(w + row * 512 + chunk * 16 + (col & 3) * 4) =
                        q_mode<MODE>() ? acc[i][jn][q] * s2c[jn] : acc[i][jn][q];
                }
#pragma unroll
            for (int rd = 0; rd < 16; rd++) {
                const int row = rd * 2 + (lane >> 5), pc = lane & 31;
                const uint4 v = lds_read16(w + row * 512 + pc * 16);
                const int m = ti.m0 + wm * 128 + i * 32 + row;
                const int col = cb + ((pc ^ (((row >> 2) & 1) << 3)) << 2);
                if (gated) {
                    // row i * 32 + row of the wave: lane (i & 1) * 32 + row of g_lo (i < 2) or g_hi
                    const float g = __shfl(i < 2 ? g_lo : g_hi, (i & 1) * 32 + row, 64);
                    const uint32_t lo = (uint32_t)f32_to_f16_sat(g * __uint_as_float(v.x)) |
                                        ((uint32_t)f32_to_f16_sat(g * __uint_as_float(v.y)) << 16);
                    const uint32_t hi2 = (uint32_t)f32_to_f16_sat(g * __uint_as_float(v.z)) |
                                         ((uint32_t)f32_to_f16_sat(g * __uint_as_float(v.w)) << 16);
                    if (m < ti.mend && col < N)
                        *reinterpret_cast<uint2 *>(slice_row<uint16_t, PLAN>(out, ti, m, N) + col) =
                            make_uint2(lo, hi2);
                } else if (m < ti.mend && col < N) {
                    if constexpr (MODE == kPlainH) {
                        // weight gradients: written once, never read here, so
                        // the stores bypass L2 and leave it to the operands
                        const f32x4_t o = {out.scale * __uint_as_float(v.x), out.scale * __uint_as_float(v.y),
                                           out.scale * __uint_as_float(v.z), out.scale * __uint_as_float(v.w)};
                        __builtin_nontemporal_store(
                            o, reinterpret_cast<f32x4_t *>(slice_row<float, PLAN>(out, ti, m, N) + col));
                    } else {
                        *reinterpret_cast<uint4 *>(slice_row<float, PLAN>(out, ti, m, N) + col) = v;
                    }
                }
            }
        }
    }
}

// A whole tile for one active-block count: the accumulators live only
// inside this function, so the variants never merge.
template <int MODE, int NACT, bool ODD, bool PLAN = false>
__device__ __forceinline__ void run_tile(const GemmThread &g, const TileInfo &ti, char *a0, char *a1, char *b0,
                                         char *b1, char *b2, int nk, int n0, int N, int wm, int wn, int lane,
                                         const GemmOut &out, const float *sc0 = nullptr, const float *sc1 = nullptr) {
    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int jn = 0; jn < 4; jn++)
#pragma unroll
            for (int q = 0; q < 16; q++) acc[i][jn][q] = 0.0f;
    main_loop<MODE, NACT, ODD>(g, a0, a1, b0, b1, b2, nk, acc);
    // the last (discarded) loads and fragment reads have landed in every
    // wave before the epilogue reuses the A buffers (16 KiB per wave)
    WAIT_VM_LGKM0();
    block_sync();
    store_tile<MODE, NACT, PLAN>(ti, n0, N, wm, wn, lane, out, sc0, sc1, acc,
                           (g.wave < 2 ? a0 : a1) + (g.wave & 1) * (kTileBytes / 2));
}

// MODE kGateUp: A = x_perm (bf16), B = W1/W3 (bf16), writes h (fp16).  With
//               a_rows, A is the unpermuted x and row m of the expert range
//               is x row a_rows[m] (the dispatch gather folded into the A
//               loads; x must then span less than 2 GiB).
// MODE kDown:   A = h (fp16), B = W2 (bf16, widened to fp16 after the LDS
//               read), writes the down projection (see GemmOut: fp32, or
//               fp16 with the row's combine weight folded in).  The d_ff
//               reduction is split into `splits` slices (work items of their
//               own, for enough work to fill the chip); each slice stores
//               its partial product and a later pass (the fix-up or the
//               combine) adds the slices in order, so the result is
//               deterministic.
//
// LDS: two A buffers and three (gate-up) or two (down) B buffers of 256 rows
// x 64 K (32 KiB each), the eight 16-byte chunks of each row XOR-swizzled by
// swz(row).  Global -> LDS with
// global_load_lds: wave w loads 8-row groups 8w .. 8w+7 of A and of B; lane
// l takes row 8g + l/8 and the logical chunk that lands at physical position
// l%8, so every wave load reads whole 128-byte lines.  Fragments: lane l
// reads row base + l%32 (base a multiple of 32), logical chunk 2s + l/32 of
// sub-step s; the swizzle of such a row is swz(l%32) ^ 4 * parity(base/32).
// PLAN (down projections of moe_forward): the device-side split plan
// (find_tile_planned, out.plan) instead of `splits` uniform slices.
template <int MODE, bool PLAN = false>
__global__ __launch_bounds__(kGemmThreads, 1) void grouped_gemm_bf16(
    const uint16_t *__restrict__ A, const int32_t *__restrict__ a_rows, const uint16_t *__restrict__ B0,
    const uint16_t *__restrict__ B1, const int32_t *__restrict__ offsets, int E, int N, int K, int ldb,
    int ntiles_n, int splits, uint32_t a_bytes, int32_t *claim, GemmOut out, const float *__restrict__ S0 = nullptr,
    const float *__restrict__ S1 = nullptr) {
    __shared__ __attribute__((aligned(1024))) char lds_a0[kTileBytes];
    __shared__ __attribute__((aligned(1024))) char lds_a1[kTileBytes];
    __shared__ __attribute__((aligned(1024))) char lds_b0[kTileBytes];
    __shared__ __attribute__((aligned(1024))) char lds_b1[kTileBytes];
    __shared__ __attribute__((aligned(1024))) char lds_b2[b_buffers<MODE>() == 3 ? kTileBytes : 1024];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    TileInfo ti;
    int k0s, nks;  // first K step and K steps of this item
    if constexpr (PLAN) {
        if (!find_tile_planned(offsets, E, ntiles_n, kBM, K / kBK, blockIdx.x, claim, reinterpret_cast<int *>(lds_a0),
                               out.plan, ti, k0s, nks))
            return;
    } else {
        if (!find_tile(offsets, E, ntiles_n, kBM, splits, blockIdx.x, claim, reinterpret_cast<int *>(lds_a0), ti,
                       true))
            return;
        nks = K / splits / kBK;
        k0s = ti.split * nks;
    }
    const int n0 = two_b<MODE>() ? ti.nt * (kBN / 2) : ti.nt * kBN;
    // bytes per weight element: 2 (bf16) or 1 (one-byte codes)
    constexpr int kWb = q_mode<MODE>() ? 1 : 2;
    const size_t wexp = (size_t)ti.e * N * ldb * kWb;
    const int k_first = k0s * kBK;  // first K element of this item

    GemmThread g;
    g.wave = wave;
    g.a_valid = ti.mend - ti.m0;
    // Buffer extents (all below 2 GiB for A, checked on the host, so an
    // offset of 2 GiB is past the end): A is x (a_bytes) when rows are
    // gathered, else the tile's valid rows; B is the expert's weight matrix
    // (below 4 GiB, also checked).
    g.a_rsrc = a_rows ? make_rsrc(A, a_bytes)
                      : make_rsrc(A + (size_t)ti.m0 * K, (uint32_t)(g.a_valid < kBM ? g.a_valid : kBM) * K * 2);
    const uint32_t w_bytes = (uint32_t)((size_t)N * ldb * kWb);
    // B's K position of this split: B rows of ldb elements, read periodically
    // when the splits of A's K range share one B (ldb < K, a multiple of ks);
    // kPlainBT: ldb is the K extent of each of B0 and B1 ([ldb][N] per
    // expert), taken in turn by consecutive K periods
    const int kb_first = k_first % ldb;
    const uint16_t *bsel = b_trans<MODE>() ? (((k_first / ldb) & 1) ? B1 : B0)
                                           : (two_b<MODE>() && wave >= 2 ? B1 : B0);
    // gate-up: waves 0-1 load B rows 0..127 (W1), waves 2-3 rows 128..255 (W3)
    g.b_rsrc = make_rsrc(reinterpret_cast<const char *>(bsel) + wexp, w_bytes);
#pragma unroll
    for (int j = 0; j < kLoadsPerOperand; j++) {
        const int grp = wave * kLoadsPerOperand + j;
        const int row = grp * kRowsPerLoad + (lane >> 3);
        const int c = (lane & 7) ^ swz(row);
        const int gm = min(ti.m0 + row, ti.mend - 1);
        const int ar = a_rows ? a_rows[gm] : gm - ti.m0;
        g.a_off[j] = grp * kRowsPerLoad < g.a_valid ? ((uint32_t)ar * K + k_first + c * 8) * 2 : kPastEnd;
        if constexpr (b_trans<MODE>()) {
            // K rows 2 grp, 2 grp + 1 of the stage (512 bytes each); lane l
            // takes the logical 16-byte chunk that lands at position l % 32,
            // chunks XOR-swizzled by 4 (row % 4)
            const int kr = 2 * grp + (lane >> 5);
            const int cl = (lane & 31) ^ (4 * (kr & 3));
            const int gc = min(n0 + 8 * cl, N - 8);
            g.b_off[j] = ((uint32_t)(kb_first + kr) * N + gc) * 2;
        } else if constexpr (!q_mode<MODE>()) {
            int gn = two_b<MODE>() ? n0 + (row & (kBN / 2 - 1)) : n0 + row;
            gn = min(gn, N - 1);
            g.b_off[j] = ((uint32_t)gn * ldb + kb_first + c * 8) * 2;
        }
    }
    g.b_kstep = (uint32_t)kBK * N * 2;
    if constexpr (q_mode<MODE>()) {
        // one-byte codes: wave w loads 16-row groups 4w .. 4w+3 of 64-byte
        // rows; lane l takes row 16g + l/4 and the logical 16-byte chunk that
        // lands at position l%4
#pragma unroll
        for (int j = 0; j < b_loads<MODE>(); j++) {
            const int grp = wave * b_loads<MODE>() + j;
            const int row = grp * 16 + (lane >> 2);
            const int c = (lane & 3) ^ swz4(row);
            int gn = two_b<MODE>() ? n0 + (row & (kBN / 2 - 1)) : n0 + row;
            gn = min(gn, N - 1);
            g.b_off[j] = (uint32_t)gn * ldb + kb_first + c * 16;
        }
    }
    const int l5 = lane & 31, hi = lane >> 5;
    const int sw0 = swz(l5);  // swizzle of row base + l5 is sw0 ^ 4 * parity(base / 32)
    const int b_rbase = two_b<MODE>() ? wn * 64 : wn * 128;
#pragma unroll
    for (int pp = 0; pp < 2; pp++)
#pragma unroll
        for (int ss = 0; ss < 4; ss++) {
            const uint32_t sw = (uint32_t)(((2 * ss + hi) ^ sw0 ^ (4 * pp)) << 4);
            g.fa[pp][ss] = (uint32_t)(wm * 128 + l5) * kRowBytes + sw;
            // one-byte codes: 8 bytes (the lane's 8 K values) of logical chunk
            // ss; row base + l5 has swizzle swz4(l5) for any base % 32 == 0
            g.fb[pp][ss] = q_mode<MODE>() ? (uint32_t)(b_rbase + l5) * 64 + ((ss ^ swz4(l5)) << 4) + hi * 8
                                          : (uint32_t)(b_rbase + l5) * kRowBytes + sw;
        }
    if constexpr (b_trans<MODE>()) {
        // block jn's base for the transposing reads: lane 16 g + 4 j' + a'
        // addresses K row 8 (g / 2) + j' (then + 4) and columns wn 128 +
        // jn 32 + 16 (g % 2) + 4 a' .. + 3, in the chunk swizzled by 4 j'
        const int gq = lane >> 4, jq = (lane >> 2) & 3, aq = lane & 3;
#pragma unroll
        for (int jn = 0; jn < 4; jn++)
            g.fb[0][jn] = (uint32_t)((8 * (gq >> 1) + jq) * 512 + 256 * wn + 64 * (jn ^ jq) + 32 * (gq & 1) + 8 * aq);
    }
    // active 32-row blocks of this wave (uniform)
    const int nact_raw = (ti.mend - (ti.m0 + wm * 128) + 31) / 32;
    const int nact = __builtin_amdgcn_readfirstlane(max(0, min(4, nact_raw)));

    const int nk = nks;
#define MOE_TILE(n)                                                                                              \
    do {                                                                                                         \
        if (b_buffers<MODE>() == 2 && (nk & 1))                                                                  \
            run_tile<MODE, n, b_buffers<MODE>() == 2, PLAN>(g, ti, lds_a0, lds_a1, lds_b0, lds_b1, lds_b2, nk, n0, \
                                                            N, wm, wn, lane, out, S0, S1);                     \
        else                                                                                                     \
            run_tile<MODE, n, false, PLAN>(g, ti, lds_a0, lds_a1, lds_b0, lds_b1, lds_b2, nk, n0, N, wm, wn,     \
                                           lane, out, S0, S1);                                                 \
    } while (0)
    switch (nact) {
        case 4: MOE_TILE(4); break;
        case 3: MOE_TILE(3); break;
        case 2: MOE_TILE(2); break;
        case 1: MOE_TILE(1); break;
        default: MOE_TILE(0); break;
    }
#undef MOE_TILE
}

// Weight gradients of the backward pass: for every expert e,
//   C_e[m][n] = sum over the expert's K window of A[m][k] B[n][k],
// A bf16 [M][ldk], B bf16 [N][ldk], C fp32 [E][M][N].  The K axis of A and
// B holds every expert's kept rows (transposed by the backward pass): expert
// e's window starts at kwin_start(offsets, e) and spans 2 Kp_e elements, Kp_e
// its row count rounded up to 64 (the rows, zero padding, then the same for
// the second operand of a hi/lo pair).  Work items are (expert, n tile, m
// tile) over uniform row ranges (unit_offsets[e] = e M); an expert without
// rows gets zeros.  The main loop, LDS layout and epilogue are those of
// grouped_gemm_bf16<kPlain>.
// H: fp16 operands holding only the first half of each window (kPlainH),
// one scaled by 2^k_e per expert (k_e = grad_scale_exp(amax[e])) and, with
// gmax, the other by 2^grad_scale_exp(*gmax); the epilogue undoes both.
template <bool H>
__global__ __launch_bounds__(kGemmThreads, 1) void grouped_gemm_wgrad(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ unit_offsets, int E, int M, int N, int ldk, int ntiles_n, float *__restrict__ C,
    const uint32_t *__restrict__ amax, const uint32_t *__restrict__ gmax) {
    __shared__ __attribute__((aligned(1024))) char lds_a0[kTileBytes];
    __shared__ __attribute__((aligned(1024))) char lds_a1[kTileBytes];
    __shared__ __attribute__((aligned(1024))) char lds_b0[kTileBytes];
    __shared__ __attribute__((aligned(1024))) char lds_b1[kTileBytes];
    __shared__ __attribute__((aligned(1024))) char lds_b2[kTileBytes];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    TileInfo ti;
    if (!find_tile(unit_offsets, E, ntiles_n, kBM, 1, blockIdx.x, nullptr, nullptr, ti)) return;
    const int e = ti.e;
    {
        // Reorder an expert's tiles in groups of kWgradGroupM m tiles, n
        // tiles outer and m inner inside a group, so that the 32 tiles an
        // XCD runs together span about 8 m tiles by 4 n tiles and share
        // both operands in its L2 (m fastest over all 56 m tiles of a
        // d_ff-sized M would fetch a distinct A tile per block).
        const int mt = (M + kBM - 1) / kBM;
        const int rem = ti.nt * mt + (ti.m0 - e * M) / kBM;
        const int grp = rem / (kWgradGroupM * ntiles_n);
        const int gm = min(kWgradGroupM, mt - grp * kWgradGroupM);
        const int j = rem - grp * kWgradGroupM * ntiles_n;
        ti.nt = __builtin_amdgcn_readfirstlane(j / gm);
        ti.m0 = __builtin_amdgcn_readfirstlane(e * M + (grp * kWgradGroupM + j % gm) * kBM);
    }
    const int rbeg = offsets[e], rows = offsets[e + 1] - rbeg;
    const int kp = (rows + kBK - 1) / kBK * kBK;
    const int kwin = kwin_start(rbeg, e);
    const int nk = __builtin_amdgcn_readfirstlane((H ? 1 : 2) * kp / kBK);
    const int m_rel = ti.m0 - e * M;
    const int n0 = ti.nt * kBN;
    GemmOut out{C, nullptr, 0, nullptr};
    if constexpr (H) out.scale = ldexpf(1.0f, -grad_scale_exp(amax[e]) - (gmax ? grad_scale_exp(*gmax) : 0));
    if (nk == 0) {
        // no rows: the tile of C_e is zero (16-byte stores, N a multiple of 64)
        const int mv = min(kBM, M - m_rel), nv = min(kBN, N - n0);
        for (int i = tid; i < mv * (kBN / 4); i += kGemmThreads) {
            const int r = i / (kBN / 4), c = (i % (kBN / 4)) * 4;
            if (c < nv)
                *reinterpret_cast<float4 *>(C + (size_t)(ti.m0 + r) * N + n0 + c) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        return;
    }

    GemmThread g;
    g.wave = wave;
    g.a_valid = min(kBM, M - m_rel);
    const int b_valid = min(kBN, N - n0);
    // per-tile buffer resources at the tile's first row and the expert's
    // window: 256 rows of ldk elements stay below 2 GiB (checked on the host)
    g.a_rsrc = make_rsrc(A + (size_t)m_rel * ldk + kwin, (uint32_t)g.a_valid * ldk * 2);
    g.b_rsrc = make_rsrc(B + (size_t)n0 * ldk + kwin, (uint32_t)b_valid * ldk * 2);
#pragma unroll
    for (int j = 0; j < kLoadsPerOperand; j++) {
        const int grp = wave * kLoadsPerOperand + j;
        const int row = grp * kRowsPerLoad + (lane >> 3);
        const int c = (lane & 7) ^ swz(row);
        g.a_off[j] = grp * kRowsPerLoad < g.a_valid ? ((uint32_t)min(row, g.a_valid - 1) * ldk + c * 8) * 2
                                                     : kPastEnd;
        g.b_off[j] = ((uint32_t)min(row, b_valid - 1) * ldk + c * 8) * 2;
    }
    const int l5 = lane & 31, hi = lane >> 5;
    const int sw0 = swz(l5);
#pragma unroll
    for (int pp = 0; pp < 2; pp++)
#pragma unroll
        for (int ss = 0; ss < 4; ss++) {
            const uint32_t sw = (uint32_t)(((2 * ss + hi) ^ sw0 ^ (4 * pp)) << 4);
            g.fa[pp][ss] = (uint32_t)(wm * 128 + l5) * kRowBytes + sw;
            g.fb[pp][ss] = (uint32_t)(wn * 128 + l5) * kRowBytes + sw;
        }
    const int nact = __builtin_amdgcn_readfirstlane(max(0, min(4, (g.a_valid - wm * 128 + 31) / 32)));
#define MOE_TILE(n)                                                                                              \
    run_tile<H ? kPlainH : kPlain, n, false>(g, ti, lds_a0, lds_a1, lds_b0, lds_b1, lds_b2, nk, n0, N, wm, wn, lane, \
                                             out)
    switch (nact) {
        case 4: MOE_TILE(4); break;
        case 3: MOE_TILE(3); break;
        case 2: MOE_TILE(2); break;
        case 1: MOE_TILE(1); break;
        default: MOE_TILE(0); break;
    }
#undef MOE_TILE
}

// ------------------------------------------------------------- skinny ----
// Small groups (every expert at most 32 rows, e.g. a decode batch): the GEMM
// is a weight stream, so the tile is one 32-row block by 128 weight rows
// (gate-up: 64 columns of h, i.e. 64 rows of W1 and the same 64 rows of W3;
// down: 128 output columns), and six LDS stages keep five K steps (80 KiB of
// weights) in flight per CU.  MFMA 16x16x32 (bf16, or fp16 for the down GEMM
// with W2 widened after the LDS read); 4 waves, each with both 16-row halves
// of the tile and 32 of its weight rows (gate-up: 16 of W1 and the same 16
// of W3).  The down projection is not split (one d_ff slice).
constexpr int kSkThreads = 256;
constexpr int kSkBM = 32;                       // rows per tile
constexpr int kSkBN = 64;                       // h columns per gate-up tile (128 weight rows)
constexpr int kSkBNd = 128;                     // output columns per down tile
constexpr int kSkA = kSkBM * kRowBytes;         // A part of a stage (4 KiB)
constexpr int kSkStage = kSkA + 2 * kSkBN * kRowBytes;  // + B part, 128 weight rows (16 KiB)
constexpr int kSkStages = 6;

template <bool F16>
__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

struct SkThread {
    const char *a_base;  // the tile's first row (or x when rows are gathered)
    const char *b_base[2];
    uint32_t a_off;      // this lane's A load row (wave w loads rows 8w .. 8w+7)
    uint32_t b_off[4];   // this lane's B load rows (gate-up: 4 groups of 8, down: 2)
    int wave;
};

// B rows per tile: 128 (gate-up: W1 rows n0.., then the same rows of W3;
// down: W2 rows n0..); loads per wave per stage: 1 A + 4 B.
template <int MODE>
__device__ __forceinline__ constexpr int sk_lb() { return 4; }

template <int MODE>
__device__ __forceinline__ void sk_issue(const SkThread &g, char *stage, uint32_t kb) {
    g2lds16(g.a_base + g.a_off + kb, stage + g.wave * 1024);
#pragma unroll
    for (int j = 0; j < sk_lb<MODE>(); j++) {
        const int grp = g.wave * sk_lb<MODE>() + j;  // 8-row group of the B part
        const int src = MODE == kGateUp ? grp >> 3 : 0;  // gate-up: groups 8.. are W3
        g2lds16((src ? g.b_base[1] : g.b_base[0]) + g.b_off[j] + kb, stage + kSkA + grp * 1024);
    }
}

template <int MODE, int NB>
__device__ __forceinline__ void sk_compute(const char *stage, int wave, int lane, f32x4_t (&acc)[2][2]) {
    constexpr bool kF16 = MODE == kDown;
    const int r16 = lane & 15, kq = lane >> 4;
    // tile row r (16-row block base + lane % 16), chunk c = 4 * sub-step +
    // lane / 16, through the stage's XOR swizzle; gate-up: W1 rows 16w.. and
    // the same W3 rows (64 further); down: W2 rows 32w.. and 32w+16..  Every
    // fragment of the stage is read, then one wait.
    const int rb0 = (MODE == kGateUp ? 16 : 32) * wave + r16;
    const int rb1 = (MODE == kGateUp ? kSkBN + 16 * wave : 32 * wave + 16) + r16;
    u32x4_t a[2][2], b[2][2];  // [sub-step][16-row block or weight fragment]
#pragma unroll
    for (int ss = 0; ss < 2; ss++) {
        const int c = 4 * ss + kq;
#pragma unroll
        for (int ib = 0; ib < 2; ib++) {
            const int row = ib * 16 + r16;
            a[ss][ib] = lds_read16_async(stage + row * kRowBytes + ((c ^ swz(row)) << 4));
        }
        b[ss][0] = lds_read16_async(stage + kSkA + rb0 * kRowBytes + ((c ^ swz(rb0)) << 4));
        b[ss][1] = lds_read16_async(stage + kSkA + rb1 * kRowBytes + ((c ^ swz(rb1)) << 4));
    }
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(a[0][0]), "+v"(a[0][1]), "+v"(a[1][0]), "+v"(a[1][1]), "+v"(b[0][0]), "+v"(b[0][1]),
                   "+v"(b[1][0]), "+v"(b[1][1])
                 :
                 : "memory");
#pragma unroll
    for (int ss = 0; ss < 2; ss++) {
        uint4 b0 = __builtin_bit_cast(uint4, b[ss][0]), b1 = __builtin_bit_cast(uint4, b[ss][1]);
        if (kF16) {
            b0 = bf16x8_to_f16x8(b0);
            b1 = bf16x8_to_f16x8(b1);
        }
#pragma unroll
        for (int ib = 0; ib < NB; ib++) {
            const uint4 av = __builtin_bit_cast(uint4, a[ss][ib]);
            acc[ib][0] = mfma16<kF16>(av, b0, acc[ib][0]);
            acc[ib][1] = mfma16<kF16>(av, b1, acc[ib][1]);
        }
    }
}

#define SK_STEP(I, cur, nxt)                                                             \
    do {                                                                                 \
        if (k0 + (I) >= nk) goto done;                                                   \
        WAIT_VMCNT((1 + sk_lb<MODE>()) * (kSkStages - 2));                               \
        block_sync();                                                                    \
        sk_issue<MODE>(g, nxt, kb(k0 + (I) + kSkStages - 1));                            \
        sk_compute<MODE, NB>(cur, g.wave, lane, acc);                                    \
    } while (0)

// The K loop: stage k lives in buffer k % 6 (six distinct LDS objects, the
// loop unrolled by six so every access names a fixed one); when step k is
// computed, steps k+1 .. k+4 are in flight and step k+5 is issued into the
// buffer step k-1 used (free: every wave passed the barrier after it).
// Loads past the last step re-read the last K slice.
template <int MODE, int NB>
__device__ __forceinline__ void sk_main(const SkThread &g, int nk, int lane, char *b0, char *b1, char *b2,
                                        char *b3, char *b4, char *b5, f32x4_t (&acc)[2][2]) {
    auto kb = [nk](int k) -> uint32_t { return (uint32_t)min(k, nk - 1) * kRowBytes; };
    sk_issue<MODE>(g, b0, kb(0));
    sk_issue<MODE>(g, b1, kb(1));
    sk_issue<MODE>(g, b2, kb(2));
    sk_issue<MODE>(g, b3, kb(3));
    sk_issue<MODE>(g, b4, kb(4));
    for (int k0 = 0;; k0 += kSkStages) {
        SK_STEP(0, b0, b5);
        SK_STEP(1, b1, b0);
        SK_STEP(2, b2, b1);
        SK_STEP(3, b3, b2);
        SK_STEP(4, b4, b3);
        SK_STEP(5, b5, b4);
    }
done:
    WAIT_VMCNT(0);
}

template <int MODE>
__global__ __launch_bounds__(kSkThreads) void grouped_gemm_skinny(
    const uint16_t *__restrict__ A, const int32_t *__restrict__ a_rows, const uint16_t *__restrict__ B0,
    const uint16_t *__restrict__ B1, const int32_t *__restrict__ offsets, int E, int N, int K, int ntiles_n,
    int splits, GemmOut out) {
    __shared__ __attribute__((aligned(1024))) char sb0[kSkStage];
    __shared__ __attribute__((aligned(1024))) char sb1[kSkStage];
    __shared__ __attribute__((aligned(1024))) char sb2[kSkStage];
    __shared__ __attribute__((aligned(1024))) char sb3[kSkStage];
    __shared__ __attribute__((aligned(1024))) char sb4[kSkStage];
    __shared__ __attribute__((aligned(1024))) char sb5[kSkStage];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    TileInfo ti;
    if (!find_tile(offsets, E, ntiles_n, kSkBM, splits, blockIdx.x, nullptr, nullptr, ti)) return;
    const int n0 = ti.nt * (MODE == kGateUp ? kSkBN : kSkBNd);
    const size_t wexp = (size_t)ti.e * N * K;
    const int ks = K / splits;
    const int k_first = ti.split * ks;

    SkThread g;
    g.wave = wave;
    g.a_base = reinterpret_cast<const char *>(a_rows ? A : A + (size_t)ti.m0 * K);
    {
        const int row = wave * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(row);
        const int gm = min(ti.m0 + row, ti.mend - 1);
        const int ar = a_rows ? a_rows[gm] : gm - ti.m0;
        g.a_off = ((uint32_t)ar * K + k_first + c * 8) * 2;
    }
    g.b_base[0] = reinterpret_cast<const char *>(B0 + wexp);
    g.b_base[1] = reinterpret_cast<const char *>((MODE == kGateUp ? B1 : B0) + wexp);
#pragma unroll
    for (int j = 0; j < sk_lb<MODE>(); j++) {
        const int grp = wave * sk_lb<MODE>() + j;
        const int row = grp * 8 + (lane >> 3);  // row of the B part
        const int c = (lane & 7) ^ swz(row);
        const int gn = min(n0 + (MODE == kGateUp ? (row & (kSkBN - 1)) : row), N - 1);
        g.b_off[j] = ((uint32_t)gn * K + k_first + c * 8) * 2;
    }
    const int nk = ks / kBK;
    f32x4_t acc[2][2];
#pragma unroll
    for (int ib = 0; ib < 2; ib++)
#pragma unroll
        for (int jb = 0; jb < 2; jb++) acc[ib][jb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int nb = ti.mend - ti.m0 > 16 ? 2 : 1;  // active 16-row blocks (uniform)
    if (nb == 2)
        sk_main<MODE, 2>(g, nk, lane, sb0, sb1, sb2, sb3, sb4, sb5, acc);
    else
        sk_main<MODE, 1>(g, nk, lane, sb0, sb1, sb2, sb3, sb4, sb5, acc);

    // epilogue: the lane holds column lane % 16, rows 4 * (lane / 16) + q
#pragma unroll
    for (int ib = 0; ib < 2; ib++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int m = ti.m0 + ib * 16 + 4 * (lane >> 4) + q;
            if (m >= ti.mend) continue;
            if (MODE == kGateUp) {
                const int col = n0 + wave * 16 + (lane & 15);
                if (col < N)
                    static_cast<uint16_t *>(out.y0)[(size_t)m * N + col] =
                        f32_to_f16_sat(silu_mul(acc[ib][0][q], acc[ib][1][q]));
            } else if (out.row_gate) {
                const float gt = out.row_gate[m];
#pragma unroll
                for (int jb = 0; jb < 2; jb++) {
                    const int col = n0 + wave * 32 + jb * 16 + (lane & 15);
                    if (col < N) slice_ptr<uint16_t>(out, ti.split)[(size_t)m * N + col] = f32_to_f16_sat(gt * acc[ib][jb][q]);
                }
            } else {
#pragma unroll
                for (int jb = 0; jb < 2; jb++) {
                    const int col = n0 + wave * 32 + jb * 16 + (lane & 15);
                    if (col < N) slice_ptr<float>(out, ti.split)[(size_t)m * N + col] = acc[ib][jb][q];
                }
            }
        }
}
#undef SK_STEP

// ------------------------------------------------------ skinny, FP8 W ----
// FP8 (OCP E4M3) expert weights with one fp32 scale per weight row,
// W[n][k] = s[n] * q[n][k], in the weight-streaming regime (every expert at
// most 32 rows).  The tile is that of the bf16 skinny kernel, but a stage
// spans 128 K elements (weight rows of 128 bytes, x or h rows of 256 bytes),
// so a stage carries as many weight bytes as there over twice the K depth.
// The q fragments are converted in registers, exactly, to bf16
// (gate-up) or fp16 (down) with the gfx950 scaled conversion at scale 1; the
// row scales multiply the fp32 accumulators in the epilogue (a row's scale
// factors out of its dot products).
constexpr int kSk8A = kSkBM * 256;                   // A part: 32 rows x 128 elements (8 KiB)
constexpr int kSk8Stage = kSk8A + 2 * kSkBN * 128;  // + 128 weight rows x 128 bytes (16 KiB)
constexpr int kSk8K = 128;                           // K elements per stage
// Three stages (72 KiB of LDS) and two blocks per CU: one block's start-up
// and drain overlap the other's streaming (up to four stages in flight per
// CU, against five for one block of six stages; measured 4% faster).
constexpr int kSk8Stages = 3;

struct Sk8Thread {
    const char *a_base;
    const char *b_base[2];
    uint32_t a_off[2];  // wave w loads A rows 8w .. 8w+7, four per load
    uint32_t b_off[4];
    int wave;
};

// Chunk swizzle of a 256-byte A row (16 chunks of 16 bytes): a fragment read
// touches one chunk of 16 consecutive rows, which the XOR spreads over all
// the banks.
__device__ __forceinline__ int swz16(int row) { return row & 15; }

template <int MODE>
__device__ __forceinline__ void sk8_issue(const Sk8Thread &g, char *stage, int k) {
    const uint32_t ka = (uint32_t)k * kSk8K * 2, kq = (uint32_t)k * kSk8K;
    g2lds16(g.a_base + g.a_off[0] + ka, stage + (2 * g.wave) * 1024);
    g2lds16(g.a_base + g.a_off[1] + ka, stage + (2 * g.wave + 1) * 1024);
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int grp = g.wave * 4 + j;                  // 8-row group of the B part
        const int src = MODE == kGateUp ? grp >> 3 : 0;  // gate-up: groups 8.. are W3
        g2lds16((src ? g.b_base[1] : g.b_base[0]) + g.b_off[j] + kq, stage + kSk8A + grp * 1024);
    }
}


template <int MODE, int NB, int FMT>
__device__ __forceinline__ void sk8_compute(const char *stage, int wave, int lane, f32x4_t (&acc)[2][2]) {
    constexpr bool kF16 = MODE == kDown;
    const int r16 = lane & 15, kq = lane >> 4;
    const int rb0 = (MODE == kGateUp ? 16 : 32) * wave + r16;
    const int rb1 = (MODE == kGateUp ? kSkBN + 16 * wave : 32 * wave + 16) + r16;
    // The stage's 128 K elements are taken in an order of their own (a dot
    // product does not depend on the order of its terms, as long as both
    // operands follow it): for sub-step pair pr, lane quarter kq reads one
    // 16-byte chunk 4 pr + kq of a weight row (16 K elements) and spends its
    // halves on sub-steps 2 pr and 2 pr + 1; the x fragments are the 8
    // elements at the same K, chunk 8 pr + 2 kq + half of the 256-byte row.
    // Every fragment of the stage is read, then one wait.
    u32x4_t q[2][2], a[2][2][2];  // [pair][weight fragment], [pair][half][16-row block]
#pragma unroll
    for (int pr = 0; pr < 2; pr++) {
        const int cb = 4 * pr + kq;
        q[pr][0] = lds_read16_async(stage + kSk8A + rb0 * 128 + ((cb ^ swz(rb0)) << 4));
        q[pr][1] = lds_read16_async(stage + kSk8A + rb1 * 128 + ((cb ^ swz(rb1)) << 4));
#pragma unroll
        for (int hf = 0; hf < 2; hf++) {
            const int c = 8 * pr + 2 * kq + hf;
#pragma unroll
            for (int ib = 0; ib < 2; ib++) {
                const int row = ib * 16 + r16;
                a[pr][hf][ib] = lds_read16_async(stage + row * 256 + ((c ^ swz16(row)) << 4));
            }
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(q[0][0]), "+v"(q[0][1]), "+v"(q[1][0]), "+v"(q[1][1]), "+v"(a[0][0][0]), "+v"(a[0][0][1]),
                   "+v"(a[0][1][0]), "+v"(a[0][1][1]), "+v"(a[1][0][0]), "+v"(a[1][0][1]), "+v"(a[1][1][0]),
                   "+v"(a[1][1][1])
                 :
                 : "memory");
#pragma unroll
    for (int pr = 0; pr < 2; pr++)
#pragma unroll
        for (int hf = 0; hf < 2; hf++) {
            const u32x4_t w0 = q[pr][0], w1 = q[pr][1];
            const uint4 b0 = fp8x8_widen<kF16, FMT>(hf ? make_uint2(w0.z, w0.w) : make_uint2(w0.x, w0.y));
            const uint4 b1 = fp8x8_widen<kF16, FMT>(hf ? make_uint2(w1.z, w1.w) : make_uint2(w1.x, w1.y));
#pragma unroll
            for (int ib = 0; ib < NB; ib++) {
                const uint4 av = __builtin_bit_cast(uint4, a[pr][hf][ib]);
                acc[ib][0] = mfma16<kF16>(av, b0, acc[ib][0]);
                acc[ib][1] = mfma16<kF16>(av, b1, acc[ib][1]);
            }
        }
}

#define SK8_STEP(I, cur, nxt)                                                            \
    do {                                                                                 \
        if (k0 + (I) >= nk) goto done;                                                   \
        WAIT_VMCNT(6 * (kSk8Stages - 2));                                                \
        block_sync();                                                                    \
        sk8_issue<MODE>(g, nxt, min(k0 + (I) + kSk8Stages - 1, nk - 1));                 \
        sk8_compute<MODE, NB, FMT>(cur, g.wave, lane, acc);                              \
    } while (0)

// The K loop of the bf16 skinny kernel, over three stages of 128 K elements.
template <int MODE, int NB, int FMT>
__device__ __forceinline__ void sk8_main(const Sk8Thread &g, int nk, int lane, char *b0, char *b1, char *b2,
                                         f32x4_t (&acc)[2][2]) {
    sk8_issue<MODE>(g, b0, 0);
    sk8_issue<MODE>(g, b1, min(1, nk - 1));
    for (int k0 = 0;; k0 += kSk8Stages) {
        SK8_STEP(0, b0, b2);
        SK8_STEP(1, b1, b0);
        SK8_STEP(2, b2, b1);
    }
done:
    WAIT_VMCNT(0);
}
#undef SK8_STEP

template <int MODE, int FMT>
__global__ __launch_bounds__(kSkThreads, 2) void grouped_gemm_skinny_fp8(
    const uint16_t *__restrict__ A, const int32_t *__restrict__ a_rows, const uint8_t *__restrict__ B0,
    const uint8_t *__restrict__ B1, const float *__restrict__ S0, const float *__restrict__ S1,
    const int32_t *__restrict__ offsets, int E, int N, int K, int ntiles_n, GemmOut out) {
    __shared__ __attribute__((aligned(1024))) char sb0[kSk8Stage];
    __shared__ __attribute__((aligned(1024))) char sb1[kSk8Stage];
    __shared__ __attribute__((aligned(1024))) char sb2[kSk8Stage];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    TileInfo ti;
    if (!find_tile(offsets, E, ntiles_n, kSkBM, 1, blockIdx.x, nullptr, nullptr, ti)) return;
    const int n0 = ti.nt * (MODE == kGateUp ? kSkBN : kSkBNd);
    const size_t wexp = (size_t)ti.e * N * K;  // bytes: one fp8 per element

    Sk8Thread g;
    g.wave = wave;
    g.a_base = reinterpret_cast<const char *>(a_rows ? A : A + (size_t)ti.m0 * K);
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int row = (2 * wave + j) * 4 + (lane >> 4);
        const int c = (lane & 15) ^ swz16(row);
        const int gm = min(ti.m0 + row, ti.mend - 1);
        const int ar = a_rows ? a_rows[gm] : gm - ti.m0;
        g.a_off[j] = ((uint32_t)ar * K + c * 8) * 2;
    }
    g.b_base[0] = reinterpret_cast<const char *>(B0 + wexp);
    g.b_base[1] = reinterpret_cast<const char *>((MODE == kGateUp ? B1 : B0) + wexp);
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int grp = wave * 4 + j;
        const int row = grp * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(row);
        const int gn = min(n0 + (MODE == kGateUp ? (row & (kSkBN - 1)) : row), N - 1);
        g.b_off[j] = (uint32_t)gn * K + c * 16;
    }
    // the row scales of the lane's output columns, fetched before the K loop
    // (they are the oldest loads, so the loop's first wait covers them)
    const float *s0e = S0 + (size_t)ti.e * N, *s1e = (MODE == kGateUp ? S1 : S0) + (size_t)ti.e * N;
    float sc[2];
#pragma unroll
    for (int jb = 0; jb < 2; jb++) {
        const int col = MODE == kGateUp ? n0 + wave * 16 + (lane & 15) : n0 + wave * 32 + jb * 16 + (lane & 15);
        sc[jb] = (MODE == kGateUp && jb == 1 ? s1e : s0e)[min(col, N - 1)];
    }
    const int nk = K / kSk8K;
    f32x4_t acc[2][2];
#pragma unroll
    for (int ib = 0; ib < 2; ib++)
#pragma unroll
        for (int jb = 0; jb < 2; jb++) acc[ib][jb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int nb = ti.mend - ti.m0 > 16 ? 2 : 1;  // active 16-row blocks (uniform)
    if (nb == 2)
        sk8_main<MODE, 2, FMT>(g, nk, lane, sb0, sb1, sb2, acc);
    else
        sk8_main<MODE, 1, FMT>(g, nk, lane, sb0, sb1, sb2, acc);

    // epilogue: the lane holds column lane % 16, rows 4 * (lane / 16) + q;
    // the weight rows' scales multiply the accumulators first
#pragma unroll
    for (int ib = 0; ib < 2; ib++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int m = ti.m0 + ib * 16 + 4 * (lane >> 4) + q;
            if (m >= ti.mend) continue;
            if (MODE == kGateUp) {
                const int col = n0 + wave * 16 + (lane & 15);
                if (col < N)
                    static_cast<uint16_t *>(out.y0)[(size_t)m * N + col] =
                        f32_to_f16_sat(silu_mul(acc[ib][0][q] * sc[0], acc[ib][1][q] * sc[1]));
            } else if (out.row_gate) {
                const float gt = out.row_gate[m];
#pragma unroll
                for (int jb = 0; jb < 2; jb++) {
                    const int col = n0 + wave * 32 + jb * 16 + (lane & 15);
                    if (col < N)
                        static_cast<uint16_t *>(out.y0)[(size_t)m * N + col] = f32_to_f16_sat(gt * (acc[ib][jb][q] * sc[jb]));
                }
            } else {
#pragma unroll
                for (int jb = 0; jb < 2; jb++) {
                    const int col = n0 + wave * 32 + jb * 16 + (lane & 15);
                    if (col < N) static_cast<float *>(out.y0)[(size_t)m * N + col] = acc[ib][jb][q] * sc[jb];
                }
            }
        }
}

// ------------------------------------------------------ skinny, INT4 W ----
// INT4 expert weights with one fp32 scale per weight row, W[n][k] = s[n] *
// q[n][k], q a two's complement nibble (-8..7), two per byte (element 2j in
// the low nibble of byte j), in the weight-streaming regime (every expert at
// most 32 rows).  The tile is that of the one-byte kernel (32 rows x 128
// weight rows) and a stage again spans 128 K elements: the A part is the
// one-byte kernel's (x or h rows of 256 bytes), the weight rows are 64 bytes.
// Five stages of 16 KiB per block and two blocks per CU keep up to eight
// stages (64 KiB of codes) in flight per CU, as the one-byte kernel does.
// The down projection takes 64 output columns per tile (one weight fragment
// per wave): with 128, a decode layer's down projection has one tile per CU
// and streams at the latency of a single block.
//
// Widening, per 32-bit word of eight codes: the word masked to its high
// nibbles holds the odd elements, and the word shifted up by four and masked
// likewise the even ones, each as a signed byte 16 q; one conversion with a
// sign-extending byte select turns such a byte into fp32, exactly, and two
// of them are packed to bf16 (gate-up) or fp16 (down), both exact for
// |16 q| <= 128.  The factor 16 leaves with the row scale in the epilogue.
constexpr int kSk4BNd = 64;               // output columns per down tile
constexpr int kSk4B = 2 * kSkBN * 64;     // B part: 128 weight rows x 64 bytes (8 KiB; down: 4 KiB used)
constexpr int kSk4Stage = kSk8A + kSk4B;  // 16 KiB
constexpr int kSk4Stages = 5;
// weight fragments per wave (16 columns each): gate-up W1 and W3, down one
template <int MODE>
__device__ __forceinline__ constexpr int sk4_nf() { return MODE == kGateUp ? 2 : 1; }

struct Sk4Thread {
    const char *a_base;
    const char *b_base[2];
    uint32_t a_off[2];  // wave w loads A rows 8w .. 8w+7, four per load
    uint32_t b_off[2];  // wave w loads B rows 16 nf w .. + 16 nf - 1, sixteen per load
    int wave;
};

// eight INT4 codes of one word -> eight values 16 q as bf16 (gate-up) or
// fp16 (down), element i from nibble i
template <bool F16>
__device__ __forceinline__ uint32_t i4x2_widen(uint32_t ev, uint32_t od, int byte) {
    const float a = (float)(int32_t)__builtin_amdgcn_sbfe(ev, 8 * byte, 8),
                b = (float)(int32_t)__builtin_amdgcn_sbfe(od, 8 * byte, 8);
    if constexpr (F16) return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
    else return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

template <bool F16>
__device__ __forceinline__ uint4 i4x8_widen(uint32_t w) {
    const uint32_t ev = (w << 4) & 0xF0F0F0F0u, od = w & 0xF0F0F0F0u;
    return make_uint4(i4x2_widen<F16>(ev, od, 0), i4x2_widen<F16>(ev, od, 1), i4x2_widen<F16>(ev, od, 2),
                      i4x2_widen<F16>(ev, od, 3));
}

template <int MODE>
__device__ __forceinline__ void sk4_issue(const Sk4Thread &g, char *stage, int k) {
    const uint32_t ka = (uint32_t)k * kSk8K * 2, kq = (uint32_t)k * (kSk8K / 2);
    g2lds16(g.a_base + g.a_off[0] + ka, stage + (2 * g.wave) * 1024);
    g2lds16(g.a_base + g.a_off[1] + ka, stage + (2 * g.wave + 1) * 1024);
#pragma unroll
    for (int j = 0; j < sk4_nf<MODE>(); j++) {
        const int grp = g.wave * sk4_nf<MODE>() + j;     // 16-row group of the B part
        const int src = MODE == kGateUp ? grp >> 2 : 0;  // gate-up: groups 4.. are W3
        g2lds16((src ? g.b_base[1] : g.b_base[0]) + g.b_off[j] + kq, stage + kSk8A + grp * 1024);
    }
}

template <int MODE, int NB>
__device__ __forceinline__ void sk4_compute(const char *stage, int wave, int lane, f32x4_t (&acc)[2][2]) {
    constexpr bool kF16 = MODE == kDown;
    const int r16 = lane & 15, kq = lane >> 4;
    constexpr int NF = sk4_nf<MODE>();
    const int rb0 = 16 * wave + r16;          // W1 rows (gate-up) or W2 rows (down)
    const int rb1 = kSkBN + 16 * wave + r16;  // gate-up: the same rows of W3
    // The stage's K elements in an order of their own (both operands follow
    // it): lane quarter kq takes elements 32 kq .. 32 kq + 31, one 16-byte
    // chunk of each weight row (64-byte rows, chunks XOR-swizzled by
    // swz4(row)), eight of them (one word) per sub-step; the x fragments are
    // the same eight elements, chunk 4 kq + ss of the 256-byte row.
    u32x4_t q[2], a[4][2];  // [weight fragment], [sub-step][16-row block]
    q[0] = lds_read16_async(stage + kSk8A + rb0 * 64 + ((kq ^ swz4(rb0)) << 4));
    q[1] = NF == 2 ? lds_read16_async(stage + kSk8A + rb1 * 64 + ((kq ^ swz4(rb1)) << 4)) : q[0];
#pragma unroll
    for (int ss = 0; ss < 4; ss++) {
        const int c = 4 * kq + ss;
#pragma unroll
        for (int ib = 0; ib < 2; ib++) {
            const int row = ib * 16 + r16;
            a[ss][ib] = lds_read16_async(stage + row * 256 + ((c ^ swz16(row)) << 4));
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(q[0]), "+v"(q[1]), "+v"(a[0][0]), "+v"(a[0][1]), "+v"(a[1][0]), "+v"(a[1][1]),
                   "+v"(a[2][0]), "+v"(a[2][1]), "+v"(a[3][0]), "+v"(a[3][1])
                 :
                 : "memory");
#pragma unroll
    for (int ss = 0; ss < 4; ss++) {
        const uint4 b0 = i4x8_widen<kF16>(q[0][ss]);
        const uint4 b1 = NF == 2 ? i4x8_widen<kF16>(q[1][ss]) : b0;
#pragma unroll
        for (int ib = 0; ib < NB; ib++) {
            const uint4 av = __builtin_bit_cast(uint4, a[ss][ib]);
            acc[ib][0] = mfma16<kF16>(av, b0, acc[ib][0]);
            if (NF == 2) acc[ib][1] = mfma16<kF16>(av, b1, acc[ib][1]);
        }
    }
}

#define SK4_STEP(I, cur, nxt)                                                            \
    do {                                                                                 \
        if (k0 + (I) >= nk) goto done;                                                   \
        WAIT_VMCNT((2 + sk4_nf<MODE>()) * (kSk4Stages - 2));                             \
        block_sync();                                                                    \
        sk4_issue<MODE>(g, nxt, min(k0 + (I) + kSk4Stages - 1, nk - 1));                 \
        sk4_compute<MODE, NB>(cur, g.wave, lane, acc);                                   \
    } while (0)

// The K loop over a ring of five stages of 128 K elements: when stage k is
// computed, stages k+1 .. k+3 are in flight and stage k+4 is issued into the
// buffer stage k-1 used (free: every wave passed the barrier after it).
// Loads past the last stage re-read the last K slice.
template <int MODE, int NB>
__device__ __forceinline__ void sk4_main(const Sk4Thread &g, int nk, int lane, char *b0, char *b1, char *b2,
                                         char *b3, char *b4, f32x4_t (&acc)[2][2]) {
    sk4_issue<MODE>(g, b0, 0);
    sk4_issue<MODE>(g, b1, min(1, nk - 1));
    sk4_issue<MODE>(g, b2, min(2, nk - 1));
    sk4_issue<MODE>(g, b3, min(3, nk - 1));
    for (int k0 = 0;; k0 += kSk4Stages) {
        SK4_STEP(0, b0, b4);
        SK4_STEP(1, b1, b0);
        SK4_STEP(2, b2, b1);
        SK4_STEP(3, b3, b2);
        SK4_STEP(4, b4, b3);
    }
done:
    WAIT_VMCNT(0);
}
#undef SK4_STEP

template <int MODE>
__global__ __launch_bounds__(kSkThreads, 2) void grouped_gemm_skinny_i4(
    const uint16_t *__restrict__ A, const int32_t *__restrict__ a_rows, const uint8_t *__restrict__ B0,
    const uint8_t *__restrict__ B1, const float *__restrict__ S0, const float *__restrict__ S1,
    const int32_t *__restrict__ offsets, int E, int N, int K, int ntiles_n, GemmOut out) {
    __shared__ __attribute__((aligned(1024))) char sb0[kSk4Stage];
    __shared__ __attribute__((aligned(1024))) char sb1[kSk4Stage];
    __shared__ __attribute__((aligned(1024))) char sb2[kSk4Stage];
    __shared__ __attribute__((aligned(1024))) char sb3[kSk4Stage];
    __shared__ __attribute__((aligned(1024))) char sb4[kSk4Stage];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    TileInfo ti;
    if (!find_tile(offsets, E, ntiles_n, kSkBM, 1, blockIdx.x, nullptr, nullptr, ti)) return;
    const int n0 = ti.nt * (MODE == kGateUp ? kSkBN : kSk4BNd);
    const size_t wexp = (size_t)ti.e * N * (K / 2);  // bytes: two codes per byte

    Sk4Thread g;
    g.wave = wave;
    g.a_base = reinterpret_cast<const char *>(a_rows ? A : A + (size_t)ti.m0 * K);
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int row = (2 * wave + j) * 4 + (lane >> 4);
        const int c = (lane & 15) ^ swz16(row);
        const int gm = min(ti.m0 + row, ti.mend - 1);
        const int ar = a_rows ? a_rows[gm] : gm - ti.m0;
        g.a_off[j] = ((uint32_t)ar * K + c * 8) * 2;
    }
    g.b_base[0] = reinterpret_cast<const char *>(B0 + wexp);
    g.b_base[1] = reinterpret_cast<const char *>((MODE == kGateUp ? B1 : B0) + wexp);
#pragma unroll
    for (int j = 0; j < sk4_nf<MODE>(); j++) {
        // 16-row group of 64-byte rows; lane l takes row 16 grp + l / 4 and
        // the logical chunk that lands at position l % 4
        const int grp = wave * sk4_nf<MODE>() + j;
        const int row = grp * 16 + (lane >> 2);
        const int c = (lane & 3) ^ swz4(row);
        const int gn = min(n0 + (MODE == kGateUp ? (row & (kSkBN - 1)) : row), N - 1);
        g.b_off[j] = (uint32_t)gn * (K / 2) + c * 16;
    }
    // the row scales of the lane's output columns (divided by the 16 of the
    // widening), fetched before the K loop
    const float *s0e = S0 + (size_t)ti.e * N, *s1e = (MODE == kGateUp ? S1 : S0) + (size_t)ti.e * N;
    float sc[2];
#pragma unroll
    for (int jb = 0; jb < 2; jb++) {
        const int col = n0 + wave * 16 + (lane & 15);
        sc[jb] = (MODE == kGateUp && jb == 1 ? s1e : s0e)[min(col, N - 1)] * 0.0625f;
    }
    const int nk = K / kSk8K;
    f32x4_t acc[2][2];
#pragma unroll
    for (int ib = 0; ib < 2; ib++)
#pragma unroll
        for (int jb = 0; jb < 2; jb++) acc[ib][jb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int nb = ti.mend - ti.m0 > 16 ? 2 : 1;  // active 16-row blocks (uniform)
    if (nb == 2)
        sk4_main<MODE, 2>(g, nk, lane, sb0, sb1, sb2, sb3, sb4, acc);
    else
        sk4_main<MODE, 1>(g, nk, lane, sb0, sb1, sb2, sb3, sb4, acc);

    // epilogue: the lane holds column lane % 16, rows 4 * (lane / 16) + q
#pragma unroll
    for (int ib = 0; ib < 2; ib++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int m = ti.m0 + ib * 16 + 4 * (lane >> 4) + q;
            if (m >= ti.mend) continue;
            if (MODE == kGateUp) {
                const int col = n0 + wave * 16 + (lane & 15);
                if (col < N)
                    static_cast<uint16_t *>(out.y0)[(size_t)m * N + col] =
                        f32_to_f16_sat(silu_mul(acc[ib][0][q] * sc[0], acc[ib][1][q] * sc[1]));
            } else {
                const int col = n0 + wave * 16 + (lane & 15);
                if (col >= N) continue;
                if (out.row_gate)
                    static_cast<uint16_t *>(out.y0)[(size_t)m * N + col] =
                        f32_to_f16_sat(out.row_gate[m] * (acc[ib][0][q] * sc[0]));
                else
                    static_cast<float *>(out.y0)[(size_t)m * N + col] = acc[ib][0][q] * sc[0];
            }
        }
}

// ---------------------------------------------------------------- fp32 ----
constexpr int kF32BM = 64, kF32BN = 64, kF32BK = 16;

template <int MODE>
__global__ __launch_bounds__(256) void grouped_gemm_f32(const float *__restrict__ A,
                                                        const int32_t *__restrict__ a_rows,
                                                        const float *__restrict__ B0,
                                                        const float *__restrict__ B1,
                                                        const int32_t *__restrict__ offsets, int E,
                                                        int N, int K, int ntiles_n,
                                                        float *__restrict__ out) {
    __shared__ float sa[kF32BK][kF32BM + 1];
    __shared__ float sb0[kF32BK][kF32BN + 1];
    __shared__ float sb1[kF32BK][kF32BN + 1];
    TileInfo ti;
    if (!find_tile(offsets, E, ntiles_n, kF32BM, 1, blockIdx.x, nullptr, nullptr, ti)) return;
    const int n0 = ti.nt * kF32BN;
    const size_t wexp = (size_t)ti.e * N * K;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;  // 4x4 outputs each
    float c0[4][4] = {}, c1[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += kF32BK) {
        for (int i = threadIdx.x; i < kF32BM * kF32BK; i += 256) {
            const int r = i / kF32BK, kk = i % kF32BK;
            int gm = ti.m0 + r;
            if (gm >= ti.mend) gm = ti.mend - 1;
            const size_t ar = a_rows ? (size_t)a_rows[gm] : (size_t)gm;
            sa[kk][r] = A[ar * K + k0 + kk];
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

}  // namespace

// Bound on sum_e ceil(rows_e / bm), the m tiles of all experts: every
// expert holds at most cap rows, and all of them at most max_rows.  The grid
// is sized by it, so a tight bound leaves few blocks without work.
static int64_t mtile_bound(int64_t max_rows, int64_t cap, int E, int bm) {
    return std::min<int64_t>(max_rows / bm + E, (int64_t)E * ((cap + bm - 1) / bm));
}

// Slices of a K reduction of `steps` K steps over (at most) `tiles` output
// tiles, among the doublings of s_min that allowed(s) accepts (at most 8):
// the count with the least cost in K steps per compute unit.  The work items
// (tiles x S) run in rounds of one per CU; an item costs its K / S steps plus
// about six steps of prologue and epilogue; fewer items than CUs leave CUs
// idle, which costs in proportion.  (Mixtral-shape down projection: 2 slices,
// 1031 us against 1134-1151 with 1 and 1042-1046 with 4; 16 experts of about
// 250 rows and K = 5632: 2 slices, 113 us against 138 with 4 and 161 with 1.)
template <typename Allowed>
static int pick_splits(int64_t tiles, int64_t steps, int s_min, Allowed allowed) {
    constexpr int64_t kCUs = 256;
    int best = s_min;
    double best_cost = -1.0;
    for (int s = s_min; s <= 8 && (s == s_min || allowed(s)); s *= 2) {
        const int64_t items = std::max<int64_t>(tiles * s, 1);
        double cost = (double)ceil_div(items, kCUs) * ((double)steps / s + 6.0);
        if (items < kCUs) cost *= (double)kCUs / (double)items;
        if (best_cost < 0.0 || cost < best_cost) best = s, best_cost = cost;
    }
    return best;
}

int ffn_splits(const moe_params &p, int64_t max_rows) {
    if (p.dtype != MOE_BF16 || max_rows <= 0) return 1;
    // small groups run the weight-streaming kernel, whose down projection is
    // one slice (a CU per 128 output columns of an expert already fills the
    // chip, and longer tiles stream better)
    const int64_t cap = capacity_rows(p);
    if (cap <= kSkBM) return 1;
    const int64_t tiles = mtile_bound(max_rows, cap, p.E, kBM) * ceil_div(p.d, kBN);
    const int64_t steps = p.d_ff / kBK;
    return pick_splits(tiles, steps, 1, [steps](int s) { return steps % (4 * s) == 0; });
}

// moe_forward's down projection on the 256-row GEMM: the split plan for
// the bound on the m tiles.  No split there (the tiles fill whole rounds):
// one slice; every tile split: that many uniform slices (when they divide
// the K steps); only a partial split runs the planned kernel, which
// re-plans for the actual m tiles on the device.  (The uniform kernel is
// the leaner one: its epilogue keeps one register fewer through the K loop.)
DownSplit forward_down_split(const moe_params &p, int64_t max_rows) {
    if (p.dtype != MOE_BF16 || max_rows <= 0 || capacity_rows(p) <= kSkBM) return DownSplit{false, 1};
    const int64_t mt = mtile_bound(max_rows, capacity_rows(p), p.E, kBM);
    const int ntn = (int)ceil_div(p.d, kBN), nk = p.d_ff / kBK;
    int G, S;
    split_plan((int)mt, ntn, nk, G, S);
    if (G == 0) return DownSplit{false, 1};
    if (G == mt && nk % S == 0) return DownSplit{false, S};
    return DownSplit{true, 1};
}

bool q4_ffn_supported(const moe_params &p) {
    // the weight-streaming kernel only (at most 32 rows per expert), which
    // steps K by 128
    return p.dtype == MOE_BF16 && capacity_rows(p) <= kSkBM && p.d % kSk8K == 0 && p.d_ff % kSk8K == 0;
}

bool fp8_ffn_supported(const moe_params &p) {
    // the weight-streaming kernel (at most 32 rows per expert) steps K by 128
    return p.dtype == MOE_BF16 && (capacity_rows(p) > kSkBM || (p.d % kSk8K == 0 && p.d_ff % kSk8K == 0));
}

namespace {

// y[r] += rest[0][r] + rest[1][r] + ... (slice order) for the rows below
// offsets[E]: the split down projection's partial products reduced into
// slice 0, deterministically.
__global__ __launch_bounds__(256) void ffn_fixup(float *__restrict__ y, const float *__restrict__ rest, int nrest,
                                                 size_t stride, const int32_t *__restrict__ offsets, int E, int d) {
    const size_t n = (size_t)offsets[E] * (d / 4);
    float4 *y4 = reinterpret_cast<float4 *>(y);
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
        float4 a = y4[i];
        for (int sl = 0; sl < nrest; sl++) {
            const float4 b = reinterpret_cast<const float4 *>(rest + (size_t)sl * stride)[i];
            a.x += b.x;
            a.y += b.y;
            a.z += b.z;
            a.w += b.w;
        }
        y4[i] = a;
    }
}

}  // namespace

template <int FMT>
static void launch_q8(const moe_params &p, int64_t mt, const void *x_perm, const int32_t *a_rows,
                      const int32_t *offsets, const uint8_t *w1, const float *s1, const uint8_t *w3, const float *s3,
                      const uint8_t *w2, const float *s2, void *h, const GemmOut &down, hipEvent_t mid,
                      hipError_t &ev, hipStream_t st) {
    const int E = p.E, d = p.d, dff = p.d_ff;
    const int nt_up = (int)ceil_div(dff, kSkBN);
    const int nt_dn = (int)ceil_div(d, kSkBNd);
    hipLaunchKernelGGL((grouped_gemm_skinny_fp8<kGateUp, FMT>), dim3((unsigned)(mt * nt_up)), dim3(kSkThreads), 0,
                       st, static_cast<const uint16_t *>(x_perm), a_rows, w1, w3, s1, s3, offsets, E, dff, d, nt_up,
                       GemmOut{h, nullptr, 0, nullptr});
    if (mid) ev = hipEventRecord(mid, st);
    hipLaunchKernelGGL((grouped_gemm_skinny_fp8<kDown, FMT>), dim3((unsigned)(mt * nt_dn)), dim3(kSkThreads), 0, st,
                       static_cast<const uint16_t *>(h), (const int32_t *)nullptr, w2, w2, s2, s2, offsets, E, d,
                       dff, nt_dn, down);
}

static void launch_q4(const moe_params &p, int64_t mt, const void *x_perm, const int32_t *a_rows,
                      const int32_t *offsets, const uint8_t *w1, const float *s1, const uint8_t *w3, const float *s3,
                      const uint8_t *w2, const float *s2, void *h, const GemmOut &down, hipEvent_t mid,
                      hipError_t &ev, hipStream_t st) {
    const int E = p.E, d = p.d, dff = p.d_ff;
    const int nt_up = (int)ceil_div(dff, kSkBN);
    const int nt_dn = (int)ceil_div(d, kSk4BNd);
    hipLaunchKernelGGL(grouped_gemm_skinny_i4<kGateUp>, dim3((unsigned)(mt * nt_up)), dim3(kSkThreads), 0, st,
                       static_cast<const uint16_t *>(x_perm), a_rows, w1, w3, s1, s3, offsets, E, dff, d, nt_up,
                       GemmOut{h, nullptr, 0, nullptr});
    if (mid) ev = hipEventRecord(mid, st);
    hipLaunchKernelGGL(grouped_gemm_skinny_i4<kDown>, dim3((unsigned)(mt * nt_dn)), dim3(kSkThreads), 0, st,
                       static_cast<const uint16_t *>(h), (const int32_t *)nullptr, w2, w2, s2, s2, offsets, E, d,
                       dff, nt_dn, down);
}

// Grid of a planned down projection over at most `tiles` tiles: the plan
// never exceeds whole rounds of kPlanCUs items (with M tiles = 256 k + r,
// 0 < r < 256: at most 256 k bulk items and 256 split items), so blocks
// beyond that would only find no work, after the claim attempts on every
// XCD's counter, at the end of the launch.  Without claim counters each XCD
// takes its own share (rounded up per XCD: 16 more).
static int64_t planned_grid(int64_t tiles, const int32_t *claim) {
    return ceil_div(tiles, (int64_t)kPlanCUs) * kPlanCUs + (claim ? 0 : 16);
}

// One-byte weights on the 256 x 256 MFMA tile (groups of more than 32 rows).
template <int GU, int DN>
static void launch_q8_mfma(const moe_params &p, int64_t mt, const void *x_perm, const int32_t *a_rows,
                           int64_t a_bytes, const int32_t *offsets, const uint8_t *w1, const float *s1,
                           const uint8_t *w3, const float *s3, const uint8_t *w2, const float *s2, void *h,
                           const GemmOut &down, int splits, int32_t *claim, hipEvent_t mid, hipError_t &ev,
                           hipStream_t st) {
    const int E = p.E, d = p.d, dff = p.d_ff;
    const int nt_up = (int)ceil_div(dff, kBN / 2);
    const int nt_dn = (int)ceil_div(d, kBN);
    hipLaunchKernelGGL(grouped_gemm_bf16<GU>, dim3((unsigned)(mt * nt_up)), dim3(kGemmThreads), 0, st,
                       static_cast<const uint16_t *>(x_perm), a_rows, reinterpret_cast<const uint16_t *>(w1),
                       reinterpret_cast<const uint16_t *>(w3), offsets, E, dff, d, d, nt_up, 1, (uint32_t)a_bytes,
                       claim, GemmOut{h, nullptr, 0, nullptr}, s1, s3);
    if (mid) ev = hipEventRecord(mid, st);
    const int64_t dn_items = down.plan ? planned_grid(mt * nt_dn, claim) : mt * nt_dn * splits;
    auto *dn = down.plan ? grouped_gemm_bf16<DN, true> : grouped_gemm_bf16<DN, false>;
    hipLaunchKernelGGL(dn, dim3((unsigned)dn_items), dim3(kGemmThreads), 0, st,
                       static_cast<const uint16_t *>(h), (const int32_t *)nullptr,
                       reinterpret_cast<const uint16_t *>(w2), reinterpret_cast<const uint16_t *>(w2), offsets, E,
                       d, dff, dff, nt_dn, splits, (uint32_t)0, claim ? claim + 8 : nullptr, down, s2, s2);
}

hipError_t launch_expert_ffn_fp8(const moe_params &p, int64_t max_rows, int64_t cap, const void *x_perm,
                                 const int32_t *a_rows, const int32_t *offsets, const uint8_t *w1, const float *s1,
                                 const uint8_t *w3, const float *s3, const uint8_t *w2, const float *s2, void *h,
                                 const GemmOut &down, int splits, int32_t *claim, hipEvent_t mid, int qfmt,
                                 hipStream_t st) {
    if (max_rows <= 0) return hipSuccess;
    if (qfmt == MOE_Q_INT4 ? !q4_ffn_supported(p) : !fp8_ffn_supported(p)) return hipErrorInvalidValue;
    hipError_t ev = hipSuccess;
    if (qfmt == MOE_Q_INT4) {
        const int64_t mt = mtile_bound(max_rows, cap, p.E, kSkBM);
        launch_q4(p, mt, x_perm, a_rows, offsets, w1, s1, w3, s3, w2, s2, h, down, mid, ev, st);
    } else if (cap <= kSkBM) {
        const int64_t mt = mtile_bound(max_rows, cap, p.E, kSkBM);
        if (qfmt == MOE_Q_INT8)
            launch_q8<kQInt8>(p, mt, x_perm, a_rows, offsets, w1, s1, w3, s3, w2, s2, h, down, mid, ev, st);
        else
            launch_q8<kQE4M3>(p, mt, x_perm, a_rows, offsets, w1, s1, w3, s3, w2, s2, h, down, mid, ev, st);
    } else {
        // gathered A rows are read from x through a buffer extent below 2 GiB
        const int64_t a_bytes = a_rows ? (int64_t)p.T * p.d * 2 : 0;
        if (a_bytes >= ((int64_t)1 << 31) || splits < 1 || (p.d_ff / kBK) % splits != 0) return hipErrorInvalidValue;
        const int64_t mt = mtile_bound(max_rows, cap, p.E, kBM);
        if (qfmt == MOE_Q_INT8)
            launch_q8_mfma<kGateUpI8, kDownI8>(p, mt, x_perm, a_rows, a_bytes, offsets, w1, s1, w3, s3, w2, s2, h,
                                               down, splits, claim, mid, ev, st);
        else
            launch_q8_mfma<kGateUpE4M3, kDownE4M3>(p, mt, x_perm, a_rows, a_bytes, offsets, w1, s1, w3, s3, w2, s2,
                                                   h, down, splits, claim, mid, ev, st);
    }
    if (ev != hipSuccess) return ev;
    return hipGetLastError();
}

hipError_t launch_expert_ffn(const moe_params &p, int64_t max_rows, int64_t cap, const void *x_perm,
                             const int32_t *a_rows, const int32_t *offsets, const void *w1,
                             const void *w3, const void *w2, void *h, const GemmOut &down, int32_t *claim,
                             hipEvent_t mid, hipStream_t st, int splits) {
    if (max_rows <= 0) return hipSuccess;
    const int E = p.E, d = p.d, dff = p.d_ff;
    const GemmOut up{h, nullptr, 0, nullptr};
    if (p.dtype == MOE_BF16 && cap <= kSkBM) {
        // every expert holds at most 32 rows: the weight-streaming kernel
        const int64_t mt = mtile_bound(max_rows, cap, E, kSkBM);
        const int nt_up = (int)ceil_div(dff, kSkBN);
        const int nt_dn = (int)ceil_div(d, kSkBNd);
        const int S = splits;
        hipLaunchKernelGGL(grouped_gemm_skinny<kGateUp>, dim3((unsigned)(mt * nt_up)), dim3(kSkThreads), 0, st,
                           static_cast<const uint16_t *>(x_perm), a_rows, static_cast<const uint16_t *>(w1),
                           static_cast<const uint16_t *>(w3), offsets, E, dff, d, nt_up, 1, up);
        if (mid && hipEventRecord(mid, st) != hipSuccess) return hipErrorLaunchFailure;
        hipLaunchKernelGGL(grouped_gemm_skinny<kDown>, dim3((unsigned)(mt * nt_dn * S)), dim3(kSkThreads), 0, st,
                           static_cast<const uint16_t *>(h), (const int32_t *)nullptr,
                           static_cast<const uint16_t *>(w2), static_cast<const uint16_t *>(w2), offsets, E, d,
                           dff, nt_dn, S, down);
        return hipGetLastError();
    }
    if (p.dtype == MOE_BF16) {
        // gathered A rows are read from x through a buffer extent below 2 GiB
        const int64_t a_bytes = a_rows ? (int64_t)p.T * d * 2 : 0;
        if (a_bytes >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
        const int64_t mt = mtile_bound(max_rows, cap, E, kBM);
        const int nt_up = (int)ceil_div(dff, kBN / 2);
        const int nt_dn = (int)ceil_div(d, kBN);
        // the split plan (down.plan) is chosen on the device: at most one
        // extra round of items; the claim counters hand them out
        const int S = down.plan ? 1 : splits;
        if (S < 1 || (dff / kBK) % S != 0) return hipErrorInvalidValue;
        const int64_t dn_items = down.plan ? planned_grid(mt * nt_dn, claim) : mt * nt_dn * S;
        auto *dn = down.plan ? grouped_gemm_bf16<kDown, true> : grouped_gemm_bf16<kDown, false>;
        hipLaunchKernelGGL(grouped_gemm_bf16<kGateUp>, dim3((unsigned)(mt * nt_up)), dim3(kGemmThreads),
                           0, st, static_cast<const uint16_t *>(x_perm), a_rows,
                           static_cast<const uint16_t *>(w1), static_cast<const uint16_t *>(w3),
                           offsets, E, dff, d, d, nt_up, 1, (uint32_t)a_bytes, claim, up);
        if (mid && hipEventRecord(mid, st) != hipSuccess) return hipErrorLaunchFailure;
        hipLaunchKernelGGL(dn, dim3((unsigned)dn_items), dim3(kGemmThreads),
                           0, st, static_cast<const uint16_t *>(h), (const int32_t *)nullptr,
                           static_cast<const uint16_t *>(w2), static_cast<const uint16_t *>(w2),
                           offsets, E, d, dff, dff, nt_dn, S, (uint32_t)0,
                           claim ? claim + 8 : nullptr, down, (const float *)nullptr, (const float *)nullptr);
    } else {
        const int64_t mt = max_rows / kF32BM + E;
        const int nt_up = (int)ceil_div(dff, kF32BN);
        const int nt_dn = (int)ceil_div(d, kF32BN);
        hipLaunchKernelGGL(grouped_gemm_f32<kGateUp>, dim3((unsigned)(mt * nt_up)), dim3(256), 0, st,
                           static_cast<const float *>(x_perm), a_rows, static_cast<const float *>(w1),
                           static_cast<const float *>(w3), offsets, E, dff, d, nt_up,
                           static_cast<float *>(h));
        if (mid && hipEventRecord(mid, st) != hipSuccess) return hipErrorLaunchFailure;
        hipLaunchKernelGGL(grouped_gemm_f32<kDown>, dim3((unsigned)(mt * nt_dn)), dim3(256), 0, st,
                           static_cast<const float *>(h), (const int32_t *)nullptr, static_cast<const float *>(w2),
                           static_cast<const float *>(w2), offsets, E, d, dff, nt_dn,
                           static_cast<float *>(down.y0));
    }
    return hipGetLastError();
}

hipError_t launch_gate_up_raw(const moe_params &p, int64_t max_rows, int64_t cap, const void *x,
                              const int32_t *a_rows, const int32_t *offsets, const void *w1, const void *w3,
                              float *a, float *b, hipStream_t st) {
    if (max_rows <= 0) return hipSuccess;
    const int64_t a_bytes = a_rows ? (int64_t)p.T * p.d * 2 : 0;
    if (p.dtype != MOE_BF16 || a_bytes >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const int64_t mt = mtile_bound(max_rows, cap, p.E, kBM);
    const int nt_up = (int)ceil_div(p.d_ff, kBN / 2);
    hipLaunchKernelGGL(grouped_gemm_bf16<kGateUpRaw>, dim3((unsigned)(mt * nt_up)), dim3(kGemmThreads), 0, st,
                       static_cast<const uint16_t *>(x), a_rows, static_cast<const uint16_t *>(w1),
                       static_cast<const uint16_t *>(w3), offsets, p.E, p.d_ff, p.d, p.d, nt_up, 1,
                       (uint32_t)a_bytes, (int32_t *)nullptr, GemmOut{a, b, 0, nullptr});
    return hipGetLastError();
}

int plain_gemm_splits(int64_t max_rows, int E, int N, int K, int ldb) {
    const int64_t tiles = (max_rows / kBM + E) * ceil_div(N, kBN);
    int s = 1;
    while (K / s > ldb) s *= 2;  // each slice's K range lies within one period of B
    while (s < 8 && tiles * s < 3 * 256 && (K / (2 * s)) % kBK == 0) s *= 2;
    return s;
}

hipError_t launch_plain_gemm(int64_t max_rows, int64_t cap, int E, const uint16_t *A, const int32_t *a_rows,
                             int64_t a_span_bytes, const int32_t *offsets, const uint16_t *B, const uint16_t *B1,
                             bool b_n_contig, int N, int K, int ldb, int S, float *C, float *rest, hipStream_t st,
                             bool a_f16, bool fixup) {
    if (max_rows <= 0) return hipSuccess;
    if (S < 1 || K % S != 0 || (K / S) % kBK != 0 || ldb % (K / S) != 0 || N % 64 != 0 ||
        a_span_bytes >= ((int64_t)1 << 31) || (int64_t)N * ldb * 2 >= ((int64_t)1 << 32))
        return hipErrorInvalidValue;
    const int64_t mt = mtile_bound(max_rows, cap, E, kBM);
    const int nt = (int)ceil_div(N, kBN);
    if (b_n_contig) {
        auto *kern = a_f16 ? grouped_gemm_bf16<kPlainBTH, false> : grouped_gemm_bf16<kPlainBT, false>;
        hipLaunchKernelGGL(kern, dim3((unsigned)(mt * nt * S)), dim3(kGemmThreads), 0, st, A, a_rows, B,
                           B1 ? B1 : B, offsets, E, N, K, ldb, nt, S, (uint32_t)a_span_bytes, (int32_t *)nullptr,
                           GemmOut{C, rest, (size_t)max_rows * N, nullptr}, (const float *)nullptr,
                           (const float *)nullptr);
    } else
        hipLaunchKernelGGL(grouped_gemm_bf16<kPlain>, dim3((unsigned)(mt * nt * S)), dim3(kGemmThreads), 0, st, A,
                           a_rows, B, B, offsets, E, N, K, ldb, nt, S, (uint32_t)a_span_bytes, (int32_t *)nullptr,
                           GemmOut{C, rest, (size_t)max_rows * N, nullptr});
    if (S > 1 && fixup) {
        const int64_t n4 = max_rows * (N / 4);
        const int grid = (int)std::min<int64_t>(ceil_div(n4, 256), 4096);
        hipLaunchKernelGGL(ffn_fixup, dim3(grid), dim3(256), 0, st, C, rest, S - 1, (size_t)max_rows * N, offsets,
                           E, N);
    }
    return hipGetLastError();
}

hipError_t launch_wgrad_gemm(int E, const uint16_t *A, const uint16_t *B, const int32_t *offsets,
                             const int32_t *unit_offsets, int M, int N, int ldk, float *C, hipStream_t st,
                             const uint32_t *amax, const uint32_t *gmax) {
    if (E <= 0 || M <= 0 || N <= 0) return hipSuccess;
    if (N % 64 != 0 || (int64_t)kBM * ldk * 2 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const int mt = (int)ceil_div(M, kBM), nt = (int)ceil_div(N, kBN);
    auto *kern = amax ? grouped_gemm_wgrad<true> : grouped_gemm_wgrad<false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)((int64_t)E * mt * nt)), dim3(kGemmThreads), 0, st, A, B, offsets,
                       unit_offsets, E, M, N, ldk, nt, C, amax, gmax);
    return hipGetLastError();
}

hipError_t launch_ffn_fixup(const moe_params &p, int64_t max_rows, const int32_t *offsets, float *y_perm,
                            const float *rest, int nrest, hipStream_t st) {
    if (max_rows <= 0 || nrest <= 0) return hipSuccess;
    const int64_t n4 = max_rows * (p.d / 4);
    const int grid = (int)std::min<int64_t>(ceil_div(n4, 256), 4096);
    hipLaunchKernelGGL(ffn_fixup, dim3(grid), dim3(256), 0, st, y_perm, rest, nrest, (size_t)max_rows * p.d,
                       offsets, p.E, p.d);
    return hipGetLastError();
}

}  // namespace moe
