// Device building blocks of libfsa's HIP kernels for gfx950 (MI355X), Fibonacci-offset
// sparse attention: element types and row fragments, MFMA blocks, LDS tiles, buffer
// loads, the slab layout, the rotary helpers and the launch helpers. Each kernel
// source (fsa_forward.hip, fsa_backward.hip, fsa_decode.hip, fsa_rope.hip) includes it.
//
//
// Operation (explainer page "Depth-Staggered Fibonacci Spacing for Sparse
// Attention: Static Schedules Beat Learned Dilation and Extrapolate Where Dense
// Attention Fails", gist.science, section "Metodologia / Arquitetura e Mecanismo
// de Atenção"): query row i attends the dense window {i-w+1 .. i} plus the keys
// i - o for each sparse offset o of the layer's table T (all o >= w), one
// softmax over the union. Static schedules run as a single boolean mask
// (section "Principais Contribuições e Resultados", item 2).
//
// Work decomposition of the bf16 window kernels (w <= 64; one workgroup = 4 wave64 =
// one 64-row tile of one head):
//  * Window band: a banded dense block on MFMA. Its K/V (or Q/dO) rows are copied
//    into LDS by direct global -> LDS loads in a chunk-swizzled row-major tile.
//    Scores are formed transposed, S^T = K Q^T, so each lane's four accumulator
//    rows are four keys of one query: the B-operand layout of the P.V product,
//    whose A operand (V^T) comes from transposing LDS reads.
//  * Sparse offsets: each offset o maps the tile's 64 query rows onto one
//    contiguous 64-row slab. Slab rows stream through a register ring in a layout
//    of their own (eight lanes per 128-byte row, so every load covers whole cache
//    lines); the per-row dot products and weighted sums run on the packed bf16 dot
//    unit with DPP row reductions.
//  * Forward: the band's softmax state moves into the slab layout and the slabs
//    continue it online.
//  * Backward: the dQ work of a tile forms dQ of its query rows (and D), storing
//    the bf16 P and dS of every sparse pair; the dK/dV work forms dK, dV of its key
//    rows from the band (recomputed) and those stored weights. Both run in one
//    launch whose dK/dV tiles wait for per-tile tokens of the dQ tiles they read
//    (two kernels when B * H is not a multiple of 8). Every output row has one
//    writer and no atomics are used.
//  * Workgroup ids are remapped so that the tiles of one head run on one XCD in
//    increasing row order, keeping that head's rows in the XCD's L2 for the
//    slab re-reads.
// The general kernels (fp32 inputs, wider windows, other scales) loop over 64-key
// chunks with an online softmax; the dense causal baseline has a kernel of its own.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "fsa_internal.h"
namespace fsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;
constexpr int kT64 = 64 + 4;    // padded LDS row (elements) of a transposed 64-row tile

// ----------------------------------------------------------------------------
// element types and row fragments
// ----------------------------------------------------------------------------

template <bool BF16>
struct Elem;
template <>
struct Elem<true> {
    using T = uint16_t;  // bf16 bits
};
template <>
struct Elem<false> {
    using T = float;
};

// The 16 elements of one 64-wide row that lane group g (lanes 16g..16g+15) owns:
// d = 32 h + 8 g + e for h in 0..1, e in 0..7, i.e. two 16-byte chunks in bf16.
// Output accumulators use the same ownership: acc[2h + b][r] holds d = 32h + 8g + 4b + r.
template <bool BF16>
struct Frag;
template <>
struct Frag<true> {
    u32x4_t c[2];  // c[h] word w = elements e = 2w (low half), 2w + 1 (high half)
};
template <>
struct Frag<false> {
    f32x4_t c[4];  // c[2h + e / 4][e % 4]
};

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// Round-to-nearest-even fp32 -> bf16 of two values, packed (first in the low half).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const f32x2_t f = {a, b};
    const bf16x2_t h = __builtin_convertvector(f, bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}

// Reinterprets a 32-bit word as two bf16. The word is taken by value on purpose:
// hipcc (clang 22, ROCm 7.2) miscompiles __builtin_bit_cast applied directly to an
// element of an ext_vector_type value, reading element 0 whatever the index.
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) {
    bf16x2_t v;
    __builtin_memcpy(&v, &w, sizeof v);
    return v;
}

// Loads row `row` of a [*, 64] matrix into lane group g's fragment.
__device__ __forceinline__ void load_frag(Frag<true> &f, const uint16_t *base, int64_t row, int g) {
    const uint16_t *p = base + row * 64 + 8 * g;
    f.c[0] = *reinterpret_cast<const u32x4_t *>(p);
    f.c[1] = *reinterpret_cast<const u32x4_t *>(p + 32);
}
__device__ __forceinline__ void load_frag(Frag<false> &f, const float *base, int64_t row, int g) {
    const float *p = base + row * 64 + 8 * g;
#pragma unroll
    for (int c = 0; c < 4; ++c) f.c[c] = *reinterpret_cast<const f32x4_t *>(p + 32 * (c >> 1) + 4 * (c & 1));
}

// Stores this lane's 16 accumulator values of row `row`, times `mul`, in the element type.
__device__ __forceinline__ void store_row(uint16_t *base, int64_t row, int g, const f32x4_t acc[4], float mul) {
    uint16_t *p = base + row * 64 + 8 * g;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const f32x4_t a = acc[2 * h] * mul, b = acc[2 * h + 1] * mul;
        const u32x4_t x = {pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]), pack_bf16(b[0], b[1]), pack_bf16(b[2], b[3])};
        *reinterpret_cast<u32x4_t *>(p + 32 * h) = x;
    }
}
__device__ __forceinline__ void store_row(float *base, int64_t row, int g, const f32x4_t acc[4], float mul) {
    float *p = base + row * 64 + 8 * g;
#pragma unroll
    for (int c = 0; c < 4; ++c) *reinterpret_cast<f32x4_t *>(p + 32 * (c >> 1) + 4 * (c & 1)) = acc[c] * mul;
}

// Partial dot product of two fragments (this lane's 16 of the 64 terms).
__device__ __forceinline__ float frag_dot(const Frag<true> &a, const Frag<true> &b) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int w = 0; w < 4; w += 2) {
            s0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.c[h][w]), as_bf16x2(b.c[h][w]), s0, false);
            s1 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.c[h][w + 1]), as_bf16x2(b.c[h][w + 1]), s1, false);
        }
    return s0 + s1;
}
__device__ __forceinline__ float frag_dot(const Frag<false> &a, const Frag<false> &b) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        s0 = fmaf(a.c[c][0], b.c[c][0], s0);
        s1 = fmaf(a.c[c][1], b.c[c][1], s1);
        s0 = fmaf(a.c[c][2], b.c[c][2], s0);
        s1 = fmaf(a.c[c][3], b.c[c][3], s1);
    }
    return s0 + s1;
}

// acc += x * f. For bf16 rows the product runs on the packed bf16 dot unit with x
// rounded to bf16 (the same rounding the MFMA path applies to probabilities):
// dot2({f_lo, f_hi}, {x, 0}) = x f_lo and dot2({f_lo, f_hi}, {0, x}) = x f_hi.
__device__ __forceinline__ void frag_axpy(f32x4_t acc[4], float x, const Frag<true> &f) {
    const bf16x2_t xl = as_bf16x2(pack_bf16(x, 0.f));
    const bf16x2_t xh = as_bf16x2(pack_bf16(0.f, x));
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const bf16x2_t v = as_bf16x2(f.c[h][w]);
            f32x4_t &a = acc[2 * h + (w >> 1)];
            const int r = 2 * (w & 1);
            a[r] = __builtin_amdgcn_fdot2_f32_bf16(v, xl, a[r], false);
            a[r + 1] = __builtin_amdgcn_fdot2_f32_bf16(v, xh, a[r + 1], false);
        }
}
__device__ __forceinline__ void frag_axpy(f32x4_t acc[4], float x, const Frag<false> &f) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] += x * f.c[c];
}

// Sum / max over the four lane groups (lanes l, l^16, l^32, l^48) with the gfx950
// row-swap permutes: permlane16_swap(x, x) yields x of lane l and of lane l^16,
// permlane32_swap(x, x) x of lane l and of lane l^32 (both VALU, no LDS trip).
__device__ __forceinline__ float swap_add16(float x) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float swap_add32(float x) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float swap_max16(float x) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float swap_max32(float x) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float group_sum(float x) { return swap_add32(swap_add16(x)); }
__device__ __forceinline__ float group_max(float x) { return swap_max32(swap_max16(x)); }

// 2^x on the hardware exponential unit; results below the normal range flush to
// zero, which only affects probabilities under 2^-126.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ----------------------------------------------------------------------------
// MFMA building blocks (16x16 output tiles; C layout: lane (col = l%16, g = l/16),
// register r holds row 4 g + r)
// ----------------------------------------------------------------------------

// acc[row][col] += sum_d A_row[d] * B_col[d]: lane (l%16, g) supplies the fragment
// of A row l%16 and of B row (= output column) l%16. Both operands present their
// 64 terms in the same fragment order, so the contraction covers every d once.
__device__ __forceinline__ f32x4_t mma_over_d(const Frag<true> &a, const Frag<true> &b, f32x4_t acc) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.c[h]),
                                                      __builtin_bit_cast(bf16x8_t, b.c[h]), acc, 0, 0, 0);
    return acc;
}
__device__ __forceinline__ f32x4_t mma_over_d(const Frag<false> &a, const Frag<false> &b, f32x4_t acc) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.c[c][r], b.c[c][r], acc, 0, 0, 0);
    return acc;
}

// Row of a transposed tile that feeds MFMA row m of output block db, chosen so
// that output register r of lane group g lands on d = 32 (db/2) + 8 g + 4 (db%2) + r.
__device__ __forceinline__ int acc_row_d(int db, int m) { return 32 * (db >> 1) + 8 * (m >> 2) + 4 * (db & 1) + (m & 3); }

// acc[db] += sum_{kk<16} At[d][kk0 + kk] * Bv[kk][col] for the four output blocks db.
// At is a transposed tile in LDS ([d][row], row stride `stride`); Bv is given in the
// C layout of an earlier product: lane (col, g) register r holds kk = 4 g + r.
__device__ __forceinline__ void mma_over_rows(f32x4_t acc[4], const uint16_t *At, int stride, int kk0, int c16,
                                              int g, const float bv[4]) {
    const u32x2_t b = {pack_bf16(bv[0], bv[1]), pack_bf16(bv[2], bv[3])};
    const i16x4_t bb = __builtin_bit_cast(i16x4_t, b);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const u32x2_t a = *reinterpret_cast<const u32x2_t *>(At + acc_row_d(db, c16) * stride + kk0 + 4 * g);
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a), bb, acc[db], 0, 0, 0);
    }
}
__device__ __forceinline__ void mma_over_rows(f32x4_t acc[4], const float *At, int stride, int kk0, int c16, int g,
                                              const float bv[4]) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const f32x4_t a = *reinterpret_cast<const f32x4_t *>(At + acc_row_d(db, c16) * stride + kk0 + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], bv[r], acc[db], 0, 0, 0);
    }
}

// ----------------------------------------------------------------------------
// LDS staging of transposed tiles: lds[d * stride + (row - row0)] = src[row][d],
// rows outside [0, n) written as zeros. Split into a load step (global -> registers)
// and a store step (registers -> LDS) so callers can issue the loads early.
// A thread covers 4 consecutive rows and 8 consecutive d (four 16-byte row loads in
// bf16); NR / 4 * 8 threads cover NR rows.
// ----------------------------------------------------------------------------

template <bool BF16>
struct StageRegs;
template <>
struct StageRegs<true> {
    u32x4_t x[4];
};
template <>
struct StageRegs<false> {
    f32x4_t x[4][2];
};

__device__ __forceinline__ void stage_load(StageRegs<true> &s, const uint16_t *src, int row0, int n, int unit) {
    const int rg = unit >> 3, dg = unit & 7;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int row = row0 + 4 * rg + rr;
        s.x[rr] = (row >= 0 && row < n) ? *reinterpret_cast<const u32x4_t *>(src + (int64_t)row * 64 + 8 * dg)
                                        : u32x4_t{0u, 0u, 0u, 0u};
    }
}
__device__ __forceinline__ void stage_load(StageRegs<false> &s, const float *src, int row0, int n, int unit) {
    const int rg = unit >> 3, dg = unit & 7;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int row = row0 + 4 * rg + rr;
        const bool ok = row >= 0 && row < n;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            s.x[rr][hh] = ok ? *reinterpret_cast<const f32x4_t *>(src + (int64_t)row * 64 + 8 * dg + 4 * hh)
                             : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
}
__device__ __forceinline__ void stage_store(uint16_t *lds, int stride, const StageRegs<true> &s, int unit) {
    const int rg = unit >> 3, dg = unit & 7;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        // d = 8 dg + 2 w (low halves) and 8 dg + 2 w + 1 (high halves) of the four rows
        const u32x2_t lo = {__builtin_amdgcn_perm(s.x[1][w], s.x[0][w], 0x05040100u),
                            __builtin_amdgcn_perm(s.x[3][w], s.x[2][w], 0x05040100u)};
        const u32x2_t hi = {__builtin_amdgcn_perm(s.x[1][w], s.x[0][w], 0x07060302u),
                            __builtin_amdgcn_perm(s.x[3][w], s.x[2][w], 0x07060302u)};
        *reinterpret_cast<u32x2_t *>(lds + (8 * dg + 2 * w) * stride + 4 * rg) = lo;
        *reinterpret_cast<u32x2_t *>(lds + (8 * dg + 2 * w + 1) * stride + 4 * rg) = hi;
    }
}
__device__ __forceinline__ void stage_store(float *lds, int stride, const StageRegs<false> &s, int unit) {
    const int rg = unit >> 3, dg = unit & 7;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const f32x4_t v = {s.x[0][c >> 2][c & 3], s.x[1][c >> 2][c & 3], s.x[2][c >> 2][c & 3], s.x[3][c >> 2][c & 3]};
        *reinterpret_cast<f32x4_t *>(lds + (8 * dg + c) * stride + 4 * rg) = v;
    }
}

// Stages rows [row0, row0 + NR) with the whole workgroup (NR = 64 or 128).
template <int NR, bool BF16>
__device__ __forceinline__ void stage_tile(typename Elem<BF16>::T *lds, int stride, const typename Elem<BF16>::T *src,
                                           int row0, int n, int tid) {
    if (tid < NR * 2) {
        StageRegs<BF16> s;
        stage_load(s, src, row0, n, tid);
        stage_store(lds, stride, s, tid);
    }
}


// ----------------------------------------------------------------------------
// Row-major LDS tiles filled by direct global -> LDS loads (bf16 window kernels)
// ----------------------------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kTileRows = 128;  // rows per LDS tile: the 64-row tile and its 64-row neighbour

// Offsets handled by the unrolled, prefetching slab code of the backward for a ring of
// r slots: whole groups of r covering at least twelve offsets (a window-64 table has
// up to eight; the narrow windows of the pages' sweep, 6 to 12, have 8 to 12).
constexpr int unrolled_slabs(int r) { return ((12 + r - 1) / r) * r; }

// Copies rows [row0, row0 + 128) of a [n, 64] bf16 matrix into an LDS tile of 128
// rows of 128 bytes. The eight 16-byte chunks of tile row r are stored XOR-swizzled:
// chunk c sits at position c ^ (r & 7) of the row, so that sixteen consecutive rows
// read at one chunk (row fragments) or four rows read at four chunks (transposed
// reads) spread over the LDS banks. Each of the four waves issues four 1 KiB
// transfers; lane l of a transfer fills tile position 16 l, so it fetches the chunk
// that belongs there. Rows outside [0, n) are read from row 0: finite values that the
// masks discard. Completion is waited for with wait_vm_all() before the workgroup
// barrier.
__device__ __forceinline__ void dma_tile(uint16_t *tile, const uint16_t *src, int row0, int n, int wave, int lane) {
    const int rl = lane >> 3;                 // row within the transfer's 8 rows (= tile row & 7)
    const int chunk = (lane & 7) ^ rl;        // chunk stored at this lane's position
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int rb = 8 * (4 * wave + k);  // first of the 8 tile rows this transfer covers
        int r = row0 + rb + rl;
        r = (r >= 0 && r < n) ? r : 0;
        __builtin_amdgcn_global_load_lds(src + (int64_t)r * 64 + 8 * chunk, (lds_void_t *)(tile + rb * 64), 16, 0, 0);
    }
}

// As dma_tile for a 64-row tile (rows [row0, row0 + 64)): two transfers per wave.
__device__ __forceinline__ void dma_tile64(uint16_t *tile, const uint16_t *src, int row0, int n, int wave, int lane) {
    const int rl = lane >> 3;
    const int chunk = (lane & 7) ^ rl;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int rb = 8 * (2 * wave + k);
        int r = row0 + rb + rl;
        r = (r >= 0 && r < n) ? r : 0;
        __builtin_amdgcn_global_load_lds(src + (int64_t)r * 64 + 8 * chunk, (lds_void_t *)(tile + rb * 64), 16, 0, 0);
    }
}

// Element offset, within a swizzled tile, of the 16-byte chunk c of tile row r.
__device__ __forceinline__ int tile_chunk(int r, int c) { return r * 64 + 8 * (c ^ (r & 7)); }

// ----------------------------------------------------------------------------
// Buffer-resource loads (bf16 window kernels): a 32-bit byte offset against a
// per-head descriptor whose range is the head's rows. Offsets outside the range
// (rows < 0 or >= n) return zeros without touching memory, so slab rows need no
// clamping; the masks discard such pairs.
// ----------------------------------------------------------------------------

constexpr int kBufferConfig = 0x00020000;  // descriptor word 3 for gfx9-family raw buffers

// `bytes` is the range in bytes (at most 2^32 - 1; the callers' ranges are at most 2^31).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), kBufferConfig);
}

// Byte range of `rows` rows of `row_bytes` bytes, formed in unsigned arithmetic (a head
// of 2^24 rows of 128 bytes spans exactly 2^31 bytes).
__device__ __forceinline__ uint32_t span_bytes(int rows, uint32_t row_bytes) {
    return static_cast<uint32_t>(rows) * row_bytes;
}

// Row fragment of row `row` (lane group g's 16 elements) from a [n, 64] bf16 head.
// Cache policy of a buffer access: kCacheNT marks data read or written once, so that
// it does not push the rows other workgroups re-read out of L2.
constexpr int kCacheNormal = 0, kCacheNT = 2;

template <int POLICY = kCacheNormal>
__device__ __forceinline__ void buf_frag(Frag<true> &f, __amdgpu_buffer_rsrc_t r, int row, int g) {
    const int off = row * 128 + 16 * g;
    f.c[0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY));
    f.c[1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off + 64, 0, POLICY));
}

__device__ __forceinline__ float buf_f32(__amdgpu_buffer_rsrc_t r, int idx) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, idx * 4, 0, 0));
}

// Row that sparse offset t pairs with row `row`: row - off[t] (sign -1) or row + off[t]
// (sign +1); t beyond the table yields an offset of 0. Used as a buffer-load row only
// (out-of-range rows read as zeros); the caller masks pairs outside the sequence.
__device__ __forceinline__ int slab_row(const AttnParams &p, int n_off, int t, int row, int sign) {
    const int o = p.off[t < FSA_MAX_OFFSETS ? t : FSA_MAX_OFFSETS - 1];
    return row + sign * (t < n_off ? o : 0);
}

// Offset t of the table, or a value no row can reach when t is past the table.
__device__ __forceinline__ int table_off(const AttnParams &p, int n_off, int t) {
    return t < n_off ? p.off[t < FSA_MAX_OFFSETS ? t : FSA_MAX_OFFSETS - 1] : 0x3fffffff;
}

// Fractional entries: the weight phi[t] of the far row (row - off[t] - 1), 0 past the
// table, and the first query row that has entry t (off[t] + (phi[t] != 0): the target
// position row - off[t] - phi[t] must not lie before the sequence start).
__device__ __forceinline__ float table_phi(const AttnParams &p, int t) {
    return t < p.n_off ? p.phi[t < FSA_MAX_OFFSETS ? t : FSA_MAX_OFFSETS - 1] : 0.f;
}
__device__ __forceinline__ int table_first(const AttnParams &p, int t) {
    const int c = t < FSA_MAX_OFFSETS ? t : FSA_MAX_OFFSETS - 1;
    return t < p.n_off ? p.off[c] + (p.phi[c] != 0.f ? 1 : 0) : 0x3fffffff;
}

// Waits for every outstanding memory operation of the wave (global -> LDS copies included).
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0); }

// Waits until at most `n` vector memory operations of the wave are outstanding
// (operations complete in issue order); LDS and scalar counters are left alone.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt holds six bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Waits until the wave's LDS operations have completed (vector memory counter left alone).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Per-lane element offsets into a swizzled tile, for blocks of 16 rows starting at a
// multiple of 8 (the swizzle then depends on the lane only, so a block's rows add a
// constant that the LDS instructions take as an immediate).
struct TileLanes {
    int frag[2];  // row fragment of row c16: chunks g and g + 4
    int tr[4];    // transposed reads, one per output block db
};

__device__ __forceinline__ TileLanes tile_lanes(int c16, int g) {
    TileLanes t;
    t.frag[0] = tile_chunk(c16, g);
    t.frag[1] = tile_chunk(c16, g + 4);
    const int row = 4 * g + (c16 >> 2);
#pragma unroll
    for (int db = 0; db < 4; ++db) t.tr[db] = tile_chunk(row, 4 * (db >> 1) + (c16 & 3)) + 4 * (db & 1);
    return t;
}

// Row fragment (lane group g's 16 elements: chunks g and g + 4) of tile row lr + c16.
__device__ __forceinline__ void lds_frag(Frag<true> &f, const uint16_t *tile, int lr, const TileLanes &tl) {
    f.c[0] = *reinterpret_cast<const u32x4_t *>(tile + lr * 64 + tl.frag[0]);
    f.c[1] = *reinterpret_cast<const u32x4_t *>(tile + lr * 64 + tl.frag[1]);
}

// acc[db] += sum_{kk<16} Tile[lr + kk][d] * Bv[kk][col] for the four output blocks db,
// i.e. the product with the transposed rows lr .. lr+15 of a swizzled tile (lr a
// multiple of 8). The A operand comes from ds_read_b64_tr_b16: within a 16-lane group,
// result lane j, slot k receives element j % 4 of the 8 bytes that group lane j / 4 + 4 k
// addresses. Lane s therefore addresses row lr + 4 g + s / 4 at column
// 32 (db / 2) + 8 (s % 4) + 4 (db % 2), i.e. half db % 2 of chunk 4 (db / 2) + s % 4,
// which hands lane j the column acc_row_d(db, j) of rows lr + 4 g + k.
__device__ __forceinline__ void mma_over_rows_tr(f32x4_t acc[4], const uint16_t *tile, int lr, const TileLanes &tl,
                                                 const float bv[4]) {
    const u32x2_t b = {pack_bf16(bv[0], bv[1]), pack_bf16(bv[2], bv[3])};
    const i16x4_t bb = __builtin_bit_cast(i16x4_t, b);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(tile + lr * 64 + tl.tr[db]));
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bb, acc[db], 0, 0, 0);
    }
}

// Splits fp32 weights into bf16 high parts and bf16 remainders (w = hi + lo to ~2^-17
// relative), packed as an MFMA B operand of four values each.
__device__ __forceinline__ void split_bf16(const float bv[4], u32x2_t &hi, u32x2_t &lo) {
    hi = u32x2_t{pack_bf16(bv[0], bv[1]), pack_bf16(bv[2], bv[3])};
    lo = u32x2_t{pack_bf16(bv[0] - bf16_lo(hi[0]), bv[1] - bf16_hi(hi[0])),
                 pack_bf16(bv[2] - bf16_lo(hi[1]), bv[3] - bf16_hi(hi[1]))};
}

// As mma_over_rows with the weights carried as bf16 high part plus bf16 remainder (two
// MFMAs on one A operand), for unnormalised gradient weights; fp32 weights go through
// the fp32 MFMA unrounded already.
__device__ __forceinline__ void mma_over_rows_exact(f32x4_t acc[4], const uint16_t *At, int stride, int kk0, int c16,
                                                    int g, const float bv[4]) {
    u32x2_t h, l;
    split_bf16(bv, h, l);
    const i16x4_t bh = __builtin_bit_cast(i16x4_t, h), bl = __builtin_bit_cast(i16x4_t, l);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const i16x4_t a =
            __builtin_bit_cast(i16x4_t, *reinterpret_cast<const u32x2_t *>(At + acc_row_d(db, c16) * stride + kk0 + 4 * g));
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bh, acc[db], 0, 0, 0);
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bl, acc[db], 0, 0, 0);
    }
}
__device__ __forceinline__ void mma_over_rows_exact(f32x4_t acc[4], const float *At, int stride, int kk0, int c16,
                                                    int g, const float bv[4]) {
    mma_over_rows(acc, At, stride, kk0, c16, g, bv);
}

// As mma_over_rows_tr2 and mma_over_rows_tr, with the weights carried as bf16 high
// part plus remainder (two MFMAs on one A operand): for products whose weights are
// large and unnormalised, where one bf16 rounding of each weight would add up.
__device__ __forceinline__ void mma_over_rows_tr2_exact(f32x4_t acc[4], const uint16_t *tile, int lr0, int lr1,
                                                        const TileLanes &tl, const float bv0[4], const float bv1[4]) {
    u32x2_t h0, l0, h1, l1;
    split_bf16(bv0, h0, l0);
    split_bf16(bv1, h1, l1);
    const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, u32x4_t{h0[0], h0[1], h1[0], h1[1]});
    const bf16x8_t bl = __builtin_bit_cast(bf16x8_t, u32x4_t{l0[0], l0[1], l1[0], l1[1]});
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const i16x4_t a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(tile + lr0 * 64 + tl.tr[db]));
        const i16x4_t a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(tile + lr1 * 64 + tl.tr[db]));
        const i16x8_t a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), bh, acc[db], 0, 0, 0);
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), bl, acc[db], 0, 0, 0);
    }
}
__device__ __forceinline__ void mma_over_rows_tr_exact(f32x4_t acc[4], const uint16_t *tile, int lr, const TileLanes &tl,
                                                       const float bv[4]) {
    u32x2_t h, l;
    split_bf16(bv, h, l);
    const i16x4_t bh = __builtin_bit_cast(i16x4_t, h), bl = __builtin_bit_cast(i16x4_t, l);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(tile + lr * 64 + tl.tr[db]));
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bh, acc[db], 0, 0, 0);
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bl, acc[db], 0, 0, 0);
    }
}

// As mma_over_rows_tr for two 16-row blocks at once (rows lr0 .. lr0+15 with weights
// bv0 and rows lr1 .. lr1+15 with bv1) on the 32-deep MFMA: k-slots 0..3 of lane group
// g are rows lr0 + 4 g + k and slots 4..7 rows lr1 + 4 g + k, in both operands.
__device__ __forceinline__ void mma_over_rows_tr2(f32x4_t acc[4], const uint16_t *tile, int lr0, int lr1,
                                                  const TileLanes &tl, const float bv0[4], const float bv1[4]) {
    const u32x4_t b = {pack_bf16(bv0[0], bv0[1]), pack_bf16(bv0[2], bv0[3]), pack_bf16(bv1[0], bv1[1]),
                       pack_bf16(bv1[2], bv1[3])};
    const bf16x8_t bb = __builtin_bit_cast(bf16x8_t, b);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const i16x4_t a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(tile + lr0 * 64 + tl.tr[db]));
        const i16x4_t a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(tile + lr1 * 64 + tl.tr[db]));
        const i16x8_t a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), bb, acc[db], 0, 0, 0);
    }
}

// As mma_over_rows_tr2 with the weights already packed as bf16 pairs: words 0-1 are
// the four weights of rows lr0 + 4 g .. + 3, words 2-3 those of rows lr1 + 4 g .. + 3.
__device__ __forceinline__ void mma_over_rows_tr2_packed(f32x4_t acc[4], const uint16_t *tile, int lr0, int lr1,
                                                         const TileLanes &tl, const u32x4_t &w) {
    const bf16x8_t bb = __builtin_bit_cast(bf16x8_t, w);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const i16x4_t a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(tile + lr0 * 64 + tl.tr[db]));
        const i16x4_t a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(tile + lr1 * 64 + tl.tr[db]));
        const i16x8_t a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), bb, acc[db], 0, 0, 0);
    }
}

// ----------------------------------------------------------------------------
// Slab layout (bf16 window kernels). The sparse-offset rows are streamed in a
// layout of their own: lane l takes rows l / 8 and 8 + l / 8 of the wave's 16 rows
// and the 16-byte chunk d = 8 (l % 8) .. 8 (l % 8) + 7 of each, so one load covers
// eight whole 128-byte rows (the MFMA operand layout touches sixteen half rows per
// load, which the L2 -> CU path serves about three times slower). Row sums run over
// eight consecutive lanes with DPP.
// ----------------------------------------------------------------------------

struct SFrag {
    u32x4_t r[2];  // bf16 chunk of the lane's first and second row
};

template <int POLICY = kCacheNormal>
__device__ __forceinline__ void sfrag_load(SFrag &f, __amdgpu_buffer_rsrc_t rs, int row_a, int row_b, int c8) {
    f.r[0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, row_a * 128 + 16 * c8, 0, POLICY));
    f.r[1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, row_b * 128 + 16 * c8, 0, POLICY));
}

// Partial dot product of two 8-element bf16 chunks, one accumulation chain (the
// accumulating form of the dot instruction then needs a zero only once).
__device__ __forceinline__ float chunk_dot(const u32x4_t &a, const u32x4_t &b) {
    float s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a[0]), as_bf16x2(b[0]), 0.f, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a[1]), as_bf16x2(b[1]), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a[2]), as_bf16x2(b[2]), s, false);
    return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a[3]), as_bf16x2(b[3]), s, false);
}

// acc[0..1] (8 fp32 values of one row) += x * chunk on the packed dot unit, with the
// bf16 weight x given as the words {x, 0} (xl) and {0, x} (xh).
__device__ __forceinline__ void chunk_axpy_words(f32x4_t acc[2], uint32_t xl, uint32_t xh, const u32x4_t &c) {
    const bf16x2_t bl = as_bf16x2(xl), bh = as_bf16x2(xh);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const bf16x2_t v = as_bf16x2(c[w]);
        f32x4_t &a = acc[w >> 1];
        const int r = 2 * (w & 1);
        a[r] = __builtin_amdgcn_fdot2_f32_bf16(v, bl, a[r], false);
        a[r + 1] = __builtin_amdgcn_fdot2_f32_bf16(v, bh, a[r + 1], false);
    }
}

// acc[0..1] += x * chunk, with x rounded to bf16.
__device__ __forceinline__ void chunk_axpy(f32x4_t acc[2], float x, const u32x4_t &c) {
    const uint32_t xb = pack_bf16(x, 0.f);
    chunk_axpy_words(acc, xb, xb << 16, c);
}

// acc[0..1] += x * chunk in fp32: the bf16 values widened (exactly) to fp32 and the
// weight x taken unrounded.
__device__ __forceinline__ void chunk_axpy_f32(f32x4_t acc[2], float x, const u32x4_t &c) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        f32x4_t &a = acc[w >> 1];
        const int r = 2 * (w & 1);
        a[r] = __builtin_fmaf(bf16_lo(c[w]), x, a[r]);
        a[r + 1] = __builtin_fmaf(bf16_hi(c[w]), x, a[r + 1]);
    }
}

// One slot of the backward's pair workspace: P and dS as two bf16 in one word, or (EXACT)
// as two fp32 words.
template <bool EXACT>
struct PairSlot {
    using T = uint32_t;
};
template <>
struct PairSlot<true> {
    using T = u32x2_t;
};

// c ? a : b for a pair slot (one or two words).
__device__ __forceinline__ uint32_t select(bool c, uint32_t a, uint32_t b) { return c ? a : b; }
__device__ __forceinline__ u32x2_t select(bool c, const u32x2_t &a, const u32x2_t &b) {
    return u32x2_t{c ? a[0] : b[0], c ? a[1] : b[1]};
}

// DPP controls: quad_perm [1,0,3,2], quad_perm [2,3,0,1], and the mirror of each half row.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141;

__device__ __forceinline__ float row8_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppXor1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppXor2, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppHalfMirror, 0xF, 0xF, false));
    return x;
}
__device__ __forceinline__ float row8_max(float x) {
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppXor1, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppXor2, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppHalfMirror, 0xF, 0xF, false)));
    return x;
}

// Sum over lanes l and l ^ 8 (DPP rotation by 8 within each 16-lane row), and over the
// two halves of a 16-lane row (DPP row mirror).
constexpr int kDppRowRor8 = 0x128, kDppRowMirror = 0x140;
__device__ __forceinline__ float xor8_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppRowRor8, 0xF, 0xF, false));
}
__device__ __forceinline__ float xor8_max(float x) {
    return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppRowRor8, 0xF, 0xF, false)));
}
__device__ __forceinline__ float row16_sum(float x) {
    x = row8_sum(x);
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppRowMirror, 0xF, 0xF, false));
}

// Stores row `row` chunk (8 values, times mul) of a slab-layout accumulator.
// (NT: a non-temporal store, for outputs no later workgroup of the kernel reads.)
template <bool NT = false>
__device__ __forceinline__ void store_chunk(uint16_t *base, int64_t row, int c8, const f32x4_t a[2], float mul) {
    const f32x4_t x = a[0] * mul, y = a[1] * mul;
    const u32x4_t v = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])};
    u32x4_t *dst = reinterpret_cast<u32x4_t *>(base + row * 64 + 8 * c8);
    if constexpr (NT) __builtin_nontemporal_store(v, dst);
    else *dst = v;
}
template <bool NT = false>
__device__ __forceinline__ void store_chunk(float *base, int64_t row, int c8, const f32x4_t a[2], float mul) {
    f32x4_t *dst = reinterpret_cast<f32x4_t *>(base + row * 64 + 8 * c8);
    if constexpr (NT) {
        __builtin_nontemporal_store(a[0] * mul, dst);
        __builtin_nontemporal_store(a[1] * mul, dst + 1);
    } else {
        dst[0] = a[0] * mul;
        dst[1] = a[1] * mul;
    }
}

// Moves a 16-row accumulator from the MFMA C layout (lane (q = l % 16, g), acc[db][r] =
// row q, d = acc_row_d(db, 4 g + r)) to the slab layout through a wave-private fp32
// area of 16 x 64 values; 16-byte units are XOR-swizzled by row to spread LDS banks.
// The writes and reads come from the same wave and are processed in order. With ADD
// the moved values are added to `out` instead of replacing it.
template <bool ADD = false>
__device__ __forceinline__ void c_to_slab(float *area, const f32x4_t acc[4], f32x4_t out[2][2], int c16, int g,
                                          int s8, int c8) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const int unit = 8 * (db >> 1) + 2 * g + (db & 1);
        *reinterpret_cast<f32x4_t *>(area + c16 * 64 + 4 * (unit ^ c16)) = acc[db];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = s8 + 8 * h;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const f32x4_t x = *reinterpret_cast<const f32x4_t *>(area + row * 64 + 4 * ((2 * c8 + b) ^ row));
            out[h][b] = ADD ? out[h][b] + x : x;
        }
    }
}

// ----------------------------------------------------------------------------
// rotary position embedding
// ----------------------------------------------------------------------------

// Channel pair (xe, xo) rotated by the angle whose cosine and sine are (c, s): the
// even channel becomes fl(c xe - fl(s xo)), the odd one fl(s xe + fl(c xo)) (one fp32
// product, then one fused multiply-add; fixed so that the stored bf16 values are
// reproducible).
__device__ __forceinline__ void rope_pair(float c, float s, float xe, float xo, float &re, float &ro) {
#pragma clang fp contract(off)
    const float sx = s * xo, cx = c * xo;
    re = __builtin_fmaf(c, xe, -sx);
    ro = __builtin_fmaf(s, xe, cx);
}

// Rotates the four channel pairs packed in a 16-byte bf16 chunk by the (cos, sin) table
// entries t01 (pairs 0, 1) and t23 (pairs 2, 3), rounding the results to bf16 exactly as
// rope_kernel does.
__device__ __forceinline__ u32x4_t rope_chunk(const u32x4_t &xv, const f32x4_t &t01, const f32x4_t &t23) {
    u32x4_t ov;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const f32x4_t &tt = k < 2 ? t01 : t23;
        const int j = 2 * (k & 1);
        float re, ro;
        rope_pair(tt[j], tt[j + 1], bf16_lo(xv[k]), bf16_hi(xv[k]), re, ro);
        ov[k] = pack_bf16(re, ro);
    }
    return ov;
}

// (cos, sin) table entries of channel pairs 4 c .. 4 c + 3 of table row `row` through a
// descriptor over table rows (rows past its range read as zeros).
__device__ __forceinline__ void rope_entries(__amdgpu_buffer_rsrc_t rt, int row, int c, f32x4_t &t01,
                                             f32x4_t &t23) {
    const int off = (row * 32 + 4 * c) * 8;
    t01 = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rt, off, 0, 0));
    t23 = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rt, off + 16, 0, 0));
}

// Rotates a slab-layout gradient chunk (channels 8 c8 .. 8 c8 + 7 of row `row`) back by
// the row's angles: the transpose of the forward rotation, (e, o) -> (c e + s o, c o - s e).
__device__ __forceinline__ void rope_back_chunk(const float *table, int row, int c8, f32x4_t a[2]) {
    const f32x4_t *tab = reinterpret_cast<const f32x4_t *>(table + ((int64_t)row * 32 + 4 * c8) * 2);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const f32x4_t tt = tab[h];  // pairs 4 c8 + 2h and 4 c8 + 2h + 1
        f32x4_t &x = a[h];
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
            const float c = tt[j], sn = tt[j + 1], e = x[j], o = x[j + 1];
            x[j] = __builtin_fmaf(c, e, sn * o);
            x[j + 1] = __builtin_fmaf(c, o, -(sn * e));
        }
    }
}

// ----------------------------------------------------------------------------
// launch helpers
// ----------------------------------------------------------------------------

template <typename Kernel>
hipError_t launch(Kernel *kernel, unsigned grid, const AttnParams &p, hipStream_t stream) {
    AttnParams a = p;
    void *args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), dim3(grid), dim3(kThreads), args, 0, stream);
}

inline unsigned tiles(const AttnParams &p) { return (unsigned)(p.bh * ((p.n + 63) / 64)); }

// Calls f(Len<k>{}) with the table length k fixed at compile time for the lengths the
// window-64 tables usually have (4 to 7 offsets below N), Len<0> (length read at run
// time) otherwise. A fixed length removes the uniform length tests from the unrolled
// slab loops. (At 8 the one-launch backward would need more than 128 VGPRs.)
template <int K>
struct Len {
    static constexpr int value = K;
};
template <typename F>
hipError_t with_table_length(int n_off, F &&f) {
    switch (n_off) {
    case 4: return f(Len<4>{});
    case 5: return f(Len<5>{});
    case 6: return f(Len<6>{});
    case 7: return f(Len<7>{});
    default: return f(Len<0>{});
    }
}

// ----------------------------------------------------------------------------
// Per-tile completion tokens within one launch (one-launch backward, rotary forward)
// ----------------------------------------------------------------------------
//
// A token names one launch: the dispatch id (the packet's index in its queue, which
// grows by one per dispatch) mixed with the queue's address (each queue counts from
// zero). A tile whose words others read writes it to that tile's flag once they are in
// L2; a workspace's earlier contents, earlier launches' tokens included, do not match it.
extern "C" __device__ uint64_t fsa_dispatch_id() __asm("llvm.amdgcn.dispatch.id");
__device__ __forceinline__ uint64_t launch_token() {
    const uint64_t q = reinterpret_cast<uint64_t>(__builtin_amdgcn_queue_ptr());
    return fsa_dispatch_id() ^ (q * 0x9E3779B97F4A7C15ull);
}

// Cache policy (sc0) for words that another workgroup of the same launch wrote, in the
// same XCD's L2 (pair words, D, rotated K rows). No CU reads them before their token is
// set, and this one bypasses the L1, so no older copy is read.
constexpr int kCachePastL1 = 1;
// Waits until flags[first .. last] all hold the token (one wave; lane l checks flags
// first + l, first + l + 64, ...; device-scope loads, which miss this CU's L1). Each
// poll requests up to 64 * BATCH flags before comparing any, so that it costs one
// round trip for up to that many tiles. The wait is bounded (p.max_polls polls with a
// short sleep between them) and looks for token ^ p.token_xor (the token itself unless
// the host forces a give-up). Returns false, uniformly over the wave, if it gave up;
// the caller then records the launch's token in p.status and stores NaN so that the
// failure shows.
template <int BATCH = 1>
__device__ __forceinline__ bool poll_tiles(const AttnParams &p, const uint64_t *flags, int first, int last,
                                           uint64_t token, int lane) {
    const uint64_t want = token ^ p.token_xor;
    for (int spin = 0;; ++spin) {
        bool ready = true;
        for (int base = first + lane; base <= last; base += 64 * BATCH) {
            // every lane loads (indices past `last` read `last` again), without branches,
            // so that the loads leave back to back
            uint64_t v[BATCH];
#pragma unroll
            for (int k = 0; k < BATCH; ++k)
                v[k] = __hip_atomic_load(flags + min(base + 64 * k, last), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int k = 0; k < BATCH; ++k) ready &= (base + 64 * k > last) | (v[k] == want);
        }
        if (__builtin_amdgcn_ballot_w64(!ready) == 0) return true;
        if (spin >= p.max_polls) return false;
        __builtin_amdgcn_s_sleep(4);
    }
}

// Records that a wait of this launch gave up: the status word takes the launch's token
// (read back by the host, see fsa_wait_status).
__device__ __forceinline__ void record_give_up(const AttnParams &p, uint64_t token) {
    __hip_atomic_store(p.status, token, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


}  // namespace
}  // namespace fsa
