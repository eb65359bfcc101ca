// HIP kernels of libfsa for gfx950 (MI355X): Fibonacci-offset sparse attention.
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
//  * Backward: two kernels. The first forms dQ of its query rows (and D), storing
//    the bf16 P and dS of every sparse pair; the second forms dK, dV of its key
//    rows from the band (recomputed) and those stored weights. Every output row
//    has one writer and no atomics are used.
//  * Workgroup ids are remapped so that the tiles of one head run on one XCD in
//    increasing row order, keeping that head's rows in the XCD's L2 for the
//    slab re-reads.
// The general kernels (fp32 inputs, wider windows, the dense baseline) loop over
// 64-key chunks with an online softmax.

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

// Hardware dispatch places workgroup b on XCD b % 8. Returns the logical tile
// index so that each XCD receives one contiguous range of logical tiles, which
// it processes in increasing order.
__device__ __forceinline__ int xcd_logical_block(int b, int nb) {
    const int x = b & 7, idx = b >> 3;
    const int per = nb >> 3, extra = nb & 7;
    return x * per + (x < extra ? x : extra) + idx;
}

// ----------------------------------------------------------------------------
// Row-major LDS tiles filled by direct global -> LDS loads (bf16 window kernels)
// ----------------------------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kTileRows = 128;  // rows per LDS tile: the 64-row tile and its 64-row neighbour

// Offsets handled by the unrolled, prefetching slab code for a ring of r slots:
// whole groups of r covering at least the eight offsets of a window-64 table.
constexpr int unrolled_slabs(int r) { return ((8 + r - 1) / r) * r; }

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

// Rotates bf16 rows into bf16 rows: one thread per 16-byte chunk (channel pairs
// 4c .. 4c + 3 of one row, eight threads per row), the same chunk of every tensor, so
// that each table entry is read once. Rows are addressed as (head, position) with
// blockIdx.y the head, so positions need no division.
__global__ void __launch_bounds__(kThreads) rope_kernel(const RopeParams p) {
    const int idx = blockIdx.x * kThreads + threadIdx.x;  // chunk within the head
    const int pos = idx >> 3, c = idx & 7;
    if (pos >= p.n) return;
    const int64_t row = ((int64_t)p.head0 + blockIdx.y) * p.n + pos;
    const f32x4_t *tab = reinterpret_cast<const f32x4_t *>(p.table + ((int64_t)pos * 32 + 4 * c) * 2);
    const f32x4_t t01 = tab[0], t23 = tab[1];  // (cos, sin) of pairs 4c, 4c + 1, then 4c + 2, 4c + 3
    u32x4_t xv[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
        if (t < p.count)
            xv[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p.x[t] + row * 64 + 8 * c));
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        if (t < p.count) {
            u32x4_t ov;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const f32x4_t &tt = k < 2 ? t01 : t23;
                const int j = 2 * (k & 1);
                float re, ro;
                rope_pair(tt[j], tt[j + 1], bf16_lo(xv[t][k]), bf16_hi(xv[t][k]), re, ro);
                ov[k] = pack_bf16(re, ro);
            }
            *reinterpret_cast<u32x4_t *>(p.out[t] + row * 64 + 8 * c) = ov;
        }
    }
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
// forward
// ----------------------------------------------------------------------------

enum FwdMode { kWide = 1, kDense = 2 };

// Sparse offsets t in [t_begin, n_off), four at a time, each with one online
// softmax update (used beyond the prefetched offsets and by the wide path).
template <bool BF16>
__device__ __forceinline__ void fwd_slabs_loop(const AttnParams &p, int t_begin, const Frag<BF16> &qf,
                                               const typename Elem<BF16>::T *K, const typename Elem<BF16>::T *V,
                                               int i, bool row_ok, int r0, int n, int g, f32x4_t acc[4], float &m2,
                                               float &lsum) {
    for (int t0 = t_begin; t0 < p.n_off; t0 += 4) {
        if (r0 + 15 < p.off[t0]) break;  // ascending offsets: no later slab reaches a key
        Frag<BF16> kf[4], vf[4];
        bool ok[4];
        int jc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = t0 + u;
            const int j = (t < p.n_off) ? i - p.off[t] : -1;
            ok[u] = row_ok && j >= 0;
            jc[u] = min(max(j, 0), n - 1);
            load_frag(kf[u], K, jc[u], g);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) load_frag(vf[u], V, jc[u], g);
        float sc[4], gm = kNegInf;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            sc[u] = ok[u] ? group_sum(frag_dot(qf, kf[u])) * p.scale_log2 : kNegInf;
            gm = fmaxf(gm, sc[u]);
        }
        const float mn = fmaxf(m2, gm);
        const float ms = (mn == kNegInf) ? 0.f : mn;
        const float al = fast_exp2(m2 - ms);
        float ps = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] *= al;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float pu = fast_exp2(sc[u] - ms);
            ps += pu;
            frag_axpy(acc, pu, vf[u]);
        }
        lsum = lsum * al + (g == 0 ? ps : 0.f);
        m2 = mn;
    }
}

template <bool BF16, bool OUT_BF16, int MODE>
__global__ void __launch_bounds__(kThreads) fwd_kernel(const AttnParams p) {
    using E = typename Elem<BF16>::T;
    using OE = typename Elem<OUT_BF16>::T;
    __shared__ __attribute__((aligned(16))) E vt[64 * kT64];  // V^T of one 64-key chunk

    const int n = p.n, w = p.w;
    const int nt = (n + 63) >> 6;
    const int lb = xcd_logical_block(blockIdx.x, p.bh * nt);
    const int bh = lb / nt, tile = lb - bh * nt;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c16 = lane & 15, g = lane >> 4;
    const int i0 = tile * 64, r0 = i0 + 16 * wave;
    const int i = r0 + c16;  // this lane's query row
    const bool row_ok = i < n;
    const int64_t head = (int64_t)bh * n * 64;
    const E *Q = static_cast<const E *>(p.q) + head;
    const E *K = static_cast<const E *>(p.k) + head;
    const E *V = static_cast<const E *>(p.v) + head;
    const float sl2 = p.scale_log2;

    Frag<BF16> qf;
    load_frag(qf, Q, row_ok ? i : n - 1, g);

    f32x4_t acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m2 = kNegInf;  // running max of log2-scaled scores
    float lsum = 0.f;    // this lane's share of the running sum

    // ---------------- wide window or dense: 64-key chunks with an online softmax ----------------
    const int jlo = max(0, i0 - w + 1), jhi = min(n - 1, i0 + 63);
    const int wlo = r0 - w + 1, whi = min(r0 + 15, n - 1);  // keys this wave needs
    for (int c0 = jlo & ~63; c0 <= jhi; c0 += 64) {
        __syncthreads();
        stage_tile<64, BF16>(vt, kT64, V, c0, n, tid);
        __syncthreads();
        if (r0 >= n) continue;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int kb0 = c0 + 16 * kb;
            if (kb0 + 15 < wlo || kb0 > whi) continue;  // uniform across the wave
            Frag<BF16> kf;
            load_frag(kf, K, min(kb0 + c16, n - 1), g);
            const f32x4_t st = mma_over_d(kf, qf, f32x4_t{0.f, 0.f, 0.f, 0.f}) * sl2;
            float sv[4], bm = kNegInf;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = kb0 + 4 * g + r;
                const bool ok = row_ok && j <= i && j > i - w;
                sv[r] = ok ? st[r] : kNegInf;
                bm = fmaxf(bm, sv[r]);
            }
            bm = group_max(bm);
            const float mn = fmaxf(m2, bm);
            const float ms = (mn == kNegInf) ? 0.f : mn;
            const float al = fast_exp2(m2 - ms);
            float pr[4], ps = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pr[r] = fast_exp2(sv[r] - ms);
                ps += pr[r];
            }
            lsum = lsum * al + ps;
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] *= al;
            m2 = mn;
            mma_over_rows(acc, vt, kT64, 16 * kb, c16, g, pr);
        }
    }
    if (MODE == kWide && r0 < n) fwd_slabs_loop(p, 0, qf, K, V, i, row_ok, r0, n, g, acc, m2, lsum);

    // ---- epilogue ----
    const float l = group_sum(lsum);
    if (row_ok) {
        store_row(static_cast<OE *>(p.out) + head, i, g, acc, 1.f / l);
        if (g == 0) p.lse_out[(int64_t)bh * n + i] = m2 * kLn2 + logf(l);
    }
}

// Forward, bf16 inputs, window w <= 64. The workgroup's band keys [i0 - 64, i0 + 64)
// are copied into LDS (K and V row-major) first. Once they have landed, the first
// sparse slabs are requested, in the slab layout, into a ring of four row pairs per
// lane, and the band runs on MFMA while those loads are in flight; its softmax state
// then moves into the slab layout and the slabs continue it as an online softmax, one
// group of four offsets at a time. The slab layout stores O and the LSE.
// With FRAC the table holds fractional entries (learned-alpha variant): entry t's key
// and value for row i are (1 - phi) row(i - off[t]) + phi row(i - off[t] - 1), so each
// entry reads two adjacent slabs (near and far); entries go two per softmax update.
// With ROPE, Q arrives unrotated (K, V as usual): the kernel rotates its own query rows
// by the table p.rope and, when p.qhat is set, stores the rotated rows there (for a
// backward to reuse).
template <bool OUT_BF16, bool FRAC, bool ROPE = false, int NOFF = 0>
__global__ void __launch_bounds__(kThreads) fwd_window_kernel(const AttnParams p) {
    using OE = typename Elem<OUT_BF16>::T;
    __shared__ __attribute__((aligned(16))) uint16_t ks[kTileRows * 64];  // band K rows, then merge areas
    __shared__ __attribute__((aligned(16))) uint16_t vs[kTileRows * 64];  // band V rows, then band row stats

    const int n = p.n, w = p.w, n_off = NOFF > 0 ? NOFF : p.n_off;
    const int nt = (n + 63) >> 6;
    const int lb = xcd_logical_block(blockIdx.x, p.bh * nt);
    const int bh = lb / nt, tile = lb - bh * nt;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c16 = lane & 15, g = lane >> 4;  // MFMA layout: row c16, lane group g
    const TileLanes tl = tile_lanes(c16, g);
    const uint16_t *ks_w = ks + 1024 * wave, *vs_w = vs + 1024 * wave;  // this wave's band rows start here
    const int s8 = lane >> 3, c8 = lane & 7;   // slab layout: rows s8 and 8 + s8, chunk c8
    const int i0 = tile * 64, r0 = i0 + 16 * wave;
    const int row_s[2] = {r0 + s8, r0 + 8 + s8};
    const int64_t head = (int64_t)bh * n * 64;
    const uint16_t *Q = static_cast<const uint16_t *>(p.q) + head;
    const uint16_t *K = static_cast<const uint16_t *>(p.k) + head;
    const uint16_t *V = static_cast<const uint16_t *>(p.v) + head;
    const __amdgpu_buffer_rsrc_t rq = head_rsrc(Q, span_bytes(n, 128)), rk = head_rsrc(K, span_bytes(n, 128));
    const __amdgpu_buffer_rsrc_t rv = head_rsrc(V, span_bytes(n, 128));
    const float sl2 = p.scale_log2;
    const int i = r0 + c16;  // MFMA-layout query row
    const bool row_ok = i < n;

    dma_tile(ks, K, i0 - 64, n, wave, lane);
    dma_tile(vs, V, i0 - 64, n, wave, lane);
    Frag<true> qf;
    buf_frag(qf, rq, i, g);
    [[maybe_unused]] __amdgpu_buffer_rsrc_t rt;
    if constexpr (ROPE) {
        // the table rows of this tile's positions (the positions past n read as zeros)
        rt = head_rsrc(p.rope + (int64_t)i0 * 64, span_bytes(min(64, n - i0), 256));
        f32x4_t a01, a23, b01, b23;
        rope_entries(rt, i - i0, g, a01, a23);      // chunk g: pairs 4g .. 4g + 3
        rope_entries(rt, i - i0, g + 4, b01, b23);  // chunk g + 4
        wait_vm_all();
        qf.c[0] = rope_chunk(qf.c[0], a01, a23);
        qf.c[1] = rope_chunk(qf.c[1], b01, b23);
    }
    wait_vm_all();
    __syncthreads();
    // the first slab rows are requested now and land while the band runs; most of them
    // are rows of neighbouring tiles whose band copies have just passed through L2
    SFrag sk[4], sv[4];  // FRAC: slot u of entries holds near rows in [2u], far rows in [2u + 1]
    auto frac_fill = [&](SFrag *f, __amdgpu_buffer_rsrc_t r, int u, int t) {
        const int n0 = slab_row(p, n_off, t, row_s[0], -1), n1 = slab_row(p, n_off, t, row_s[1], -1);
        sfrag_load(f[2 * u], r, n0, n1, c8);
        sfrag_load(f[2 * u + 1], r, n0 - 1, n1 - 1, c8);
    };
    if constexpr (FRAC) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            frac_fill(sk, rk, u, u);
            frac_fill(sv, rv, u, u);
        }
    } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (u < n_off) {  // uniform
                sfrag_load(sk[u], rk, slab_row(p, n_off, u, row_s[0], -1), slab_row(p, n_off, u, row_s[1], -1), c8);
                sfrag_load(sv[u], rv, slab_row(p, n_off, u, row_s[0], -1), slab_row(p, n_off, u, row_s[1], -1), c8);
            }
        }
    }

    // ---- window band on MFMA: rows r0..r0+15 (row c16 of the lane) see key blocks qb-4 .. qb ----
    // Scores stay unscaled (the scale, > 0 on this path, enters each exponent through
    // one fma). Blocks wholly outside the sequence or the window are computed like the
    // others and masked: their tile rows hold finite values (row 0 stands in for rows
    // outside [0, n)).
    const int qb = r0 >> 4;
    float sc[5][4];
    float bm = kNegInf;
#pragma unroll
    for (int b = 0; b < 5; ++b) {
        const int kb0 = 16 * (qb - 4 + b);
        const bool full = kb0 >= 0 && kb0 + 15 <= r0 && kb0 >= r0 + 16 - w && r0 + 15 < n;
        Frag<true> kf;
        lds_frag(kf, ks_w, 16 * b, tl);
        f32x4_t st = mma_over_d(kf, qf, f32x4_t{0.f, 0.f, 0.f, 0.f});
        if (!full) {  // uniform: edge blocks only
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = kb0 + 4 * g + r;
                if (!(row_ok && j <= i && j > i - w && j >= 0)) st[r] = kNegInf;
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sc[b][r] = st[r];
            bm = fmaxf(bm, st[r]);
        }
    }
    // scaled row maximum; a valid row always attends itself, so it is finite there
    const float m_b = row_ok ? group_max(bm) * sl2 : kNegInf;
    const float msb = row_ok ? m_b : 0.f;
    f32x4_t acc_b[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc_b[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float pr[5][4], lsum_b = 0.f;
#pragma unroll
    for (int b = 0; b < 5; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pr[b][r] = fast_exp2(__builtin_fmaf(sc[b][r], sl2, -msb));
            lsum_b += pr[b][r];
        }
    mma_over_rows_tr2(acc_b, vs_w, 0, 16, tl, pr[0], pr[1]);
    mma_over_rows_tr2(acc_b, vs_w, 32, 48, tl, pr[2], pr[3]);
    mma_over_rows_tr(acc_b, vs_w, 64, tl, pr[4]);
    const float l_b = group_sum(lsum_b);

    // ---- the band state, moved into the slab layout, starts the slabs' online softmax ----
    __syncthreads();  // every wave is done with the band tiles
    float *area = reinterpret_cast<float *>(ks) + wave * 1024;
    float *stat = reinterpret_cast<float *>(vs) + wave * 32;
    if (g == 0) {
        stat[c16] = m_b;
        stat[16 + c16] = l_b;
    }
    float m_s[2], l_s[2];  // scaled running maximum, running sum
    f32x4_t acc_s[2][2];
    c_to_slab(area, acc_b, acc_s, c16, g, s8, c8);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        m_s[h] = stat[s8 + 8 * h];
        l_s[h] = stat[16 + s8 + 8 * h];
    }

    // ---- sparse slabs: keys row - off[t], four offsets per online-softmax update ----
    SFrag qs;
    if constexpr (ROPE) {
        // the rotated query rows, already in registers in the MFMA layout (row c16, chunks
        // g and g + 4), move to the slab layout through this wave's 2 KB of the V tile,
        // free since the barrier above
        uint16_t *qa = vs + 1024 * wave + 512;
        *reinterpret_cast<u32x4_t *>(qa + c16 * 64 + 8 * g) = qf.c[0];
        *reinterpret_cast<u32x4_t *>(qa + c16 * 64 + 8 * (g + 4)) = qf.c[1];
        uint16_t *QH = p.qhat ? static_cast<uint16_t *>(p.qhat) + head : nullptr;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            qs.r[h] = *reinterpret_cast<const u32x4_t *>(qa + (s8 + 8 * h) * 64 + 8 * c8);
            if (p.qhat && row_s[h] < n)  // uniform test of the pointer
                *reinterpret_cast<u32x4_t *>(QH + (int64_t)row_s[h] * 64 + 8 * c8) = qs.r[h];
        }
    } else {
        sfrag_load(qs, rq, row_s[0], row_s[1], c8);
    }
    // moves the state to a new maximum; skipped (uniformly) when no row's maximum grew,
    // which the band's 64 keys make the common case
    auto rescale = [&](const float mn[2]) {
        if (__builtin_amdgcn_ballot_w64((mn[0] > m_s[0]) | (mn[1] > m_s[1])) != 0) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float al = fast_exp2(m_s[h] - (mn[h] == kNegInf ? 0.f : mn[h]));
                acc_s[h][0] *= al;
                acc_s[h][1] *= al;
                l_s[h] *= al;
                m_s[h] = mn[h];
            }
        }
    };
    if constexpr (FRAC) {
        // entries two at a time; the ring slot of an entry is refilled with the entry
        // two further on as soon as its rows have been used
        for (int t0 = 0; t0 < n_off; t0 += 2) {
            if (r0 + 15 < p.off[t0]) break;  // ascending entries: no row of the wave has one
            float ss[2][2], ph[2], gm[2] = {kNegInf, kNegInf};
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int t = t0 + u, first = table_first(p, t);
                ph[u] = table_phi(p, t);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const bool ok = (row_s[h] < n) & (row_s[h] >= first);
                    const float dn = chunk_dot(qs.r[h], sk[2 * u].r[h]);
                    const float df = chunk_dot(qs.r[h], sk[2 * u + 1].r[h]);
                    const float d = row8_sum(__builtin_fmaf(ph[u], df - dn, dn));
                    ss[u][h] = ok ? d : kNegInf;
                    gm[h] = fmaxf(gm[h], ss[u][h]);
                }
                if (t + 2 < n_off) frac_fill(sk, rk, u, t + 2);  // uniform
            }
            const float mn[2] = {fmaxf(m_s[0], gm[0] * sl2), fmaxf(m_s[1], gm[1] * sl2)};
            rescale(mn);
            const float ms[2] = {m_s[0] == kNegInf ? 0.f : m_s[0], m_s[1] == kNegInf ? 0.f : m_s[1]};
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (t0 + u < n_off) {  // uniform
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const float pt = fast_exp2(__builtin_fmaf(ss[u][h], sl2, -ms[h]));
                        const float pf = pt * ph[u];
                        l_s[h] += pt;
                        chunk_axpy(acc_s[h], pt - pf, sv[2 * u].r[h]);
                        chunk_axpy(acc_s[h], pf, sv[2 * u + 1].r[h]);
                    }
                }
                if (t0 + u + 2 < n_off) frac_fill(sv, rv, u, t0 + u + 2);  // uniform
            }
        }
    } else {
#pragma unroll
        for (int t0 = 0; t0 < 8; t0 += 4) {
            if (t0 >= n_off || r0 + 15 < p.off[t0]) break;  // ascending offsets
            float ss[4][2], gm[2] = {kNegInf, kNegInf};    // unscaled scores
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int o = table_off(p, n_off, t0 + u);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    ss[u][h] = kNegInf;
                    if (t0 + u < n_off) {  // uniform: slots past the table only refill
                        const bool ok = (row_s[h] < n) & (row_s[h] - o >= 0);
                        const float d = row8_sum(chunk_dot(qs.r[h], sk[u].r[h]));
                        ss[u][h] = ok ? d : kNegInf;
                        gm[h] = fmaxf(gm[h], ss[u][h]);
                    }
                }
                if (t0 == 0 && u + 4 < n_off)  // uniform
                    sfrag_load(sk[u], rk, slab_row(p, n_off, u + 4, row_s[0], -1), slab_row(p, n_off, u + 4, row_s[1], -1), c8);
            }
            const float mn[2] = {fmaxf(m_s[0], gm[0] * sl2), fmaxf(m_s[1], gm[1] * sl2)};
            rescale(mn);
            const float ms[2] = {m_s[0] == kNegInf ? 0.f : m_s[0], m_s[1] == kNegInf ? 0.f : m_s[1]};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (t0 + u < n_off) {  // uniform
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const float pt = fast_exp2(__builtin_fmaf(ss[u][h], sl2, -ms[h]));
                        l_s[h] += pt;
                        chunk_axpy(acc_s[h], pt, sv[u].r[h]);
                    }
                }
                if (t0 == 0 && u + 4 < n_off)  // uniform
                    sfrag_load(sv[u], rv, slab_row(p, n_off, u + 4, row_s[0], -1), slab_row(p, n_off, u + 4, row_s[1], -1), c8);
            }
        }
        for (int t = 8; t < n_off; ++t) {  // tables longer than eight offsets
            if (r0 + 15 < p.off[t]) break;
            SFrag kt, vt;
            sfrag_load(kt, rk, row_s[0] - p.off[t], row_s[1] - p.off[t], c8);
            sfrag_load(vt, rv, row_s[0] - p.off[t], row_s[1] - p.off[t], c8);
            float sv1[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bool ok = (row_s[h] < n) & (row_s[h] - p.off[t] >= 0);
                sv1[h] = ok ? row8_sum(chunk_dot(qs.r[h], kt.r[h])) : kNegInf;
            }
            const float mn[2] = {fmaxf(m_s[0], sv1[0] * sl2), fmaxf(m_s[1], sv1[1] * sl2)};
            rescale(mn);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float pt = fast_exp2(__builtin_fmaf(sv1[h], sl2, -(m_s[h] == kNegInf ? 0.f : m_s[h])));
                l_s[h] += pt;
                chunk_axpy(acc_s[h], pt, vt.r[h]);
            }
        }

    }
    // ---- normalise, store ----
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (row_s[h] < n) {
            store_chunk(static_cast<OE *>(p.out) + head, row_s[h], c8, acc_s[h], 1.f / l_s[h]);
            if (c8 == 0) p.lse_out[(int64_t)bh * n + row_s[h]] = m_s[h] * kLn2 + logf(l_s[h]);
        }
    }
}

// One thread's share of a 64-row K and V tile: the 16-byte chunks q = tid and
// q = tid + 256 (tile row q / 8, chunk q % 8) of each.
struct TileChunks {
    u32x4_t k[2], v[2];
};

// Fetches key rows [row0, row0 + 64) into registers (rows past the sequence read as zeros).
__device__ __forceinline__ void fetch_tile(TileChunks &c, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                           int row0, int tid) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int q = tid + 256 * h;
        const int off = (row0 + (q >> 3)) * 128 + 16 * (q & 7);
        c.k[h] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
        c.v[h] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    }
}

// Writes fetched chunks into swizzled 64-row LDS tiles (chunk c of row r at c ^ (r & 7)).
__device__ __forceinline__ void stage_tile(uint16_t *kt, uint16_t *vt, const TileChunks &c, int tid) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int q = tid + 256 * h;
        const int e = tile_chunk(q >> 3, q & 7);
        *reinterpret_cast<u32x4_t *>(kt + e) = c.k[h];
        *reinterpret_cast<u32x4_t *>(vt + e) = c.v[h];
    }
}

// Dense causal forward (the baseline), bf16 inputs, positive scale. One workgroup =
// one 64-row query tile; it walks the key tiles 0 .. tile with an online softmax whose
// accumulator is rescaled only when a row maximum grows. Each key tile is fetched into
// registers two tiles ahead of its use and written into one of two swizzled LDS stages
// one tile ahead, so its fetch has two tiles of compute to land. Row sums are taken
// over the bf16-rounded probabilities that the P.V product uses. The tile order pairs
// light and heavy tiles on a CU: within each head the upper half of the tiles runs in
// reverse, so the blocks that dispatch places on one CU (32 apart in an XCD's range)
// hold tiles t and T - 1 - t.
template <bool OUT_BF16>
__global__ void __launch_bounds__(kThreads) fwd_dense_kernel(const AttnParams p) {
    using OE = typename Elem<OUT_BF16>::T;
    __shared__ __attribute__((aligned(16))) uint16_t kt[2][64 * 64];
    __shared__ __attribute__((aligned(16))) uint16_t vt[2][64 * 64];

    const int n = p.n, nt = (n + 63) >> 6, half = nt >> 1;
    const int lb = xcd_logical_block(blockIdx.x, p.bh * nt);
    const int bh = lb / nt, u = lb - bh * nt;
    const int tile = u < half ? u : nt - 1 + half - u;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15, g = lane >> 4;
    const TileLanes tl = tile_lanes(c16, g);
    const int i0 = tile * 64, i = i0 + 16 * wave + c16;
    const bool row_ok = i < n;
    const int64_t head = (int64_t)bh * n * 64;
    const __amdgpu_buffer_rsrc_t rk = head_rsrc(static_cast<const uint16_t *>(p.k) + head, span_bytes(n, 128));
    const __amdgpu_buffer_rsrc_t rv = head_rsrc(static_cast<const uint16_t *>(p.v) + head, span_bytes(n, 128));
    const float sl2 = p.scale_log2;

    Frag<true> qf;
    buf_frag(qf, head_rsrc(static_cast<const uint16_t *>(p.q) + head, span_bytes(n, 128)), i, g);
    // ring[x] holds the fetched key tile that is next staged at a step of parity x ^ 1.
    // Fetches and stages run unconditionally, past the last tile on a copy of it, so that
    // the wait before each stage counts exactly the loads issued after its fetch.
    TileChunks ring[2];
    fetch_tile(ring[0], rk, rv, 0, tid);
    fetch_tile(ring[1], rk, rv, 64 * min(1, tile), tid);
    stage_tile(kt[0], vt[0], ring[0], tid);
    fetch_tile(ring[0], rk, rv, 64 * min(2, tile), tid);

    float m = kNegInf, lsum = 0.f;  // unscaled running maximum, running sum (lane partial)
    f32x4_t acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // step j: key tile j from stage b = j & 1; tile j + 1 goes from ring[b ^ 1] into the
    // other stage, and ring[b ^ 1] then fetches tile j + 3
    auto step = [&](int j, uint16_t *ks, uint16_t *vs, uint16_t *ks_next, uint16_t *vs_next, TileChunks &next) {
        __syncthreads();  // key tile j is in its stage; every wave is done with tile j - 1
        stage_tile(ks_next, vs_next, next, tid);
        fetch_tile(next, rk, rv, 64 * min(j + 3, tile), tid);
        float sc[4][4], bm = kNegInf;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            Frag<true> kf;
            lds_frag(kf, ks, 16 * b, tl);
            f32x4_t st = mma_over_d(kf, qf, f32x4_t{0.f, 0.f, 0.f, 0.f});
            if (j == tile) {  // uniform: the diagonal tile is causal-masked
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (!(row_ok && 64 * j + 16 * b + 4 * g + r <= i)) st[r] = kNegInf;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sc[b][r] = st[r];
                bm = fmaxf(bm, st[r]);
            }
        }
        const float mn = fmaxf(m, group_max(bm));
        if (__builtin_amdgcn_ballot_w64(mn > m) != 0) {  // some row's maximum grew
            const float al = fast_exp2(m == kNegInf ? kNegInf : (m - mn) * sl2);  // 0 while m is still -inf
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] *= al;
            lsum *= al;
            m = mn;
        }
        const float ms = m == kNegInf ? 0.f : m * sl2;
        // probabilities rounded to bf16 once: the P.V product and the row sum use the same values
        u32x4_t pw[2];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            float pr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(__builtin_fmaf(sc[b][r], sl2, -ms));
            pw[b >> 1][2 * (b & 1)] = pack_bf16(pr[0], pr[1]);
            pw[b >> 1][2 * (b & 1) + 1] = pack_bf16(pr[2], pr[3]);
        }
        const bf16x2_t ones = as_bf16x2(0x3F803F80u);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int w = 0; w < 4; ++w) lsum = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pw[h][w]), ones, lsum, false);
        mma_over_rows_tr2_packed(acc, vs, 0, 16, tl, pw[0]);
        mma_over_rows_tr2_packed(acc, vs, 32, 48, tl, pw[1]);
    };
    int j = 0;
    for (; j < tile; j += 2) {
        step(j, kt[0], vt[0], kt[1], vt[1], ring[1]);
        step(j + 1, kt[1], vt[1], kt[0], vt[0], ring[0]);
    }
    if (j == tile) step(j, kt[0], vt[0], kt[1], vt[1], ring[1]);
    const float l = group_sum(lsum);
    if (row_ok) {
        store_row(static_cast<OE *>(p.out) + head, i, g, acc, 1.f / l);
        if (g == 0) p.lse_out[(int64_t)bh * n + i] = m * sl2 * kLn2 + logf(l);
    }
}

// ----------------------------------------------------------------------------
// backward: D = rowsum(dO * O)
// ----------------------------------------------------------------------------

// D = rowsum(dO * O): eight lanes per 64-wide row, 16 bytes each (bf16); a workgroup
// covers 32 rows per pass and two passes.
template <bool BF16>
__global__ void __launch_bounds__(kThreads) delta_kernel(const AttnParams p) {
    using E = typename Elem<BF16>::T;
    constexpr int kPer = 16 / sizeof(E);  // elements per lane and load
    constexpr int kLanesPerRow = 64 / kPer;
    constexpr int kRowsPerPass = kThreads / kLanesPerRow;
    const int64_t rows = (int64_t)p.bh * p.n;
    const int part = threadIdx.x % kLanesPerRow;
    float acc[2];
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const int64_t row = ((int64_t)blockIdx.x * 2 + pass) * kRowsPerPass + threadIdx.x / kLanesPerRow;
        acc[pass] = 0.f;
        if (row < rows) {
            const E *o = static_cast<const E *>(p.o) + row * 64 + kPer * part;
            const E *d = static_cast<const E *>(p.dout) + row * 64 + kPer * part;
            if constexpr (BF16) {
                const u32x4_t a = *reinterpret_cast<const u32x4_t *>(o);
                const u32x4_t b = *reinterpret_cast<const u32x4_t *>(d);
                float s = 0.f;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a[k]), as_bf16x2(b[k]), s, false);
                acc[pass] = s;
            } else {
                const f32x4_t a = *reinterpret_cast<const f32x4_t *>(o);
                const f32x4_t b = *reinterpret_cast<const f32x4_t *>(d);
                acc[pass] = a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
            }
        }
    }
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        float s = acc[pass];
#pragma unroll
        for (int sh = 1; sh < kLanesPerRow; sh <<= 1) s += __shfl_xor(s, sh);
        const int64_t row = ((int64_t)blockIdx.x * 2 + pass) * kRowsPerPass + threadIdx.x / kLanesPerRow;
        if (row < rows && part == 0) p.delta[row] = s;
    }
}

// ----------------------------------------------------------------------------
// backward: dQ (query-owned) then dK, dV (key-owned) of one 64-row tile
// ----------------------------------------------------------------------------

template <bool BF16, bool OUT_BF16>
__global__ void __launch_bounds__(kThreads) bwd_generic_kernel(const AttnParams p) {
    using E = typename Elem<BF16>::T;
    using OE = typename Elem<OUT_BF16>::T;
    __shared__ __attribute__((aligned(16))) E t0s[64 * kT64];  // transposed tile (K^T, or Q^T)
    __shared__ __attribute__((aligned(16))) E t1s[64 * kT64];  // transposed tile (dO^T)
    __shared__ float lse_s[64], del_s[64];

    const int n = p.n, w = p.w;
    const int nt = (n + 63) >> 6;
    const int lb = xcd_logical_block(blockIdx.x, p.bh * nt);
    const int bh = lb / nt, tile = lb - bh * nt;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c16 = lane & 15, g = lane >> 4;
    const int t0 = tile * 64, r0 = t0 + 16 * wave;
    const int64_t head = (int64_t)bh * n * 64;
    const E *Q = static_cast<const E *>(p.q) + head;
    const E *K = static_cast<const E *>(p.k) + head;
    const E *V = static_cast<const E *>(p.v) + head;
    const E *DO = static_cast<const E *>(p.dout) + head;
    const float *LSE = p.lse_in + (int64_t)bh * n;
    const float *DEL = p.delta + (int64_t)bh * n;
    const float sl2 = p.scale_log2;

    // =========================== dQ of query rows ===========================
    {
        const int i = r0 + c16;
        const bool row_ok = i < n;
        const int ic = row_ok ? i : n - 1;
        Frag<BF16> qf, df;
        load_frag(qf, Q, ic, g);
        load_frag(df, DO, ic, g);
        const float lse2 = LSE[ic] * kLog2e;
        const float di = DEL[ic];
        f32x4_t acc[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        const int jlo = max(0, t0 - w + 1), jhi = min(n - 1, t0 + 63);
        const int wlo = r0 - w + 1, whi = min(r0 + 15, n - 1);
        for (int c0 = jlo & ~63; c0 <= jhi; c0 += 64) {
            __syncthreads();
            stage_tile<64, BF16>(t0s, kT64, K, c0, n, tid);
            __syncthreads();
            if (r0 >= n) continue;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int kb0 = c0 + 16 * kb;
                if (kb0 + 15 < wlo || kb0 > whi) continue;
                Frag<BF16> kf, vf;
                const int jr = min(kb0 + c16, n - 1);
                load_frag(kf, K, jr, g);
                load_frag(vf, V, jr, g);
                const f32x4_t st = mma_over_d(kf, qf, f32x4_t{0.f, 0.f, 0.f, 0.f});
                const f32x4_t dpt = mma_over_d(vf, df, f32x4_t{0.f, 0.f, 0.f, 0.f});
                float ds[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = kb0 + 4 * g + r;
                    const bool ok = row_ok && j <= i && j > i - w;
                    const float pv = ok ? fast_exp2(__builtin_fmaf(st[r], sl2, -lse2)) : 0.f;
                    ds[r] = pv * (dpt[r] - di);
                }
                mma_over_rows_exact(acc, t0s, kT64, 16 * kb, c16, g, ds);
            }
        }
        if (r0 < n) {
            for (int t = 0; t < p.n_off; ++t) {
                const int o = p.off[t];
                if (r0 + 15 < o) break;
                const int j = i - o;
                const bool ok = row_ok && j >= 0;
                const int jc = min(max(j, 0), n - 1);
                Frag<BF16> kf, vf;
                load_frag(kf, K, jc, g);
                load_frag(vf, V, jc, g);
                const float s = group_sum(frag_dot(qf, kf));
                const float dp = group_sum(frag_dot(df, vf));
                const float pv = ok ? fast_exp2(__builtin_fmaf(s, sl2, -lse2)) : 0.f;
                frag_axpy(acc, pv * (dp - di), kf);
            }
        }
        if (row_ok) store_row(static_cast<OE *>(p.dq) + head, i, g, acc, p.scale);
    }

    // ========================= dK, dV of key rows ==========================
    {
        const int j = r0 + c16;  // this lane's key row
        const bool key_ok = j < n;
        const int jc = key_ok ? j : n - 1;
        Frag<BF16> kf, vf;
        load_frag(kf, K, jc, g);
        load_frag(vf, V, jc, g);
        f32x4_t dk[4], dv[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            dk[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            dv[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        // window: queries i in [j, j + w - 1]
        const int ihi_wg = (int)min((int64_t)n - 1, (int64_t)t0 + 63 + w - 1);
        const int ilo = r0, ihi = (int)min((int64_t)n - 1, (int64_t)r0 + 15 + w - 1);
        for (int c0 = t0; c0 <= ihi_wg; c0 += 64) {
            __syncthreads();
            stage_tile<64, BF16>(t0s, kT64, Q, c0, n, tid);
            stage_tile<64, BF16>(t1s, kT64, DO, c0, n, tid);
            if (tid < 64) {
                const int row = c0 + tid;
                lse_s[tid] = (row < n) ? LSE[row] * kLog2e : 0.f;
                del_s[tid] = (row < n) ? DEL[row] : 0.f;
            }
            __syncthreads();
            if (r0 >= n) continue;
#pragma unroll
            for (int qb = 0; qb < 4; ++qb) {
                const int qb0 = c0 + 16 * qb;
                if (qb0 + 15 < ilo || qb0 > ihi) continue;
                Frag<BF16> qf, df;
                const int ir = min(qb0 + c16, n - 1);
                load_frag(qf, Q, ir, g);
                load_frag(df, DO, ir, g);
                const f32x4_t sq = mma_over_d(qf, kf, f32x4_t{0.f, 0.f, 0.f, 0.f});  // rows: queries
                const f32x4_t dpq = mma_over_d(df, vf, f32x4_t{0.f, 0.f, 0.f, 0.f});
                float pr[4], ds[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int qi = 16 * qb + 4 * g + r;  // row within the chunk
                    const int iq = c0 + qi;
                    const bool ok = key_ok && iq < n && iq >= j && iq - j < w;
                    pr[r] = ok ? fast_exp2(__builtin_fmaf(sq[r], sl2, -lse_s[qi])) : 0.f;
                    ds[r] = pr[r] * (dpq[r] - del_s[qi]);
                }
                mma_over_rows_exact(dv, t1s, kT64, 16 * qb, c16, g, pr);
                mma_over_rows_exact(dk, t0s, kT64, 16 * qb, c16, g, ds);
            }
        }
        // sparse offsets: queries i = j + o
        if (r0 < n) {
            for (int t = 0; t < p.n_off; ++t) {
                const int o = p.off[t];
                if (r0 + o >= n) break;  // ascending offsets: no query row left
                const int iq = j + o;
                const bool ok = key_ok && iq < n;
                const int ic = ok ? iq : n - 1;
                Frag<BF16> qf, df;
                load_frag(qf, Q, ic, g);
                load_frag(df, DO, ic, g);
                const float s = group_sum(frag_dot(qf, kf));
                const float dp = group_sum(frag_dot(df, vf));
                const float pv = ok ? fast_exp2(__builtin_fmaf(s, sl2, -(LSE[ic] * kLog2e))) : 0.f;
                const float dsv = pv * (dp - DEL[ic]);
                frag_axpy(dv, pv, df);
                frag_axpy(dk, dsv, qf);
            }
        }
        if (key_ok) {
            store_row(static_cast<OE *>(p.dk) + head, j, g, dk, p.scale);
            store_row(static_cast<OE *>(p.dv) + head, j, g, dv, 1.f);
        }
    }
}

// Backward on the window path (bf16 inputs, w <= 64) runs as two kernels over 64-row
// tiles. The first forms dQ of its query rows and, for every sparse pair (query i,
// key i - off[t]), stores P and dS rounded to bf16 (the weights the gradient products
// use) in a pair workspace [BH, N, S] of 32-bit words (P in the low half). The
// second forms dK and dV of its key rows from the window band, recomputed on MFMA, and
// from the stored weights of the sparse pairs (key j, query j + off[t]), so no score is
// formed twice on the vector units. Each kernel keeps one pair of operands resident
// (K, V for dQ; Q, dO for dK and dV), which halves the data an XCD's L2 has to hold.

constexpr int kRingQ = 4, kPreQ = 2;    // dQ kernel: slab slots in the ring; slots requested before the band
constexpr int kRingKV = 3, kPreKV = 1;  // dK/dV kernel

// ---- one-launch backward: per-tile completion tokens ----
//
// A token names one launch: the dispatch id (the packet's index in its queue, which
// grows by one per dispatch) mixed with the queue's address (each queue counts from
// zero). The dQ work of a tile writes it to that tile's flag; a workspace's earlier
// contents, earlier launches' tokens included, do not match it.
extern "C" __device__ uint64_t fsa_dispatch_id() __asm("llvm.amdgcn.dispatch.id");
__device__ __forceinline__ uint64_t launch_token() {
    const uint64_t q = reinterpret_cast<uint64_t>(__builtin_amdgcn_queue_ptr());
    return fsa_dispatch_id() ^ (q * 0x9E3779B97F4A7C15ull);
}

// Cache policy (sc0) for the pair words and D that another workgroup of the same launch
// wrote, in the same XCD's L2. No CU reads them before their token is set, so no L1
// holds an older copy.
constexpr int kCachePastL1 = 1;

// Polls before giving up; with the sleep below they span tens of milliseconds, far
// beyond any real wait (the dQ work of a whole launch takes tens of microseconds).
constexpr int kMaxSpins = 1 << 18;

// Waits until flags[first .. last] all hold the token (one wave; lane l checks flags
// first + l, first + l + 64, ...; device-scope loads, which miss this CU's L1). Each
// poll requests up to 64 * BATCH flags before comparing any, so that it costs one
// round trip for up to that many tiles. Returns false, uniformly over the wave, if it
// gave up; the caller then stores NaN so that the failure shows.
template <int BATCH = 1>
__device__ __forceinline__ bool poll_tiles(const uint64_t *flags, int first, int last, uint64_t token, int lane) {
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
            for (int k = 0; k < BATCH; ++k) ready &= (base + 64 * k > last) | (v[k] == token);
        }
        if (__builtin_amdgcn_ballot_w64(!ready) == 0) return true;
        if (spin == kMaxSpins) return false;
        __builtin_amdgcn_s_sleep(4);
    }
}

// Descriptor over the pair-workspace words of head bh ([N, S] words, S = pair_slots):
// rows past the sequence end read as zero words.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pair_rsrc(const AttnParams &p, int n_off, int bh) {
    const int slots = pair_slots(n_off);
    return head_rsrc(p.pairs + (int64_t)bh * p.n * slots, span_bytes(p.n, 4u * slots));
}

// dQ of query rows [t0, t0 + 64): the band keys [t0 - 64, t0 + 64) (K, V in LDS) on
// MFMA first, then the slab keys i - off[t] in the slab layout through a register ring,
// storing each sparse pair's P and dS on the way. With WITH_D the kernel also forms
// D = rowsum(dO * O) of its rows from O (instead of reading it) and stores it for the
// dK/dV kernel.
//
// With FRAC (fractional entries, WITH_D) each entry's key and value mix the near row
// i - off[t] and the far row i - off[t] - 1 with weights 1 - phi and phi. The kernel
// stores two words per pair, the near and the far share of P and dS, and adds up, per
// entry, the derivative of the loss with respect to the entry's distance over its rows
// (one partial per workgroup and entry; see reduce_alpha_grad).
//
// The body works on logical tile lb with the caller's LDS: ta, tb (band K and V rows,
// kTileRows * 64 each, then merge areas), d_s (64 floats: D of the tile's rows, WITH_D)
// and dd_s (4 * FSA_MAX_OFFSETS floats, FRAC).
template <bool OUT_BF16, bool WITH_D, bool FRAC, int NOFF = 0, bool PUBLISH = false>
__device__ __forceinline__ void dq_tile(const AttnParams &p, const int lb, uint16_t *ta, uint16_t *tb, float *d_s,
                                        float *dd_s) {
    static_assert(!FRAC || WITH_D, "the fractional backward forms D in the dQ kernel");
    using OE = typename Elem<OUT_BF16>::T;

    const int n = p.n, w = p.w, n_off = NOFF > 0 ? NOFF : p.n_off;
    const int nt = (n + 63) >> 6;
    const int bh = lb / nt, tile = lb - bh * nt;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c16 = lane & 15, g = lane >> 4;  // MFMA layout
    const TileLanes tl = tile_lanes(c16, g);
    const uint16_t *ta_w = ta + 1024 * wave, *tb_w = tb + 1024 * wave;  // this wave's band rows start here
    const int s8 = lane >> 3, c8 = lane & 7;   // slab layout
    const int t0 = tile * 64, r0 = t0 + 16 * wave;
    const int row_s[2] = {r0 + s8, r0 + 8 + s8};
    const int i = r0 + c16;  // MFMA-layout query row
    const bool i_ok = i < n;
    const int64_t head = (int64_t)bh * n * 64;
    const uint16_t *Q = static_cast<const uint16_t *>(p.q) + head;
    const uint16_t *K = static_cast<const uint16_t *>(p.k) + head;
    const uint16_t *V = static_cast<const uint16_t *>(p.v) + head;
    const uint16_t *DO = static_cast<const uint16_t *>(p.dout) + head;
    const __amdgpu_buffer_rsrc_t rq = head_rsrc(Q, span_bytes(n, 128)), rk = head_rsrc(K, span_bytes(n, 128));
    const __amdgpu_buffer_rsrc_t rv = head_rsrc(V, span_bytes(n, 128)), rdo = head_rsrc(DO, span_bytes(n, 128));
    const __amdgpu_buffer_rsrc_t rl = head_rsrc(p.lse_in + (int64_t)bh * n, span_bytes(n, 4));
    const __amdgpu_buffer_rsrc_t rd = head_rsrc(p.delta + (int64_t)bh * n, span_bytes(n, 4));
    const float sl2 = p.scale_log2;

    dma_tile(ta, K, t0 - 64, n, wave, lane);
    dma_tile(tb, V, t0 - 64, n, wave, lane);
    Frag<true> qf, df;
    buf_frag(qf, rq, i, g);
    buf_frag(df, rdo, i, g);
    const float lse2_i = buf_f32(rl, i) * kLog2e;
    float di[2];  // D of the slab-layout rows
    if constexpr (WITH_D) {
        // D from the slab layout (whole rows per load); the band reads it back from LDS
        SFrag dos, os;
        sfrag_load(dos, rdo, row_s[0], row_s[1], c8);
        sfrag_load<kCacheNT>(os, head_rsrc(static_cast<const uint16_t *>(p.o) + head, span_bytes(n, 128)), row_s[0], row_s[1], c8);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            di[h] = row8_sum(chunk_dot(dos.r[h], os.r[h]));
            if (c8 == 0) {
                d_s[16 * wave + s8 + 8 * h] = di[h];
                if (row_s[h] < n) p.delta[(int64_t)bh * n + row_s[h]] = di[h];
            }
        }
    } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) di[h] = buf_f32(rd, row_s[h]);
    }
    wait_vm_all();
    __syncthreads();
    const float di_i = WITH_D ? d_s[16 * wave + c16] : buf_f32(rd, i);

    // the first slab rows land while the band runs
    SFrag sk[kRingQ], sv[kRingQ];  // FRAC: entry slot u holds near rows in [2u], far rows in [2u + 1]
    auto fill = [&](int u, int t) {
        sfrag_load(sk[u], rk, slab_row(p, n_off, t, row_s[0], -1), slab_row(p, n_off, t, row_s[1], -1), c8);
        sfrag_load(sv[u], rv, slab_row(p, n_off, t, row_s[0], -1), slab_row(p, n_off, t, row_s[1], -1), c8);
    };
    // FRAC: K rows of two entries in flight (slot u: near rows in sk[2u], far rows in
    // sk[2u + 1]), V rows of one (sv[0] near, sv[1] far), requested as soon as the
    // previous entry's V rows have been used
    auto frac_load_k = [&](int u, int t) {
        const int n0 = slab_row(p, n_off, t, row_s[0], -1), n1 = slab_row(p, n_off, t, row_s[1], -1);
        sfrag_load(sk[2 * u], rk, n0, n1, c8);
        sfrag_load(sk[2 * u + 1], rk, n0 - 1, n1 - 1, c8);
    };
    auto frac_load_v = [&](int t) {
        const int n0 = slab_row(p, n_off, t, row_s[0], -1), n1 = slab_row(p, n_off, t, row_s[1], -1);
        sfrag_load(sv[0], rv, n0, n1, c8);
        sfrag_load(sv[1], rv, n0 - 1, n1 - 1, c8);
    };
    if constexpr (FRAC) {
        frac_load_k(0, 0);
        frac_load_v(0);
        if (threadIdx.x < 4 * FSA_MAX_OFFSETS) dd_s[threadIdx.x] = 0.f;  // read after the last barrier
    } else {
#pragma unroll
        for (int u = 0; u < kPreQ; ++u)
            if (u < n_off) fill(u, u);  // uniform
    }

    // band on MFMA: query row i sees key blocks qb-4 .. qb (blocks outside the sequence
    // or the window are masked like edge blocks: their tile rows hold finite values)
    f32x4_t acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int qb = r0 >> 4;
    auto block_ds = [&](int b, float ds[4]) {
        const int kb0 = 16 * (qb - 4 + b);
        const bool full = kb0 >= 0 && kb0 + 15 <= r0 && kb0 >= r0 + 16 - w && r0 + 15 < n;
        Frag<true> kf, vf;
        lds_frag(kf, ta_w, 16 * b, tl);
        lds_frag(vf, tb_w, 16 * b, tl);
        const f32x4_t st = mma_over_d(kf, qf, f32x4_t{0.f, 0.f, 0.f, 0.f});
        const f32x4_t dpt = mma_over_d(vf, df, f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int r = 0; r < 4; ++r) ds[r] = fast_exp2(__builtin_fmaf(st[r], sl2, -lse2_i)) * (dpt[r] - di_i);
        if (!full) {  // uniform: edge blocks only
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = kb0 + 4 * g + r;
                if (!(i_ok && j <= i && j > i - w && j >= 0)) ds[r] = 0.f;
            }
        }
    };
    {
        float d0[4], d1[4];
        // the band's dS weights go in as bf16 high part plus remainder (see bwd_dkdv_kernel)
        block_ds(0, d0);
        block_ds(1, d1);
        mma_over_rows_tr2_exact(acc, ta_w, 0, 16, tl, d0, d1);
        block_ds(2, d0);
        block_ds(3, d1);
        mma_over_rows_tr2_exact(acc, ta_w, 32, 48, tl, d0, d1);
        block_ds(4, d0);
        mma_over_rows_tr_exact(acc, ta_w, 64, tl, d0);
    }
    if constexpr (FRAC) {
        frac_load_k(1, 1);
    } else {
#pragma unroll
        for (int u = kPreQ; u < kRingQ; ++u)
            if (u < n_off) fill(u, u);  // uniform
    }
    __syncthreads();  // every wave is done with the band tiles
    f32x4_t dq_s[2][2];
    c_to_slab(reinterpret_cast<float *>(ta) + wave * 1024, acc, dq_s, c16, g, s8, c8);

    // sparse offsets: keys i - o, in the slab layout
    SFrag qs, dos;
    sfrag_load<kCacheNT>(qs, rq, row_s[0], row_s[1], c8);  // second and last read of these rows
    sfrag_load<kCacheNT>(dos, rdo, row_s[0], row_s[1], c8);
    float lse2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) lse2[h] = buf_f32(rl, row_s[h]) * kLog2e;
    // pair words of this head's rows: [n, slots]; lane c8 of a row keeps the word of
    // slot c8 of the unrolled part and the eight lanes store them with one 32-byte write
    const int slots = pair_slots(n_off);
    uint32_t *pairs = p.pairs + (int64_t)bh * n * slots;
    if constexpr (FRAC) {
        // pair words [n, slots, 2]: the near word {(1 - phi) P, (1 - phi) dS} and the far
        // word {phi P, phi dS} of every entry, each rounded once to bf16, stored by the lane
        // c8 = t mod 8 of each row
        uint2 *pairs2 = reinterpret_cast<uint2 *>(p.pairs) + (int64_t)bh * n * slots;
        auto entry = [&](int t, const SFrag &kn, const SFrag &kf) {
            const int a = p.off[t], first = table_first(p, t);
            const float ph = table_phi(p, t);
            float pn[2], pd[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                pn[h] = row8_sum(chunk_dot(dos.r[h], sv[0].r[h]));
                pd[h] = row8_sum(chunk_dot(dos.r[h], sv[1].r[h])) - pn[h];
            }
            if (t + 1 < n_off) frac_load_v(t + 1);  // uniform
            float ddl = 0.f;  // this lane's rows' share of d(loss)/d(d_t)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row = row_s[h];
                const bool ok = (row < n) & (row >= first);
                const float sn = row8_sum(chunk_dot(qs.r[h], kn.r[h]));
                const float sd = row8_sum(chunk_dot(qs.r[h], kf.r[h])) - sn;
                const float sc = __builtin_fmaf(ph, sd, sn), dp = __builtin_fmaf(ph, pd[h], pn[h]);
                const float pv = ok ? fast_exp2(__builtin_fmaf(sc, sl2, -lse2[h])) : 0.f;
                const float ds = pv * (dp - di[h]);
                const float pf = pv * ph, dsf = ds * ph;
                const uint2 pw = {pack_bf16(pv - pf, ds - dsf), pack_bf16(pf, dsf)};
                if (c8 == (t & 7) && row < n) pairs2[(int64_t)row * slots + t] = pw;
                chunk_axpy_words(dq_s[h], pw.x >> 16, pw.x & 0xffff0000u, kn.r[h]);
                chunk_axpy_words(dq_s[h], pw.y >> 16, pw.y & 0xffff0000u, kf.r[h]);
                // moving the target distance moves the key and value along far - near
                // (the piece [a, a + 1)); rows without the far row contribute nothing
                if (ok & (row - a - 1 >= 0)) ddl += __builtin_fmaf(p.scale * ds, sd, pv * pd[h]);
            }
            // wave total: the eight lanes of a row hold the same value, so sum over rows
            const float tot = group_sum(xor8_add(ddl));
            if (lane == 0) dd_s[wave * FSA_MAX_OFFSETS + t] = tot;
        };
        for (int t0 = 0; t0 < n_off; t0 += 2) {
            if (r0 + 15 < p.off[t0]) break;  // ascending entries: no row of the wave has one
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (t0 + u < n_off) entry(t0 + u, sk[2 * u], sk[2 * u + 1]);  // uniform
                if (t0 + u + 2 < n_off) frac_load_k(u, t0 + u + 2);         // uniform
            }
        }
    } else {
        uint32_t keep[2] = {0u, 0u};
        auto slab = [&](int t, int o, const SFrag &kt, const SFrag &vt) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bool ok = (row_s[h] < n) & (row_s[h] - o >= 0);
                const float s = row8_sum(chunk_dot(qs.r[h], kt.r[h]));
                const float dp = row8_sum(chunk_dot(dos.r[h], vt.r[h]));
                const float pv = ok ? fast_exp2(__builtin_fmaf(s, sl2, -lse2[h])) : 0.f;
                const uint32_t pw = pack_bf16(pv, pv * (dp - di[h]));
                if (t < 8)
                    keep[h] = c8 == t ? pw : keep[h];
                else if (c8 == 0 && row_s[h] < n)
                    pairs[(int64_t)row_s[h] * slots + t] = pw;
                chunk_axpy_words(dq_s[h], pw >> 16, pw & 0xffff0000u, kt.r[h]);
            }
        };
#pragma unroll
        for (int s0 = 0; s0 < unrolled_slabs(kRingQ); s0 += kRingQ) {
            if (s0 >= n_off || r0 + 15 < p.off[s0]) break;  // ascending offsets: no key left
#pragma unroll
            for (int u = 0; u < kRingQ; ++u) {
                if (s0 + u < n_off) slab(s0 + u, table_off(p, n_off, s0 + u), sk[u], sv[u]);  // uniform
                if (s0 + u + kRingQ < min(n_off, unrolled_slabs(kRingQ))) fill(u, s0 + u + kRingQ);  // uniform
            }
        }
        static_assert(unrolled_slabs(kRingQ) == 8, "the kept pair words cover slots 0..7");
        if (n_off > 0) {  // uniform
#pragma unroll
            for (int h = 0; h < 2; ++h)
                if (row_s[h] < n) pairs[(int64_t)row_s[h] * slots + c8] = keep[h];
        }
        for (int t = unrolled_slabs(kRingQ); t < n_off; ++t) {  // longer tables
            if (r0 + 15 < p.off[t]) break;
            fill(0, t);
            slab(t, p.off[t], sk[0], sv[0]);
        }
    }
    if (p.rope) {  // uniform: gradients with respect to the unrotated rows
#pragma unroll
        for (int h = 0; h < 2; ++h)
            if (row_s[h] < n) rope_back_chunk(p.rope, row_s[h], c8, dq_s[h]);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
        if (row_s[h] < n) store_chunk<true>(static_cast<OE *>(p.dq) + head, row_s[h], c8, dq_s[h], p.scale);
    if constexpr (FRAC) {  // partials [n_off, tiles]: entry t's partials are contiguous
        __syncthreads();
        const int t = threadIdx.x;
        if (t < n_off) {
            const float part = (dd_s[t] + dd_s[FSA_MAX_OFFSETS + t]) +
                               (dd_s[2 * FSA_MAX_OFFSETS + t] + dd_s[3 * FSA_MAX_OFFSETS + t]);
            float *dst = p.dd_part + (int64_t)t * (p.bh * nt) + lb;
            if constexpr (PUBLISH)  // read in the same launch, possibly from another XCD
                __hip_atomic_store(dst, part, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
                *dst = part;
        }
    }
}

template <bool OUT_BF16, bool WITH_D, bool FRAC>
__global__ void __launch_bounds__(kThreads) bwd_dq_kernel(const AttnParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t ta[kTileRows * 64];
    __shared__ __attribute__((aligned(16))) uint16_t tb[kTileRows * 64];
    __shared__ float d_s[64];
    __shared__ float dd_s[FRAC ? 4 * FSA_MAX_OFFSETS : 1];
    dq_tile<OUT_BF16, WITH_D, FRAC>(p, xcd_logical_block(blockIdx.x, p.bh * ((p.n + 63) >> 6)), ta, tb, d_s, dd_s);
}

// Alpha gradient of the fractional backward, run by one whole workgroup: d(loss)/d(d_t)
// is the sum of the dQ kernel's per-tile partials of entry t, and d(loss)/d(alpha) =
// sum_t fbase[t] * d(loss)/d(d_t), since every target distance is alpha times its base
// value. Wave v sums entries v, v + 4, ... (lanes stride over the tiles, fp64), then one
// thread forms the outputs in entry order: a fixed order, so the result is reproducible.
// Entries that no row reaches (trimmed from the table) get 0. `red` holds 48 doubles.
template <bool SAME_LAUNCH = false>
__device__ void reduce_alpha_grad(const AttnParams &p, double *red) {
    const int n_tiles = p.bh * ((p.n + 63) >> 6);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int t = wave; t < p.n_off; t += kThreads / 64) {
        const float *part = p.dd_part + (int64_t)t * n_tiles;
        double x = 0.0;
        for (int i = lane; i < n_tiles; i += 64)
            x += SAME_LAUNCH ? __hip_atomic_load(part + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : part[i];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
        if (lane == 0) red[t] = x;
    }
    __syncthreads();
    if (tid == 0) {
        double ga = 0.0;
        for (int t = 0; t < p.n_entries; ++t) {
            const double tot = t < p.n_off ? red[t] : 0.0;
            if (p.doffs) p.doffs[t] = static_cast<float>(tot);
            ga += static_cast<double>(p.fbase[t]) * tot;
        }
        p.dalpha[0] = static_cast<float>(ga);
    }
}

// dK, dV of key rows [t0, t0 + 64): the band queries [t0, t0 + 128) (Q, dO, LSE, D in
// LDS) on MFMA first, then the slab queries j + off[t] in the slab layout with the
// pair weights that bwd_dq_kernel stored.
//
// With FRAC, key row j receives entry t from two queries: j + off[t], whose key mixes
// row j with weight 1 - phi (its near word), and j + off[t] + 1, whose key mixes row j
// with weight phi (its far word).
//
// The body works on logical tile lb with the caller's LDS: ta, tb (band Q and dO rows,
// then merge areas), lse_s and del_s (log2-scaled LSE and D of the band queries,
// kTileRows floats each). With FUSED the dQ work of the same call runs in the same
// launch (bwd_fused_kernel): D and the pair words are read only once the tiles that
// write them have published this launch's token (poll_tiles, while the band rows load).
// FROM_DQ: D comes from that dQ work (otherwise the caller gave it).
template <bool OUT_BF16, bool FRAC, bool FUSED = false, bool FROM_DQ = false, int NOFF = 0>
__device__ __forceinline__ void dkdv_tile(const AttnParams &p, const int lb, uint16_t *ta, uint16_t *tb, float *lse_s,
                                          float *del_s, [[maybe_unused]] const uint64_t token = 0) {
    static_assert(FUSED || !FROM_DQ, "D comes from the same launch only in the one-launch backward");
    using OE = typename Elem<OUT_BF16>::T;

    const int n = p.n, w = p.w, n_off = NOFF > 0 ? NOFF : p.n_off;
    const int nt = (n + 63) >> 6;
    const int bh = lb / nt, tile = lb - bh * nt;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15, g = lane >> 4;  // MFMA layout
    const TileLanes tl = tile_lanes(c16, g);
    const uint16_t *ta_w = ta + 1024 * wave, *tb_w = tb + 1024 * wave;  // this wave's band rows start here
    const int s8 = lane >> 3, c8 = lane & 7;   // slab layout
    const int t0 = tile * 64, r0 = t0 + 16 * wave;
    const int row_s[2] = {r0 + s8, r0 + 8 + s8};
    const int j = r0 + c16;  // MFMA-layout key row
    const bool j_ok = j < n;
    const int64_t head = (int64_t)bh * n * 64;
    const uint16_t *Q = static_cast<const uint16_t *>(p.q) + head;
    const uint16_t *K = static_cast<const uint16_t *>(p.k) + head;
    const uint16_t *V = static_cast<const uint16_t *>(p.v) + head;
    const uint16_t *DO = static_cast<const uint16_t *>(p.dout) + head;
    const float *LSE = p.lse_in + (int64_t)bh * n;
    const float *DEL = p.delta + (int64_t)bh * n;
    const __amdgpu_buffer_rsrc_t rq = head_rsrc(Q, span_bytes(n, 128)), rk = head_rsrc(K, span_bytes(n, 128));
    const __amdgpu_buffer_rsrc_t rv = head_rsrc(V, span_bytes(n, 128)), rdo = head_rsrc(DO, span_bytes(n, 128));
    const float sl2 = p.scale_log2;

    dma_tile(ta, Q, t0, n, wave, lane);
    dma_tile(tb, DO, t0, n, wave, lane);
    if (tid < kTileRows) {
        const int row = t0 + tid;
        lse_s[tid] = (row < n) ? LSE[row] * kLog2e : 0.f;
        if constexpr (!FROM_DQ) del_s[tid] = (row < n) ? DEL[row] : 0.f;
    }
    Frag<true> kf, vf;
    buf_frag<kCacheNT>(kf, rk, j, g);  // read once by this kernel
    buf_frag<kCacheNT>(vf, rv, j, g);
    // scales of the stored dK and dV: NaN if the wait below gave up, so that it shows
    float k_mul = p.scale, v_mul = 1.f;
    if constexpr (FUSED) {
        // D of the band queries (tiles tile and tile + 1) and the pair words of the slab
        // queries (up to row + max offset) come from this launch's dQ work: wait for
        // those tiles while the band rows are in flight
        __shared__ int gave_up;
        if (wave == 0) {
            const int far = n_off > 0 ? t0 + 63 + p.off[n_off - 1] + (FRAC ? 1 : 0) : t0;
            const int last = min(nt - 1, max(FROM_DQ ? tile + 1 : tile, far >> 6));
            const bool ok = poll_tiles(p.flags + (int64_t)bh * nt, tile, last, token, lane);
            if (lane == 0) gave_up = ok ? 0 : 1;
        }
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(gave_up)) {
            k_mul = __builtin_nanf("");
            v_mul = k_mul;
        }
        if constexpr (FROM_DQ) {
            if (tid < kTileRows) {
                const int row = t0 + tid;
                del_s[tid] = (row < n) ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                             head_rsrc(DEL, span_bytes(n, 4)), row * 4, 0, kCachePastL1))
                                       : 0.f;
            }
        }
        wait_vm_all();
        __syncthreads();
    } else {
        wait_vm_all();
        __syncthreads();
    }

    // slot u: query rows row + off[t] (Q, dO) and their pair weights (word t of each row)
    // slot u of the ring. FRAC: the ring runs over half entries, 2t (the near queries
    // j + off[t] with their near words) and 2t + 1 (the far queries j + off[t] + 1 with
    // their far words)
    SFrag sq[kRingKV], sd[kRingKV];
    uint32_t pw[kRingKV][2];
    const int slots = pair_slots(n_off);
    const __amdgpu_buffer_rsrc_t rp =
        FRAC ? head_rsrc(p.pairs + (int64_t)bh * n * slots * 2, span_bytes(n, 8u * slots)) : pair_rsrc(p, n_off, bh);
    auto fill_words = [&](int u, int x) {
        const int t = FRAC ? x >> 1 : x, far = FRAC ? x & 1 : 0;
        const int iq0 = slab_row(p, n_off, t, row_s[0], 1) + far, iq1 = slab_row(p, n_off, t, row_s[1], 1) + far;
        if constexpr (FRAC) {
            pw[u][0] = __builtin_amdgcn_raw_buffer_load_b32(rp, ((iq0 * slots + t) * 2 + far) * 4, 0,
                                                            FUSED ? kCachePastL1 : 0);
            pw[u][1] = __builtin_amdgcn_raw_buffer_load_b32(rp, ((iq1 * slots + t) * 2 + far) * 4, 0,
                                                            FUSED ? kCachePastL1 : 0);
        } else {
            pw[u][0] = __builtin_amdgcn_raw_buffer_load_b32(rp, (iq0 * slots + t) * 4, 0, FUSED ? kCachePastL1 : 0);
            pw[u][1] = __builtin_amdgcn_raw_buffer_load_b32(rp, (iq1 * slots + t) * 4, 0, FUSED ? kCachePastL1 : 0);
        }
    };
    auto fill_rows = [&](int u, int x) {
        const int t = FRAC ? x >> 1 : x, far = FRAC ? x & 1 : 0;
        const int iq0 = slab_row(p, n_off, t, row_s[0], 1) + far, iq1 = slab_row(p, n_off, t, row_s[1], 1) + far;
        sfrag_load(sq[u], rq, iq0, iq1, c8);
        sfrag_load(sd[u], rdo, iq0, iq1, c8);
    };
    auto fill = [&](int u, int x) {
        fill_rows(u, x);
        fill_words(u, x);
    };
#pragma unroll
    for (int u = 0; u < kPreKV; ++u)
        if (u < (FRAC ? 2 * n_off : n_off)) fill(u, u);  // uniform; FRAC: half entries

    // band on MFMA: key row j sees query blocks r0 + 16 b (blocks past the sequence or
    // the window are masked like edge blocks)
    f32x4_t dk[4], dv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        dk[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        dv[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    auto block_pds = [&](int b, float pr[4], float ds[4]) {
        const int qb0 = r0 + 16 * b;
        const bool full = qb0 >= r0 + 15 && qb0 + 15 <= r0 + w - 1 && qb0 + 15 < n && r0 + 15 < n;
        const int lr = 16 * b;  // band rows of this block, relative to the wave's first
        Frag<true> qf, df;
        lds_frag(qf, ta_w, lr, tl);
        lds_frag(df, tb_w, lr, tl);
        const f32x4_t sq4 = mma_over_d(qf, kf, f32x4_t{0.f, 0.f, 0.f, 0.f});  // rows: queries
        const f32x4_t dp4 = mma_over_d(df, vf, f32x4_t{0.f, 0.f, 0.f, 0.f});
        const f32x4_t l4 = *reinterpret_cast<const f32x4_t *>(lse_s + 16 * wave + lr + 4 * g);
        const f32x4_t d4 = *reinterpret_cast<const f32x4_t *>(del_s + 16 * wave + lr + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(__builtin_fmaf(sq4[r], sl2, -l4[r]));
        if (!full) {  // uniform: edge blocks only
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int q = qb0 + 4 * g + r;
                if (!(j_ok && q < n && q >= j && q - j < w)) pr[r] = 0.f;
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) ds[r] = pr[r] * (dp4[r] - d4[r]);
    };
    {
        float p0[4], s0[4], p1[4], s1[4];
        block_pds(0, p0, s0);
        block_pds(1, p1, s1);
        // dV = sum_i P_ij dO_i and dK = sum_i dS_ij q_i are unnormalised sums that reach
        // several units at early keys, where the band's weights are large: the weights go
        // in as bf16 high part plus remainder
        mma_over_rows_tr2_exact(dv, tb_w, 0, 16, tl, p0, p1);
        mma_over_rows_tr2_exact(dk, ta_w, 0, 16, tl, s0, s1);
        block_pds(2, p0, s0);
        block_pds(3, p1, s1);
        mma_over_rows_tr2_exact(dv, tb_w, 32, 48, tl, p0, p1);
        mma_over_rows_tr2_exact(dk, ta_w, 32, 48, tl, s0, s1);
        block_pds(4, p0, s0);
        mma_over_rows_tr_exact(dv, tb_w, 64, tl, p0);
        mma_over_rows_tr_exact(dk, ta_w, 64, tl, s0);
    }
#pragma unroll
    for (int u = kPreKV; u < kRingKV; ++u)
        if (u < (FRAC ? 2 * n_off : n_off)) fill(u, u);  // uniform; FRAC: half entries
    __syncthreads();  // every wave is done with the band tiles
    f32x4_t dk_s[2][2], dv_s[2][2];
    c_to_slab(reinterpret_cast<float *>(ta) + wave * 1024, dk, dk_s, c16, g, s8, c8);
    c_to_slab(reinterpret_cast<float *>(tb) + wave * 1024, dv, dv_s, c16, g, s8, c8);

    // sparse offsets: queries j + o, weights P (low half) and dS (high half) as stored;
    // pairs past the sequence end read as zero words
    auto slab = [&](const uint32_t pwt[2], const SFrag &qt, const SFrag &dt) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t x = pwt[h];
            chunk_axpy_words(dv_s[h], x & 0xffffu, x << 16, dt.r[h]);
            chunk_axpy_words(dk_s[h], x >> 16, x & 0xffff0000u, qt.r[h]);
        }
    };
    if constexpr (FRAC) {
        const int n_half = 2 * n_off;
        for (int x0 = 0; x0 < n_half; x0 += kRingKV) {
            if (r0 + p.off[x0 >> 1] >= n) break;  // ascending entries: no query row left
#pragma unroll
            for (int u = 0; u < kRingKV; ++u) {
                if (x0 + u < n_half) slab(pw[u], sq[u], sd[u]);          // uniform
                if (x0 + u + kRingKV < n_half) fill(u, x0 + u + kRingKV);  // uniform
            }
        }
    } else {
#pragma unroll
        for (int s0 = 0; s0 < unrolled_slabs(kRingKV); s0 += kRingKV) {
            if (s0 >= n_off || r0 + p.off[s0] >= n) break;  // ascending offsets: no query row left
#pragma unroll
            for (int u = 0; u < kRingKV; ++u) {
                if (s0 + u < n_off) slab(pw[u], sq[u], sd[u]);  // uniform
                if (s0 + u + kRingKV < min(n_off, unrolled_slabs(kRingKV))) fill(u, s0 + u + kRingKV);  // uniform
            }
        }
        for (int t = unrolled_slabs(kRingKV); t < n_off; ++t) {  // longer tables
            if (r0 + p.off[t] >= n) break;
            fill(0, t);
            slab(pw[0], sq[0], sd[0]);
        }
    }
    if (p.rope) {  // uniform: gradients with respect to the unrotated rows
#pragma unroll
        for (int h = 0; h < 2; ++h)
            if (row_s[h] < n) rope_back_chunk(p.rope, row_s[h], c8, dk_s[h]);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (row_s[h] < n) {
            store_chunk<true>(static_cast<OE *>(p.dk) + head, row_s[h], c8, dk_s[h], k_mul);
            store_chunk<true>(static_cast<OE *>(p.dv) + head, row_s[h], c8, dv_s[h], v_mul);
        }
    }
    // FRAC: the dQ kernel, which ran before this one on the stream, left the alpha
    // gradient's partials; the last tile of head 0, whose keys no later query reaches
    // through the sparse entries, has the least work and reduces them
    if constexpr (FRAC) {
        if (bh == 0 && tile == nt - 1) {  // uniform over the workgroup
            if constexpr (FUSED) {
                // every tile's partials come from this launch's dQ work, on any XCD
                __shared__ int all_ok;
                if (wave == 0) {
                    const bool ok = poll_tiles<16>(p.flags, 0, p.bh * nt - 1, token, lane);
                    if (lane == 0) all_ok = ok ? 1 : 0;
                }
                __syncthreads();  // also: the LDS tiles are free again
                if (!all_ok) {    // uniform: the wait gave up
                    if (tid == 0) p.dalpha[0] = __builtin_nanf("");
                    return;
                }
                reduce_alpha_grad<true>(p, reinterpret_cast<double *>(ta));
            } else {
                __syncthreads();  // the LDS tiles are free again
                reduce_alpha_grad(p, reinterpret_cast<double *>(ta));
            }
        }
    }
}

template <bool OUT_BF16, bool FRAC>
__global__ void __launch_bounds__(kThreads) bwd_dkdv_kernel(const AttnParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t ta[kTileRows * 64];
    __shared__ __attribute__((aligned(16))) uint16_t tb[kTileRows * 64];
    __shared__ __attribute__((aligned(16))) float lse_s[kTileRows];
    __shared__ __attribute__((aligned(16))) float del_s[kTileRows];
    dkdv_tile<OUT_BF16, FRAC>(p, xcd_logical_block(blockIdx.x, p.bh * ((p.n + 63) >> 6)), ta, tb, lse_s, del_s);
}

// The static backward in one launch: blocks [0, tiles) do the dQ work of tile
// xcd_logical_block(b), blocks [tiles, 2 tiles) the dK/dV work of tile
// xcd_logical_block(b - tiles). A dQ tile publishes this launch's token in p.flags once
// its pair words are in L2; a dK/dV tile waits for the tokens of the tiles whose pair
// words it reads (D it forms itself, or reads from the caller).
// Workgroups are dispatched in block order, so every dQ tile has been dispatched before
// any dK/dV tile waits, and dQ tiles wait for nothing: the waits end. The host launches
// this only when B * H is a multiple of 8: every XCD then holds whole heads, so a tile
// and the tiles it waits for share one XCD and its L2.
template <bool OUT_BF16, bool WITH_D, int NOFF = 0, bool FRAC = false>
__global__ void __launch_bounds__(kThreads) bwd_fused_kernel(const AttnParams p) {
    static_assert(!FRAC || (WITH_D && NOFF == 0), "the fractional form runs with D formed, any table length");
    constexpr int kFb = FRAC ? 4 * FSA_MAX_OFFSETS : kTileRows;
    __shared__ __attribute__((aligned(16))) uint16_t ta[kTileRows * 64];
    __shared__ __attribute__((aligned(16))) uint16_t tb[kTileRows * 64];
    __shared__ __attribute__((aligned(16))) float fa[kTileRows];  // dQ: D of its rows; dK/dV: LSE of the band
    __shared__ __attribute__((aligned(16))) float fb[kFb];        // dQ: per-wave entry sums (FRAC); dK/dV: D of the band
    const int tiles = p.bh * ((p.n + 63) >> 6);
    const uint64_t token = launch_token();
    if (static_cast<int>(blockIdx.x) < tiles) {
        const int lb = xcd_logical_block(blockIdx.x, tiles);
        dq_tile<OUT_BF16, WITH_D, FRAC, NOFF, true>(p, lb, ta, tb, fa, fb);
        // every wave's stores (pair words, D, dQ) have reached L2 before the token does
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_store(p.flags + lb, token, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        dkdv_tile<OUT_BF16, FRAC, true, WITH_D, NOFF>(p, xcd_logical_block(blockIdx.x - tiles, tiles), ta, tb, fa,
                                                      fb, token);
    }
}

// The alpha-gradient reduction on its own (an empty problem: writes the zeros).
__global__ void __launch_bounds__(kThreads) frac_alpha_kernel(const AttnParams p) {
    __shared__ double red[FSA_MAX_OFFSETS];
    reduce_alpha_grad(p, red);
}

// ----------------------------------------------------------------------------
// decode: the newest query of each sequence against a key/value cache
// ----------------------------------------------------------------------------

// One workgroup per (b, h). The newest token of sequence b, at position i = L_b - 1
// (L_b clamped into [1, lmax]), attends the cached keys i - o for o in {0 .. w-1} and
// the table entries o <= i, one softmax over them, as the forward does for row i. Key
// rows are gathered kRows per wave and load (kLanes lanes of 16 bytes per 64-element
// row), the four waves taking interleaved groups, through a ring of kDepth loads in
// flight per wave. Every group of kLanes lanes keeps an online softmax over the keys
// it takes (log2 domain, scale applied: any finite scale); the groups of a wave merge
// through lane exchanges and the four waves through LDS.
//
// With FRAC the table holds fractional entries (learned-alpha variant): entry t is
// present when i >= off[t] + (phi[t] != 0), and its key and value are the fp32 mix
// (1 - phi) row(i - off[t]) + phi row(i - off[t] - 1) of the two cached rows.
template <bool BF16, bool OUT_BF16, bool FRAC>
__global__ void __launch_bounds__(kThreads) decode_kernel(const AttnParams p) {
    using E = typename Elem<BF16>::T;
    using OE = typename Elem<OUT_BF16>::T;
    constexpr int kPer = 16 / sizeof(E);   // elements per lane and load: 8 (bf16) or 4 (fp32)
    constexpr int kLanes = 64 / kPer;      // lanes per row: 8 or 16
    constexpr int kRows = 64 / kLanes;     // rows per wave and load: 8 or 4
    constexpr int kDepth = 4;              // loads in flight per wave
    __shared__ float part[4][2 + 64];      // per wave: maximum, sum, accumulator (64 elements)

    const int64_t hid = blockIdx.x;  // b * H + h
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int L = min(max(p.seq_lens[hid / p.heads], 1), p.lmax);
    const int i = L - 1;
    const int kg = lane / kLanes, c = lane % kLanes;  // row group, chunk
    const E *K = static_cast<const E *>(p.k) + hid * p.lmax * 64 + kPer * c;
    const E *V = static_cast<const E *>(p.v) + hid * p.lmax * 64 + kPer * c;
    const int wl = min(p.w, L);
    int nt = 0;  // table entries that reach a key (the table is sorted)
    while (nt < p.n_off && (FRAC ? table_first(p, nt) : p.off[nt]) <= i) ++nt;
    const int nkeys = wl + nt;
    const int n_iter = (nkeys + 4 * kRows - 1) / (4 * kRows);  // loads per wave
    const float sl2 = p.scale_log2;

    auto to_f32 = [&](const u32x4_t &w4, float out[kPer]) {
        if constexpr (BF16) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                out[2 * e] = bf16_lo(w4[e]);
                out[2 * e + 1] = bf16_hi(w4[e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = __uint_as_float(w4[e]);
        }
    };
    float qv[kPer];
    to_f32(*reinterpret_cast<const u32x4_t *>(static_cast<const E *>(p.q) + hid * 64 + kPer * c), qv);

    // key of load `it` for this lane's row group: index (4 it + wave) kRows + kg; `ph` is
    // the weight of the row below it (fractional entries only, else 0)
    auto key_row = [&](int it, bool &valid, float &ph) {
        const int idx = (4 * it + wave) * kRows + kg;
        valid = idx < nkeys;
        const int t = min(max(idx - wl, 0), FSA_MAX_OFFSETS - 1);
        ph = (FRAC && valid && idx >= wl) ? p.phi[t] : 0.f;
        return valid ? i - (idx < wl ? idx : p.off[t]) : i;  // a valid key lies in [0, i]
    };
    u32x4_t kr[kDepth], vr[kDepth];
    u32x4_t kr2[FRAC ? kDepth : 1], vr2[FRAC ? kDepth : 1];  // FRAC: the rows below
    auto issue = [&](int u, int it) {
        bool valid;
        float ph;
        const int j = key_row(it, valid, ph);
        kr[u] = *reinterpret_cast<const u32x4_t *>(K + (int64_t)j * 64);
        vr[u] = *reinterpret_cast<const u32x4_t *>(V + (int64_t)j * 64);
        if constexpr (FRAC) {
            const int j2 = ph != 0.f ? j - 1 : j;  // a present entry with phi > 0 has j >= 1
            kr2[u] = *reinterpret_cast<const u32x4_t *>(K + (int64_t)j2 * 64);
            vr2[u] = *reinterpret_cast<const u32x4_t *>(V + (int64_t)j2 * 64);
        }
    };
#pragma unroll
    for (int u = 0; u < kDepth; ++u) issue(u, u);  // rows of loads past the keys are row i: in bounds

    float m = kNegInf, l = 0.f, acc[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
    for (int it0 = 0; it0 < n_iter; it0 += kDepth) {
#pragma unroll
        for (int u = 0; u < kDepth; ++u) {
            const int it = it0 + u;
            if (it < n_iter) {  // uniform
                bool valid;
                float ph;
                key_row(it, valid, ph);
                float kv[kPer], vv[kPer];
                to_f32(kr[u], kv);
                to_f32(vr[u], vv);
                if constexpr (FRAC) {
                    float k2[kPer], v2[kPer];
                    to_f32(kr2[u], k2);
                    to_f32(vr2[u], v2);
#pragma unroll
                    for (int e = 0; e < kPer; ++e) {
                        kv[e] = __builtin_fmaf(ph, k2[e] - kv[e], kv[e]);
                        vv[e] = __builtin_fmaf(ph, v2[e] - vv[e], vv[e]);
                    }
                }
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < kPer; ++e) d = __builtin_fmaf(qv[e], kv[e], d);
                d = BF16 ? row8_sum(d) : row16_sum(d);
                const float sc = valid ? d * sl2 : kNegInf;
                const float mn = fmaxf(m, sc);
                const float ms = mn == kNegInf ? 0.f : mn;
                const float al = fast_exp2(m - ms), pv = fast_exp2(sc - ms);
#pragma unroll
                for (int e = 0; e < kPer; ++e) acc[e] = __builtin_fmaf(pv, vv[e], acc[e] * al);
                l = __builtin_fmaf(l, al, pv);
                m = mn;
                if (it + kDepth < n_iter) issue(u, it + kDepth);
            }
        }
    }
    // merge the row groups of the wave (lanes of equal chunk c)
    float mw = m;
    if constexpr (BF16) mw = xor8_max(mw);
    mw = swap_max32(swap_max16(mw));
    const float f = mw == kNegInf ? 0.f : fast_exp2(m - mw);
    float lw = l * f;
    if constexpr (BF16) lw = xor8_add(lw);
    lw = group_sum(lw);
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        float x = acc[e] * f;
        if constexpr (BF16) x = xor8_add(x);
        acc[e] = group_sum(x);
    }
    // merge the four waves; the newest key (offset 0, wave 0) makes the maximum finite
    if (kg == 0) {
#pragma unroll
        for (int e = 0; e < kPer; ++e) part[wave][2 + kPer * c + e] = acc[e];
        if (c == 0) {
            part[wave][0] = mw;
            part[wave][1] = lw;
        }
    }
    __syncthreads();
    if (wave == 0 && kg == 0) {
        float ma = kNegInf;
#pragma unroll
        for (int v = 0; v < 4; ++v) ma = fmaxf(ma, part[v][0]);
        float la = 0.f, oa[kPer];
#pragma unroll
        for (int e = 0; e < kPer; ++e) oa[e] = 0.f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float fv = part[v][0] == kNegInf ? 0.f : fast_exp2(part[v][0] - ma);
            la = __builtin_fmaf(part[v][1], fv, la);
#pragma unroll
            for (int e = 0; e < kPer; ++e) oa[e] = __builtin_fmaf(part[v][2 + kPer * c + e], fv, oa[e]);
        }
#pragma unroll
        for (int e = 0; e < kPer; ++e) oa[e] /= la;
        OE *o = static_cast<OE *>(p.out) + hid * 64 + kPer * c;
        if constexpr (OUT_BF16) {
            if constexpr (BF16) {
                const u32x4_t w4 = {pack_bf16(oa[0], oa[1]), pack_bf16(oa[2], oa[3]), pack_bf16(oa[4], oa[5]),
                                    pack_bf16(oa[6], oa[7])};
                *reinterpret_cast<u32x4_t *>(o) = w4;
            } else {
                const u32x2_t w2 = {pack_bf16(oa[0], oa[1]), pack_bf16(oa[2], oa[3])};
                *reinterpret_cast<u32x2_t *>(o) = w2;
            }
        } else {
#pragma unroll
            for (int e = 0; e < kPer; e += 4)
                *reinterpret_cast<f32x4_t *>(o + e) = f32x4_t{oa[e], oa[e + 1], oa[e + 2], oa[e + 3]};
        }
        if (c == 0) p.lse_out[hid] = ma * kLn2 + logf(la);
    }
}

template <typename Kernel>
hipError_t launch(Kernel *kernel, unsigned grid, const AttnParams &p, hipStream_t stream) {
    AttnParams a = p;
    void *args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), dim3(grid), dim3(kThreads), args, 0, stream);
}

unsigned tiles(const AttnParams &p) { return (unsigned)(p.bh * ((p.n + 63) / 64)); }

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

template <int MODE>
hipError_t launch_generic_forward(fsa_dtype_t dt, fsa_dtype_t out_dt, const AttnParams &p, hipStream_t s) {
    if (dt == FSA_BF16)
        return out_dt == FSA_BF16 ? launch(&fwd_kernel<true, true, MODE>, tiles(p), p, s)
                                  : launch(&fwd_kernel<true, false, MODE>, tiles(p), p, s);
    return out_dt == FSA_BF16 ? launch(&fwd_kernel<false, true, MODE>, tiles(p), p, s)
                              : launch(&fwd_kernel<false, false, MODE>, tiles(p), p, s);
}

}  // namespace

bool window_path(fsa_dtype_t dt, const AttnParams &p) { return window_path(dt, p.w, p.n); }

hipError_t launch_forward(fsa_dtype_t dt, fsa_dtype_t out_dt, const AttnParams &p, hipStream_t s) {
    if (window_path(dt, p) && p.scale_log2 > 0.f)  // the window kernel folds a positive scale into exponents
        return with_table_length(p.n_off, [&](auto len) {
            constexpr int L = decltype(len)::value;
            return out_dt == FSA_BF16 ? launch(&fwd_window_kernel<true, false, false, L>, tiles(p), p, s)
                                      : launch(&fwd_window_kernel<false, false, false, L>, tiles(p), p, s);
        });
    return launch_generic_forward<kWide>(dt, out_dt, p, s);
}

hipError_t launch_dense_forward(fsa_dtype_t dt, fsa_dtype_t out_dt, const AttnParams &p, hipStream_t s) {
    if (dt == FSA_BF16 && p.n <= (1 << 24) && p.scale_log2 > 0.f)
        return out_dt == FSA_BF16 ? launch(&fwd_dense_kernel<true>, tiles(p), p, s)
                                  : launch(&fwd_dense_kernel<false>, tiles(p), p, s);
    return launch_generic_forward<kDense>(dt, out_dt, p, s);
}

hipError_t launch_backward_delta(fsa_dtype_t dt, const AttnParams &p, hipStream_t s) {
    const int64_t rows = (int64_t)p.bh * p.n;
    const int64_t per_block = dt == FSA_BF16 ? 64 : 32;  // two passes of 32 (bf16) or 16 (fp32) rows
    const unsigned grid = (unsigned)((rows + per_block - 1) / per_block);
    return dt == FSA_BF16 ? launch(&delta_kernel<true>, grid, p, s) : launch(&delta_kernel<false>, grid, p, s);
}

hipError_t launch_decode(fsa_dtype_t dt, fsa_dtype_t out_dt, const AttnParams &p, hipStream_t s) {
    const unsigned grid = (unsigned)p.bh;  // one workgroup per (b, h)
    if (dt == FSA_BF16)
        return out_dt == FSA_BF16 ? launch(&decode_kernel<true, true, false>, grid, p, s)
                                  : launch(&decode_kernel<true, false, false>, grid, p, s);
    return out_dt == FSA_BF16 ? launch(&decode_kernel<false, true, false>, grid, p, s)
                              : launch(&decode_kernel<false, false, false>, grid, p, s);
}

hipError_t launch_frac_decode(fsa_dtype_t dt, fsa_dtype_t out_dt, const AttnParams &p, hipStream_t s) {
    const unsigned grid = (unsigned)p.bh;  // one workgroup per (b, h)
    if (dt == FSA_BF16)
        return out_dt == FSA_BF16 ? launch(&decode_kernel<true, true, true>, grid, p, s)
                                  : launch(&decode_kernel<true, false, true>, grid, p, s);
    return out_dt == FSA_BF16 ? launch(&decode_kernel<false, true, true>, grid, p, s)
                              : launch(&decode_kernel<false, false, true>, grid, p, s);
}

hipError_t launch_backward_grads(fsa_dtype_t dt, fsa_dtype_t out_dt, const AttnParams &p, hipStream_t s,
                                 bool with_delta) {
    if (window_backward(dt, p.w, p.n, p.n_off)) {
        // one launch when every XCD holds whole heads (its waits stay within one L2)
        if (p.flags && p.n_off > 0 && p.bh % 8 == 0) {
            const unsigned grid = 2 * tiles(p);
            return with_table_length(p.n_off, [&](auto len) {
                constexpr int L = decltype(len)::value;
                if (with_delta)
                    return out_dt == FSA_BF16 ? launch(&bwd_fused_kernel<true, true, L>, grid, p, s)
                                              : launch(&bwd_fused_kernel<false, true, L>, grid, p, s);
                return out_dt == FSA_BF16 ? launch(&bwd_fused_kernel<true, false, L>, grid, p, s)
                                          : launch(&bwd_fused_kernel<false, false, L>, grid, p, s);
            });
        }
        hipError_t e;
        if (with_delta)
            e = out_dt == FSA_BF16 ? launch(&bwd_dq_kernel<true, true, false>, tiles(p), p, s)
                                   : launch(&bwd_dq_kernel<false, true, false>, tiles(p), p, s);
        else
            e = out_dt == FSA_BF16 ? launch(&bwd_dq_kernel<true, false, false>, tiles(p), p, s)
                                   : launch(&bwd_dq_kernel<false, false, false>, tiles(p), p, s);
        if (e != hipSuccess) return e;
        return out_dt == FSA_BF16 ? launch(&bwd_dkdv_kernel<true, false>, tiles(p), p, s)
                                  : launch(&bwd_dkdv_kernel<false, false>, tiles(p), p, s);
    }
    if (with_delta) {  // the generic kernel reads D: form it first
        const hipError_t e = launch_backward_delta(dt, p, s);
        if (e != hipSuccess) return e;
    }
    if (dt == FSA_BF16)
        return out_dt == FSA_BF16 ? launch(&bwd_generic_kernel<true, true>, tiles(p), p, s)
                                  : launch(&bwd_generic_kernel<true, false>, tiles(p), p, s);
    return out_dt == FSA_BF16 ? launch(&bwd_generic_kernel<false, true>, tiles(p), p, s)
                              : launch(&bwd_generic_kernel<false, false>, tiles(p), p, s);
}

hipError_t launch_rope(const RopeParams &p, hipStream_t s) {
    const int64_t chunks = (int64_t)p.n * 8;  // per head
    const int64_t heads = p.rows / p.n;
    constexpr int64_t kMaxY = 65535;  // heads per launch (grid y)
    for (int64_t h0 = 0; h0 < heads; h0 += kMaxY) {
        const dim3 grid((unsigned)((chunks + kThreads - 1) / kThreads), (unsigned)std::min(kMaxY, heads - h0));
        RopeParams a = p;
        a.head0 = h0;
        void *args[] = {&a};
        const hipError_t e =
            hipLaunchKernel(reinterpret_cast<const void *>(&rope_kernel), grid, dim3(kThreads), args, 0, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_rope_forward(fsa_dtype_t out_dt, const AttnParams &p, hipStream_t s) {
    return with_table_length(p.n_off, [&](auto len) {
        constexpr int L = decltype(len)::value;
        return out_dt == FSA_BF16 ? launch(&fwd_window_kernel<true, false, true, L>, tiles(p), p, s)
                                  : launch(&fwd_window_kernel<false, false, true, L>, tiles(p), p, s);
    });
}

hipError_t launch_frac_forward(fsa_dtype_t out_dt, const AttnParams &p, hipStream_t s) {
    return out_dt == FSA_BF16 ? launch(&fwd_window_kernel<true, true>, tiles(p), p, s)
                              : launch(&fwd_window_kernel<false, true>, tiles(p), p, s);
}

hipError_t launch_frac_backward(fsa_dtype_t out_dt, const AttnParams &p, hipStream_t s) {
    if (tiles(p) == 0) return launch(&frac_alpha_kernel, 1, p, s);  // writes the zeros of an empty problem
    if (p.flags && p.n_off > 0 && p.bh % 8 == 0)  // one launch, as for the static tables
        return out_dt == FSA_BF16 ? launch(&bwd_fused_kernel<true, true, 0, true>, 2 * tiles(p), p, s)
                                  : launch(&bwd_fused_kernel<false, true, 0, true>, 2 * tiles(p), p, s);
    const hipError_t e = out_dt == FSA_BF16 ? launch(&bwd_dq_kernel<true, true, true>, tiles(p), p, s)
                                            : launch(&bwd_dq_kernel<false, true, true>, tiles(p), p, s);
    if (e != hipSuccess) return e;
    // the dK/dV kernel also reduces the alpha gradient
    return out_dt == FSA_BF16 ? launch(&bwd_dkdv_kernel<true, true>, tiles(p), p, s)
                              : launch(&bwd_dkdv_kernel<false, true>, tiles(p), p, s);
}

}  // namespace fsa
