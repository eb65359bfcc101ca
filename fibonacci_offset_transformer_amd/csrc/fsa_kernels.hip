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
// Work decomposition (one workgroup = 4 wave64 = one 64-row tile of one head):
//  * Window band: a banded dense block, computed on MFMA. Scores are formed
//    transposed, S^T = K Q^T, so each lane's four accumulator rows are four keys
//    of one query; that accumulator layout is exactly the B-operand layout of
//    the 16x16x16 MFMA, so P^T feeds the P.V product with no data movement. V
//    (and, in the backward, K, Q and dO) is staged transposed in LDS to serve
//    as the A operand of those key-contracting products.
//  * Sparse offsets: each offset o maps the tile's 64 query rows onto one
//    contiguous 64-row K/V slab. Lanes read their rows with coalesced vector
//    loads and form the per-row diagonal dot products on VALU, reducing across
//    the four lane groups with cross-lane shuffles.
//  * One online (running max / running sum) fp32 softmax covers both parts.
//  * Lane ownership of a 64-wide row: lane group g = lane / 16 holds the 16
//    elements d = 16 s + 4 g + u (s, u in 0..3). The d-contracting MFMAs read
//    their operands in that order (any fixed assignment of d to k-slots that A
//    and B share gives the same sum), so the band, the sparse slabs and the
//    output accumulators all use one layout.
//  * Workgroup ids are remapped so that the tiles of one head run on one XCD in
//    increasing row order, keeping that head's K/V in the XCD's L2 for the
//    slab re-reads.
//  * Backward: one kernel computes D = rowsum(dO * O); the main kernel gives
//    each workgroup dQ of its 64 query rows and dK, dV of the same 64 key rows,
//    recomputing P on both sides, so every output row has one writer and no
//    atomics are used.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fsa_internal.h"

namespace fsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;
constexpr int kT64 = 64 + 4;    // padded LDS row (elements) of a transposed 64-row tile
constexpr int kT128 = 128 + 4;  // padded LDS row (elements) of a transposed 128-row tile
constexpr int kSlabRegs = 8;    // sparse offsets whose rows are prefetched into registers

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

__device__ __forceinline__ float frag_elem(const Frag<true> &f, int h, int e) {
    const uint32_t w = f.c[h][e >> 1];
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}
__device__ __forceinline__ float frag_elem(const Frag<false> &f, int h, int e) { return f.c[2 * h + (e >> 2)][e & 3]; }

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
            s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.c[h][w]),
                                                 __builtin_bit_cast(bf16x2_t, b.c[h][w]), s0, false);
            s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.c[h][w + 1]),
                                                 __builtin_bit_cast(bf16x2_t, b.c[h][w + 1]), s1, false);
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
    const bf16x2_t xl = __builtin_bit_cast(bf16x2_t, pack_bf16(x, 0.f));
    const bf16x2_t xh = __builtin_bit_cast(bf16x2_t, pack_bf16(0.f, x));
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const bf16x2_t v = __builtin_bit_cast(bf16x2_t, f.c[h][w]);
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

// Sum / max over the four lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float group_sum(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}
__device__ __forceinline__ float group_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

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
// forward
// ----------------------------------------------------------------------------

enum FwdMode { kWindow = 0, kWide = 1, kDense = 2 };

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
        const float al = exp2f(m2 - ms);
        float ps = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] *= al;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float pu = exp2f(sc[u] - ms);
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
    // window mode: V^T of keys [i0 - 64, i0 + 64); wide/dense: V^T of one 64-key chunk
    __shared__ __attribute__((aligned(16))) E vt[MODE == kWindow ? 64 * kT128 : 64 * kT64];

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

    if constexpr (MODE == kWindow) {
        // ---------------- window of at most 64 keys: every load issued up front ----------------
        StageRegs<BF16> vs;
        stage_load(vs, V, i0 - 64, n, tid);
        const int qb = r0 >> 4;  // the wave's 16-row block; its keys lie in blocks qb-4 .. qb
        Frag<BF16> kf[5];
#pragma unroll
        for (int b = 0; b < 5; ++b) load_frag(kf[b], K, min(max(16 * (qb - 4 + b) + c16, 0), n - 1), g);
        Frag<BF16> sk[kSlabRegs], sv[kSlabRegs];
        int sj[kSlabRegs];
        bool sok[kSlabRegs];
#pragma unroll
        for (int t = 0; t < kSlabRegs; ++t) {
            const int j = (t < p.n_off) ? i - p.off[t] : -1;
            sok[t] = row_ok && j >= 0;
            sj[t] = min(max(j, 0), n - 1);
            if (t < p.n_off) load_frag(sk[t], K, sj[t], g);
        }
        stage_store(vt, kT128, vs, tid);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < kSlabRegs; ++t)
            if (t < p.n_off) load_frag(sv[t], V, sj[t], g);

        // window band: all 20 scores of the lane, one max, then P.V on MFMA
        const int klo = max(0, r0 - w + 1), khi = min(r0 + 15, n - 1);  // keys the wave needs
        float sc[5][4];
        float bm = kNegInf;
#pragma unroll
        for (int b = 0; b < 5; ++b) {
            const int kb0 = 16 * (qb - 4 + b);
            const bool active = kb0 + 15 >= klo && kb0 <= khi;
            const bool full = kb0 >= 0 && kb0 + 15 <= r0 && kb0 >= r0 + 16 - w && r0 + 15 < n;
            f32x4_t st = {kNegInf, kNegInf, kNegInf, kNegInf};
            if (active) st = mma_over_d(kf[b], qf, f32x4_t{0.f, 0.f, 0.f, 0.f}) * sl2;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = kb0 + 4 * g + r;
                const bool ok = full || (active && row_ok && j <= i && j > i - w && j >= 0);
                sc[b][r] = ok ? st[r] : kNegInf;
                bm = fmaxf(bm, sc[b][r]);
            }
        }
        m2 = group_max(bm);
        const float ms = row_ok ? m2 : 0.f;
#pragma unroll
        for (int b = 0; b < 5; ++b) {
            const int kb0 = 16 * (qb - 4 + b);
            const bool active = kb0 + 15 >= klo && kb0 <= khi;
            float pr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pr[r] = exp2f(sc[b][r] - ms);
                lsum += pr[r];
            }
            if (active) mma_over_rows(acc, vt, kT128, 16 * (wave + b), c16, g, pr);
        }

        // prefetched sparse offsets: scores, one rescale, then the P.V terms
        float ss[kSlabRegs];
        float gm = kNegInf;
#pragma unroll
        for (int t = 0; t < kSlabRegs; ++t) {
            ss[t] = kNegInf;
            if (t < p.n_off) {
                const float d = group_sum(frag_dot(qf, sk[t]));
                ss[t] = sok[t] ? d * sl2 : kNegInf;
            }
            gm = fmaxf(gm, ss[t]);
        }
        const float mn = fmaxf(m2, gm);
        const float ms2 = (mn == kNegInf) ? 0.f : mn;
        const float al = exp2f(m2 - ms2);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] *= al;
        float ps = 0.f;
#pragma unroll
        for (int t = 0; t < kSlabRegs; ++t) {
            if (t < p.n_off) {
                const float pt = exp2f(ss[t] - ms2);
                ps += pt;
                frag_axpy(acc, pt, sv[t]);
            }
        }
        lsum = lsum * al + (g == 0 ? ps : 0.f);
        m2 = mn;
        if (p.n_off > kSlabRegs && r0 < n) fwd_slabs_loop(p, kSlabRegs, qf, K, V, i, row_ok, r0, n, g, acc, m2, lsum);
    } else {
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
                const float al = exp2f(m2 - ms);
                float pr[4], ps = 0.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pr[r] = exp2f(sv[r] - ms);
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
    }

    // ---- epilogue ----
    const float l = group_sum(lsum);
    if (row_ok) {
        store_row(static_cast<OE *>(p.out) + head, i, g, acc, 1.f / l);
        if (g == 0) p.lse_out[(int64_t)bh * n + i] = m2 * kLn2 + logf(l);
    }
}

// ----------------------------------------------------------------------------
// backward: D = rowsum(dO * O)
// ----------------------------------------------------------------------------

template <bool BF16>
__global__ void __launch_bounds__(kThreads) delta_kernel(const AttnParams p) {
    using E = typename Elem<BF16>::T;
    const int64_t rows = (int64_t)p.bh * p.n;
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int part = threadIdx.x & 15;  // 4 elements each
    float acc = 0.f;
    if (row < rows) {
        const E *o = static_cast<const E *>(p.o) + row * 64 + 4 * part;
        const E *d = static_cast<const E *>(p.dout) + row * 64 + 4 * part;
        if constexpr (BF16) {
            const u32x2_t a = *reinterpret_cast<const u32x2_t *>(o);
            const u32x2_t b = *reinterpret_cast<const u32x2_t *>(d);
            acc = bf16_lo(a.x) * bf16_lo(b.x) + bf16_hi(a.x) * bf16_hi(b.x) + bf16_lo(a.y) * bf16_lo(b.y) +
                  bf16_hi(a.y) * bf16_hi(b.y);
        } else {
            const f32x4_t a = *reinterpret_cast<const f32x4_t *>(o);
            const f32x4_t b = *reinterpret_cast<const f32x4_t *>(d);
            acc = a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
        }
    }
#pragma unroll
    for (int sh = 1; sh < 16; sh <<= 1) acc += __shfl_xor(acc, sh);
    if (row < rows && part == 0) p.delta[row] = acc;
}

// ----------------------------------------------------------------------------
// backward: dQ (query-owned) then dK, dV (key-owned) of one 64-row tile
// ----------------------------------------------------------------------------

template <bool BF16, bool OUT_BF16>
__global__ void __launch_bounds__(kThreads) bwd_kernel(const AttnParams p) {
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
                    const float pv = ok ? exp2f(st[r] * sl2 - lse2) : 0.f;
                    ds[r] = pv * (dpt[r] - di);
                }
                mma_over_rows(acc, t0s, kT64, 16 * kb, c16, g, ds);
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
                const float pv = ok ? exp2f(s * sl2 - lse2) : 0.f;
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
                    pr[r] = ok ? exp2f(sq[r] * sl2 - lse_s[qi]) : 0.f;
                    ds[r] = pr[r] * (dpq[r] - del_s[qi]);
                }
                mma_over_rows(dv, t1s, kT64, 16 * qb, c16, g, pr);
                mma_over_rows(dk, t0s, kT64, 16 * qb, c16, g, ds);
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
                const float pv = ok ? exp2f(s * sl2 - LSE[ic] * kLog2e) : 0.f;
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

template <bool BF16, bool OUT_BF16, int MODE>
hipError_t launch_forward_t(const AttnParams &p, hipStream_t stream) {
    const int nt = (p.n + 63) / 64;
    const dim3 grid(p.bh * nt), block(kThreads);
    AttnParams a = p;
    void *args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void *>(&fwd_kernel<BF16, OUT_BF16, MODE>), grid, block, args, 0,
                           stream);
}

template <int MODE>
hipError_t launch_forward_mode(fsa_dtype_t dt, fsa_dtype_t out_dt, const AttnParams &p, hipStream_t stream) {
    if (dt == FSA_BF16)
        return out_dt == FSA_BF16 ? launch_forward_t<true, true, MODE>(p, stream)
                                  : launch_forward_t<true, false, MODE>(p, stream);
    return out_dt == FSA_BF16 ? launch_forward_t<false, true, MODE>(p, stream)
                              : launch_forward_t<false, false, MODE>(p, stream);
}

template <bool BF16>
hipError_t launch_delta_t(const AttnParams &p, hipStream_t stream) {
    AttnParams a = p;
    void *args[] = {&a};
    const int64_t rows = (int64_t)p.bh * p.n;
    const dim3 grid((unsigned)((rows + 15) / 16)), block(kThreads);
    return hipLaunchKernel(reinterpret_cast<const void *>(&delta_kernel<BF16>), grid, block, args, 0, stream);
}

template <bool BF16, bool OUT_BF16>
hipError_t launch_grads_t(const AttnParams &p, hipStream_t stream) {
    AttnParams a = p;
    void *args[] = {&a};
    const int nt = (p.n + 63) / 64;
    const dim3 grid(p.bh * nt), block(kThreads);
    return hipLaunchKernel(reinterpret_cast<const void *>(&bwd_kernel<BF16, OUT_BF16>), grid, block, args, 0,
                           stream);
}

}  // namespace

hipError_t launch_forward(fsa_dtype_t dt, fsa_dtype_t out_dt, const AttnParams &p, hipStream_t stream) {
    return p.w <= 64 ? launch_forward_mode<kWindow>(dt, out_dt, p, stream)
                     : launch_forward_mode<kWide>(dt, out_dt, p, stream);
}

hipError_t launch_dense_forward(fsa_dtype_t dt, fsa_dtype_t out_dt, const AttnParams &p, hipStream_t stream) {
    return launch_forward_mode<kDense>(dt, out_dt, p, stream);
}

hipError_t launch_backward_delta(fsa_dtype_t dt, const AttnParams &p, hipStream_t stream) {
    return dt == FSA_BF16 ? launch_delta_t<true>(p, stream) : launch_delta_t<false>(p, stream);
}

hipError_t launch_backward_grads(fsa_dtype_t dt, fsa_dtype_t out_dt, const AttnParams &p, hipStream_t stream) {
    if (dt == FSA_BF16)
        return out_dt == FSA_BF16 ? launch_grads_t<true, true>(p, stream) : launch_grads_t<true, false>(p, stream);
    return out_dt == FSA_BF16 ? launch_grads_t<false, true>(p, stream) : launch_grads_t<false, false>(p, stream);
}

}  // namespace fsa
