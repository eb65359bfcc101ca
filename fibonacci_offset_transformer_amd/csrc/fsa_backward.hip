// Backward kernels of libfsa (gfx950): D = rowsum(dO * O), the general kernel, and
// the bf16 window path's dQ and dK/dV work (two kernels, or one launch joined by
// per-tile tokens), static and learned-alpha; with their launchers.
#include "fsa_device.h"

namespace fsa {
namespace {

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

// Backward on the window path (bf16 inputs, w <= 64) has two parts over 64-row tiles.
// The dQ part forms dQ of its query rows and, for every sparse pair (query i, key
// i - off[t]), stores P and dS rounded to bf16 (the weights the gradient products use)
// in a pair workspace [BH, N, S] of 32-bit words (P in the low half). The dK/dV part
// forms dK and dV of its key rows from the window band, recomputed on MFMA, and from
// the stored weights of the sparse pairs (key j, query j + off[t]), so no score is
// formed twice on the vector units. Each part keeps one pair of operands resident (K, V
// for dQ; Q, dO for dK and dV), which halves the data an XCD's L2 has to hold. The two
// parts run as two kernels (bwd_dq_kernel, bwd_dkdv_kernel) or, when B * H is a
// multiple of 8, in one launch (bwd_fused_kernel) joined by per-tile tokens.

constexpr int kRingQ = 4, kPreQ = 2;    // dQ kernel: slab slots in the ring; slots requested before the band
constexpr int kRingKV = 3, kPreKV = 1;  // dK/dV kernel

// Descriptor over the pair-workspace words of head bh ([N, S, WORDS] words, S =
// pair_slots): rows past the sequence end read as zero words.
template <int WORDS>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pair_rsrc(const AttnParams &p, int n_off, int bh) {
    const int slots = pair_slots(n_off);
    return head_rsrc(p.pairs + (int64_t)bh * p.n * slots * WORDS, span_bytes(p.n, 4u * slots * WORDS));
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
// With EXACT (windows narrower than 64, static tables) each pair slot holds P and dS as
// two fp32 words, and the sparse part of dQ takes dS unrounded.
//
// The body works on logical tile lb with the caller's LDS: ta, tb (band K and V rows,
// kTileRows * 64 each, then merge areas), d_s (64 floats: D of the tile's rows, WITH_D)
// and dd_s (4 * FSA_MAX_OFFSETS floats, FRAC). With PUBLISH (one-launch backward) the
// tile sets its flag to `token` once its D, pair words and partials are in L2, before
// it stores dQ, which nothing in the launch reads.
template <bool OUT_BF16, bool WITH_D, bool FRAC, int NOFF = 0, bool PUBLISH = false, bool EXACT = false>
__device__ __forceinline__ void dq_tile(const AttnParams &p, const int lb, uint16_t *ta, uint16_t *tb, float *d_s,
                                        float *dd_s, [[maybe_unused]] const uint64_t token = 0) {
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
    if (w == 64 && r0 >= 64 && r0 + 15 < n) {  // uniform: a full window of 64 keys for every row
        // only the oldest block and the newest are cut, at the same lane position: key
        // 4 g + r of the block against row c16 (no branch, so the blocks' LDS reads and
        // MFMAs interleave)
        auto fast_ds = [&](auto bc, float ds[4]) {
            constexpr int b = decltype(bc)::value;
            Frag<true> kf, vf;
            lds_frag(kf, ta_w, 16 * b, tl);
            lds_frag(vf, tb_w, 16 * b, tl);
            const f32x4_t st = mma_over_d(kf, qf, f32x4_t{0.f, 0.f, 0.f, 0.f});
            const f32x4_t dpt = mma_over_d(vf, df, f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool newer = 4 * g + r > c16;
                const float x = fast_exp2(__builtin_fmaf(st[r], sl2, -lse2_i)) * (dpt[r] - di_i);
                ds[r] = (b == 0 && !newer) || (b == 4 && newer) ? 0.f : x;
            }
        };
        float d0[4], d1[4];
        fast_ds(Len<0>{}, d0);
        fast_ds(Len<1>{}, d1);
        mma_over_rows_tr2_exact(acc, ta_w, 0, 16, tl, d0, d1);
        __builtin_amdgcn_sched_barrier(0);  // keeps the next pair's reads from piling up registers
        fast_ds(Len<2>{}, d0);
        fast_ds(Len<3>{}, d1);
        mma_over_rows_tr2_exact(acc, ta_w, 32, 48, tl, d0, d1);
        __builtin_amdgcn_sched_barrier(0);
        fast_ds(Len<4>{}, d0);
        mma_over_rows_tr_exact(acc, ta_w, 64, tl, d0);
    } else {
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
    // Q and dO rows move from the MFMA layout (row c16, chunks g and g + 4) to the slab
    // layout through this wave's 4 KB of the V tile, free since the barrier above (chunk
    // c of row r at position c ^ (r & 7), so that neither side conflicts on banks)
    SFrag qs, dos;
    {
        uint16_t *qa = tb + 2048 * wave, *da = qa + 1024;
        const int w0 = c16 * 64 + 8 * (g ^ (c16 & 7)), w1 = c16 * 64 + 8 * ((g + 4) ^ (c16 & 7));
        *reinterpret_cast<u32x4_t *>(qa + w0) = qf.c[0];
        *reinterpret_cast<u32x4_t *>(qa + w1) = qf.c[1];
        *reinterpret_cast<u32x4_t *>(da + w0) = df.c[0];
        *reinterpret_cast<u32x4_t *>(da + w1) = df.c[1];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = (s8 + 8 * h) * 64 + 8 * (c8 ^ s8);
            qs.r[h] = *reinterpret_cast<const u32x4_t *>(qa + r);
            dos.r[h] = *reinterpret_cast<const u32x4_t *>(da + r);
        }
    }
    float lse2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) lse2[h] = buf_f32(rl, row_s[h]) * kLog2e;
    const int slots = pair_slots(n_off);
    if constexpr (FRAC) {
        // pair words [n, slots, 2]: the near word {(1 - phi) P, (1 - phi) dS} and the far
        // word {phi P, phi dS} of every entry, each rounded once to bf16 (EXACT: [n, slots,
        // 4], the same four values as fp32 words), stored by the lane c8 = t mod 8 of each row
        uint2 *pairs2 = reinterpret_cast<uint2 *>(p.pairs) + (int64_t)bh * n * slots;
        uint4 *pairs4 = reinterpret_cast<uint4 *>(p.pairs) + (int64_t)bh * n * slots;
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
                if constexpr (EXACT) {
                    if (c8 == (t & 7) && row < n)
                        pairs4[(int64_t)row * slots + t] = uint4{__float_as_uint(pv - pf), __float_as_uint(ds - dsf),
                                                                 __float_as_uint(pf), __float_as_uint(dsf)};
                    chunk_axpy_f32(dq_s[h], ds - dsf, kn.r[h]);
                    chunk_axpy_f32(dq_s[h], dsf, kf.r[h]);
                } else {
                    const uint2 pw = {pack_bf16(pv - pf, ds - dsf), pack_bf16(pf, dsf)};
                    if (c8 == (t & 7) && row < n) pairs2[(int64_t)row * slots + t] = pw;
                    chunk_axpy_words(dq_s[h], pw.x >> 16, pw.x & 0xffff0000u, kn.r[h]);
                    chunk_axpy_words(dq_s[h], pw.y >> 16, pw.y & 0xffff0000u, kf.r[h]);
                }
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
        // pair slots of this head's rows: [n, slots]; lane c8 of a row keeps slot c8 of the
        // unrolled part and the eight lanes store them with one 32-byte (EXACT: 64-byte) write
        using PairT = typename PairSlot<EXACT>::T;
        PairT *pairs = reinterpret_cast<PairT *>(p.pairs) + (int64_t)bh * n * slots;
        PairT keep[2] = {PairT{}, PairT{}};
        auto slab = [&](int t, int o, const SFrag &kt, const SFrag &vt) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bool ok = (row_s[h] < n) & (row_s[h] - o >= 0);
                const float s = row8_sum(chunk_dot(qs.r[h], kt.r[h]));
                const float dp = row8_sum(chunk_dot(dos.r[h], vt.r[h]));
                const float pv = ok ? fast_exp2(__builtin_fmaf(s, sl2, -lse2[h])) : 0.f;
                const float ds = pv * (dp - di[h]);
                PairT pw;
                if constexpr (EXACT) {
                    pw = PairT{__float_as_uint(pv), __float_as_uint(ds)};
                    chunk_axpy_f32(dq_s[h], ds, kt.r[h]);
                } else {
                    pw = pack_bf16(pv, ds);
                    chunk_axpy_words(dq_s[h], pw >> 16, pw & 0xffff0000u, kt.r[h]);
                }
                if (t < 8)
                    keep[h] = select(c8 == t, pw, keep[h]);
                else if (c8 == 0 && row_s[h] < n)
                    pairs[(int64_t)row_s[h] * slots + t] = pw;
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
        static_assert(unrolled_slabs(kRingQ) >= 8, "the kept pair words cover slots 0..7");
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
    if constexpr (PUBLISH) {
        // every wave's stores of the words others read (pair words, D, the partials) have
        // reached L2 before the token does; dQ, read by no one in the launch, follows it
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_store(p.flags + lb, token, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
        if (row_s[h] < n) store_chunk<true>(static_cast<OE *>(p.dq) + head, row_s[h], c8, dq_s[h], p.scale);
}

template <bool OUT_BF16, bool WITH_D, bool FRAC, bool EXACT = false>
__global__ void __launch_bounds__(kThreads) bwd_dq_kernel(const AttnParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t ta[kTileRows * 64];
    __shared__ __attribute__((aligned(16))) uint16_t tb[kTileRows * 64];
    __shared__ float d_s[64];
    __shared__ float dd_s[FRAC ? 4 * FSA_MAX_OFFSETS : 1];
    dq_tile<OUT_BF16, WITH_D, FRAC, 0, false, EXACT>(p, xcd_logical_block(blockIdx.x, p.bh * ((p.n + 63) >> 6)), ta,
                                                     tb, d_s, dd_s);
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
// FROM_DQ: D comes from that dQ work (otherwise the caller gave it). EXACT: the pair
// slots hold P and dS as fp32 words (see dq_tile), which weight the rows unrounded.
template <bool OUT_BF16, bool FRAC, bool FUSED = false, bool FROM_DQ = false, int NOFF = 0, bool EXACT = false>
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
            const bool ok = poll_tiles(p, p.flags + (int64_t)bh * nt, tile, last, token, lane);
            if (lane == 0) {
                gave_up = ok ? 0 : 1;
                if (!ok) record_give_up(p, token);
            }
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
    using PairT = typename PairSlot<EXACT>::T;
    SFrag sq[kRingKV], sd[kRingKV];
    PairT pw[kRingKV][2];
    const int slots = pair_slots(n_off);
    constexpr int kFracWords = EXACT ? 4 : 2;  // FRAC: words per slot (near and far share)
    const __amdgpu_buffer_rsrc_t rp = FRAC    ? head_rsrc(p.pairs + (int64_t)bh * n * slots * kFracWords,
                                                          span_bytes(n, 4u * kFracWords * slots))
                                      : EXACT ? pair_rsrc<2>(p, n_off, bh)
                                              : pair_rsrc<1>(p, n_off, bh);
    auto fill_words = [&](int u, int x) {
        const int t = FRAC ? x >> 1 : x, far = FRAC ? x & 1 : 0;
        const int iq0 = slab_row(p, n_off, t, row_s[0], 1) + far, iq1 = slab_row(p, n_off, t, row_s[1], 1) + far;
        if constexpr (FRAC && EXACT) {  // the share's two fp32 words
            pw[u][0] = __builtin_bit_cast(PairT, __builtin_amdgcn_raw_buffer_load_b64(rp, ((iq0 * slots + t) * 2 + far) * 8,
                                                                                      0, FUSED ? kCachePastL1 : 0));
            pw[u][1] = __builtin_bit_cast(PairT, __builtin_amdgcn_raw_buffer_load_b64(rp, ((iq1 * slots + t) * 2 + far) * 8,
                                                                                      0, FUSED ? kCachePastL1 : 0));
        } else if constexpr (FRAC) {
            pw[u][0] = __builtin_amdgcn_raw_buffer_load_b32(rp, ((iq0 * slots + t) * 2 + far) * 4, 0,
                                                            FUSED ? kCachePastL1 : 0);
            pw[u][1] = __builtin_amdgcn_raw_buffer_load_b32(rp, ((iq1 * slots + t) * 2 + far) * 4, 0,
                                                            FUSED ? kCachePastL1 : 0);
        } else if constexpr (EXACT) {
            pw[u][0] = __builtin_bit_cast(
                PairT, __builtin_amdgcn_raw_buffer_load_b64(rp, (iq0 * slots + t) * 8, 0, FUSED ? kCachePastL1 : 0));
            pw[u][1] = __builtin_bit_cast(
                PairT, __builtin_amdgcn_raw_buffer_load_b64(rp, (iq1 * slots + t) * 8, 0, FUSED ? kCachePastL1 : 0));
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

    // sparse offsets: queries j + o, weights P (low half, or first word) and dS (high
    // half, or second word) as stored; pairs past the sequence end read as zero words
    auto slab = [&](const PairT pwt[2], const SFrag &qt, const SFrag &dt) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if constexpr (EXACT) {
                chunk_axpy_f32(dv_s[h], __uint_as_float(pwt[h][0]), dt.r[h]);
                chunk_axpy_f32(dk_s[h], __uint_as_float(pwt[h][1]), qt.r[h]);
            } else {
                const uint32_t x = pwt[h];
                chunk_axpy_words(dv_s[h], x & 0xffffu, x << 16, dt.r[h]);
                chunk_axpy_words(dk_s[h], x >> 16, x & 0xffff0000u, qt.r[h]);
            }
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
                    const bool ok = poll_tiles<16>(p, p.flags, 0, p.bh * nt - 1, token, lane);
                    if (lane == 0) {
                        all_ok = ok ? 1 : 0;
                        if (!ok) record_give_up(p, token);
                    }
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

template <bool OUT_BF16, bool FRAC, bool EXACT = false>
__global__ void __launch_bounds__(kThreads) bwd_dkdv_kernel(const AttnParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t ta[kTileRows * 64];
    __shared__ __attribute__((aligned(16))) uint16_t tb[kTileRows * 64];
    __shared__ __attribute__((aligned(16))) float lse_s[kTileRows];
    __shared__ __attribute__((aligned(16))) float del_s[kTileRows];
    dkdv_tile<OUT_BF16, FRAC, false, false, 0, EXACT>(p, xcd_logical_block(blockIdx.x, p.bh * ((p.n + 63) >> 6)), ta,
                                                      tb, lse_s, del_s);
}

// The static backward in one launch: blocks [0, tiles) do the dQ work of tile
// xcd_logical_block(b), blocks [tiles, 2 tiles) the dK/dV work of tile
// xcd_logical_block(b - tiles). A dQ tile publishes this launch's token in p.flags once
// its D and pair words are in L2 (before its dQ store); a dK/dV tile waits for the tokens of the tiles whose pair
// words it reads (D it forms itself, or reads from the caller).
// Workgroups are dispatched in block order, so every dQ tile has been dispatched before
// any dK/dV tile waits, and dQ tiles wait for nothing: the waits end. The host launches
// this only when B * H is a multiple of 8: every XCD then holds whole heads, so a tile
// and the tiles it waits for share one XCD and its L2.
template <bool OUT_BF16, bool WITH_D, int NOFF = 0, bool FRAC = false, bool EXACT = false>
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
        dq_tile<OUT_BF16, WITH_D, FRAC, NOFF, true, EXACT>(p, lb, ta, tb, fa, fb, token);
    } else {
        dkdv_tile<OUT_BF16, FRAC, true, WITH_D, NOFF, EXACT>(p, xcd_logical_block(blockIdx.x - tiles, tiles), ta, tb,
                                                             fa, fb, token);
    }
}

// The alpha-gradient reduction on its own (an empty problem: writes the zeros).
__global__ void __launch_bounds__(kThreads) frac_alpha_kernel(const AttnParams p) {
    __shared__ double red[FSA_MAX_OFFSETS];
    reduce_alpha_grad(p, red);
}

// Static window backward with pair slots of one format (EXACT: fp32 P and dS).
template <bool EXACT>
hipError_t launch_window_backward(fsa_dtype_t out_dt, const AttnParams &p, hipStream_t s, bool with_delta) {
    // one launch when every XCD holds whole heads (its waits stay within one L2)
    if (one_launch_backward(p)) {
        const unsigned grid = 2 * tiles(p);
        auto fused = [&](auto len) {
            constexpr int L = decltype(len)::value;
            if (with_delta)
                return out_dt == FSA_BF16 ? launch(&bwd_fused_kernel<true, true, L, false, EXACT>, grid, p, s)
                                          : launch(&bwd_fused_kernel<false, true, L, false, EXACT>, grid, p, s);
            return out_dt == FSA_BF16 ? launch(&bwd_fused_kernel<true, false, L, false, EXACT>, grid, p, s)
                                      : launch(&bwd_fused_kernel<false, false, L, false, EXACT>, grid, p, s);
        };
        // the narrow windows that take EXACT slots have long tables: the run-time length only
        if constexpr (EXACT) return fused(Len<0>{});
        else return with_table_length(p.n_off, fused);
    }
    hipError_t e;
    if (with_delta)
        e = out_dt == FSA_BF16 ? launch(&bwd_dq_kernel<true, true, false, EXACT>, tiles(p), p, s)
                               : launch(&bwd_dq_kernel<false, true, false, EXACT>, tiles(p), p, s);
    else
        e = out_dt == FSA_BF16 ? launch(&bwd_dq_kernel<true, false, false, EXACT>, tiles(p), p, s)
                               : launch(&bwd_dq_kernel<false, false, false, EXACT>, tiles(p), p, s);
    if (e != hipSuccess) return e;
    return out_dt == FSA_BF16 ? launch(&bwd_dkdv_kernel<true, false, EXACT>, tiles(p), p, s)
                              : launch(&bwd_dkdv_kernel<false, false, EXACT>, tiles(p), p, s);
}

}  // namespace

hipError_t launch_backward_delta(fsa_dtype_t dt, const AttnParams &p, hipStream_t s) {
    const int64_t rows = (int64_t)p.bh * p.n;
    const int64_t per_block = dt == FSA_BF16 ? 64 : 32;  // two passes of 32 (bf16) or 16 (fp32) rows
    const unsigned grid = (unsigned)((rows + per_block - 1) / per_block);
    return dt == FSA_BF16 ? launch(&delta_kernel<true>, grid, p, s) : launch(&delta_kernel<false>, grid, p, s);
}

hipError_t launch_backward_grads(fsa_dtype_t dt, fsa_dtype_t out_dt, const AttnParams &p, hipStream_t s,
                                 bool with_delta) {
    if (window_backward(dt, p.w, p.n, p.n_off)) {
        if (pair_slot_words(p.w) == 2) return launch_window_backward<true>(out_dt, p, s, with_delta);
        return launch_window_backward<false>(out_dt, p, s, with_delta);
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

// Learned-alpha backward with pair slots of one format (EXACT: fp32 shares, below w = 64).
template <bool EXACT>
hipError_t launch_frac_window_backward(fsa_dtype_t out_dt, const AttnParams &p, hipStream_t s) {
    if (one_launch_backward(p))  // one launch, as for the static tables
        return out_dt == FSA_BF16 ? launch(&bwd_fused_kernel<true, true, 0, true, EXACT>, 2 * tiles(p), p, s)
                                  : launch(&bwd_fused_kernel<false, true, 0, true, EXACT>, 2 * tiles(p), p, s);
    const hipError_t e = out_dt == FSA_BF16 ? launch(&bwd_dq_kernel<true, true, true, EXACT>, tiles(p), p, s)
                                            : launch(&bwd_dq_kernel<false, true, true, EXACT>, tiles(p), p, s);
    if (e != hipSuccess) return e;
    // the dK/dV kernel also reduces the alpha gradient
    return out_dt == FSA_BF16 ? launch(&bwd_dkdv_kernel<true, true, EXACT>, tiles(p), p, s)
                              : launch(&bwd_dkdv_kernel<false, true, EXACT>, tiles(p), p, s);
}

hipError_t launch_frac_backward(fsa_dtype_t out_dt, const AttnParams &p, hipStream_t s) {
    if (tiles(p) == 0) return launch(&frac_alpha_kernel, 1, p, s);  // writes the zeros of an empty problem
    if (frac_pair_words(p.w) == 4) return launch_frac_window_backward<true>(out_dt, p, s);
    return launch_frac_window_backward<false>(out_dt, p, s);
}

}  // namespace fsa
