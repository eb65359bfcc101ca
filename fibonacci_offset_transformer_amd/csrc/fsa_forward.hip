// Forward kernels of libfsa (gfx950): the general kernel (fp32 inputs, wide windows,
// other scales), the bf16 window kernel with its learned-alpha and rotary
// instantiations, and the dense causal baseline; with their launchers.
#include "fsa_device.h"

namespace fsa {
namespace {

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

// Key row row - off[t] of a slab, or -1 (a row the buffer loads return as zeros without
// touching memory) when BAND and the row lies in the band tiles, which hold rows
// i0 - 64 .. i0 + 63: such rows are read from LDS after the band instead.
template <bool BAND>
__device__ __forceinline__ int band_slab_row(const AttnParams &p, int n_off, int t, int row, int i0) {
    const int x = slab_row(p, n_off, t, row, -1);
    return BAND && x >= i0 - 64 ? -1 : x;
}

// Forward, bf16 inputs, window w <= 64. The workgroup's band keys [i0 - 64, i0 + 64)
// are copied into LDS (K and V row-major) first, with its query rows (read from there
// in the MFMA and in the slab layout; with ROPE they go to registers, to be rotated).
// Once they have landed, the first sparse slabs are requested, in the slab layout, into
// a ring of four row pairs per lane (rows the band tiles hold are read from LDS after
// the band), and the band runs on MFMA while those loads are in flight; its softmax state
// then moves into the slab layout and the slabs continue it as an online softmax, one
// group of four offsets at a time. The slab layout stores O and the LSE.
// With FRAC the table holds fractional entries (learned-alpha variant): entry t's key
// and value for row i are (1 - phi) row(i - off[t]) + phi row(i - off[t] - 1), so each
// entry reads two adjacent slabs (near and far); entries go two per softmax update.
// With ROPE, Q arrives unrotated: the kernel rotates its own query rows by the table
// p.rope and, when p.qhat is set, stores the rotated rows there (for a backward to
// reuse). K arrives rotated (a rotation pass ran first), or, with FUSEK, unrotated: then
// each tile rotates the band rows it copied into LDS, stores its own 64 rows to p.khat,
// publishes this launch's token in its flag once they are in L2, and reads its slab K
// rows from p.khat after the tiles that hold them have published (earlier tiles of the
// same head, dispatched before it on the same XCD, so the waits end; bounded, as in the
// one-launch backward, with NaN output and the status word if a wait gives up).
template <bool OUT_BF16, bool FRAC, bool ROPE = false, int NOFF = 0, bool FUSEK = false>
__global__ void __launch_bounds__(kThreads) fwd_window_kernel(const AttnParams p) {
    static_assert(!FUSEK || (ROPE && !FRAC), "the in-kernel K rotation belongs to the static rotary forward");
    using OE = typename Elem<OUT_BF16>::T;
    __shared__ __attribute__((aligned(16))) uint16_t ks[kTileRows * 64];  // band K rows, then merge areas
    __shared__ __attribute__((aligned(16))) uint16_t vs[kTileRows * 64];  // band V rows, then band row stats
    __shared__ __attribute__((aligned(16))) uint16_t qt[ROPE ? 8 : 64 * 64];  // the tile's query rows

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
    // slab K rows: the caller's (pre-rotated) K, or with FUSEK the rotated rows the tiles store
    const uint16_t *KS = FUSEK ? static_cast<const uint16_t *>(p.khat) + head : K;
    const __amdgpu_buffer_rsrc_t rq = head_rsrc(Q, span_bytes(n, 128)), rk = head_rsrc(KS, span_bytes(n, 128));
    const __amdgpu_buffer_rsrc_t rv = head_rsrc(V, span_bytes(n, 128));
    constexpr int kSlabK = FUSEK ? kCachePastL1 : kCacheNormal;  // rows other tiles wrote in this launch
    const float sl2 = p.scale_log2;
    const int i = r0 + c16;  // MFMA-layout query row
    const bool row_ok = i < n;

    // K and Q first, V after them: the scores start once K and Q (and, with ROPE, the
    // table rows that rotate Q) have landed, while V is still in flight
    [[maybe_unused]] f32x4_t a01, a23, b01, b23;
    if constexpr (ROPE) {
        // the table rows of this tile's positions (the positions past n read as zeros)
        const __amdgpu_buffer_rsrc_t rt = head_rsrc(p.rope + (int64_t)i0 * 64, span_bytes(min(64, n - i0), 256));
        rope_entries(rt, i - i0, g, a01, a23);      // chunk g: pairs 4g .. 4g + 3
        rope_entries(rt, i - i0, g + 4, b01, b23);  // chunk g + 4
    }
    // FUSEK: the band's K rows are rotated in LDS once they have all landed. The tile's own
    // rows (tile rows 64..127, positions i0 ..) take the query rows' table entries (lane
    // (c16, g) of wave w: row 16 w + c16, chunks g and g + 4); the rows before it (tile
    // rows 0..63) take entries of their own, two chunks per lane (positions before 0
    // read as zeros)
    [[maybe_unused]] f32x4_t ktab[2][2];
    if constexpr (FUSEK) {
        const int pos0 = max(i0 - 64, 0);
        const __amdgpu_buffer_rsrc_t rb = head_rsrc(p.rope + (int64_t)pos0 * 64, span_bytes(min(64, n - pos0), 256));
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int idx = threadIdx.x + 256 * j;  // chunk idx & 7 of tile row idx >> 3
            rope_entries(rb, i0 - 64 + (idx >> 3) - pos0, idx & 7, ktab[j][0], ktab[j][1]);
        }
    }
    dma_tile(ks, K, i0 - 64, n, wave, lane);
    Frag<true> qf;
    if constexpr (ROPE) buf_frag(qf, rq, i, g);
    else dma_tile64(qt, Q, i0, n, wave, lane);  // read in both layouts from LDS
    // FUSEK: V is requested once the rotated K rows' stores have completed and the tile's
    // token is out, so that the wait for those stores does not wait for V
    if constexpr (!FUSEK) dma_tile(vs, V, i0 - 64, n, wave, lane);
    // a bare barrier (the compiler's __syncthreads would first wait for every copy into LDS)
    if constexpr (FUSEK) wait_vm_all();
    else wait_vm<4>();  // the four V copies of this wave may still be in flight
    __asm__ volatile("" ::: "memory");
    if constexpr (ROPE) {
        qf.c[0] = rope_chunk(qf.c[0], a01, a23);
        qf.c[1] = rope_chunk(qf.c[1], b01, b23);
    }
    if constexpr (FUSEK) {
        // every wave's K copies have landed; rotate in place with the rotation pass's
        // arithmetic, and store the tile's own rows for the other tiles' slabs and for a
        // backward
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int idx = threadIdx.x + 256 * j, r = idx >> 3, c = idx & 7;
            u32x4_t *slot = reinterpret_cast<u32x4_t *>(ks + r * 64 + 8 * (c ^ (r & 7)));
            *slot = rope_chunk(*slot, ktab[j][0], ktab[j][1]);
        }
        uint16_t *KH = static_cast<uint16_t *>(p.khat) + head;
        const int r = 64 + 16 * wave + c16, pos = i0 + 16 * wave + c16;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int c = g + 4 * h;
            u32x4_t *slot = reinterpret_cast<u32x4_t *>(ks + r * 64 + 8 * (c ^ (r & 7)));
            const u32x4_t x = rope_chunk(*slot, h == 0 ? a01 : b01, h == 0 ? a23 : b23);
            *slot = x;
            if (pos < n) *reinterpret_cast<u32x4_t *>(KH + (int64_t)pos * 64 + 8 * c) = x;
        }
        // the load counter counts stores too: with nothing else outstanding, waiting for
        // zero waits for exactly these stores to reach L2 (V is requested after the token)
        wait_vm_all();
        wait_lds();  // the rotated rows are in LDS before the barrier lets the other waves read them
    }
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    if constexpr (!ROPE) lds_frag(qf, qt, 16 * wave, tl);
    [[maybe_unused]] uint64_t token = 0;
    if constexpr (FUSEK) {
        // every wave's rotated rows are in L2: this tile's token goes out, then V is requested
        token = launch_token();
        if (threadIdx.x == 0) __hip_atomic_store(p.flags + lb, token, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        dma_tile(vs, V, i0 - 64, n, wave, lane);
    }
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
                // rows the band tiles hold are read from LDS after the band instead
                const int a = band_slab_row<!FUSEK>(p, n_off, u, row_s[0], i0);
                const int b = band_slab_row<!FUSEK>(p, n_off, u, row_s[1], i0);
                if constexpr (!FUSEK)  // with FUSEK the K rows follow the wait for their tiles
                    sfrag_load(sk[u], rk, a, b, c8);
                sfrag_load(sv[u], rv, a, b, c8);
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
    if (w == 64 && r0 >= 64 && r0 + 15 < n) {  // uniform: a full window of 64 keys for every row
        // only the oldest block (keys older than the window) and the newest (keys after the
        // row) are cut, at the same lane position: key 4 g + r of the block against row c16
#pragma unroll
        for (int b = 0; b < 5; ++b) {
            Frag<true> kf;
            lds_frag(kf, ks_w, 16 * b, tl);
            const f32x4_t st = mma_over_d(kf, qf, f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool newer = 4 * g + r > c16;
                sc[b][r] = (b == 0 && !newer) || (b == 4 && newer) ? kNegInf : st[r];
                bm = fmaxf(bm, sc[b][r]);
            }
        }
    } else {
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
    // the V copies were issued before the slab loads (at most 4 x 4 of them per wave; the
    // learned-alpha ring always requests its 16; with FUSEK 4 x 2, the V rows only)
    if constexpr (FUSEK) {
        if (n_off >= 4) wait_vm<8>();
        else wait_vm_all();
    } else {
        if (FRAC || n_off >= 4) wait_vm<16>();
        else wait_vm_all();
    }
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    mma_over_rows_tr2(acc_b, vs_w, 0, 16, tl, pr[0], pr[1]);
    mma_over_rows_tr2(acc_b, vs_w, 32, 48, tl, pr[2], pr[3]);
    mma_over_rows_tr(acc_b, vs_w, 64, tl, pr[4]);
    const float l_b = group_sum(lsum_b);

    // FUSEK: wait for the tiles whose rotated rows the slabs read, then request them
    [[maybe_unused]] float o_mul = 1.f;  // NaN if the wait gave up, so that it shows
    if constexpr (FUSEK) {
        __shared__ int gave_up;
        if (wave == 0) {
            // key rows row - off[t] of rows [i0, i0 + 64): tiles (i0 - max off) / 64 .. this
            // one (its own rows it stored itself); earlier tiles only
            const int first = max(0, i0 - p.off[n_off > 0 ? n_off - 1 : 0]) >> 6;
            bool ok = true;
            if (n_off > 0 && first < tile)  // uniform
                ok = poll_tiles(p, p.flags + (int64_t)bh * nt, first, tile - 1, token, lane);
            if (lane == 0) {
                gave_up = ok ? 0 : 1;
                if (!ok) record_give_up(p, token);
            }
        }
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(gave_up)) o_mul = __builtin_nanf("");
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (u < n_off)  // uniform
                sfrag_load<kSlabK>(sk[u], rk, slab_row(p, n_off, u, row_s[0], -1), slab_row(p, n_off, u, row_s[1], -1), c8);
    }

    if constexpr (!FRAC && !FUSEK) {
        // the ring's rows that lie in the band tiles (tile row r = row - i0 + 64 >= 0; r <
        // 128 since every offset is >= 1) come from LDS: offsets below 128 at w = 64, most
        // of the ring at the narrow windows
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (u < n_off) {  // uniform
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = slab_row(p, n_off, u, row_s[h], -1) - i0 + 64;
                    if (r >= 0) {
                        sk[u].r[h] = *reinterpret_cast<const u32x4_t *>(ks + tile_chunk(r, c8));
                        sv[u].r[h] = *reinterpret_cast<const u32x4_t *>(vs + tile_chunk(r, c8));
                    }
                }
            }
        }
    }
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
#pragma unroll
        for (int h = 0; h < 2; ++h) qs.r[h] = *reinterpret_cast<const u32x4_t *>(qt + tile_chunk(16 * wave + s8 + 8 * h, c8));
    }
    // moves the state to a new maximum. Unconditional: where no maximum grew the factor
    // is 2^0 = 1. (Skipping it when no row's maximum grew, the common case after the
    // band's 64 keys, made the compiler copy the whole state around the branch.)
    auto rescale = [&](const float mn[2]) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float al = fast_exp2(m_s[h] - (mn[h] == kNegInf ? 0.f : mn[h]));
            acc_s[h][0] *= al;
            acc_s[h][1] *= al;
            l_s[h] *= al;
            m_s[h] = mn[h];
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
                    sfrag_load<kSlabK>(sk[u], rk, slab_row(p, n_off, u + 4, row_s[0], -1), slab_row(p, n_off, u + 4, row_s[1], -1), c8);
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
            sfrag_load<kSlabK>(kt, rk, row_s[0] - p.off[t], row_s[1] - p.off[t], c8);
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
            // hardware reciprocal and log2 (1 ulp): l >= 1, since the row maximum's term is 1.
            // O goes out with non-temporal stores, which keep it from evicting the K and V
            // rows that other workgroups' slabs still gather from L2
            const float rl = FUSEK ? __builtin_amdgcn_rcpf(l_s[h]) * o_mul : __builtin_amdgcn_rcpf(l_s[h]);
            store_chunk<true>(static_cast<OE *>(p.out) + head, row_s[h], c8, acc_s[h], rl);
            if (c8 == 0)
                p.lse_out[(int64_t)bh * n + row_s[h]] =
                    FUSEK ? (m_s[h] + __builtin_amdgcn_logf(l_s[h])) * kLn2 * o_mul : (m_s[h] + __builtin_amdgcn_logf(l_s[h])) * kLn2;
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

template <int MODE>
hipError_t launch_generic_forward(fsa_dtype_t dt, fsa_dtype_t out_dt, const AttnParams &p, hipStream_t s) {
    if (dt == FSA_BF16)
        return out_dt == FSA_BF16 ? launch(&fwd_kernel<true, true, MODE>, tiles(p), p, s)
                                  : launch(&fwd_kernel<true, false, MODE>, tiles(p), p, s);
    return out_dt == FSA_BF16 ? launch(&fwd_kernel<false, true, MODE>, tiles(p), p, s)
                              : launch(&fwd_kernel<false, false, MODE>, tiles(p), p, s);
}

}  // namespace

hipError_t launch_forward(fsa_dtype_t dt, fsa_dtype_t out_dt, const AttnParams &p, hipStream_t s) {
    if (window_path(dt, p.w, p.n) && p.scale_log2 > 0.f)  // the window kernel folds a positive scale into exponents
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

hipError_t launch_rope_forward(fsa_dtype_t out_dt, const AttnParams &p, hipStream_t s) {
    return with_table_length(p.n_off, [&](auto len) {
        constexpr int L = decltype(len)::value;
        if (p.khat)  // K rotated in the kernel (the caller set the flags and the status word)
            return out_dt == FSA_BF16 ? launch(&fwd_window_kernel<true, false, true, L, true>, tiles(p), p, s)
                                      : launch(&fwd_window_kernel<false, false, true, L, true>, tiles(p), p, s);
        return out_dt == FSA_BF16 ? launch(&fwd_window_kernel<true, false, true, L>, tiles(p), p, s)
                                  : launch(&fwd_window_kernel<false, false, true, L>, tiles(p), p, s);
    });
}

hipError_t launch_frac_forward(fsa_dtype_t out_dt, const AttnParams &p, hipStream_t s) {
    return out_dt == FSA_BF16 ? launch(&fwd_window_kernel<true, true>, tiles(p), p, s)
                              : launch(&fwd_window_kernel<false, true>, tiles(p), p, s);
}

}  // namespace fsa
