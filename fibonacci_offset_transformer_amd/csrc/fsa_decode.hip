// Decode kernel of libfsa (gfx950): the newest query of each sequence against its
// key/value cache, static and learned-alpha tables; with its launchers.
#include "fsa_device.h"

namespace fsa {
namespace {

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

}  // namespace

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

}  // namespace fsa
