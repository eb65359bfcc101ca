// C-ABI layer of libfsa: argument validation, offset-table construction and
// kernel launch on the caller's stream. Declarations and contracts: fsa.h.
//
// Offset tables follow the explainer page "Depth-Staggered Fibonacci Spacing for
// Sparse Attention: Static Schedules Beat Learned Dilation and Extrapolate Where
// Dense Attention Fails" (gist.science), section "Metodologia / Arquitetura e
// Mecanismo de Atenção", items "Conjunto Atendido" (window plus Fibonacci offsets)
// and "Escalonamento" (d_k = alpha * f_k), and section "Controles" (power-of-2
// base). Rounding, reach and deduplication are the library's stated reading:
// round half to even on the double product, base values F < R, set semantics.
//
// This file must be compiled without -ffast-math: the table depends on exact
// IEEE double rounding of alpha * F.

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "fsa_internal.h"

namespace {

thread_local std::string g_last_error;

fsa_status_t fail(fsa_status_t st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

fsa_status_t fail(fsa_status_t st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

fsa_status_t ok() {
    g_last_error.clear();
    return FSA_OK;
}

// Nearest integer to a finite, non-negative double; exact ties go to the even
// neighbour. x - floor(x) is exact in double arithmetic for these magnitudes.
int64_t round_half_even(double x) {
    const double f = std::floor(x);
    const double r = x - f;
    int64_t n = static_cast<int64_t>(f);
    if (r > 0.5 || (r == 0.5 && (n & 1))) ++n;
    return n;
}

// Builds T into out[0..FSA_MAX_OFFSETS) and returns |T|, or -1 with the error set.
int build_table(fsa_base_t base, double alpha, int32_t w, int32_t R, int32_t *out,
                fsa_status_t *st) {
    if (base != FSA_BASE_FIB && base != FSA_BASE_POW2) {
        *st = fail(FSA_E_ARG, "unknown offset base %d", static_cast<int>(base));
        return -1;
    }
    if (!std::isfinite(alpha) || !(alpha > 0.0)) {
        *st = fail(FSA_E_ARG, "alpha must be finite and > 0 (got %g)", alpha);
        return -1;
    }
    if (w < 1) {
        *st = fail(FSA_E_ARG, "window w must be >= 1 (got %d)", w);
        return -1;
    }
    if (R < 1) {
        *st = fail(FSA_E_ARG, "reach R must be >= 1 (got %d)", R);
        return -1;
    }
    int count = 0;
    int64_t a = 1, b = 2;  // Fibonacci: 1, 2, 3, 5, ...; powers of two: 1, 2, 4, ...
    while (a < R) {
        const double x = alpha * static_cast<double>(a);
        // round(x) <= 2^31 - 1 exactly when x < 2^31 - 1/2 (the tie rounds to even 2^31)
        if (!(x < 2147483647.5)) {
            *st = fail(FSA_E_ARG, "alpha * %lld = %.17g does not fit in int32",
                       static_cast<long long>(a), x);
            return -1;
        }
        const int64_t o = round_half_even(x);
        if (o >= w) {
            // insert into the sorted, duplicate-free list
            int pos = 0;
            while (pos < count && out[pos] < o) ++pos;
            if (pos == count || out[pos] != o) {
                if (count == FSA_MAX_OFFSETS) {
                    *st = fail(FSA_E_ARG, "offset table exceeds %d entries", FSA_MAX_OFFSETS);
                    return -1;
                }
                for (int t = count; t > pos; --t) out[t] = out[t - 1];
                out[pos] = static_cast<int32_t>(o);
                ++count;
            }
        }
        if (base == FSA_BASE_FIB) {
            const int64_t c = a + b;
            a = b;
            b = c;
        } else {
            a *= 2;
        }
    }
    return count;
}

// Fractional table of the learned-alpha variant: d = alpha * F (one double product,
// not rounded) for F in the base list below R, kept when d >= w, increasing. Entry t
// gets whole[t] = floor(d), frac[t] = d - floor(d) rounded to float, fb[t] = F.
// Returns the count, or -1 with the error set.
int build_frac_table(fsa_base_t base, double alpha, int32_t w, int32_t R, int32_t *whole, float *frac,
                     int32_t *fb, fsa_status_t *st) {
    int32_t tmp[FSA_MAX_OFFSETS];
    if (build_table(base, alpha, w, R, tmp, st) < 0) return -1;  // the same argument checks
    int count = 0;
    int64_t a = 1, b = 2;
    while (a < R) {
        const double x = alpha * static_cast<double>(a);
        if (!(x < 2147483647.0)) {
            *st = fail(FSA_E_ARG, "alpha * %lld = %.17g does not fit in int32", static_cast<long long>(a), x);
            return -1;
        }
        if (x >= static_cast<double>(w)) {
            if (count == FSA_MAX_OFFSETS) {
                *st = fail(FSA_E_ARG, "fractional table exceeds %d entries", FSA_MAX_OFFSETS);
                return -1;
            }
            const double f = std::floor(x);
            whole[count] = static_cast<int32_t>(f);
            frac[count] = static_cast<float>(x - f);
            fb[count] = static_cast<int32_t>(a);
            ++count;
        }
        if (base == FSA_BASE_FIB) {
            const int64_t c = a + b;
            a = b;
            b = c;
        } else {
            a *= 2;
        }
    }
    return count;  // base values increase and alpha > 0, so d increases
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Shape {
    int32_t B, H, N, d;
};

// Shape, dtype and scale checks common to every attention call.
fsa_status_t check_common(fsa_dtype_t dt, fsa_dtype_t out_dt, const Shape &s, float scale) {
    if (dt != FSA_F32 && dt != FSA_BF16)
        return fail(FSA_E_UNSUPPORTED, "unsupported dtype %d", static_cast<int>(dt));
    if (out_dt != FSA_F32 && out_dt != FSA_BF16)
        return fail(FSA_E_UNSUPPORTED, "unsupported output dtype %d", static_cast<int>(out_dt));
    if (s.B < 0 || s.H < 0 || s.N < 0)
        return fail(FSA_E_ARG, "negative size B=%d H=%d N=%d", s.B, s.H, s.N);
    if (s.d < 1) return fail(FSA_E_ARG, "head size d must be >= 1 (got %d)", s.d);
    if (s.d != fsa::kHeadDim)
        return fail(FSA_E_UNSUPPORTED, "head size d=%d (only 64 is implemented)", s.d);
    if (!std::isfinite(scale)) return fail(FSA_E_ARG, "scale must be finite");
    const int64_t bh = static_cast<int64_t>(s.B) * s.H;
    if (bh > INT32_MAX) return fail(FSA_E_ARG, "B*H=%lld too large", static_cast<long long>(bh));
    const int64_t tiles = (static_cast<int64_t>(s.N) + fsa::kTile - 1) / fsa::kTile;
    if (bh * tiles > INT32_MAX)
        return fail(FSA_E_ARG, "B*H*ceil(N/64)=%lld workgroups exceed the grid limit",
                    static_cast<long long>(bh * tiles));
    return FSA_OK;
}

fsa_status_t check_ptrs(const char *const *names, const void *const *ptrs, int n) {
    for (int i = 0; i < n; ++i) {
        if (!ptrs[i]) return fail(FSA_E_ARG, "%s is NULL", names[i]);
        if (!aligned16(ptrs[i])) return fail(FSA_E_ARG, "%s is not 16-byte aligned", names[i]);
    }
    return FSA_OK;
}

fsa_status_t check_no_alias(const char *const *names, const void *const *ptrs, int n_in, int n) {
    for (int i = n_in; i < n; ++i)
        for (int j = 0; j < n; ++j)
            if (j != i && ptrs[i] == ptrs[j])
                return fail(FSA_E_ARG, "%s aliases %s", names[i], names[j]);
    return FSA_OK;
}

// Keeps only offsets that reach a key for some row (offset < N); sorted input.
int trim_offsets(int32_t *off, int count, int32_t N) {
    int c = 0;
    while (c < count && off[c] < N) ++c;
    return c;
}

// Set by fsa_debug_force_wait_timeout: the one-launch backward's waits then look for a
// value no workgroup publishes and give up after a few polls.
std::atomic<int> g_force_give_up{0};

void set_wait_limits(fsa::AttnParams &p) {
    const bool forced = g_force_give_up.load(std::memory_order_relaxed) != 0;
    p.max_polls = forced ? 16 : fsa::kMaxPolls;
    p.token_xor = forced ? 1u : 0u;
}

fsa_status_t launched(hipError_t e, const char *what) {
    if (e != hipSuccess)
        return fail(FSA_E_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

namespace fsa {
// Sets the calling thread's error text (for the C-ABI functions of other sources).
fsa_status_t set_error(fsa_status_t st, const char *msg) { return fail(st, "%s", msg); }
}  // namespace fsa

extern "C" {

fsa_status_t fsa_build_offsets(fsa_base_t base, double alpha, int32_t w, int32_t R,
                               int32_t *out, int32_t capacity, int32_t *count) {
    if (!count) return fail(FSA_E_ARG, "count is NULL");
    if (capacity < 0) return fail(FSA_E_ARG, "capacity must be >= 0");
    int32_t tab[FSA_MAX_OFFSETS];
    fsa_status_t st = FSA_OK;
    const int n = build_table(base, alpha, w, R, tab, &st);
    if (n < 0) return st;
    *count = n;
    if (n > capacity)
        return fail(FSA_E_CAPACITY, "offset table has %d entries, capacity is %d", n, capacity);
    if (n > 0 && !out) return fail(FSA_E_ARG, "out is NULL");
    if (n > 0) std::memcpy(out, tab, sizeof(int32_t) * static_cast<size_t>(n));
    return ok();
}

fsa_status_t fsa_forward(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k, const void *v, void *o,
                         float *lse, int32_t B, int32_t H, int32_t N, int32_t d, float scale,
                         fsa_base_t base, double alpha, int32_t w, int32_t R, void *stream) {
    const Shape s{B, H, N, d};
    fsa_status_t st = check_common(dt, out_dt, s, scale);
    if (st != FSA_OK) return st;
    fsa::AttnParams p{};
    const int n_off = build_table(base, alpha, w, R, p.off, &st);
    if (n_off < 0) return st;
    if (static_cast<int64_t>(B) * H * N == 0) return ok();
    const char *names[] = {"q", "k", "v", "o", "lse"};
    const void *ptrs[] = {q, k, v, o, lse};
    if ((st = check_ptrs(names, ptrs, 5)) != FSA_OK) return st;
    if ((st = check_no_alias(names, ptrs, 3, 5)) != FSA_OK) return st;
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = o;
    p.lse_out = lse;
    p.bh = B * H;
    p.n = N;
    p.w = w;
    p.n_off = trim_offsets(p.off, n_off, N);
    p.scale = scale;
    p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    return launched(fsa::launch_forward(dt, out_dt, p, static_cast<hipStream_t>(stream)), "forward");
}

fsa_status_t fsa_backward_delta(fsa_dtype_t dt, const void *o, const void *dout, float *delta_ws,
                                int32_t B, int32_t H, int32_t N, int32_t d, void *stream) {
    const Shape s{B, H, N, d};
    fsa_status_t st = check_common(dt, dt, s, 1.0f);
    if (st != FSA_OK) return st;
    if (static_cast<int64_t>(B) * H * N == 0) return ok();
    const char *names[] = {"o", "dout", "delta_ws"};
    const void *ptrs[] = {o, dout, delta_ws};
    if ((st = check_ptrs(names, ptrs, 3)) != FSA_OK) return st;
    if ((st = check_no_alias(names, ptrs, 2, 3)) != FSA_OK) return st;
    fsa::AttnParams p{};
    p.o = o;
    p.dout = dout;
    p.delta = delta_ws;
    p.bh = B * H;
    p.n = N;
    return launched(fsa::launch_backward_delta(dt, p, static_cast<hipStream_t>(stream)), "backward delta");
}

namespace {

// Validates the arguments of the gradient stage and fills its kernel parameters.
fsa_status_t prepare_grads(fsa::AttnParams &p, fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q,
                           const void *k, const void *v, const float *lse, const void *dout,
                           const float *delta, void *dq, void *dk, void *dv, void *pair_ws,
                           uint64_t pair_ws_bytes, int32_t B, int32_t H, int32_t N, int32_t d, float scale,
                           fsa_base_t base, double alpha, int32_t w, int32_t R, bool *empty) {
    const Shape s{B, H, N, d};
    fsa_status_t st = check_common(dt, out_dt, s, scale);
    if (st != FSA_OK) return st;
    const int n_off = build_table(base, alpha, w, R, p.off, &st);
    if (n_off < 0) return st;
    *empty = static_cast<int64_t>(B) * H * N == 0;
    if (*empty) return FSA_OK;
    p.n_off = trim_offsets(p.off, n_off, N);
    const int64_t words = fsa::pair_words(dt, w, N, static_cast<int64_t>(B) * H, p.n_off);
    const uint64_t need = fsa::pair_ws_bytes(dt, w, N, static_cast<int64_t>(B) * H, p.n_off);
    const int np = need > 0 ? 10 : 9;  // the pair workspace is checked only when it is used
    const char *names[] = {"q", "k", "v", "lse", "dout", "delta", "dq", "dk", "dv", "pair_ws"};
    const void *ptrs[] = {q, k, v, lse, dout, delta, dq, dk, dv, pair_ws};
    if ((st = check_ptrs(names, ptrs, np)) != FSA_OK) return st;
    if ((st = check_no_alias(names, ptrs, 6, np)) != FSA_OK) return st;
    if (pair_ws_bytes < need)
        return fail(FSA_E_ARG, "pair_ws holds %llu bytes, this problem needs %llu",
                    static_cast<unsigned long long>(pair_ws_bytes), static_cast<unsigned long long>(need));
    p.q = q;
    p.k = k;
    p.v = v;
    p.lse_in = lse;
    p.dout = dout;
    p.delta = const_cast<float *>(delta);
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.pairs = need > 0 ? static_cast<uint32_t *>(pair_ws) : nullptr;
    p.flags = need > 0 ? reinterpret_cast<uint64_t *>(static_cast<char *>(pair_ws) + fsa::pair_ws_flags_offset(words))
                       : nullptr;
    p.status = need > 0 ? reinterpret_cast<uint64_t *>(static_cast<char *>(pair_ws) +
                                                       fsa::pair_ws_status_offset(words, static_cast<int64_t>(B) * H, N))
                        : nullptr;
    set_wait_limits(p);
    p.bh = B * H;
    p.n = N;
    p.w = w;
    p.scale = scale;
    p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    return FSA_OK;
}

}  // namespace

fsa_status_t fsa_backward_workspace_bytes(fsa_dtype_t dt, int32_t B, int32_t H, int32_t N, int32_t d,
                                          fsa_base_t base, double alpha, int32_t w, int32_t R,
                                          uint64_t *bytes) {
    if (!bytes) return fail(FSA_E_ARG, "bytes is NULL");
    const Shape s{B, H, N, d};
    fsa_status_t st = check_common(dt, dt, s, 1.0f);
    if (st != FSA_OK) return st;
    int32_t tab[FSA_MAX_OFFSETS];
    const int n_off = build_table(base, alpha, w, R, tab, &st);
    if (n_off < 0) return st;
    *bytes = fsa::pair_ws_bytes(dt, w, N, static_cast<int64_t>(B) * H, trim_offsets(tab, n_off, N));
    return ok();
}

fsa_status_t fsa_backward_grads(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k,
                                const void *v, const float *lse, const void *dout,
                                const float *delta, void *dq, void *dk, void *dv, void *pair_ws,
                                uint64_t pair_ws_bytes, int32_t B, int32_t H, int32_t N, int32_t d,
                                float scale, fsa_base_t base, double alpha, int32_t w, int32_t R,
                                void *stream) {
    fsa::AttnParams p{};
    bool empty = false;
    fsa_status_t st = prepare_grads(p, dt, out_dt, q, k, v, lse, dout, delta, dq, dk, dv, pair_ws,
                                    pair_ws_bytes, B, H, N, d, scale, base, alpha, w, R, &empty);
    if (st != FSA_OK) return st;
    if (empty) return ok();
    return launched(fsa::launch_backward_grads(dt, out_dt, p, static_cast<hipStream_t>(stream), false),
                    "backward grads");
}

fsa_status_t fsa_backward(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k, const void *v,
                          const void *o, const float *lse, const void *dout, void *dq, void *dk,
                          void *dv, float *delta_ws, void *pair_ws, uint64_t pair_ws_bytes, int32_t B,
                          int32_t H, int32_t N, int32_t d, float scale, fsa_base_t base, double alpha,
                          int32_t w, int32_t R, void *stream) {
    fsa::AttnParams p{};
    bool empty = false;
    fsa_status_t st = prepare_grads(p, dt, out_dt, q, k, v, lse, dout, delta_ws, dq, dk, dv, pair_ws,
                                    pair_ws_bytes, B, H, N, d, scale, base, alpha, w, R, &empty);
    if (st != FSA_OK) return st;
    if (empty) return ok();
    // delta_ws is written here, so it must not alias any input either
    const bool use_pairs = p.pairs != nullptr;
    const int np = use_pairs ? 11 : 10;
    const char *names[] = {"q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "delta_ws", "pair_ws"};
    const void *ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv, delta_ws, pair_ws};
    if ((st = check_ptrs(names, ptrs, np)) != FSA_OK) return st;
    if ((st = check_no_alias(names, ptrs, 6, np)) != FSA_OK) return st;
    p.o = o;
    return launched(fsa::launch_backward_grads(dt, out_dt, p, static_cast<hipStream_t>(stream), true),
                    "backward");
}

fsa_status_t fsa_decode(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k_cache,
                        const void *v_cache, const int32_t *seq_lens, void *o, float *lse, int32_t B, int32_t H,
                        int32_t Lmax, int32_t d, float scale, fsa_base_t base, double alpha, int32_t w, int32_t R,
                        void *stream) {
    const Shape s{B, H, Lmax, d};
    fsa_status_t st = check_common(dt, out_dt, s, scale);
    if (st != FSA_OK) return st;
    fsa::AttnParams p{};
    const int n_off = build_table(base, alpha, w, R, p.off, &st);
    if (n_off < 0) return st;
    if (static_cast<int64_t>(B) * H == 0) return ok();
    if (Lmax < 1) return fail(FSA_E_ARG, "Lmax must be >= 1 (the cache holds at least the newest token)");
    const char *names[] = {"q", "k_cache", "v_cache", "o", "lse"};
    const void *ptrs[] = {q, k_cache, v_cache, o, lse};
    if ((st = check_ptrs(names, ptrs, 5)) != FSA_OK) return st;
    if (!seq_lens) return fail(FSA_E_ARG, "seq_lens is NULL");
    if (reinterpret_cast<uintptr_t>(seq_lens) & 3u) return fail(FSA_E_ARG, "seq_lens is not 4-byte aligned");
    const char *names6[] = {"q", "k_cache", "v_cache", "seq_lens", "o", "lse"};
    const void *ptrs6[] = {q, k_cache, v_cache, seq_lens, o, lse};
    if ((st = check_no_alias(names6, ptrs6, 4, 6)) != FSA_OK) return st;
    p.q = q;
    p.k = k_cache;
    p.v = v_cache;
    p.out = o;
    p.lse_out = lse;
    p.seq_lens = seq_lens;
    p.bh = B * H;
    p.heads = H;
    p.lmax = Lmax;
    p.n = Lmax;
    p.w = w;
    p.n_off = trim_offsets(p.off, n_off, Lmax);
    p.scale = scale;
    p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    return launched(fsa::launch_decode(dt, out_dt, p, static_cast<hipStream_t>(stream)), "decode");
}

fsa_status_t fsa_dense_forward(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k, const void *v,
                               void *o, float *lse, int32_t B, int32_t H, int32_t N, int32_t d,
                               float scale, void *stream) {
    const Shape s{B, H, N, d};
    fsa_status_t st = check_common(dt, out_dt, s, scale);
    if (st != FSA_OK) return st;
    if (static_cast<int64_t>(B) * H * N == 0) return ok();
    const char *names[] = {"q", "k", "v", "o", "lse"};
    const void *ptrs[] = {q, k, v, o, lse};
    if ((st = check_ptrs(names, ptrs, 5)) != FSA_OK) return st;
    if ((st = check_no_alias(names, ptrs, 3, 5)) != FSA_OK) return st;
    // Dense causal attention is the window case with w = N and no sparse offsets.
    fsa::AttnParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = o;
    p.lse_out = lse;
    p.bh = B * H;
    p.n = N;
    p.w = N;
    p.n_off = 0;
    p.scale = scale;
    p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    return launched(fsa::launch_dense_forward(dt, out_dt, p, static_cast<hipStream_t>(stream)), "dense forward");
}

fsa_status_t fsa_frac_offsets(fsa_base_t base, double alpha, int32_t w, int32_t R, int32_t *whole,
                              float *frac, int32_t *base_value, int32_t capacity, int32_t *count) {
    if (!count) return fail(FSA_E_ARG, "count is NULL");
    if (capacity < 0) return fail(FSA_E_ARG, "capacity must be >= 0");
    int32_t wh[FSA_MAX_OFFSETS], fb[FSA_MAX_OFFSETS];
    float fr[FSA_MAX_OFFSETS];
    fsa_status_t st = FSA_OK;
    const int n = build_frac_table(base, alpha, w, R, wh, fr, fb, &st);
    if (n < 0) return st;
    *count = n;
    if (n > capacity)
        return fail(FSA_E_CAPACITY, "fractional table has %d entries, capacity is %d", n, capacity);
    if (n > 0 && (!whole || !frac || !base_value)) return fail(FSA_E_ARG, "an output array is NULL");
    for (int t = 0; t < n; ++t) {
        whole[t] = wh[t];
        frac[t] = fr[t];
        base_value[t] = fb[t];
    }
    return ok();
}

namespace {

// Checks shared by the fractional calls and their table, trimmed to the entries some
// row of length N reaches (first row floor(d) + (frac != 0) < N).
fsa_status_t prepare_frac(fsa::AttnParams &p, fsa_dtype_t dt, fsa_dtype_t out_dt, int32_t B, int32_t H, int32_t N,
                          int32_t d, float scale, fsa_base_t base, double alpha, int32_t w, int32_t R) {
    const Shape s{B, H, N, d};
    fsa_status_t st = check_common(dt, out_dt, s, scale);
    if (st != FSA_OK) return st;
    int32_t fb[FSA_MAX_OFFSETS];
    const int n = build_frac_table(base, alpha, w, R, p.off, p.phi, fb, &st);
    if (n < 0) return st;
    if (dt != FSA_BF16) return fail(FSA_E_UNSUPPORTED, "fractional entries are implemented for bf16 inputs only");
    if (w > 64) return fail(FSA_E_UNSUPPORTED, "fractional entries need a window w <= 64 (got %d)", w);
    if (N > (1 << 24)) return fail(FSA_E_UNSUPPORTED, "fractional entries need N <= 2^24 (got %d)", N);
    if (!(scale > 0.f)) return fail(FSA_E_UNSUPPORTED, "fractional entries need a positive scale");
    int used = 0;
    while (used < n && p.off[used] + (p.phi[used] != 0.f ? 1 : 0) < N) ++used;
    if (!fsa::pair_offsets_fit(N, used, fsa::frac_pair_words(w)))
        return fail(FSA_E_UNSUPPORTED, "fractional entries: N = %d with %d entries exceeds 32-bit pair offsets", N, used);
    for (int t = 0; t < n; ++t) p.fbase[t] = static_cast<float>(fb[t]);
    p.n_entries = n;
    p.n_off = used;
    p.bh = B * H;
    p.n = N;
    p.w = w;
    p.scale = scale;
    p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    return FSA_OK;
}

}  // namespace

fsa_status_t fsa_frac_forward(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k, const void *v,
                              void *o, float *lse, int32_t B, int32_t H, int32_t N, int32_t d, float scale,
                              fsa_base_t base, double alpha, int32_t w, int32_t R, void *stream) {
    fsa::AttnParams p{};
    fsa_status_t st = prepare_frac(p, dt, out_dt, B, H, N, d, scale, base, alpha, w, R);
    if (st != FSA_OK) return st;
    if (static_cast<int64_t>(B) * H * N == 0) return ok();
    const char *names[] = {"q", "k", "v", "o", "lse"};
    const void *ptrs[] = {q, k, v, o, lse};
    if ((st = check_ptrs(names, ptrs, 5)) != FSA_OK) return st;
    if ((st = check_no_alias(names, ptrs, 3, 5)) != FSA_OK) return st;
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = o;
    p.lse_out = lse;
    return launched(fsa::launch_frac_forward(out_dt, p, static_cast<hipStream_t>(stream)), "fractional forward");
}

fsa_status_t fsa_frac_backward_workspace_bytes(fsa_dtype_t dt, int32_t B, int32_t H, int32_t N, int32_t d,
                                               fsa_base_t base, double alpha, int32_t w, int32_t R,
                                               uint64_t *bytes) {
    if (!bytes) return fail(FSA_E_ARG, "bytes is NULL");
    fsa::AttnParams p{};
    const fsa_status_t st = prepare_frac(p, dt, dt, B, H, N, d, 1.0f, base, alpha, w, R);
    if (st != FSA_OK) return st;
    *bytes = fsa::frac_workspace(static_cast<int64_t>(B) * H, N, p.n_off, w).total;
    return ok();
}

fsa_status_t fsa_frac_backward(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k, const void *v,
                               const void *o, const float *lse, const void *dout, void *dq, void *dk, void *dv,
                               float *dalpha, float *doffs, void *ws, uint64_t ws_bytes, int32_t B, int32_t H,
                               int32_t N, int32_t d, float scale, fsa_base_t base, double alpha, int32_t w,
                               int32_t R, void *stream) {
    fsa::AttnParams p{};
    fsa_status_t st = prepare_frac(p, dt, out_dt, B, H, N, d, scale, base, alpha, w, R);
    if (st != FSA_OK) return st;
    if (!dalpha) return fail(FSA_E_ARG, "dalpha is NULL");
    if (reinterpret_cast<uintptr_t>(dalpha) & 3u) return fail(FSA_E_ARG, "dalpha is not 4-byte aligned");
    if (doffs && (reinterpret_cast<uintptr_t>(doffs) & 3u)) return fail(FSA_E_ARG, "doffs is not 4-byte aligned");
    const bool empty = static_cast<int64_t>(B) * H * N == 0;
    if (!empty) {
        const uint64_t need = fsa::frac_workspace(static_cast<int64_t>(B) * H, N, p.n_off, w).total;
        const char *names[] = {"q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "ws"};
        const void *ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv, ws};
        if ((st = check_ptrs(names, ptrs, 10)) != FSA_OK) return st;
        if ((st = check_no_alias(names, ptrs, 6, 10)) != FSA_OK) return st;
        if (ws_bytes < need)
            return fail(FSA_E_ARG, "ws holds %llu bytes, this problem needs %llu",
                        static_cast<unsigned long long>(ws_bytes), static_cast<unsigned long long>(need));
    }
    // the gradient outputs are written by the kernels, so they must not alias each other or inputs
    const void *outs[] = {dalpha, doffs, dq, dk, dv, ws, q, k, v, o, lse, dout};
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 12; ++j)
            if (j != i && outs[i] && outs[i] == outs[j])
                return fail(FSA_E_ARG, "%s aliases another argument", i == 0 ? "dalpha" : "doffs");
    p.dalpha = dalpha;
    p.doffs = doffs;
    if (!empty) {
        const fsa::FracWorkspace lay = fsa::frac_workspace(p.bh, N, p.n_off, w);
        char *base_ws = static_cast<char *>(ws);
        p.q = q;
        p.k = k;
        p.v = v;
        p.o = o;
        p.lse_in = lse;
        p.dout = dout;
        p.dq = dq;
        p.dk = dk;
        p.dv = dv;
        p.delta = reinterpret_cast<float *>(base_ws + lay.delta);
        p.pairs = reinterpret_cast<uint32_t *>(base_ws + lay.pairs);
        p.dd_part = reinterpret_cast<float *>(base_ws + lay.partials);
        p.flags = reinterpret_cast<uint64_t *>(base_ws + lay.flags);
        p.status = reinterpret_cast<uint64_t *>(base_ws + lay.status);
        set_wait_limits(p);
    } else {
        p.bh = 0;  // no tiles: only the alpha reduction runs, writing zeros
    }
    return launched(fsa::launch_frac_backward(out_dt, p, static_cast<hipStream_t>(stream)), "fractional backward");
}

fsa_status_t fsa_rope_table(int32_t n_pos, int32_t d, double rope_base, float *table) {
    if (n_pos < 0) return fail(FSA_E_ARG, "n_pos must be >= 0 (got %d)", n_pos);
    if (d < 2 || (d & 1)) return fail(FSA_E_ARG, "d must be even and >= 2 (got %d)", d);
    if (!std::isfinite(rope_base) || !(rope_base > 0.0))
        return fail(FSA_E_ARG, "rope_base must be finite and > 0 (got %g)", rope_base);
    if (n_pos > 0 && !table) return fail(FSA_E_ARG, "table is NULL");
    const int half = d / 2;
    for (int m = 0; m < half; ++m) {
        const double theta = std::pow(rope_base, -2.0 * m / d);
        for (int32_t pos = 0; pos < n_pos; ++pos) {
            const double a = pos * theta;
            table[(static_cast<int64_t>(pos) * half + m) * 2] = static_cast<float>(std::cos(a));
            table[(static_cast<int64_t>(pos) * half + m) * 2 + 1] = static_cast<float>(std::sin(a));
        }
    }
    return ok();
}

namespace {

// Rotates `count` bf16 tensors [B*H*N, 64] on the stream (x[t] -> out[t]).
hipError_t rotate_rows(const void *const *x, void *const *out, int count, const float *rope, int64_t rows,
                       int32_t n, hipStream_t stream) {
    fsa::RopeParams rp{};
    for (int t = 0; t < count; ++t) {
        rp.x[t] = static_cast<const uint16_t *>(x[t]);
        rp.out[t] = static_cast<uint16_t *>(out[t]);
    }
    rp.table = rope;
    rp.rows = rows;
    rp.n = n;
    rp.count = count;
    return fsa::launch_rope(rp, stream);
}


// Path checks shared by the fused rotary calls.
// n_off: the table's length before trimming to N.
fsa_status_t check_rope_path(fsa_dtype_t dt, int32_t w, int32_t N, float scale, int32_t n_pos, int32_t n_off) {
    if (dt != FSA_BF16) return fail(FSA_E_UNSUPPORTED, "the rotary path stores rotated rows in bf16: bf16 inputs only");
    if (w > 64) return fail(FSA_E_UNSUPPORTED, "the rotary path needs a window w <= 64 (got %d)", w);
    if (N > (1 << 24)) return fail(FSA_E_UNSUPPORTED, "the rotary path needs N <= 2^24 (got %d)", N);
    if (!fsa::pair_offsets_fit(N, n_off, fsa::pair_slot_words(w)))
        return fail(FSA_E_UNSUPPORTED, "the rotary path: N = %d with %d offsets exceeds 32-bit pair offsets", N, n_off);
    if (!(scale > 0.f)) return fail(FSA_E_UNSUPPORTED, "the rotary path needs a positive scale");
    if (n_pos < N) return fail(FSA_E_ARG, "the rotary table has %d positions, the sequence %d", n_pos, N);
    return FSA_OK;
}

struct RopeLayout {
    uint64_t qhat, khat, fflags, fstatus, delta, pairs, fwd, bwd;  // byte offsets into ws and the two sizes
    int64_t words;                                                // pair words of the static backward's workspace
};

// The forward's part: rotated Q rows, rotated K rows, then the forward's per-tile tokens
// and status word (the forward that rotates K itself, B * H a multiple of 8).
RopeLayout rope_layout(int64_t bh, int32_t n, int32_t n_off, int32_t w) {
    RopeLayout l;
    const uint64_t rows = static_cast<uint64_t>(bh) * n;
    l.qhat = 0;
    l.khat = fsa::align256(rows * 128);
    l.fflags = l.khat + fsa::align256(rows * 128);
    l.fstatus = l.fflags + 8ull * static_cast<uint64_t>(bh) * ((n + 63) / 64);
    l.fwd = fsa::align256(l.fstatus + 8);
    l.delta = l.fwd;
    l.pairs = l.delta + fsa::align256(rows * 4);
    l.words = fsa::pair_words(FSA_BF16, w, n, bh, n_off);
    l.bwd = l.pairs + fsa::align256(fsa::pair_ws_bytes(FSA_BF16, w, n, bh, n_off));
    return l;
}

}  // namespace

fsa_status_t fsa_rope_rotate(fsa_dtype_t dt, const void *x, const float *rope, int32_t n_pos, void *out, int32_t B,
                             int32_t H, int32_t N, int32_t d, void *stream) {
    const Shape s{B, H, N, d};
    fsa_status_t st = check_common(dt, dt, s, 1.0f);
    if (st != FSA_OK) return st;
    if (dt != FSA_BF16) return fail(FSA_E_UNSUPPORTED, "rotation is implemented for bf16 rows only");
    if (N > (1 << 24)) return fail(FSA_E_UNSUPPORTED, "rotation needs N <= 2^24 (got %d)", N);
    if (n_pos < N) return fail(FSA_E_ARG, "the rotary table has %d positions, the sequence %d", n_pos, N);
    if (static_cast<int64_t>(B) * H * N == 0) return ok();
    const char *names[] = {"x", "rope", "out"};
    const void *ptrs[] = {x, rope, out};
    if ((st = check_ptrs(names, ptrs, 3)) != FSA_OK) return st;
    if ((st = check_no_alias(names, ptrs, 2, 3)) != FSA_OK) return st;
    const void *xs[] = {x};
    void *outs[] = {out};
    return launched(rotate_rows(xs, outs, 1, rope, static_cast<int64_t>(B) * H * N, N, static_cast<hipStream_t>(stream)),
                    "rotary rotation");
}

fsa_status_t fsa_rope_workspace_bytes(fsa_dtype_t dt, int32_t B, int32_t H, int32_t N, int32_t d, fsa_base_t base,
                                      double alpha, int32_t w, int32_t R, uint64_t *fwd_bytes, uint64_t *bwd_bytes) {
    if (!fwd_bytes || !bwd_bytes) return fail(FSA_E_ARG, "fwd_bytes or bwd_bytes is NULL");
    const Shape s{B, H, N, d};
    fsa_status_t st = check_common(dt, dt, s, 1.0f);
    if (st != FSA_OK) return st;
    int32_t tab[FSA_MAX_OFFSETS];
    const int n_off = build_table(base, alpha, w, R, tab, &st);
    if (n_off < 0) return st;
    if ((st = check_rope_path(dt, w, N, 1.0f, N, n_off)) != FSA_OK) return st;
    const RopeLayout l = rope_layout(static_cast<int64_t>(B) * H, N, trim_offsets(tab, n_off, N), w);
    *fwd_bytes = static_cast<int64_t>(B) * H * N == 0 ? 0 : l.fwd;
    *bwd_bytes = static_cast<int64_t>(B) * H * N == 0 ? 0 : l.bwd;
    return ok();
}

fsa_status_t fsa_rope_forward(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k, const void *v,
                              const float *rope, int32_t n_pos, void *o, float *lse, void *ws, uint64_t ws_bytes,
                              int32_t keep_rotated, int32_t B, int32_t H, int32_t N, int32_t d, float scale,
                              fsa_base_t base, double alpha, int32_t w, int32_t R, void *stream) {
    const Shape s{B, H, N, d};
    fsa_status_t st = check_common(dt, out_dt, s, scale);
    if (st != FSA_OK) return st;
    fsa::AttnParams p{};
    const int n_off = build_table(base, alpha, w, R, p.off, &st);
    if (n_off < 0) return st;
    if ((st = check_rope_path(dt, w, N, scale, n_pos, n_off)) != FSA_OK) return st;
    if (static_cast<int64_t>(B) * H * N == 0) return ok();
    const char *names[] = {"q", "k", "v", "rope", "o", "lse", "ws"};
    const void *ptrs[] = {q, k, v, rope, o, lse, ws};
    if ((st = check_ptrs(names, ptrs, 7)) != FSA_OK) return st;
    if ((st = check_no_alias(names, ptrs, 4, 7)) != FSA_OK) return st;
    p.n_off = trim_offsets(p.off, n_off, N);
    const RopeLayout l = rope_layout(static_cast<int64_t>(B) * H, N, p.n_off, w);
    if (ws_bytes < l.fwd)
        return fail(FSA_E_ARG, "ws holds %llu bytes, this problem needs %llu",
                    static_cast<unsigned long long>(ws_bytes), static_cast<unsigned long long>(l.fwd));
    char *wsb = static_cast<char *>(ws);
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    // The forward kernel rotates its own Q rows (and leaves them in ws with keep_rotated).
    // With B * H a multiple of 8 (each XCD holds whole heads) it also rotates K: every tile
    // rotates the band rows it copies and stores its own rows in ws, where the other tiles'
    // slabs read them once its token is set. Otherwise a rotation pass rotates K first.
    p.q = q;
    if (static_cast<int64_t>(B) * H % 8 == 0) {
        p.k = k;
        p.khat = wsb + l.khat;
        p.flags = reinterpret_cast<uint64_t *>(wsb + l.fflags);
        p.status = reinterpret_cast<uint64_t *>(wsb + l.fstatus);
        set_wait_limits(p);
    } else {
        const void *xs[] = {k};
        void *hats[] = {wsb + l.khat};
        const hipError_t e = rotate_rows(xs, hats, 1, rope, static_cast<int64_t>(B) * H * N, N, hs);
        if (e != hipSuccess) return launched(e, "rotary rotation");
        p.k = hats[0];
    }
    p.v = v;
    p.out = o;
    p.lse_out = lse;
    p.rope = rope;
    p.qhat = keep_rotated ? wsb + l.qhat : nullptr;
    p.bh = B * H;
    p.n = N;
    p.w = w;
    p.scale = scale;
    p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    return launched(fsa::launch_rope_forward(out_dt, p, hs), "rotary forward");
}

fsa_status_t fsa_rope_backward(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k, const void *v,
                               const float *rope, int32_t n_pos, const void *o, const float *lse, const void *dout,
                               void *dq, void *dk, void *dv, void *ws, uint64_t ws_bytes, int32_t reuse_rotated,
                               int32_t B, int32_t H, int32_t N, int32_t d, float scale, fsa_base_t base, double alpha,
                               int32_t w, int32_t R, void *stream) {
    const Shape s{B, H, N, d};
    fsa_status_t st = check_common(dt, out_dt, s, scale);
    if (st != FSA_OK) return st;
    fsa::AttnParams p{};
    const int n_off = build_table(base, alpha, w, R, p.off, &st);
    if (n_off < 0) return st;
    if ((st = check_rope_path(dt, w, N, scale, n_pos, n_off)) != FSA_OK) return st;
    if (static_cast<int64_t>(B) * H * N == 0) return ok();
    const char *names[] = {"q", "k", "v", "rope", "o", "lse", "dout", "dq", "dk", "dv", "ws"};
    const void *ptrs[] = {q, k, v, rope, o, lse, dout, dq, dk, dv, ws};
    if ((st = check_ptrs(names, ptrs, 11)) != FSA_OK) return st;
    if ((st = check_no_alias(names, ptrs, 7, 11)) != FSA_OK) return st;
    p.n_off = trim_offsets(p.off, n_off, N);
    const RopeLayout l = rope_layout(static_cast<int64_t>(B) * H, N, p.n_off, w);
    if (ws_bytes < l.bwd)
        return fail(FSA_E_ARG, "ws holds %llu bytes, this problem needs %llu",
                    static_cast<unsigned long long>(ws_bytes), static_cast<unsigned long long>(l.bwd));
    char *wsb = static_cast<char *>(ws);
    const void *xs[] = {q, k};
    void *hats[] = {wsb + l.qhat, wsb + l.khat};
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    if (!reuse_rotated) {  // otherwise ws already holds the forward's rotated rows of these q, k
        const hipError_t e = rotate_rows(xs, hats, 2, rope, static_cast<int64_t>(B) * H * N, N, hs);
        if (e != hipSuccess) return launched(e, "rotary rotation");
    }
    p.q = hats[0];
    p.k = hats[1];
    p.v = v;
    p.o = o;
    p.lse_in = lse;
    p.dout = dout;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.delta = reinterpret_cast<float *>(wsb + l.delta);
    p.pairs = p.n_off > 0 ? reinterpret_cast<uint32_t *>(wsb + l.pairs) : nullptr;
    p.flags = p.n_off > 0 ? reinterpret_cast<uint64_t *>(wsb + l.pairs + fsa::pair_ws_flags_offset(l.words)) : nullptr;
    p.status = p.n_off > 0 ? reinterpret_cast<uint64_t *>(
                                 wsb + l.pairs + fsa::pair_ws_status_offset(l.words, static_cast<int64_t>(B) * H, N))
                           : nullptr;
    set_wait_limits(p);
    p.rope = rope;
    p.bh = B * H;
    p.n = N;
    p.w = w;
    p.scale = scale;
    p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    return launched(fsa::launch_backward_grads(dt, out_dt, p, hs, true), "rotary backward");
}

fsa_status_t fsa_frac_decode(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k_cache,
                             const void *v_cache, const int32_t *seq_lens, void *o, float *lse, int32_t B, int32_t H,
                             int32_t Lmax, int32_t d, float scale, fsa_base_t base, double alpha, int32_t w,
                             int32_t R, void *stream) {
    const Shape s{B, H, Lmax, d};
    fsa_status_t st = check_common(dt, out_dt, s, scale);
    if (st != FSA_OK) return st;
    fsa::AttnParams p{};
    int32_t fb[FSA_MAX_OFFSETS];
    const int n = build_frac_table(base, alpha, w, R, p.off, p.phi, fb, &st);
    if (n < 0) return st;
    if (static_cast<int64_t>(B) * H == 0) return ok();
    if (Lmax < 1) return fail(FSA_E_ARG, "Lmax must be >= 1 (the cache holds at least the newest token)");
    const char *names[] = {"q", "k_cache", "v_cache", "o", "lse"};
    const void *ptrs[] = {q, k_cache, v_cache, o, lse};
    if ((st = check_ptrs(names, ptrs, 5)) != FSA_OK) return st;
    if (!seq_lens) return fail(FSA_E_ARG, "seq_lens is NULL");
    if (reinterpret_cast<uintptr_t>(seq_lens) & 3u) return fail(FSA_E_ARG, "seq_lens is not 4-byte aligned");
    const char *names6[] = {"q", "k_cache", "v_cache", "seq_lens", "o", "lse"};
    const void *ptrs6[] = {q, k_cache, v_cache, seq_lens, o, lse};
    if ((st = check_no_alias(names6, ptrs6, 4, 6)) != FSA_OK) return st;
    int used = 0;  // entries some cached position reaches: first row floor(d) + (frac != 0) < Lmax
    while (used < n && p.off[used] + (p.phi[used] != 0.f ? 1 : 0) < Lmax) ++used;
    p.q = q;
    p.k = k_cache;
    p.v = v_cache;
    p.out = o;
    p.lse_out = lse;
    p.seq_lens = seq_lens;
    p.bh = B * H;
    p.heads = H;
    p.lmax = Lmax;
    p.n = Lmax;
    p.w = w;
    p.n_off = used;
    p.n_entries = n;
    p.scale = scale;
    p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    return launched(fsa::launch_frac_decode(dt, out_dt, p, static_cast<hipStream_t>(stream)), "fractional decode");
}

// ---- RoPE before the gather, then the learned-alpha variant's interpolated entries ----

namespace {

struct RopeFracLayout {
    uint64_t qhat, khat, frac, fwd, bwd;  // byte offsets into ws (frac: the fractional workspace) and sizes
};

RopeFracLayout rope_frac_layout(int64_t bh, int32_t n, int32_t n_off, int32_t w) {
    RopeFracLayout l;
    const uint64_t rows = static_cast<uint64_t>(bh) * n;
    l.qhat = 0;
    l.khat = fsa::align256(rows * 128);
    l.fwd = l.khat + fsa::align256(rows * 128);
    l.frac = l.fwd;
    l.bwd = l.frac + fsa::frac_workspace(bh, n, n_off, w).total;
    return l;
}

}  // namespace

fsa_status_t fsa_rope_frac_workspace_bytes(fsa_dtype_t dt, int32_t B, int32_t H, int32_t N, int32_t d,
                                           fsa_base_t base, double alpha, int32_t w, int32_t R, uint64_t *fwd_bytes,
                                           uint64_t *bwd_bytes) {
    if (!fwd_bytes || !bwd_bytes) return fail(FSA_E_ARG, "fwd_bytes or bwd_bytes is NULL");
    fsa::AttnParams p{};
    const fsa_status_t st = prepare_frac(p, dt, dt, B, H, N, d, 1.0f, base, alpha, w, R);
    if (st != FSA_OK) return st;
    const bool empty = static_cast<int64_t>(B) * H * N == 0;
    const RopeFracLayout l = rope_frac_layout(static_cast<int64_t>(B) * H, N, p.n_off, w);
    *fwd_bytes = empty ? 0 : l.fwd;
    *bwd_bytes = empty ? 0 : l.bwd;
    return ok();
}

fsa_status_t fsa_rope_frac_forward(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k, const void *v,
                                   const float *rope, int32_t n_pos, void *o, float *lse, void *ws,
                                   uint64_t ws_bytes, int32_t B, int32_t H, int32_t N, int32_t d, float scale,
                                   fsa_base_t base, double alpha, int32_t w, int32_t R, void *stream) {
    fsa::AttnParams p{};
    fsa_status_t st = prepare_frac(p, dt, out_dt, B, H, N, d, scale, base, alpha, w, R);
    if (st != FSA_OK) return st;
    if (n_pos < N) return fail(FSA_E_ARG, "the rotary table has %d positions, the sequence %d", n_pos, N);
    if (static_cast<int64_t>(B) * H * N == 0) return ok();
    const char *names[] = {"q", "k", "v", "rope", "o", "lse", "ws"};
    const void *ptrs[] = {q, k, v, rope, o, lse, ws};
    if ((st = check_ptrs(names, ptrs, 7)) != FSA_OK) return st;
    if ((st = check_no_alias(names, ptrs, 4, 7)) != FSA_OK) return st;
    const RopeFracLayout l = rope_frac_layout(p.bh, N, p.n_off, w);
    if (ws_bytes < l.fwd)
        return fail(FSA_E_ARG, "ws holds %llu bytes, this problem needs %llu",
                    static_cast<unsigned long long>(ws_bytes), static_cast<unsigned long long>(l.fwd));
    char *wsb = static_cast<char *>(ws);
    const void *xs[] = {q, k};
    void *hats[] = {wsb + l.qhat, wsb + l.khat};
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    const hipError_t e = rotate_rows(xs, hats, 2, rope, static_cast<int64_t>(B) * H * N, N, hs);
    if (e != hipSuccess) return launched(e, "rotary rotation");
    p.q = hats[0];
    p.k = hats[1];
    p.v = v;
    p.out = o;
    p.lse_out = lse;
    return launched(fsa::launch_frac_forward(out_dt, p, hs), "rotary fractional forward");
}

fsa_status_t fsa_rope_frac_backward(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k,
                                    const void *v, const float *rope, int32_t n_pos, const void *o, const float *lse,
                                    const void *dout, void *dq, void *dk, void *dv, float *dalpha, float *doffs,
                                    void *ws, uint64_t ws_bytes, int32_t reuse_rotated, int32_t B, int32_t H,
                                    int32_t N, int32_t d, float scale, fsa_base_t base, double alpha, int32_t w,
                                    int32_t R, void *stream) {
    fsa::AttnParams p{};
    fsa_status_t st = prepare_frac(p, dt, out_dt, B, H, N, d, scale, base, alpha, w, R);
    if (st != FSA_OK) return st;
    if (n_pos < N) return fail(FSA_E_ARG, "the rotary table has %d positions, the sequence %d", n_pos, N);
    if (!dalpha) return fail(FSA_E_ARG, "dalpha is NULL");
    if (reinterpret_cast<uintptr_t>(dalpha) & 3u) return fail(FSA_E_ARG, "dalpha is not 4-byte aligned");
    if (doffs && (reinterpret_cast<uintptr_t>(doffs) & 3u)) return fail(FSA_E_ARG, "doffs is not 4-byte aligned");
    const bool empty = static_cast<int64_t>(B) * H * N == 0;
    RopeFracLayout l{};
    if (!empty) {
        l = rope_frac_layout(p.bh, N, p.n_off, w);
        const char *names[] = {"q", "k", "v", "rope", "o", "lse", "dout", "dq", "dk", "dv", "ws"};
        const void *ptrs[] = {q, k, v, rope, o, lse, dout, dq, dk, dv, ws};
        if ((st = check_ptrs(names, ptrs, 11)) != FSA_OK) return st;
        if ((st = check_no_alias(names, ptrs, 7, 11)) != FSA_OK) return st;
        if (ws_bytes < l.bwd)
            return fail(FSA_E_ARG, "ws holds %llu bytes, this problem needs %llu",
                        static_cast<unsigned long long>(ws_bytes), static_cast<unsigned long long>(l.bwd));
    }
    const void *outs[] = {dalpha, doffs, dq, dk, dv, ws, q, k, v, o, lse, dout, rope};
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 13; ++j)
            if (j != i && outs[i] && outs[i] == outs[j])
                return fail(FSA_E_ARG, "%s aliases another argument", i == 0 ? "dalpha" : "doffs");
    p.dalpha = dalpha;
    p.doffs = doffs;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    if (empty) {
        p.bh = 0;
        return launched(fsa::launch_frac_backward(out_dt, p, hs), "rotary fractional backward");
    }
    char *wsb = static_cast<char *>(ws);
    const void *xs[] = {q, k};
    void *hats[] = {wsb + l.qhat, wsb + l.khat};
    if (!reuse_rotated) {
        const hipError_t e = rotate_rows(xs, hats, 2, rope, static_cast<int64_t>(B) * H * N, N, hs);
        if (e != hipSuccess) return launched(e, "rotary rotation");
    }
    const fsa::FracWorkspace fl = fsa::frac_workspace(p.bh, N, p.n_off, w);
    char *fw = wsb + l.frac;
    p.q = hats[0];
    p.k = hats[1];
    p.v = v;
    p.o = o;
    p.lse_in = lse;
    p.dout = dout;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.delta = reinterpret_cast<float *>(fw + fl.delta);
    p.pairs = reinterpret_cast<uint32_t *>(fw + fl.pairs);
    p.dd_part = reinterpret_cast<float *>(fw + fl.partials);
    p.flags = reinterpret_cast<uint64_t *>(fw + fl.flags);
    p.status = reinterpret_cast<uint64_t *>(fw + fl.status);
    set_wait_limits(p);
    p.rope = rope;
    return launched(fsa::launch_frac_backward(out_dt, p, hs), "rotary fractional backward");
}

fsa_status_t fsa_wait_status(fsa_ws_kind_t kind, fsa_dtype_t dt, int32_t B, int32_t H, int32_t N, int32_t d,
                             fsa_base_t base, double alpha, int32_t w, int32_t R, const void *ws,
                             uint64_t ws_bytes, int32_t *gave_up, void *stream) {
    if (!gave_up) return fail(FSA_E_ARG, "gave_up is NULL");
    *gave_up = 0;
    const int64_t bh = static_cast<int64_t>(B) * H;
    bool one_launch = false;
    uint64_t flags = 0, status = 0, need = 0;  // byte offsets of the token array and status word, ws size
    fsa_status_t st = FSA_OK;
    if (kind == FSA_WS_BACKWARD_NOALLOC) {
        // the library's scratch on the current device: D, then the static backward's workspace
        if (bh * N == 0) return ok();
        uint64_t pair_bytes = 0;
        if ((st = fsa_backward_workspace_bytes(dt, B, H, N, d, base, alpha, w, R, &pair_bytes)) != FSA_OK) return st;
        const uint64_t delta_bytes = fsa::align256(4ull * static_cast<uint64_t>(bh) * N);
        if (delta_bytes + pair_bytes > fsa::kScratchBytes) return ok();  // the call refused this size
        void *p = nullptr;
        const hipError_t e = fsa::scratch_address(&p);
        if (e != hipSuccess) return fail(FSA_E_HIP, "looking up the scratch array failed: %s", hipGetErrorString(e));
        ws = static_cast<const char *>(p) + delta_bytes;
        ws_bytes = pair_bytes;
        kind = FSA_WS_BACKWARD;
    }
    if (kind == FSA_WS_BACKWARD || kind == FSA_WS_ROPE_BACKWARD) {
        const Shape s{B, H, N, d};
        if ((st = check_common(dt, dt, s, 1.0f)) != FSA_OK) return st;
        int32_t tab[FSA_MAX_OFFSETS];
        const int n_all = build_table(base, alpha, w, R, tab, &st);
        if (n_all < 0) return st;
        const int n_off = trim_offsets(tab, n_all, N);
        uint64_t pairs = 0;  // start of the static backward's workspace within ws
        if (kind == FSA_WS_ROPE_BACKWARD) {
            if ((st = check_rope_path(dt, w, N, 1.0f, N, n_all)) != FSA_OK) return st;
            const RopeLayout l = rope_layout(bh, N, n_off, w);
            pairs = l.pairs;
            need = l.bwd;
        } else {
            need = fsa::pair_ws_bytes(dt, w, N, bh, n_off);
        }
        const int64_t words = fsa::pair_words(dt, w, N, bh, n_off);
        one_launch = words > 0 && n_off > 0 && bh % 8 == 0;
        flags = pairs + fsa::pair_ws_flags_offset(words);
        status = pairs + fsa::pair_ws_status_offset(words, bh, N);
    } else if (kind == FSA_WS_ROPE_FORWARD) {
        const Shape s{B, H, N, d};
        if ((st = check_common(dt, dt, s, 1.0f)) != FSA_OK) return st;
        int32_t tab[FSA_MAX_OFFSETS];
        const int n_all = build_table(base, alpha, w, R, tab, &st);
        if (n_all < 0) return st;
        if ((st = check_rope_path(dt, w, N, 1.0f, N, n_all)) != FSA_OK) return st;
        const RopeLayout l = rope_layout(bh, N, trim_offsets(tab, n_all, N), w);
        need = l.fwd;
        one_launch = bh * N > 0 && bh % 8 == 0;
        flags = l.fflags;
        status = l.fstatus;
    } else if (kind == FSA_WS_FRAC_BACKWARD || kind == FSA_WS_ROPE_FRAC_BACKWARD) {
        fsa::AttnParams p{};
        if ((st = prepare_frac(p, dt, dt, B, H, N, d, 1.0f, base, alpha, w, R)) != FSA_OK) return st;
        const fsa::FracWorkspace fl = fsa::frac_workspace(bh, N, p.n_off, w);
        uint64_t frac = 0;
        need = fl.total;
        if (kind == FSA_WS_ROPE_FRAC_BACKWARD) {
            const RopeFracLayout l = rope_frac_layout(bh, N, p.n_off, w);
            frac = l.frac;
            need = l.bwd;
        }
        one_launch = bh * N > 0 && p.n_off > 0 && bh % 8 == 0;
        flags = frac + fl.flags;
        status = frac + fl.status;
    } else {
        return fail(FSA_E_ARG, "unknown workspace kind %d", static_cast<int>(kind));
    }
    if (!one_launch) return ok();  // no waits on this path
    if (!ws) return fail(FSA_E_ARG, "ws is NULL");
    if (ws_bytes < need)
        return fail(FSA_E_ARG, "ws holds %llu bytes, this problem needs %llu",
                    static_cast<unsigned long long>(ws_bytes), static_cast<unsigned long long>(need));
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    uint64_t words[2] = {0, 0};
    const char *b = static_cast<const char *>(ws);
    hipError_t e = hipMemcpyAsync(&words[0], b + flags, 8, hipMemcpyDeviceToHost, hs);
    if (e == hipSuccess) e = hipMemcpyAsync(&words[1], b + status, 8, hipMemcpyDeviceToHost, hs);
    if (e == hipSuccess) e = hipStreamSynchronize(hs);
    if (e != hipSuccess) return fail(FSA_E_HIP, "reading the wait status failed: %s", hipGetErrorString(e));
    *gave_up = words[0] == words[1] ? 1 : 0;
    return ok();
}

fsa_status_t fsa_debug_tile_order(int32_t nb, int32_t *tile_of_block) {
    if (nb < 0) return fail(FSA_E_ARG, "nb must be >= 0 (got %d)", nb);
    if (nb > 0 && !tile_of_block) return fail(FSA_E_ARG, "tile_of_block is NULL");
    for (int32_t b = 0; b < nb; ++b) tile_of_block[b] = fsa::xcd_logical_block(b, nb);
    return ok();
}

fsa_status_t fsa_debug_force_wait_timeout(int32_t enable) {
    g_force_give_up.store(enable != 0 ? 1 : 0, std::memory_order_relaxed);
    return ok();
}

const char *fsa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
