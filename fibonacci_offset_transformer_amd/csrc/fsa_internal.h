// Internal interface between the C-ABI layer (fsa_abi.cpp) and the HIP kernels
// (fsa_*.hip). Not installed; the public interface is include/fsa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fsa.h"

namespace fsa {

constexpr int kHeadDim = 64;   // head size supported by the kernels
constexpr int kTile = 64;      // query (or key) rows owned by one workgroup
constexpr int kThreads = 256;  // four wave64 per workgroup, 16 rows each

// Hardware dispatch places workgroup b on XCD b % 8. Returns the logical tile of
// workgroup b of a grid of nb so that each XCD receives one contiguous range of
// logical tiles, which it processes in increasing order (shared with the host, which
// exports it for tests: fsa_debug_tile_order).
__host__ __device__ inline int xcd_logical_block(int b, int nb) {
    const int x = b & 7, idx = b >> 3;
    const int per = nb >> 3, extra = nb & 7;
    return x * per + (x < extra ? x : extra) + idx;
}

// Kernel arguments, passed by value. Offsets are the sparse table T after the
// host dropped entries >= N (they attend nothing); all entries are >= w.
struct AttnParams {
    const void *q, *k, *v;   // [BH, N, 64]
    const void *o;           // forward output (backward input)
    const void *dout;        // upstream gradient (backward)
    void *out;               // forward: O
    void *dq, *dk, *dv;      // backward outputs
    const float *lse_in;     // backward: forward LSE
    float *lse_out;          // forward: LSE
    float *delta;            // backward: D workspace [BH, N]
    uint32_t *pairs;         // backward: per-pair workspace [BH, N, pair_slots(n_off)] (window path)
    int32_t bh;              // B * H
    int32_t n;               // sequence length
    int32_t w;               // window (offsets 0..w-1)
    int32_t n_off;           // entries used in off[]
    float scale;             // score scale
    float scale_log2;        // scale * log2(e)
    int32_t off[FSA_MAX_OFFSETS];
    const int32_t *seq_lens;  // decode: cached length of each sequence [B]
    int32_t heads;            // decode: H (heads per sequence)
    int32_t lmax;             // decode: rows allocated per cached head
    // Fractional entries (learned-alpha variant): entry t targets distance
    // off[t] + phi[t] (off = floor, phi in [0, 1)) and scales base value fbase[t].
    float phi[FSA_MAX_OFFSETS];
    float fbase[FSA_MAX_OFFSETS];
    float *dd_part;           // backward: per-tile partials of d(loss)/d(d_t) [tiles, n_off]
    float *dalpha;            // backward: d(loss)/d(alpha), one float
    float *doffs;             // backward: d(loss)/d(d_t) per table entry, or null
    int32_t n_entries;        // table entries before trimming (length of doffs)
    // Rotary embedding: when set, the backward kernels rotate dQ and dK of row r back by
    // its position's angles before storing them (table [n_pos, 32, 2] of cos, sin).
    const float *rope;
    void *qhat;               // rotary forward: rotated Q rows written here [BH, N, 64]
    void *khat;               // rotary forward with the K rotation in the kernel: the rotated K
                              // rows [BH, N, 64], written by their tile and read by the slabs
    // One-launch backward: one 64-bit completion token per tile [BH * tiles per head], and
    // the status word a waiting workgroup that gave up sets to the launch's token.
    uint64_t *flags;
    uint64_t *status;
    int32_t max_polls;        // polls a wait makes before it gives up
    uint32_t token_xor;       // waits look for token ^ token_xor (0; nonzero only to force a give-up)
};

// Rotary embedding of up to two [rows, 64] bf16 tensors (x[t] -> out[t]); rows come in
// heads of n, row r sits at position r mod n. table: [n_pos, 32, 2] float32 (cos, sin),
// n_pos >= n.
struct RopeParams {
    const uint16_t *x[2];
    uint16_t *out[2];
    const float *table;
    int64_t rows;
    int64_t head0;  // first head of the launch (set by the launcher)
    int32_t n;
    int32_t count;  // tensors to rotate: 1 or 2
};

// The bf16 window kernels (w <= 64) address each head with 32-bit byte offsets.
inline bool window_path(fsa_dtype_t dt, int32_t w, int32_t n) { return dt == FSA_BF16 && w <= 64 && n <= (1 << 24); }

// Backward pair workspace on the window path: [BH, N, pair_slots(n_off)] slots, slot t of a
// query row holding P and dS of the pair (row, row - off[t]). Slots come in groups of 8 so
// that one row's first eight slots are written by one store. None elsewhere.
__host__ __device__ inline int32_t pair_slots(int32_t n_off) { return 8 * ((n_off + 7) / 8); }

// Format of a slot. With a window of 64 keys or more every query that has a sparse pair
// also has at least 64 window keys, and one 32-bit word of two bf16 (P in the low half,
// dS in the high half) carries the pair. With a narrower window a row's few keys can each
// hold most of its probability: a bf16 rounding of such a weight (up to 2^-8 of it)
// times an upstream gradient of a few units would take most of a 1e-2 error budget, so
// P and dS travel unrounded as two fp32 words.
constexpr int32_t kCompactPairWindow = 64;
__host__ __device__ inline int32_t pair_slot_words(int32_t w) { return w >= kCompactPairWindow ? 1 : 2; }

// The window backward addresses one head's pair words with 32-bit offsets: [N, slots,
// words_per_slot] words (the learned-alpha path stores two words per slot).
inline bool pair_offsets_fit(int32_t n, int32_t n_off, int words_per_slot) {
    return static_cast<int64_t>(n) * pair_slots(n_off) * 4 * words_per_slot <= INT32_MAX;
}
// The static backward takes the window kernels (and their pair workspace) when the
// window path applies and the pair words of a head fit 32-bit offsets.
inline bool window_backward(fsa_dtype_t dt, int32_t w, int32_t n, int32_t n_off) {
    return window_path(dt, w, n) && pair_offsets_fit(n, n_off, pair_slot_words(w));
}
inline int64_t pair_words(fsa_dtype_t dt, int32_t w, int32_t n, int64_t bh, int32_t n_off) {
    return window_backward(dt, w, n, n_off)
               ? static_cast<int64_t>(pair_slots(n_off)) * pair_slot_words(w) * bh * n
               : 0;
}
inline uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

// The static backward's workspace on the window path: the pair words, then (256-byte
// aligned) one 64-bit completion token per 64-row tile, which the one-launch backward
// uses, then one 64-bit status word (the token of a one-launch backward whose dK/dV
// work gave up waiting; see fsa_backward_status). Empty when the table has no sparse
// offsets.
inline uint64_t pair_ws_flags_offset(int64_t words) { return align256(4ull * static_cast<uint64_t>(words)); }
inline uint64_t pair_ws_status_offset(int64_t words, int64_t bh, int32_t n) {
    return pair_ws_flags_offset(words) + 8ull * static_cast<uint64_t>(bh) * ((n + 63) / 64);
}
inline uint64_t pair_ws_bytes(fsa_dtype_t dt, int32_t w, int32_t n, int64_t bh, int32_t n_off) {
    const int64_t words = pair_words(dt, w, n, bh, n_off);
    if (words == 0) return 0;
    return pair_ws_status_offset(words, bh, n) + 8;
}

// Fractional-entry backward workspace on the window path: D [BH, N] floats, then the
// pair words [BH, N, pair_slots(n_off), 2] (the near and far weights of every
// entry), then the per-tile partials [n_off, tiles], then one 64-bit completion token
// per tile (the one-launch backward), then the 64-bit status word; each part 256-byte
// aligned.
struct FracWorkspace {
    uint64_t delta, pairs, partials, flags, status, total;  // byte offsets of the parts, total size
};
// Words per pair slot of the learned-alpha backward: the near and the far share, each
// P and dS as two bf16 in one word at w >= 64, as four fp32 words below (the same
// reading as the static slots).
__host__ __device__ inline int32_t frac_pair_words(int32_t window) { return 2 * pair_slot_words(window); }
inline FracWorkspace frac_workspace(int64_t bh, int32_t n, int32_t n_off, int32_t window) {
    FracWorkspace w;
    const uint64_t tiles = static_cast<uint64_t>(bh) * ((n + 63) / 64);
    w.delta = 0;
    w.pairs = align256(4ull * bh * n);
    w.partials = w.pairs + align256(4ull * frac_pair_words(window) * pair_slots(n_off) * bh * n);
    w.flags = w.partials + align256(4ull * tiles * n_off);
    w.status = w.flags + align256(8ull * tiles);
    w.total = w.status + (tiles > 0 ? 256 : 0);
    return w;
}

// Polls of a bounded wait before it gives up: with the sleep between polls they span
// tens of milliseconds, far beyond any real wait (the dQ work of a whole launch takes
// tens of microseconds).
constexpr int32_t kMaxPolls = 1 << 18;

// The one-launch backward runs when it has sparse offsets, a token array and B * H a
// multiple of 8 (every XCD then holds whole heads).
inline bool one_launch_backward(const AttnParams &p) { return p.flags && p.n_off > 0 && p.bh % 8 == 0; }

// Sets the calling thread's error text, returns st (fsa_abi.cpp).
fsa_status_t set_error(fsa_status_t st, const char *msg);
// Device address of the library's static scratch array on the current device, looked up
// once per device (fsa_noalloc.hip); its size in bytes.
extern const uint64_t kScratchBytes;
hipError_t scratch_address(void **ptr);

hipError_t launch_forward(fsa_dtype_t dt, fsa_dtype_t out_dt, const AttnParams &p, hipStream_t stream);
hipError_t launch_dense_forward(fsa_dtype_t dt, fsa_dtype_t out_dt, const AttnParams &p, hipStream_t stream);
hipError_t launch_backward_delta(fsa_dtype_t dt, const AttnParams &p, hipStream_t stream);
hipError_t launch_decode(fsa_dtype_t dt, fsa_dtype_t out_dt, const AttnParams &p, hipStream_t stream);
hipError_t launch_frac_decode(fsa_dtype_t dt, fsa_dtype_t out_dt, const AttnParams &p, hipStream_t stream);
// Gradient stage. With `with_delta`, D is formed from p.o and p.dout and written to
// p.delta on the way (by the dQ kernel on the window path, by the delta kernel
// elsewhere); otherwise p.delta is read as given.
hipError_t launch_backward_grads(fsa_dtype_t dt, fsa_dtype_t out_dt, const AttnParams &p, hipStream_t stream,
                                 bool with_delta);
// Fractional entries (bf16 window path, positive scale): the forward, and the
// backward (dQ with D, dK/dV, then the reduction of the alpha gradient).
hipError_t launch_frac_forward(fsa_dtype_t out_dt, const AttnParams &p, hipStream_t stream);
hipError_t launch_rope(const RopeParams &p, hipStream_t stream);
// Rotary forward on the bf16 window path: Q unrotated (rotated in the kernel and stored
// to p.qhat), K already rotated.
hipError_t launch_rope_forward(fsa_dtype_t out_dt, const AttnParams &p, hipStream_t stream);
hipError_t launch_frac_backward(fsa_dtype_t out_dt, const AttnParams &p, hipStream_t stream);

}  // namespace fsa
