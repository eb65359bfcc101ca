/*
 * fsa.h - C ABI of libfsa, Fibonacci-offset sparse attention for AMD MI355X (gfx950).
 *
 * The operation (cited from the explainer page "Depth-Staggered Fibonacci Spacing
 * for Sparse Attention: Static Schedules Beat Learned Dilation and Extrapolate
 * Where Dense Attention Fails", gist.science, Portuguese edition, section
 * "Metodologia / Arquitetura e Mecanismo de Atenção"): causal attention in which
 * query row i attends a dense local window of w keys (offsets 0..w-1, itself
 * included) plus the keys i - round(alpha * F) for F in a base list (Fibonacci
 * numbers 1, 2, 3, 5, ... or, for the power-of-2 control of section "Controles",
 * 1, 2, 4, 8, ...), with one per-layer scalar alpha (item "Escalonamento").
 * Static schedules run as one boolean mask (section "Principais Contribuições e
 * Resultados", item 2), so every key is attended at most once and one softmax
 * covers window and sparse keys together.
 *
 * Conventions shared by every call:
 *  - Tensors Q, K, V, O, dO, dQ, dK, dV are contiguous row-major [B, H, N, d] in
 *    device memory, each 16-byte aligned; d must be 64. Inputs Q, K, V (and, in
 *    the backward, O and dO) have the input dtype `dt`; the outputs O (forward)
 *    and dQ, dK, dV (backward) have the output dtype `out_dt`. Arithmetic does
 *    not depend on out_dt: a bf16 output is the round-to-nearest-even image of
 *    the float32 output of the same call.
 *  - LSE and the backward workspace are float32 [B, H, N] in device memory; LSE
 *    is the natural-log row log-sum-exp of the scaled scores.
 *  - Device buffers are owned by the caller. The library never allocates, frees
 *    or synchronises; each call enqueues its kernels on `stream` (a hipStream_t,
 *    NULL for the default stream) and returns without waiting. Faults inside a
 *    kernel surface at the caller's next synchronisation.
 *  - Outputs are overwritten, never accumulated; outputs must not alias inputs.
 *  - B, H or N equal to 0 is an empty problem: FSA_OK, nothing is launched.
 *  - Arguments are validated before any HIP call; on any non-OK status nothing
 *    has been enqueued and no output has been written. fsa_last_error() then
 *    returns a text for the calling thread.
 *  - Offset tables are rebuilt on the host on every call (a few dozen integer
 *    operations) and passed to the kernels by value; the library keeps no global
 *    state besides a thread-local error string. All calls are thread-safe.
 */
#ifndef FSA_H
#define FSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FSA_OK = 0,
    FSA_E_ARG = 1,          /* invalid argument (null pointer, bad size, alpha, w, R, alignment) */
    FSA_E_UNSUPPORTED = 2,  /* valid but not implemented (head size other than 64, unknown dtype) */
    FSA_E_CAPACITY = 3,     /* output array too small; *count holds the size needed */
    FSA_E_HIP = 4           /* the HIP runtime refused a launch; see fsa_last_error() */
} fsa_status_t;

typedef enum { FSA_BASE_FIB = 0, FSA_BASE_POW2 = 1 } fsa_base_t;

typedef enum { FSA_F32 = 0, FSA_BF16 = 1 } fsa_dtype_t;

/* Largest number of sparse offsets any table can hold (Fibonacci values below 2^31). */
#define FSA_MAX_OFFSETS 48

/*
 * fsa_build_offsets - the sparse offset table T of one layer, in host memory.
 *
 * T = sorted, duplicate-free { round(alpha * F) : F in base, F < R } restricted
 * to values >= w (smaller ones already lie in the dense window). Base list:
 * Fibonacci 1, 2, 3, 5, 8, ... (recurrence F_{k+1} = F_k + F_{k-1}; page section
 * "Metodologia / Arquitetura e Mecanismo de Atenção", item "Conjunto Atendido")
 * or powers of two 1, 2, 4, ... (section "Controles"). alpha * F is one IEEE
 * double product, rounded half to even. R is exclusive and caps the base value
 * before scaling, so scaled offsets may exceed R. T does not depend on N.
 *
 *   base      FSA_BASE_FIB or FSA_BASE_POW2
 *   alpha     finite, > 0; alpha * F must round to at most 2^31 - 1
 *   w         window size, >= 1
 *   R         reach, >= 1
 *   out       host array receiving T in increasing order (may be NULL if capacity == 0)
 *   capacity  entries available in out
 *   count     receives |T| (also on FSA_E_CAPACITY)
 */
fsa_status_t fsa_build_offsets(fsa_base_t base, double alpha, int32_t w, int32_t R,
                               int32_t *out, int32_t capacity, int32_t *count);

/*
 * fsa_forward - sparse attention forward: O and LSE.
 *
 * For every (b, h) and row i < N:
 *   J(i) = { i - o : o in {0..w-1} u T(base, alpha, w, R), i - o >= 0 }
 *   s_ij = scale * <q_i, k_j>, P_ij = softmax_j(s_ij) over J(i),
 *   o_i = sum_j P_ij v_j (written in out_dt),
 *   lse_i = ln sum_j exp(s_ij) (float32).
 * Arithmetic: products and softmax in fp32 (bf16 inputs: bf16 MFMA for the
 * window, probabilities rounded to bf16 for the window's P.V product).
 *
 *   dt              FSA_F32 or FSA_BF16: dtype of q, k, v
 *   out_dt          FSA_F32 or FSA_BF16: dtype of o
 *   q, k, v         inputs [B,H,N,d]
 *   o               output [B,H,N,d]
 *   lse             output float32 [B,H,N]
 *   scale           finite score scale (1/sqrt(d) in the usual setting)
 *   base, alpha, w, R   offset table parameters as in fsa_build_offsets
 *   stream          hipStream_t to enqueue on
 */
fsa_status_t fsa_forward(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k,
                         const void *v, void *o, float *lse, int32_t B, int32_t H, int32_t N, int32_t d,
                         float scale, fsa_base_t base, double alpha, int32_t w, int32_t R,
                         void *stream);

/*
 * fsa_backward - gradients of sum(dO * O) with respect to Q, K and V.
 *
 * The textbook softmax-attention gradient restricted to the same mask as
 * fsa_forward (the pages train through this mask, section "Metodologia"):
 *   D_i = <dO_i, o_i>, P_ij = exp(s_ij - lse_i), dS_ij = P_ij (<dO_i, v_j> - D_i),
 *   dQ_i = scale sum_j dS_ij k_j, dK_j = scale sum_i dS_ij q_i, dV_j = sum_i P_ij dO_i.
 * o and lse must be the outputs of fsa_forward for the same inputs and table.
 * Every output row is written by exactly one workgroup (no atomics), so results
 * are bitwise reproducible.
 *
 *   dt                  dtype of q, k, v, o, dout
 *   out_dt              dtype of dq, dk, dv
 *   q, k, v, o, dout    inputs [B,H,N,d]
 *   lse                 input float32 [B,H,N]
 *   dq, dk, dv          outputs [B,H,N,d]
 *   delta_ws            caller-owned float32 [B,H,N] workspace, overwritten with D
 *   pair_ws             caller-owned device workspace of at least
 *                       fsa_backward_workspace_bytes(...) bytes, 16-byte aligned,
 *                       overwritten; its contents on entry do not matter. It may
 *                       be NULL when that size is 0. Two calls that overlap in
 *                       time must not share one.
 *   pair_ws_bytes       size of pair_ws in bytes; FSA_E_ARG if smaller than needed
 */
fsa_status_t fsa_backward(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k,
                          const void *v, const void *o, const float *lse, const void *dout,
                          void *dq, void *dk, void *dv, float *delta_ws, void *pair_ws,
                          uint64_t pair_ws_bytes, int32_t B, int32_t H, int32_t N, int32_t d, float scale,
                          fsa_base_t base, double alpha, int32_t w, int32_t R, void *stream);

/*
 * fsa_backward_workspace_bytes - bytes of pair workspace the backward needs.
 *
 * On the bf16 window path (dt = FSA_BF16, w <= 64, N <= 2^24, and 4 * S * W * N < 2^31
 * with S and W below) the gradient stage has two parts: the dQ part stores, for every
 * query row i and sparse offset o of the table (offsets >= N dropped), P and dS of the
 * pair (i, i - o); the dK/dV part reads them. A pair takes W 32-bit words: W = 1 (two
 * bf16) when w >= 64, W = 2 (two fp32) for narrower windows, where a query's few keys
 * can each carry most of its probability and one bf16 rounding of such a weight would
 * weigh on the gradients. When B * H is a multiple of 8 both parts run in one launch:
 * each 64-row tile's dQ part then publishes a 64-bit token naming the launch (from the
 * hardware dispatch id), and the dK/dV parts wait for the tokens of the tiles they read.
 * That wait is bounded: if it ever gave up, the tile's dK and dV would be NaN and a
 * status word in the workspace would name the launch (fsa_wait_status reads it).
 * Otherwise the parts run as two kernels. The size is 4 * S * W * B * H * N bytes of pair
 * words, S = |T| rounded up to a multiple of 8 (slots per query row), rounded up to a
 * multiple of 256, plus 8 * B * H * ceil(N / 64) bytes of tokens and 8 bytes of status;
 * 0 on every other path or when no offset is below N. Arguments as in fsa_backward;
 * *bytes receives the size.
 */
fsa_status_t fsa_backward_workspace_bytes(fsa_dtype_t dt, int32_t B, int32_t H, int32_t N, int32_t d,
                                          fsa_base_t base, double alpha, int32_t w, int32_t R,
                                          uint64_t *bytes);

/*
 * fsa_backward_delta and fsa_backward_grads - the two stages of fsa_backward,
 * exposed so that a caller can schedule (or time) them separately.
 * fsa_backward_delta writes D_i = <dO_i, o_i> (float32 [B,H,N]) into delta_ws;
 * fsa_backward_grads then computes dQ, dK, dV from q, k, v, lse, dout and that
 * D. fsa_backward(...) is exactly fsa_backward_delta followed by
 * fsa_backward_grads on the same stream. Arguments as in fsa_backward.
 */
fsa_status_t fsa_backward_delta(fsa_dtype_t dt, const void *o, const void *dout, float *delta_ws,
                                int32_t B, int32_t H, int32_t N, int32_t d, void *stream);
fsa_status_t fsa_backward_grads(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k,
                                const void *v, const float *lse, const void *dout,
                                const float *delta, void *dq, void *dk, void *dv, void *pair_ws,
                                uint64_t pair_ws_bytes, int32_t B, int32_t H, int32_t N, int32_t d,
                                float scale, fsa_base_t base, double alpha, int32_t w, int32_t R,
                                void *stream);

/*
 * fsa_decode - one decoding step: the newest query of each sequence against a
 * key/value cache (the inference workload of the method; the same attended set
 * as fsa_forward's last row).
 *
 * For every (b, h), with L = seq_lens[b] clamped into [1, Lmax] and i = L - 1:
 *   J = { i - o : o in {0..w-1} u T(base, alpha, w, R), i - o >= 0 },
 *   o[b,h] = sum_{j in J} softmax_j(scale * <q[b,h], k_cache[b,h,j]>) v_cache[b,h,j],
 *   lse[b,h] = ln sum_{j in J} exp(scale * <q[b,h], k_cache[b,h,j]>).
 * Arithmetic in fp32 (inputs converted exactly). A window w >= Lmax makes this
 * dense decoding.
 *
 *   dt, out_dt          dtypes as in fsa_forward (q, k_cache, v_cache; o)
 *   q                   [B,H,d]: the newest token's query
 *   k_cache, v_cache    [B,H,Lmax,d]: row j of a sequence holds position j; rows
 *                       0 .. L-1 must be filled, the newest token's key and value
 *                       included (appending them is the caller's step)
 *   seq_lens            device int32 [B], 4-byte aligned: L of each sequence;
 *                       values outside [1, Lmax] are clamped into it
 *   o                   output [B,H,d] in out_dt
 *   lse                 output float32 [B,H]
 *   Lmax                rows allocated per cached head, >= 1
 *   scale, base, alpha, w, R   as in fsa_forward (table entries >= Lmax dropped)
 */
fsa_status_t fsa_decode(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k_cache,
                        const void *v_cache, const int32_t *seq_lens, void *o, float *lse, int32_t B, int32_t H,
                        int32_t Lmax, int32_t d, float scale, fsa_base_t base, double alpha, int32_t w, int32_t R,
                        void *stream);

/*
 * fsa_dense_forward - dense causal attention baseline (every j <= i attended),
 * the same architecture with full attention (page section "Controles").
 * Arguments as in fsa_forward.
 */
fsa_status_t fsa_dense_forward(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q,
                               const void *k, const void *v, void *o, float *lse, int32_t B, int32_t H, int32_t N, int32_t d,
                               float scale, void *stream);

/*
 * Learned-alpha variant: fractional entries.
 *
 * With a learned per-layer alpha (page section "Variáveis Experimentais", item
 * "Aprendido") the targets d = alpha * F are not integers; the model then reads
 * keys and values linearly interpolated between the two rows around the target
 * position, so that a gradient reaches alpha (section "Metodologia / Arquitetura",
 * item "Implementação"). The library's reading of that sentence:
 *   - d = alpha * F is one IEEE double product, not rounded; entries with d >= w
 *     are kept (the same threshold as the static table), one per base value, in
 *     increasing d. Entry t has a = floor(d), phi = d - a.
 *   - Query row i has entry t when i - d >= 0. Its key is
 *     (1 - phi) k_{i-a} + phi k_{i-a-1}, its value the same mix of v; every entry
 *     is one more column of the row's single softmax over window and entries.
 *   - At alpha * F integral (phi = 0) the entry is the static key i - d, so alpha
 *     values with integral products reproduce fsa_forward exactly in exact
 *     arithmetic.
 *   - The derivative with respect to d is that of the piece [a, a + 1):
 *     k_{i-a-1} - k_{i-a} (and the same for v); rows without row i - a - 1
 *     contribute none. d(loss)/d(alpha) = sum_t F_t d(loss)/d(d_t).
 * Supported for bf16 inputs, w <= 64, N <= 2^24, scale > 0, d = 64, and 8 * S * N <
 * 2^31 (S: the entries some row reaches, rounded up to a multiple of 8; one head's
 * pair words are addressed with 32-bit offsets); other valid arguments return
 * FSA_E_UNSUPPORTED.
 */

/*
 * fsa_frac_offsets - the fractional table of one layer, in host memory.
 *
 *   base, alpha, w, R   as in fsa_build_offsets
 *   whole               receives floor(d) of each entry (int32)
 *   frac                receives d - floor(d), rounded to float
 *   base_value          receives the base value F of each entry
 *   capacity            entries available in each of the three arrays
 *   count               receives the number of entries (also on FSA_E_CAPACITY)
 */
fsa_status_t fsa_frac_offsets(fsa_base_t base, double alpha, int32_t w, int32_t R, int32_t *whole,
                              float *frac, int32_t *base_value, int32_t capacity, int32_t *count);

/*
 * fsa_frac_forward - forward of the learned-alpha variant: O and LSE.
 *
 * For every (b, h) and row i < N, the columns of row i are the window keys
 * k_{i-o} (o in 0..w-1, o <= i) and, for each entry t with d_t <= i, the
 * interpolated key above; s = scale * <q_i, key>, P = softmax over the columns,
 * o_i = sum P * value (interpolated for the entries), lse_i = ln sum exp(s).
 * Arithmetic as in fsa_forward (bf16 MFMA window, fp32 dot products for the
 * entries, each entry's two value weights rounded to bf16). Arguments as in
 * fsa_forward.
 */
fsa_status_t fsa_frac_forward(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k,
                              const void *v, void *o, float *lse, int32_t B, int32_t H, int32_t N, int32_t d,
                              float scale, fsa_base_t base, double alpha, int32_t w, int32_t R, void *stream);

/*
 * fsa_frac_backward - gradients of sum(dO * O) of fsa_frac_forward with respect to
 * Q, K, V and alpha.
 *
 * dQ, dK, dV: the softmax-attention gradient through the interpolation (an entry
 * column's key and value gradients reach row i - a with weight 1 - phi and row
 * i - a - 1 with weight phi). dalpha: d(loss)/d(alpha) summed over b, h and rows
 * (alpha is one scalar per layer), reduced in a fixed order (reproducible).
 * o and lse must be the outputs of fsa_frac_forward for the same inputs and table.
 *
 *   dt, out_dt, q, k, v, o, lse, dout, dq, dk, dv, scale, base, alpha, w, R, stream
 *                       as in fsa_backward
 *   dalpha              device float32 [1], 4-byte aligned: receives d(loss)/d(alpha);
 *                       written also for an empty problem (0)
 *   doffs               device float32 [count of fsa_frac_offsets], 4-byte aligned,
 *                       or NULL: receives d(loss)/d(d_t) per entry (0 for entries
 *                       no row reaches)
 *   ws                  caller-owned device workspace of at least
 *                       fsa_frac_backward_workspace_bytes(...) bytes, 16-byte aligned,
 *                       overwritten; its contents on entry do not matter (it holds D,
 *                       the near and far weights of every pair (bf16 at w = 64, fp32
 *                       below, as fsa_backward's pair slots), the per-tile
 *                       partials of the alpha gradient and one 64-bit token per tile:
 *                       with B * H a multiple of 8 the dQ and dK/dV parts run in one
 *                       launch, as in fsa_backward). May be NULL for an empty problem.
 *                       Two calls that overlap in time must not share one.
 *   ws_bytes            size of ws; FSA_E_ARG if smaller than needed
 */
fsa_status_t fsa_frac_backward(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k,
                               const void *v, const void *o, const float *lse, const void *dout, void *dq,
                               void *dk, void *dv, float *dalpha, float *doffs, void *ws, uint64_t ws_bytes,
                               int32_t B, int32_t H, int32_t N, int32_t d, float scale, fsa_base_t base,
                               double alpha, int32_t w, int32_t R, void *stream);

/*
 * fsa_frac_backward_workspace_bytes - bytes of ws fsa_frac_backward needs:
 * 4 B H N (D) + 4 W S B H N (W words per pair: 2 at w = 64, the near and far
 * shares' P and dS as bf16 pairs, and 4 below, as fp32 words; S = number of entries
 * some row reaches, rounded up to a multiple of 8) + 4 B H ceil(N/64) S' (partials, S' the
 * unrounded count) + 8 B H ceil(N/64) (tokens) + 8 (status word, see fsa_wait_status),
 * each part rounded up to 256 bytes. Arguments as in fsa_frac_backward; *bytes receives
 * the size.
 */
fsa_status_t fsa_frac_backward_workspace_bytes(fsa_dtype_t dt, int32_t B, int32_t H, int32_t N, int32_t d,
                                               fsa_base_t base, double alpha, int32_t w, int32_t R,
                                               uint64_t *bytes);

/*
 * fsa_frac_decode - one decoding step of the learned-alpha variant: as fsa_decode,
 * with the fractional entries of fsa_frac_offsets in place of the static table. For
 * the newest position i = L - 1, entry t is present when i - d_t >= 0, and its key
 * and value are (1 - phi_t) row(i - a_t) + phi_t row(i - a_t - 1) of the caches,
 * mixed in fp32. Any scale, bf16 or float32 inputs; arguments as in fsa_decode
 * (entries no cached position reaches are dropped).
 */
fsa_status_t fsa_frac_decode(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k_cache,
                             const void *v_cache, const int32_t *seq_lens, void *o, float *lse, int32_t B, int32_t H,
                             int32_t Lmax, int32_t d, float scale, fsa_base_t base, double alpha, int32_t w,
                             int32_t R, void *stream);

/*
 * Rotary position embedding before the attention.
 *
 * The pages rotate queries and keys with rotary position embeddings before the
 * rows are gathered, vanilla RoPE without scaling (section "Metodologia /
 * Arquitetura", item "Implementação", and the limitations paragraph). The
 * library's reading: channel pairs (2m, 2m + 1) of a row at position p (the row
 * index) are rotated by the angle p * theta_m, theta_m = rope_base^(-2m/d) (10000
 * for vanilla RoPE); values are not rotated.
 *
 * The rotated rows enter the attention in bf16, as a separate rotation step would
 * store them. Each rotated value is fixed exactly: with (c, s) the table entries,
 * channel 2m becomes fma(c, x_2m, -(s * x_2m+1)) and channel 2m + 1 becomes
 * fma(s, x_2m, c * x_2m+1) in float32, then each is rounded to bf16 (nearest, ties
 * to even). The attention over the rotated rows is fsa_forward / fsa_backward's.
 * The backward returns gradients with respect to the unrotated Q and K: the
 * rotated-row gradients rotated back by each row's angles (the transpose), with the
 * bf16 rounding passing gradients unchanged.
 *
 * Each key row is gathered by about |T| + 2 query tiles, so the calls rotate K once
 * per row into a workspace (one memory-bound pass) instead of once per gather; the
 * forward kernel rotates its own Q rows, the backward rotates Q and K by the same
 * pass (or reuses the forward's), and its inverse rotation is fused into the store
 * of dQ and dK.
 * Supported for bf16 inputs, w <= 64, N <= 2^24, scale > 0, d = 64, and 4 * S * N <
 * 2^31 (S: the table's offsets rounded up to a multiple of 8); other valid arguments
 * return FSA_E_UNSUPPORTED.
 */

/*
 * fsa_rope_table - the rotary table, in host memory: table[(p * d/2 + m) * 2] =
 * cos(p * theta_m) and table[... + 1] = sin(p * theta_m), each computed in double
 * precision with the C library's cos and sin and rounded once to float32, for
 * p = 0 .. n_pos - 1 and m = 0 .. d/2 - 1. Copy it to the device for the calls below.
 *
 *   n_pos       positions, >= 0 (at least N of the calls that use the table)
 *   d           head size, even, >= 2
 *   rope_base   frequency base, finite, > 0 (10000: vanilla RoPE)
 *   table       host float32 array of n_pos * d floats (NULL allowed when n_pos = 0)
 */
fsa_status_t fsa_rope_table(int32_t n_pos, int32_t d, double rope_base, float *table);

/*
 * fsa_rope_rotate - the rotation step on its own: out = the rotated rows of x,
 * bf16 [B,H,N,d] -> bf16 [B,H,N,d] (exactly as described above; row i of each head
 * at position i).
 *
 *   dt          FSA_BF16 (FSA_F32 returns FSA_E_UNSUPPORTED)
 *   x, out      device [B,H,N,d], 16-byte aligned, out must not alias x
 *   rope        device copy of fsa_rope_table(n_pos, d, ...), 16-byte aligned
 *   n_pos       positions in the table, >= N
 *   N           <= 2^24 (larger returns FSA_E_UNSUPPORTED)
 */
fsa_status_t fsa_rope_rotate(fsa_dtype_t dt, const void *x, const float *rope, int32_t n_pos, void *out, int32_t B,
                             int32_t H, int32_t N, int32_t d, void *stream);

/*
 * fsa_rope_workspace_bytes - bytes of ws the rotary forward and backward need:
 * forward 2 B H N d * 2 (the rotated Q and K, each part rounded up to 256 bytes) plus
 * 8 bytes per 64-row tile and an 8-byte status word (rounded up to 256);
 * backward that plus 4 B H N (D) plus fsa_backward_workspace_bytes for the same window
 * (pair words, tokens and status word).
 * Arguments as in fsa_rope_forward; 0 and 0 for an empty problem.
 */
fsa_status_t fsa_rope_workspace_bytes(fsa_dtype_t dt, int32_t B, int32_t H, int32_t N, int32_t d, fsa_base_t base,
                                      double alpha, int32_t w, int32_t R, uint64_t *fwd_bytes, uint64_t *bwd_bytes);

/*
 * fsa_rope_forward - fsa_forward on the rotated Q and K: O and LSE.
 *
 *   q, k, v         unrotated inputs [B,H,N,d] (bf16)
 *   rope, n_pos     device rotary table (fsa_rope_table) and its positions, n_pos >= N
 *   o, lse          outputs as in fsa_forward
 *   ws, ws_bytes    caller-owned device workspace of at least the forward size of
 *                   fsa_rope_workspace_bytes, 16-byte aligned, overwritten (holds
 *                   the rotated K, the rotated Q when keep_rotated, and per-tile
 *                   tokens); its contents on entry do not matter
 *   keep_rotated    nonzero: the rotated Q rows are also stored in ws, so that
 *                   fsa_rope_backward can reuse them (reuse_rotated); 0 (inference)
 *                   skips that store. The attention kernel rotates its own Q rows.
 *                   With B * H a multiple of 8 it rotates K as well: each 64-row tile
 *                   rotates the K rows it copies for its window, stores its own rows
 *                   in ws and publishes a token, and the tiles whose sparse offsets
 *                   reach those rows read them there after a bounded wait for the
 *                   token (as in fsa_backward's one-launch path: a wait that gives up
 *                   stores NaN O and LSE for its tile and sets the status word that
 *                   fsa_wait_status reads with FSA_WS_ROPE_FORWARD). Otherwise a
 *                   separate pass rotates K first.
 *   other arguments as in fsa_forward
 */
fsa_status_t fsa_rope_forward(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k, const void *v,
                              const float *rope, int32_t n_pos, void *o, float *lse, void *ws, uint64_t ws_bytes,
                              int32_t keep_rotated, int32_t B, int32_t H, int32_t N, int32_t d, float scale,
                              fsa_base_t base, double alpha, int32_t w, int32_t R, void *stream);

/*
 * fsa_rope_backward - gradients of sum(dO * O) of fsa_rope_forward with respect to
 * the unrotated Q and K, and V. o and lse must be fsa_rope_forward's outputs for
 * the same inputs, table and offsets.
 *
 *   q, k, v, rope, n_pos   as in fsa_rope_forward
 *   o, lse, dout           as in fsa_backward
 *   dq, dk, dv             outputs [B,H,N,d] in out_dt
 *   ws, ws_bytes           caller-owned device workspace of at least the backward size
 *                          of fsa_rope_workspace_bytes, 16-byte aligned, overwritten
 *   reuse_rotated          0: the call rotates q and k itself, and the contents of ws on
 *                          entry do not matter. Nonzero: ws's first forward-size bytes
 *                          still hold the rotated rows fsa_rope_forward wrote there, with
 *                          keep_rotated, for these same q, k and table (the activations a training step
 *                          keeps for its backward); the rotation is skipped. Nothing
 *                          checks this: other contents give wrong gradients.
 *   other arguments as in fsa_backward
 */
fsa_status_t fsa_rope_backward(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k, const void *v,
                               const float *rope, int32_t n_pos, const void *o, const float *lse, const void *dout,
                               void *dq, void *dk, void *dv, void *ws, uint64_t ws_bytes, int32_t reuse_rotated,
                               int32_t B, int32_t H, int32_t N, int32_t d, float scale, fsa_base_t base, double alpha,
                               int32_t w, int32_t R, void *stream);

/*
 * The learned-alpha variant with rotary embedding, as the pages describe it: Q and K
 * are rotated (as in fsa_rope_forward, stored in bf16), then the attention of
 * fsa_frac_forward runs over the rotated rows, so each fractional entry interpolates
 * rotated key rows (and unrotated value rows). The backward returns dQ, dK with
 * respect to the unrotated rows, dV, dalpha and doffs (as fsa_frac_backward).
 *
 * fsa_rope_frac_workspace_bytes: forward 2 B H N d * 2 (rotated Q and K); backward
 * that plus fsa_frac_backward_workspace_bytes (each part rounded up to 256 bytes).
 * fsa_rope_frac_forward / fsa_rope_frac_backward: arguments as in fsa_rope_forward /
 * fsa_rope_backward, plus dalpha and doffs as in fsa_frac_backward; reuse_rotated as
 * in fsa_rope_backward (ws then holds fsa_rope_frac_forward's rotated rows). Supported
 * for bf16 inputs, w <= 64, N <= 2^24, scale > 0, d = 64, within the pair-offset limit
 * of the fractional calls.
 */
fsa_status_t fsa_rope_frac_workspace_bytes(fsa_dtype_t dt, int32_t B, int32_t H, int32_t N, int32_t d,
                                           fsa_base_t base, double alpha, int32_t w, int32_t R, uint64_t *fwd_bytes,
                                           uint64_t *bwd_bytes);
fsa_status_t fsa_rope_frac_forward(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k, const void *v,
                                   const float *rope, int32_t n_pos, void *o, float *lse, void *ws,
                                   uint64_t ws_bytes, int32_t B, int32_t H, int32_t N, int32_t d, float scale,
                                   fsa_base_t base, double alpha, int32_t w, int32_t R, void *stream);
fsa_status_t fsa_rope_frac_backward(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k,
                                    const void *v, const float *rope, int32_t n_pos, const void *o, const float *lse,
                                    const void *dout, void *dq, void *dk, void *dv, float *dalpha, float *doffs,
                                    void *ws, uint64_t ws_bytes, int32_t reuse_rotated, int32_t B, int32_t H,
                                    int32_t N, int32_t d, float scale, fsa_base_t base, double alpha, int32_t w,
                                    int32_t R, void *stream);

/*
 * fsa_backward_noalloc - fsa_backward for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 *
 * Computes exactly what fsa_backward computes (the same kernels, bitwise the same
 * results), with its two workspaces (D, and the pair weights, tokens and status word of
 * fsa_backward_workspace_bytes) taken from a static device array of the library: 32 MiB
 * per GPU, held by every GPU the library runs on until the process ends. The caller
 * passes inputs and outputs only; the call allocates nothing and makes no allocating
 * library call. Problems whose D (4 B H N bytes, rounded up to 256) plus pair workspace
 * exceed 32 MiB are refused with FSA_E_CAPACITY (fsa_backward with caller workspaces
 * takes them). Every call on one GPU shares that GPU's array and leaves its contents
 * behind (nothing in it has to start at zero): two calls that overlap in time on one
 * GPU, on different streams or threads, race and must not be issued. fsa_wait_status
 * with FSA_WS_BACKWARD_NOALLOC reads this array's status word.
 *
 * Arguments as in fsa_backward, without delta_ws, pair_ws and pair_ws_bytes.
 */
fsa_status_t fsa_backward_noalloc(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k,
                                  const void *v, const void *o, const float *lse, const void *dout,
                                  void *dq, void *dk, void *dv, int32_t B, int32_t H, int32_t N, int32_t d,
                                  float scale, fsa_base_t base, double alpha, int32_t w, int32_t R, void *stream);

/*
 * fsa_wait_status - whether the last one-launch backward (or rotary forward that
 * rotates K itself) that ran with a workspace gave up one of its bounded waits.
 *
 * The one-launch backward (B * H a multiple of 8, sparse offsets below N) is correct
 * only if the GPU dispatches its workgroups in block order and places block b on XCD
 * b mod 8; its dK/dV workgroups then never wait for a workgroup that has not started.
 * The rotary forward with B * H a multiple of 8 rests on the same two facts (its tiles
 * wait only for earlier tiles of their head). Each wait is bounded nonetheless: a
 * workgroup that gives up stores NaN results (dK and dV; the learned-alpha reduction's
 * dalpha; the rotary forward's O and LSE) instead of hanging, and writes the launch's
 * token into the workspace's status word. This call reads that word and the token of
 * the workspace's most recent launch (published by its first tile, whose work never
 * waits) and reports whether they match. It synchronises `stream` and copies 16 bytes
 * to the host (the one call of the library that waits). Call it after the backward or
 * forward, with the same arguments, before the workspace is reused.
 *
 *   kind        which call's workspace: FSA_WS_BACKWARD (fsa_backward,
 *               fsa_backward_grads: pair_ws), FSA_WS_FRAC_BACKWARD (fsa_frac_backward:
 *               ws), FSA_WS_ROPE_BACKWARD (fsa_rope_backward: ws),
 *               FSA_WS_ROPE_FRAC_BACKWARD (fsa_rope_frac_backward: ws),
 *               FSA_WS_BACKWARD_NOALLOC (fsa_backward_noalloc: the library's scratch
 *               on the current device; ws and ws_bytes are ignored),
 *               FSA_WS_ROPE_FORWARD (fsa_rope_forward: ws; its waits are those of the
 *               tiles that read rotated K rows other tiles stored)
 *   dt, B, H, N, d, base, alpha, w, R   the arguments the backward ran with
 *   ws, ws_bytes   that workspace and its size
 *   gave_up     receives 1 if a wait of that launch gave up, else 0 (also 0 when the
 *               problem does not take the one-launch path)
 *   stream      the stream the backward ran on
 */
typedef enum {
    FSA_WS_BACKWARD = 0,
    FSA_WS_FRAC_BACKWARD = 1,
    FSA_WS_ROPE_BACKWARD = 2,
    FSA_WS_ROPE_FRAC_BACKWARD = 3,
    FSA_WS_BACKWARD_NOALLOC = 4,
    FSA_WS_ROPE_FORWARD = 5
} fsa_ws_kind_t;
fsa_status_t fsa_wait_status(fsa_ws_kind_t kind, fsa_dtype_t dt, int32_t B, int32_t H, int32_t N, int32_t d,
                             fsa_base_t base, double alpha, int32_t w, int32_t R, const void *ws,
                             uint64_t ws_bytes, int32_t *gave_up, void *stream);

/*
 * fsa_debug_force_wait_timeout - diagnostic hook for tests of the failure path (not
 * part of the method). With enable != 0, later one-launch backward and rotary forward
 * calls of this process wait for a value no workgroup publishes and give up after 16
 * polls, so every kernel still exits and fsa_wait_status then reports the give-up;
 * enable = 0 restores normal waits. Process-wide; returns FSA_OK.
 */
fsa_status_t fsa_debug_force_wait_timeout(int32_t enable);

/*
 * fsa_debug_tile_order - diagnostic hook for tests of the dispatch assumptions (not part
 * of the method). Writes, for each workgroup b of a window-kernel grid of nb workgroups
 * (nb = B * H * ceil(N / 64); the one-launch backward runs two such grids back to back),
 * the logical tile it processes (head b_h = tile / ceil(N / 64), row tile = tile mod
 * ceil(N / 64)) into tile_of_block[b] (host memory, nb entries, caller-owned). The
 * kernels rely on the hardware placing workgroup b on XCD b mod 8 and dispatching in
 * increasing b; this order gives each XCD one contiguous range of tiles (whole heads
 * when B * H is a multiple of 8), taken in increasing order. Returns FSA_E_ARG for
 * nb < 0 or a NULL array with nb > 0.
 */
fsa_status_t fsa_debug_tile_order(int32_t nb, int32_t *tile_of_block);

/* Text describing the calling thread's last non-OK status ("" if none). */
const char *fsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FSA_H */
