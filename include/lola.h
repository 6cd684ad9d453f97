/*
 * lola.h — C ABI of the LoLA hot path on AMD MI355X (gfx950): causal linear attention with a
 * fixed-size memory (H, s), a sliding window of exact KV, and a bounded sparse cache of exact KV
 * whose members are chosen by self-recall error (SRE).
 *
 * Source of the method: "LoLA: Low-Rank Linear Attention With Sparse Caching" reading notes
 * (cc.laoqi.cc, paper 2505.23666 v3), part 2 ("Method"):
 *   2.2 Eqs. (3)-(5)   H += phi(k) v^T, s += phi(k); linear read-out H^T phi(q) / phi(q)^T s
 *   2.3 Eq. (10)       SRE(k, v | H, s) = || H^T phi(k) / (phi(k)^T s) - v ||_2
 *   2.4 Eqs. (11)-(13) candidates = cache + the token leaving the window; keep the lambda largest
 *                      SRE (scored against the state before the update); fold the rest into H, s
 *   2.5 Eq. (14)       y = [H^T phi(q) + sum_cache a v + sum_window a v] / [phi(q)^T s + sum a + sum a],
 *                      a = exp(q^T k / sqrt(d_k))
 *   2.6 Eq. (15)       chunked prefill: allocation once per chunk of C tokens against the chunk-start
 *                      state; candidates = cache + the window tokens that leave during the chunk
 *
 * Semantics fixed where the notes leave a step open:
 *   - the window of query t is positions max(0, t-eta+1) .. t; token i leaves it at time i + eta;
 *   - a folded token that was leaving the window becomes visible in (H, s) at its exit time; a folded
 *     former cache member becomes visible at the chunk start; each step scores, folds, then reads out;
 *   - lambda == 0 or eta >= C - 1 (a chunk may only promote tokens all its queries have seen);
 *   - if phi(k)^T s == 0 the recall is zero, so SRE = ||v||;
 *   - exactly lambda are kept; equal SRE keeps the older position.
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers owned by the caller.  The library never allocates,
 *     frees or synchronises; all work is enqueued on `stream` (a hipStream_t; NULL = default stream),
 *     or on a second stream the caller hands to lola_prefill_ex (lola_overlap), and the call returns
 *     before it completes.
 *   - Arguments are validated on the host before anything is enqueued.  A failed validation returns
 *     LOLA_EINVAL or LOLA_EUNSUPPORTED and leaves the state (device arrays and `t`) untouched.
 *     A launch failure returns LOLA_EDEVICE (the state may then be partially updated).
 *   - No global state: the library keeps no stream, event, lock or cached device property between
 *     calls, so distinct states may be driven from different threads and streams.  (The one exception
 *     is lola_prefill_noalloc's scratch array and its per-device address, below.)
 *   - Supported shapes (v1): d_k == d_v in {64, 128}, D == 128, 0 <= lambda <= 1024, 1 <= C <= 128,
 *     eta >= 0, positions below 2^31.
 *   - Device arrays must be 16-byte aligned.
 */
#ifndef LOLA_H
#define LOLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t lola_status;
#define LOLA_OK 0
#define LOLA_EINVAL (-1)        /* bad argument: null pointer, bad size, misalignment, small workspace */
#define LOLA_EUNSUPPORTED (-2)  /* well-formed but outside the shapes the kernels are built for */
#define LOLA_EDEVICE (-3)       /* a HIP launch or runtime call failed */

/* Storage type of q, k, v, y and of the window / cache K, V.  H and s are always fp32. */
#define LOLA_F32 0
#define LOLA_BF16 1

/* Feature map phi: R^{d_k} -> R^D (section 2.2).  W is shared by queries, keys, heads and batches.
 *   LOLA_PHI_ELU1:       phi(x) = elu(xW) + 1,                     W: [d_k][D]   fp32 row-major
 *   LOLA_PHI_SOFTMAX_PM: phi(x) = [softmax(xW); softmax(-xW)],     W: [d_k][D/2] fp32 row-major */
#define LOLA_PHI_ELU1 0
#define LOLA_PHI_SOFTMAX_PM 1

typedef struct lola_phi {
    int32_t kind;      /* LOLA_PHI_* */
    int32_t d_k;       /* must equal the state's d_k */
    int32_t D;         /* feature dimension; must equal the state's D */
    int32_t reserved;
    const float *W;    /* device, fp32, row-major, see above */
} lola_phi;

/* The persistent per-layer state of B sequences x n_heads heads (section 2.4's three memories).
 * The struct itself lives in host memory; the arrays it points to are device memory.
 *   H         [B][n_heads][d_v][D]  fp32   H transposed: entry (i, j) of H (feature i, value j) is at
 *                                          offset j*D + i within a head
 *   s         [B][n_heads][D]       fp32
 *   win_k     [B][n_heads][eta][d_k]       dtype; ring: position p lives in slot p mod eta
 *   win_v     [B][n_heads][eta][d_v]       dtype
 *   cache_k   [B][n_heads][lambda][d_k]    dtype; slot order is arbitrary
 *   cache_v   [B][n_heads][lambda][d_v]    dtype
 *   cache_pos [B][n_heads][lambda]  int32  absolute position held by each slot, -1 = empty
 *   t                                      tokens consumed by every sequence (host value, advanced
 *                                          by lola_prefill and lola_decode_step)
 * Pointers for zero-sized arrays (eta == 0 or lambda == 0) may be NULL. */
typedef struct lola_state {
    int32_t B, n_heads, d_k, d_v, D, eta, lambda, dtype;
    int64_t t;
    float *H;
    float *s;
    void *win_k, *win_v;
    void *cache_k, *cache_v;
    int32_t *cache_pos;
    /* Query-accumulated cache scores (section 4.5, Table 4), used only by the LOLA_SCORE_* rules other
     * than LOLA_SCORE_SRE and otherwise ignored (may be NULL):
     *   win_score   [B][n_heads][eta]     fp32  score gathered so far by the window token in each ring slot
     *   cache_score [B][n_heads][lambda]  fp32  final score of the key in each cache slot
     * A state keeps one scoring rule for its whole life; lola_state_init zeroes both. */
    float *win_score;
    float *cache_score;
    /* Chunked decode (lola_decode_step_ex with decode_chunk > 1; may be NULL otherwise):
     *   dec_fold  [B][n_heads] uint64, device: which of the open group's leaving tokens are folded at
     *             their exit (bit = exit time mod decode_chunk)
     *   dec_chunk host: the decode_chunk of the group still open (0: none).  lola_state_init sets 0.
     *             While a group is open only lola_decode_step_ex with the same decode_chunk accepts the
     *             state; every other entry point returns LOLA_EINVAL. */
    uint64_t *dec_fold;
    int32_t dec_chunk;
    int32_t reserved_state;
} lola_state;

/* Read-branch masks (section 4.8, Table 12): the memories a query reads in Eq. (14).  Storage and
 * allocation do not depend on the mask: a hidden memory keeps its keys, its terms just leave both the
 * numerator and the denominator.  Every mask contains LOLA_READ_WINDOW, the one memory that always
 * holds the current token. */
#define LOLA_READ_STATE 1    /* the linear state H, s (with the chunk's newly folded tokens) */
#define LOLA_READ_SPARSE 2   /* the sparse cache of exact KV */
#define LOLA_READ_WINDOW 4   /* the sliding window */
#define LOLA_READ_ALL 7

/* Cache-scoring rules (section 4.5, Table 4).  LOLA_SCORE_SRE ranks the candidates by self-recall error
 * against the chunk-start state (Eq. (10)).  The others give each key a score accumulated over the
 * queries whose window holds it, from one query's e = exp(q.k / sqrt(d_k)) and p = phi(q).phi(k):
 * (e - p)^2, |e - p|, p / e, or e.  An allocation at a chunk start uses what the queries before it have
 * added; a key's score is fixed once it leaves the window.  Every rule keeps the lambda largest scores,
 * ties to the older position. */
#define LOLA_SCORE_SRE 0
#define LOLA_SCORE_KERNEL_SQ 1
#define LOLA_SCORE_KERNEL_ABS 2
#define LOLA_SCORE_RATIO 3
#define LOLA_SCORE_ATTN 4

/* Resources for the overlapped prefill schedule, created and owned by the caller.  With them, the
 * read-out of chunk ranges the allocation chain has finished runs on `stream` below, beside the chain's
 * next range, which keeps running on the call's stream.  The second stream forks from the call's stream
 * and joins back into it through `events`, so the whole call still completes in the call's stream order
 * (later work on that stream sees all of it).  The library creates, keeps and destroys nothing.
 *   stream  hipStream_t, not NULL and not the call's stream.  Keep it at the default priority.
 *   events  LOLA_OVERLAP_EVENTS hipEvent_t handles, none NULL (hipEventDisableTiming is enough).
 * A block may serve any number of calls one after another, also calls whose device work is still
 * running.  Two calls enqueued at the same time from different host threads must not share a block
 * (the events are re-recorded by every call). */
#define LOLA_OVERLAP_EVENTS 9
typedef struct lola_overlap {
    void *stream;
    void *events[LOLA_OVERLAP_EVENTS];
} lola_overlap;

typedef struct lola_options {
    int32_t read_mask;    /* LOLA_READ_* bits, containing LOLA_READ_WINDOW */
    int32_t score_rule;   /* LOLA_SCORE_* */
    int32_t decode_chunk; /* lola_decode_step_ex only: 0 or 1 = allocate every step; 2..64 = chunked decode */
    int32_t reserved;     /* must be 0 */
    /* nullable: without it every kernel of the call runs on the call's stream, one after another */
    const lola_overlap *overlap;
} lola_options;

/* Bytes of device scratch lola_prefill needs for calls of up to n_max tokens with chunk C, for the
 * state's shape.  Returns 0 if the shape is invalid or unsupported. */
size_t lola_workspace_bytes(const lola_state *st, int64_t n_max, int32_t C);

/* Empties the state: H = 0, s = 0, every cache slot empty (cache_pos = -1), t = 0.
 * Window and cache K/V contents are left as they are (they are dead until written). */
lola_status lola_state_init(lola_state *st, void *stream);

/* Chunked prefill (section 2.6, Eq. (15)) of n new tokens for every sequence and head, every kernel on
 * `stream` in turn (lola_prefill_ex with an overlap block runs the read-out beside the chain).
 *   q, k: [B][n_heads][n][d_k], v: [B][n_heads][n][d_v], y (output): [B][n_heads][n][d_v], all in
 *   the state's dtype, contiguous.  Chunk boundaries are t, t+C, t+2C, ... (relative to the call's
 *   starting t).  fold_at (nullable) [B][n_heads][n] int32 receives, for each input token, the
 *   call-local chunk index at which it was folded into (H, s), or -1.
 *   workspace: device scratch of at least lola_workspace_bytes(st, n, C) bytes, 256-byte aligned;
 *   it may be reused once the enqueued work has finished.  On return st->t has advanced by n.
 *   n == 0 is a no-op. */
lola_status lola_prefill(lola_state *st, const lola_phi *phi, const void *q, const void *k,
                         const void *v, int64_t n, int32_t C, void *y, int32_t *fold_at,
                         void *workspace, size_t workspace_bytes, void *stream);

/* lola_prefill plus kernel-boundary timing.  A prefill enqueues four kernels: features, allocation
 * chain, read-out and commit.  events[0] is recorded before the feature kernel, events[i] after the
 * i-th kernel (events[4] after the commit kernel), all on `stream`.  events[i] are hipEvent_t handles
 * created by the caller (any may be NULL).  Arguments, validation and results are those of
 * lola_prefill; nothing is recorded when n == 0 or validation fails. */
lola_status lola_prefill_profiled(lola_state *st, const lola_phi *phi, const void *q, const void *k,
                                  const void *v, int64_t n, int32_t C, void *y, int32_t *fold_at,
                                  void *workspace, size_t workspace_bytes, void *stream,
                                  void *const events[5]);

/* lola_prefill with options (NULL = LOLA_READ_ALL, LOLA_SCORE_SRE and no overlap, which is
 * lola_prefill).  A rule other than LOLA_SCORE_SRE needs the state's win_score and cache_score (16-byte
 * aligned).  LOLA_EINVAL for a mask without the window or with other bits, an unknown rule, non-zero
 * reserved fields, missing score arrays, or an overlap block with a NULL handle or whose stream is the
 * call's own.  The overlap changes where the kernels run, never what they compute: results are
 * bit-identical with and without it. */
lola_status lola_prefill_ex(lola_state *st, const lola_phi *phi, const void *q, const void *k, const void *v,
                            int64_t n, int32_t C, const lola_options *opt, void *y, int32_t *fold_at,
                            void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): lola_prefill_ex without a workspace argument.  The scratch is a
 * device array of LOLA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the process
 * ends; its address is looked up once per device.  A call needs lola_workspace_bytes(st, n, C) <=
 * LOLA_NOALLOC_SCRATCH_BYTES, else LOLA_EUNSUPPORTED before anything is queued.  Calls on one GPU share
 * its array: calls whose device work overlaps on one GPU race (order them on one stream, or wait).
 * Results equal lola_prefill_ex's.  Allocates and frees nothing. */
#define LOLA_NOALLOC_SCRATCH_BYTES (64u << 20)
lola_status lola_prefill_noalloc(lola_state *st, const lola_phi *phi, const void *q, const void *k,
                                 const void *v, int64_t n, int32_t C, const lola_options *opt, void *y,
                                 int32_t *fold_at, void *stream);

/* One decode token for every sequence and head (section 2.4 single-token update, then Eq. (14)):
 * the token leaving the window (if any) joins the candidates, one candidate is folded when the cache
 * overflows, and y is read out.  q, k: [B][n_heads][d_k], v, y: [B][n_heads][d_v] in the state's
 * dtype.  folded_pos (nullable) [B][n_heads] int32 receives the position folded by this step or -1.
 * On return st->t has advanced by 1. */
lola_status lola_decode_step(lola_state *st, const lola_phi *phi, const void *q, const void *k,
                             const void *v, void *y, int32_t *folded_pos, void *stream);

/* lola_decode_step with options (NULL = defaults, which is lola_decode_step).  The read mask applies as
 * in lola_prefill_ex.  A scoring rule other than LOLA_SCORE_SRE returns LOLA_EUNSUPPORTED here: such
 * states decode through lola_prefill_ex with n = C = 1 (or several tokens per call), which is the same
 * single-token update and needs the workspace this entry point does not take.
 *
 * Chunked decode (section 2.6, Eq. (15), Fig. 2, for one token at a time): with decode_chunk = Cd in
 * 2..64 the allocation runs once per group of steps, groups covering the exit times [a, b) with b the
 * next multiple of Cd after a (from a state with t a multiple of Cd every group is Cd steps).  At a
 * group's first step the cache and the tokens that leave the window during the group are scored against
 * the state (as one prefill chunk: same candidates, same top-lambda, ties to the older position); the
 * losing cache members are folded at once, the losing leaving tokens at their own exit step, and the
 * kept leaving tokens take the freed slots.  Each step reads out over the window, the cache members
 * that have left the window and the state, so Cd steps give what lola_prefill with C = Cd gives on
 * the same tokens.  Needs st->dec_fold (8-byte aligned), folded_pos == NULL (a group step may fold
 * several tokens) and lambda == 0 or eta >= Cd - 1; LOLA_EINVAL otherwise.  The group's last step closes
 * it (st->dec_chunk back to 0). */
lola_status lola_decode_step_ex(lola_state *st, const lola_phi *phi, const void *q, const void *k, const void *v,
                                const lola_options *opt, void *y, int32_t *folded_pos, void *stream);

/* SRE collision map of the prefill call that just ran (section 4.4, Fig. 3; relative form Fig. 10 and
 * Eq. (26)): the self-recall error (Eq. (10)) of each of the call's tokens against the linear state at
 * the end of each of the call's chunks.
 *   Row r (0 <= r < R = ceil(n / C)) is the state (H, s) at the end of call-local chunk r; for r < R - 1
 *   it is read from the chunk records the call left in `workspace`, the last row is st's current H, s.
 *   out [B][n_heads][R][n] fp32 (device): out[.., r, i] = SRE(phi(k_i), v_i | H_r, s_r) if
 *   0 <= fold_at[i] <= r (token i is in that state), else 0 (still in the window or the cache, or never
 *   folded).  relative = 1: each entry minus the same token's entry at row fold_at[i], so that row is
 *   0 (Eq. (26) is a difference, not a ratio).  phi(k_i) is the feature row the call stored in the
 *   workspace.
 *   Contract: call it after the lola_prefill(st, ..., v, n, C, ..., fold_at, workspace, ...) it maps, in
 *   stream order, with the same st, v, n, C, fold_at (non-NULL there) and workspace, and before anything
 *   else writes the workspace or advances the state.  Otherwise the map is meaningless; every access
 *   still stays inside the buffers sized by these arguments.  v, fold_at, out: 16-byte aligned.
 *   n == 0 is a no-op.  LOLA_EINVAL for NULL or misaligned pointers, relative outside {0, 1}, or a
 *   workspace smaller than lola_workspace_bytes(st, n, C). */
lola_status lola_sre_collisions(const lola_state *st, const void *v, const int32_t *fold_at, int64_t n,
                                int32_t C, const void *workspace, size_t workspace_bytes, int32_t relative,
                                float *out, void *stream);

/* ---------------------------------------------------------------------------------------------
 * HOLA variant (the HOLA reading notes, cc.laoqi.cc paper 2607.02303 v1, part 2 "Method"): a gated
 * delta-rule state (3.1 Eq. (1), 3.5) plus an exact KV cache chosen by write magnitude (3.3 Eqs. (5)-(6)),
 * read through RMS-normalised queries and keys (3.4 Eq. (7)).  For each sequence and head, from an empty
 * memory:
 *   e_t = v_t - alpha_t S_{t-1}^T k^_t,   S_t = alpha_t S_{t-1} + beta_t k^_t e_t^T,   o_t = S_t^T q^_t
 * with k^, q^ the unit-L2-norm key and query; m_t = beta_t ||e_t||_2.  The persistent cache at the start
 * of chunk c (chunks of C tokens) holds the w positions of earlier chunks with the largest m (ties: the
 * older).  Query t of chunk c reads by softmax over that cache, the chunk's tokens up to t, and a null
 * sink (logit sink[h], value 0), with logits (gamma_q*q/rms(q)).(gamma_k*k/rms(k)) / sqrt(d),
 * rms(x) = sqrt(mean(x^2) + 1e-6).  y_t = o_t + sigmoid(gate[h]) * that read-out.
 * --------------------------------------------------------------------------------------------- */

/* Bytes of device scratch hola_prefill needs (0 if the arguments are invalid or unsupported). */
size_t hola_workspace_bytes(int32_t B, int32_t n_heads, int32_t d, int32_t dtype, int64_t n, int32_t C);

/* One HOLA layer call over n tokens of B sequences x n_heads heads (all device pointers):
 *   q, k, v, y [B][n_heads][n][d] in dtype (LOLA_F32 or LOLA_BF16), 16-byte aligned, d in {64, 128, 256};
 *   alpha, beta [B][n_heads][n] fp32 gates (alpha in (0, 1], beta in [0, 1]);
 *   gamma_q, gamma_k [n_heads][d] fp32 cache-path scales; sink, gate [n_heads] fp32;
 *   S_out (nullable) [B][n_heads][d][d] fp32 final state, row = key dimension;
 *   cache_pos_out, cache_score_out (nullable) [B][n_heads][w]: the final persistent cache sorted by
 *   position (-1 / 0 where fewer than w tokens exist) and its write magnitudes.
 * 1 <= C <= 1024, 0 <= w <= 64 (LOLA_EUNSUPPORTED beyond).  workspace: hola_workspace_bytes(...) bytes,
 * 256-byte aligned.  n == 0 is a no-op.  The state path is serial in t within a (sequence, head). */
lola_status hola_prefill(int32_t B, int32_t n_heads, int32_t d, int32_t dtype, int64_t n, int32_t C, int32_t w,
                         const void *q, const void *k, const void *v, const float *alpha, const float *beta,
                         const float *gamma_q, const float *gamma_k, const float *sink, const float *gate,
                         void *y, float *S_out, int32_t *cache_pos_out, float *cache_score_out,
                         void *workspace, size_t workspace_bytes, void *stream);

/* HOLA decode (the same notes, part 2: 3.5 sizes one head's runtime memory as the state plus at most
 * w + C exact key-value rows).  Decode keeps the prefill's chunk grid (chunks of C positions from
 * position 0).  Between tokens the memory of a (sequence, head) is the state S, the persistent cache
 * at the start of the open chunk and the open chunk's tokens so far; a token that closes its chunk
 * merges the chunk into the cache (the w largest magnitudes, ties: the older; sorted by position).
 * Buffers are device memory owned by the caller, rows 16-byte aligned:
 *   S            [B][n_heads][d][d]  fp32   row = key dimension
 *   cache_pos    [B][n_heads][w]     int32  positions, ascending, then -1 for empty slots
 *   cache_score  [B][n_heads][w]     fp32   their write magnitudes (0 for empty slots)
 *   cache_k, cache_v [B][n_heads][w][d] dtype  raw keys and values of the cached tokens
 *   open_k, open_v   [B][n_heads][C][d] dtype  the open chunk's tokens (t mod C of them)
 *   open_score   [B][n_heads][C]     fp32   their magnitudes
 * The cache_* pointers may be NULL when w == 0.  t (host) counts the tokens seen; C and w are fixed
 * for the state's life. */
typedef struct hola_state {
    int32_t B, n_heads, d, dtype, C, w;
    int64_t t;
    float *S;
    int32_t *cache_pos;
    float *cache_score;
    void *cache_k, *cache_v;
    void *open_k, *open_v;
    float *open_score;
} hola_state;

/* An empty memory: t = 0, S = 0, every cache slot empty (enqueued on stream).  LOLA_EINVAL for a
 * malformed state, LOLA_EUNSUPPORTED for sizes hola_prefill does not take. */
lola_status hola_state_init(hola_state *st, void *stream);

/* hola_prefill over n tokens from the empty memory st (st->t must be 0: LOLA_EUNSUPPORTED otherwise),
 * with B, n_heads, d, dtype, C, w taken from st; also leaves the decode memory in st (S, the cache at
 * the start of the open chunk, the open chunk's tokens) and sets st->t = n.  Other arguments and the
 * workspace (hola_workspace_bytes with st's sizes) as for hola_prefill. */
lola_status hola_prefill_state(hola_state *st, int64_t n, const void *q, const void *k, const void *v,
                               const float *alpha, const float *beta, const float *gamma_q, const float *gamma_k,
                               const float *sink, const float *gate, void *y, void *workspace,
                               size_t workspace_bytes, void *stream);

/* One decode token for every (sequence, head) of st: q, k, v, y [B][n_heads][d] in st->dtype; alpha,
 * beta [B][n_heads] fp32; gamma_q, gamma_k [n_heads][d], sink, gate [n_heads] fp32 (all device).
 * The token is written into the state, read out by y_t = S_t^T q^_t + sigmoid(gate) * (softmax over
 * the cache, the open chunk's earlier tokens, the token itself and the sink), joins the open chunk,
 * and st->t advances by one.  No workspace; one kernel on stream. */
lola_status hola_decode_step(hola_state *st, const void *q, const void *k, const void *v, const float *alpha,
                             const float *beta, const float *gamma_q, const float *gamma_k, const float *sink,
                             const float *gate, void *y, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Measurement probes (not part of the method): the device's attainable rates, measured beside the
 * vendor's peaks so that roofline fractions can be stated against both.
 * --------------------------------------------------------------------------------------------- */

/* A dense bf16 matrix loop: `workgroups` workgroups of 4 waves; each wave issues 4 * iters
 * v_mfma_f32_32x32x16_bf16 (32768 FLOP each) from register operands, so one launch performs
 * workgroups * 4 * 4 * iters * 32768 FLOP.  out: device, workgroups * 256 floats, 16-byte aligned
 * (one sum per lane, written so the work is kept).  LOLA_EINVAL for non-positive sizes or a bad out. */
lola_status lola_peak_mfma_bf16(int32_t workgroups, int32_t iters, float *out, void *stream);

/* A streaming device-to-device copy of `bytes` (a multiple of 16; src and dst 16-byte aligned and not
 * overlapping): each byte is read once and written once.  LOLA_EINVAL for bad pointers or sizes. */
lola_status lola_peak_copy(const void *src, void *dst, size_t bytes, void *stream);

/* Static, human-readable text for a status code. */
const char *lola_status_string(lola_status status);

#ifdef __cplusplus
}
#endif

#endif /* LOLA_H */
