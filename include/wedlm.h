/*
 * wedlm.h -- C ABI of the WeDLM streaming-decode step on MI355X (gfx950).
 *
 * One decode step of WeDLM (causal-attention diffusion decoding) is three
 * calls on one HIP stream:
 *
 *   wedlm_reorder        Topological Reordering of the window, RoPE at the
 *                        slots' logical positions, append of the window's
 *                        K/V to the paged prefix cache.
 *   wedlm_step_attn      windowed causal grouped-query attention of the
 *                        reordered window over the cached prefix.
 *   wedlm_select_commit  per-slot confidence (entropy, argmax) over the
 *                        vocabulary, commit of the leading filled run, the
 *                        distance-penalised fill rule (Eq. 11) and refill of
 *                        the window with new masks.
 *
 * wedlm_decode_step runs the same three in one call with fewer launches.
 *
 * The operations are defined on these pages (cited by title and section):
 *  - "WeDLM: Reconciling Diffusion Language Models with Standard Causal
 *    Attention for Fast Inference", paper-summary page (bud-325.pages.dev):
 *    "Key claims" (paper sec. 3.2; sec. 4.1, Eq. 5-6; sec. 5.2) and "Method"
 *    (inference paragraph, Eq. 11);
 *  - the same title's ICML 2026 oral page, abstract;
 *  - risewithvishwas.com WeDLM page, "Core Technical Architecture" table.
 *
 * Conventions shared by every call
 *  - Pointers named "device" are HIP device memory owned by the caller; the
 *    library keeps no pointer after a call returns.  Host pointers are only
 *    the shape structs and scalars.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and never synchronise the device.
 *  - Return value: WEDLM_OK, or an error status after which nothing was
 *    enqueued; wedlm_last_error() then holds a message (thread-local).
 *    Errors from the HIP runtime at launch are WEDLM_ERR_HIP.
 *  - Device-side checks: conditions only the data can reveal (a context
 *    length beyond the block table, a page id outside the pool, a
 *    permutation entry outside the window, non-increasing positions) are
 *    OR-ed as WEDLM_DEV_* bits into *dev_status (device int32, may be NULL).
 *    No out-of-range access is ever made.  BAD_CTX: the sequence is skipped
 *    (no cache write; attention outputs zero).  BAD_PAGE: the reorder skips
 *    that row's append; attention reads page 0 in place of the bad page, so
 *    that sequence's outputs are meaningless.  BAD_PERM: the row is not
 *    written.  BAD_POS is reported only (RoPE is applied at the positions
 *    given).  The caller reads dev_status whenever it likes.
 *  - Layouts are row-major (last index fastest).  dtype WEDLM_BF16 tensors
 *    hold bfloat16 bit patterns; WEDLM_F32 tensors hold float.
 *  - KV cache: pages of page_size (= 16) tokens; k_cache and v_cache are
 *    [num_pages][Hkv][page_size][D]; token t of sequence b sits in page
 *    block_table[b * max_pages + t / page_size], row t % page_size.
 *  - Window state per sequence b: W slots in logical (slot) order; filled
 *    flags (1 = observed token, 0 = mask), logical positions (strictly
 *    increasing along the slots), ctx_len[b] = committed prefix length.
 */
#ifndef WEDLM_H
#define WEDLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    WEDLM_OK = 0,
    WEDLM_ERR_ARG = 1,          /* NULL pointer or bad scalar */
    WEDLM_ERR_SHAPE = 2,        /* inconsistent or out-of-range sizes */
    WEDLM_ERR_UNSUPPORTED = 3,  /* valid but not built: e.g. D not 64/128 */
    WEDLM_ERR_HIP = 4,          /* HIP runtime error at launch */
    WEDLM_ERR_WORKSPACE = 5     /* workspace missing or too small */
} wedlm_status;

typedef enum { WEDLM_F32 = 0, WEDLM_BF16 = 1 } wedlm_dtype;

/* device-side status bits */
#define WEDLM_DEV_BAD_CTX 1u   /* ctx_len[b] < 0, ctx_len[b] + W > max_pages * page_size, or
                                  (attention) ctx_len[b] > the call's max_ctx_len */
#define WEDLM_DEV_BAD_PAGE 2u  /* a needed block_table entry is outside [0, num_pages) */
#define WEDLM_DEV_BAD_PERM 4u  /* a permutation entry is outside [0, W) */
#define WEDLM_DEV_BAD_POS 8u   /* positions negative or not strictly increasing */
#define WEDLM_DEV_BAD_TOKEN 16u /* a window token id outside [0, vocab] (wedlm_model_step) */

typedef struct {
    int32_t B;          /* sequences */
    int32_t W;          /* window slots per sequence, 1..64 */
    int32_t Hq;         /* query heads */
    int32_t Hkv;        /* KV heads; Hq % Hkv == 0, Hq / Hkv <= 16 */
    int32_t D;          /* head dim: 64 or 128 */
    int32_t page_size;  /* tokens per KV page: must be 16 */
    int32_t max_pages;  /* block_table row length */
    int32_t num_pages;  /* pages in the k_cache / v_cache pool */
    int32_t dtype;      /* wedlm_dtype of q, k, v, caches, q_phys, out */
} wedlm_shape;

/*
 * wedlm_reorder -- Topological Reordering + logical RoPE + KV append.
 * (paper-summary page, "Key claims", sec. 4.1 Eq. 5-6: observed tokens move
 * to the physical front while RoPE keeps their logical positions; "Method",
 * inference paragraph: the decode window is put in this order before every
 * causal pass over the cached prefix.)
 *
 * For each sequence b the physical order is: filled slots in slot order,
 * then masked slots in slot order (perm[b][r] = logical slot at physical
 * row r).  Physical row r = slot i = perm[b][r] at position p = pos[b][i]:
 *   q_phys[b][r][h][:]                  = RoPE_p(q[b][i][h][:])     h < Hq
 *   k_cache at token ctx_len[b] + r     = RoPE_p(k[b][i][g][:])     g < Hkv
 *   v_cache at token ctx_len[b] + r     = v[b][i][g][:]
 * RoPE pairs coordinate c with c + D/2 and turns the pair by the angle
 * p * rope_base^(-2c/D) (computed in float64, rotation in float64, result
 * rounded once to the storage dtype).
 *
 *   filled  [B][W] uint8 device        pos [B][W] int32 device
 *   q       [B][W][Hq][D]  device, logical slot order, before RoPE
 *   k, v    [B][W][Hkv][D] device, logical slot order, before RoPE
 *   q_phys  [B][W][Hq][D]  device out, physical order
 *   k_cache, v_cache       device in/out; only tokens ctx_len[b] .. +W-1
 *                          of each sequence are written
 *   block_table [B][max_pages] int32 device; ctx_len [B] int32 device
 *   perm    [B][W] int32 device out
 *   dev_status  device int32 or NULL (WEDLM_DEV_BAD_CTX/PAGE/POS)
 */
int wedlm_reorder(const wedlm_shape *s, const uint8_t *filled, const int32_t *pos,
                  const void *q, const void *k, const void *v, void *q_phys,
                  void *k_cache, void *v_cache, const int32_t *block_table,
                  const int32_t *ctx_len, int32_t *perm, double rope_base,
                  int32_t *dev_status, void *stream);

/*
 * wedlm_step_attn_workspace -- bytes of device workspace wedlm_step_attn
 * needs for this shape when every ctx_len[b] <= max_ctx_len.  May be 0.
 */
size_t wedlm_step_attn_workspace(const wedlm_shape *s, int32_t max_ctx_len);

/*
 * wedlm_step_attn -- windowed causal GQA attention of one decode step.
 * (paper-summary page, "Key claims", sec. 3.2 and 5.2: the step is an
 * ordinary causal pass of the window over the cached prefix; after the
 * reordering every masked slot sees all observed tokens; risewithvishwas
 * page, "Attention Mechanism": plain lower-triangular mask.)
 *
 * For sequence b (L = ctx_len[b], the window's K/V already appended at
 * tokens L .. L+W-1 by wedlm_reorder), query head h, KV head g = h/(Hq/Hkv),
 * physical row r:
 *     o = sum_{t <= L + r} softmax_t(scale * q_phys[b][r][h] . K_t) V_t
 * written to out[b][perm[b][r]][h][:] (logical slot order), in dtype.
 *
 *   q_phys [B][W][Hq][D] device      k_cache, v_cache  device (see top)
 *   block_table, ctx_len, perm       device (as produced by wedlm_reorder)
 *   out    [B][W][Hq][D] device out
 *   scale  softmax scale; 0 means 1/sqrt(D)
 *   max_ctx_len  host upper bound on every ctx_len[b]; sizes the split grid
 *                (a larger ctx_len on the device is reported as BAD_CTX);
 *                max_ctx_len + W <= 524288 (WEDLM_ERR_UNSUPPORTED beyond)
 *   workspace / ws_bytes  device scratch of at least
 *                wedlm_step_attn_workspace(s, max_ctx_len) bytes (NULL if 0);
 *                contents need no initialisation and are not preserved
 *   dev_status   device int32 or NULL (WEDLM_DEV_BAD_CTX/PAGE/PERM)
 */
int wedlm_step_attn(const wedlm_shape *s, const void *q_phys, const void *k_cache,
                    const void *v_cache, const int32_t *block_table, const int32_t *ctx_len,
                    const int32_t *perm, void *out, float scale, int32_t max_ctx_len,
                    void *workspace, size_t ws_bytes, int32_t *dev_status, void *stream);

/*
 * wedlm_step_attn_noalloc -- wedlm_step_attn without a workspace argument,
 * for callers that cannot allocate device memory (code recorded into a HIP
 * graph, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, result bytes and errors as wedlm_step_attn with the workspace
 * removed; the split partials go to a library-owned device array of
 * wedlm_step_attn_noalloc_limit() bytes (32 MiB), one per GPU, held until
 * the process ends.  The call allocates nothing.
 *   Errors: as wedlm_step_attn; WEDLM_ERR_WORKSPACE (nothing enqueued) when
 *   wedlm_step_attn_workspace(s, max_ctx_len) exceeds the limit.
 *   Concurrency: every call on one GPU shares that GPU's array, so calls
 *   that may overlap on one GPU (different streams, different host
 *   threads) race and corrupt each other's results; serialise them (one
 *   stream) or use wedlm_step_attn with separate workspaces.  Nothing in
 *   the array needs to start at any value, and a call leaves it holding
 *   that call's partials.
 */
size_t wedlm_step_attn_noalloc_limit(void);
int wedlm_step_attn_noalloc(const wedlm_shape *s, const void *q_phys, const void *k_cache,
                            const void *v_cache, const int32_t *block_table, const int32_t *ctx_len,
                            const int32_t *perm, void *out, float scale, int32_t max_ctx_len,
                            int32_t *dev_status, void *stream);

/*
 * wedlm_select_commit_workspace -- bytes of device workspace for
 * wedlm_select_commit at (B, W, V): one 16-byte partial per slot and
 * vocabulary part (a row is cut into ceil(V / 16384) parts of equal
 * length unless wedlm_set_select_parts asks for more).  Contents need no
 * initialisation and are not preserved; calls that run at the same time
 * must not share one workspace.
 */
size_t wedlm_select_commit_workspace(int32_t B, int32_t W, int32_t V);

/*
 * wedlm_set_select_parts -- process-wide override of the vocabulary parts
 * per row (1..4096; still at least V / 16384 and at most V / 4), 0 restores
 * the automatic choice.  Affects later workspace queries and calls alike,
 * so a workspace sized before a change may be too small after it (the call
 * then fails with WEDLM_ERR_WORKSPACE).  A tuning knob; results agree with
 * the automatic plan up to the rounding order of the merged sums.
 */
int wedlm_set_select_parts(int32_t parts);

/*
 * wedlm_select_commit -- confidence, commit, Eq. 11 select and refill.
 * (paper-summary page, "Method", inference paragraph, Eq. 11 and "Key
 * claims", sec. 5.2; ICML abstract: confident tokens are committed into a
 * growing left-to-right prefix and the window keeps a fixed size.)
 *
 * Per sequence b, in this order:
 *  1. commit: k = length of the leading run of filled slots;
 *     committed[b][i] = tok[b][i] for i < k, else -1; n_commit[b] = k;
 *     ctx_len[b] += k.  (Those slots' K/V already sit at cache tokens
 *     L .. L+k-1, so nothing is copied.)
 *  2. select: for every masked slot j: a_j = argmax of logits[b][j][:]
 *     (lowest index on ties), H_j = entropy in nats of softmax(logits[b][j]).
 *     j0 = leftmost masked slot; Ht_j = fmaf(alpha, (float)(j - j0), H_j),
 *     all in fp32.  Every masked slot with Ht_j < tau is filled
 *     (tok = a_j, filled = 1); if none is, only the masked slot with the
 *     smallest Ht_j (lowest j on ties) is.  The strict threshold, the
 *     fallback and the tie-breaks are this library's reading of the rule.
 *  3. refill: slots shift left by k; k masks (tok = mask_id, filled = 0)
 *     enter at the right; pos[b][i] = ctx_len[b] + i.
 *  4. counters (if given): counters[b][0] += k (N_new: tokens committed to
 *     the cached prefix) and counters[b][1] += W (N_total: window slots this
 *     step ran through the model), so that the prefix cacheability of the
 *     stream is P_c = N_new / N_total ("Key claims", sec. 3.1, Eq. 4).
 *
 *   logits   [B][W][V] fp32 device (rows of filled slots are not read)
 *   tok, filled, pos [B][W], ctx_len [B]   device, updated in place
 *   n_commit [B], committed [B][W]         device out
 *   argmax_out [B][W] int32, entropy_out [B][W] fp32   device out or NULL;
 *            masked slots get a_j / H_j, filled slots -1 / -1.0f
 *   counters [B][2] int64 device, accumulated in place (the caller zeroes
 *            it at the start of a stream), or NULL
 *   workspace / ws_bytes  see wedlm_select_commit_workspace
 * Logits must be finite.  W <= 64, V >= 1, and B * W * parts below 2^24
 * (WEDLM_ERR_SHAPE otherwise).
 */
int wedlm_select_commit(int32_t B, int32_t W, int32_t V, const float *logits, int32_t *tok,
                        uint8_t *filled, int32_t *pos, int32_t *ctx_len, int32_t *n_commit,
                        int32_t *committed, int32_t *argmax_out, float *entropy_out,
                        int64_t *counters, float alpha, float tau, int32_t mask_id,
                        void *workspace, size_t ws_bytes, void *stream);

/*
 * wedlm_lmhead_select_commit_workspace -- bytes of device workspace for
 * wedlm_lmhead_select_commit at (B, W, V, Dm): the masked-row list, one
 * 16-byte partial per (masked row, 256-entry vocabulary tile) and one per
 * row.  0 if the shape is not supported.  Contents need no initialisation
 * and are not preserved; calls that run at the same time must not share
 * one workspace.
 */
size_t wedlm_lmhead_select_commit_workspace(int32_t B, int32_t W, int32_t V, int32_t Dm);

/*
 * wedlm_lmhead_select_commit -- the LM head fused with the select step.
 * (paper-summary page, "Method", inference paragraph: masked slots are
 * scored by the entropy of the model's predictive distribution and filled
 * with its most likely token; TL;DR: the backbone is Qwen3-8B, hidden size
 * 4096, vocabulary 151936.)
 *
 * Same as wedlm_select_commit with
 *     logits[b][j][v] = sum_k hidden[b][j][k] * lm_head[v][k]
 * taken from bf16 operands with fp32 accumulation (MFMA) and folded into the
 * per-slot statistics as they are produced: no logit is written.  Only the
 * masked slots' rows are computed.
 *
 *   hidden   [B][W][Dm] bf16 device, the window's final hidden states in
 *            logical slot order (16-byte aligned)
 *   lm_head  [V][Dm] bf16 device, row v = output embedding of token v
 *            (16-byte aligned)
 *   other arguments as for wedlm_select_commit; workspace / ws_bytes see
 *   wedlm_lmhead_select_commit_workspace.
 * Dm: a multiple of 64, 64..65536.  B*W <= 4096, W <= 64, V >= 1.
 * Errors: WEDLM_ERR_SHAPE / WEDLM_ERR_ARG / WEDLM_ERR_WORKSPACE before any
 * launch; WEDLM_ERR_HIP if a launch fails.
 */
int wedlm_lmhead_select_commit(int32_t B, int32_t W, int32_t V, int32_t Dm, const void *hidden,
                               const void *lm_head, int32_t *tok, uint8_t *filled, int32_t *pos,
                               int32_t *ctx_len, int32_t *n_commit, int32_t *committed,
                               int32_t *argmax_out, float *entropy_out, int64_t *counters,
                               float alpha, float tau, int32_t mask_id, void *workspace,
                               size_t ws_bytes, void *stream);

/*
 * wedlm_dual_stream_attn_workspace -- bytes of device workspace for
 * wedlm_dual_stream_attn (the paged K/V cache of both streams, rotated
 * queries, block tables and the attention partials); 0 if the shape is not
 * supported.
 */
size_t wedlm_dual_stream_attn_workspace(const wedlm_shape *s, int32_t N);

/*
 * wedlm_dual_stream_attn -- Dual-Stream Masking attention, forward.
 * (paper-summary page, "Method", training paragraph, and "Key claims",
 * sec. 4.2, Eq. 8-10: a clean memory stream and a block-masked prediction
 * stream share position ids; prediction tokens of block i attend to the
 * memory tokens whose logical positions precede block i.)
 *
 * For each of s->B sequences of N tokens at logical positions 0..N-1:
 *   memory token t      sees memory tokens 0..t (causal);
 *   prediction token t  of block i = t / b sees memory tokens 0..i*b-1 and
 *                       the prediction tokens u of its own block with
 *                       (u observed and (t masked or u <= t)) or
 *                       (both masked and u <= t)
 * (Topological Reordering under the causal mask inside the block; the
 * memory rule inside the stream and the block rule are this library's
 * reading of the page).  Both streams take RoPE at the logical positions
 * as in wedlm_reorder; softmax scale 1/sqrt(D).  Computed as two
 * (wedlm_reorder, wedlm_step_attn) pairs on one paged cache: the memory
 * stream as all-observed 64-token windows, each prediction block as one
 * decode-step window over the memory prefix.
 *
 *   s        B = sequences, W = block size b (16, 32 or 64), Hq, Hkv, D,
 *            dtype as for wedlm_step_attn; page_size 16; max_pages and
 *            num_pages are ignored
 *   N        tokens per sequence, a multiple of 64
 *   qm, km, vm  memory stream [B][N][Hq|Hkv][D] device, before RoPE
 *   qp, kp, vp  prediction stream, same layout
 *   flags    [B][N] uint8 device, 1 = observed, 0 = masked (prediction)
 *   out_m, out_p  [B][N][Hq][D] device out, logical order
 *   workspace / ws_bytes  see wedlm_dual_stream_attn_workspace
 *   dev_status  device int32 or NULL
 */
int wedlm_dual_stream_attn(const wedlm_shape *s, int32_t N, const void *qm, const void *km, const void *vm,
                           const void *qp, const void *kp, const void *vp, const uint8_t *flags,
                           void *out_m, void *out_p, double rope_base, void *workspace, size_t ws_bytes,
                           int32_t *dev_status, void *stream);

/*
 * A synthetic decoder for wedlm_model_step: per layer the pre-norm block
 *   h = RMSNorm(x) * attn_norm;  q, k, v = h Wq^T, h Wk^T, h Wv^T
 *   x += (windowed causal attention of the reordered window, as
 *         wedlm_reorder + wedlm_step_attn on this layer's cache) Wo^T
 *   h = RMSNorm(x) * mlp_norm;  x += (silu(h Wg^T) * (h Wu^T)) Wd^T
 * (TL;DR of the paper-summary page: a Qwen3-8B backbone; the block itself
 * is this library's plain reading.)  All weights bf16, row-major with the
 * input dimension contiguous: wq [Hq*D][d_model], wk, wv [Hkv*D][d_model],
 * wo [d_model][Hq*D], w_gate, w_up [d_ff][d_model], w_down [d_model][d_ff];
 * norms [d_model].  k_cache / v_cache: this layer's paged cache as for
 * wedlm_reorder.  Every weight pointer (here and in wedlm_model) must be
 * 16-byte aligned; wedlm_model_step returns WEDLM_ERR_ARG otherwise.
 */
typedef struct {
    const void *attn_norm, *wq, *wk, *wv, *wo, *mlp_norm, *w_gate, *w_up, *w_down;
    void *k_cache, *v_cache;
} wedlm_layer_weights;

typedef struct {
    int32_t n_layers, d_model, d_ff, vocab;
    float rms_eps;
    const void *embed;        /* [vocab + 1][d_model] bf16; row vocab = the mask token */
    const void *final_norm;   /* [d_model] bf16 */
    const void *lm_head;      /* [vocab][d_model] bf16 */
    const wedlm_layer_weights *layers;   /* host array of n_layers */
} wedlm_model;

/*
 * wedlm_model_step_workspace -- bytes of device workspace for
 * wedlm_model_step (activations, split-K partial products, attention and
 * LM-head scratch); 0 if the shapes are not supported.
 */
size_t wedlm_model_step_workspace(const wedlm_model *m, const wedlm_shape *s, int32_t max_ctx_len);

/*
 * wedlm_model_step -- one WeDLM streaming decode step of a whole synthetic
 * decoder: embed the window tokens (tok, logical order; masked slots hold
 * mask_id = vocab), run every layer on its cache with the window reordered
 * by `filled` and RoPE at `pos`, apply the final RMSNorm, then the fused LM
 * head + commit / Eq. 11 select / refill of wedlm_lmhead_select_commit.
 * (paper-summary page, "Method", inference paragraph, and "Key claims",
 * sec. 4.1 and 5.2.)
 *
 *   s        B, W (<= 64), Hq, Hkv, D (64 or 128), page_size 16, max_pages,
 *            num_pages of the layer caches; dtype WEDLM_BF16
 *   block_table [B][max_pages], shared by every layer's cache
 *   tok, filled, pos, ctx_len, n_commit, committed, argmax_out,
 *   entropy_out, counters, alpha, tau  as for wedlm_select_commit
 *            (mask_id = vocab)
 *   hidden_out  [B][W][d_model] bf16 device out (the final normalised
 *            hidden states) or NULL
 *   rope_base, max_ctx_len   as for wedlm_reorder / wedlm_step_attn
 * d_model = Hq * D; d_model and d_ff multiples of 256; B*W <= 4096.
 * Device-side problems are OR-ed into *dev_status (may be NULL).
 */
int wedlm_model_step(const wedlm_model *m, const wedlm_shape *s, const int32_t *block_table, int32_t *tok,
                     uint8_t *filled, int32_t *pos, int32_t *ctx_len, int32_t *n_commit, int32_t *committed,
                     int32_t *argmax_out, float *entropy_out, int64_t *counters, void *hidden_out,
                     float alpha, float tau, double rope_base, int32_t max_ctx_len, void *workspace,
                     size_t ws_bytes, int32_t *dev_status, void *stream);

/*
 * wedlm_decode_step -- one whole streaming decode step: wedlm_reorder, then
 * wedlm_step_attn, then wedlm_select_commit, with the results of those three
 * calls in that order byte for byte, in three kernel launches instead of
 * five.  (paper-summary page, "Method", inference paragraph and Eq. 11:
 * the order of one step's work; "Key claims", sec. 5.2: the per-step
 * forward is short enough that launch overhead matters, which the pages
 * address with captured graphs.)
 *
 * The launches pair work that shares no memory: the reorder with the
 * vocabulary statistics (both only read the window flags); the split-KV
 * attention alone; the split combine with the commit / select / refill
 * (the combine reads only the split partials and perm, the commit rewrites
 * the window state and ctx_len).  On the small windows this removes two
 * launch latencies from the step's critical path.
 *
 * Every pointer in *io means what the argument of the same name means in
 * those three calls (shapes in s; V, max_ctx_len, mask_id, scale, alpha,
 * tau, rope_base host values as there).  argmax_out, entropy_out, counters
 * and dev_status may be NULL.
 *   workspace / ws_bytes  device scratch of at least
 *         wedlm_decode_step_workspace(s, max_ctx_len, V) bytes (the split
 *         partials, then the vocabulary partials); contents need no
 *         initialisation and are not preserved.
 *   Errors: as the three calls (nothing is enqueued when a check fails).
 */
typedef struct {
    /* window state, device, updated in place */
    int32_t *tok;
    uint8_t *filled;
    int32_t *pos;
    int32_t *ctx_len;
    /* this step's inputs, device */
    const void *q;          /* [B][W][Hq][D] logical slot order, before RoPE */
    const void *k;          /* [B][W][Hkv][D] */
    const void *v;          /* [B][W][Hkv][D] */
    const float *logits;    /* [B][W][V] fp32 */
    /* paged cache, device */
    void *k_cache;
    void *v_cache;
    const int32_t *block_table;
    /* outputs, device */
    void *q_phys;           /* [B][W][Hq][D] */
    int32_t *perm;          /* [B][W] */
    void *out;              /* [B][W][Hq][D] logical slot order */
    int32_t *n_commit;      /* [B] */
    int32_t *committed;     /* [B][W] */
    int32_t *argmax_out;    /* [B][W] or NULL */
    float *entropy_out;     /* [B][W] or NULL */
    int64_t *counters;      /* [B][2] accumulated, or NULL */
    int32_t *dev_status;    /* or NULL */
    /* host parameters */
    int32_t V;
    int32_t max_ctx_len;
    int32_t mask_id;
    float scale;            /* 0 means 1/sqrt(D) */
    float alpha;
    float tau;
    double rope_base;
} wedlm_step_io;

size_t wedlm_decode_step_workspace(const wedlm_shape *s, int32_t max_ctx_len, int32_t V);
int wedlm_decode_step(const wedlm_shape *s, const wedlm_step_io *io, void *workspace, size_t ws_bytes,
                      void *stream);

/*
 * wedlm_decode_step_timed -- wedlm_decode_step whose attention launch (the
 * split kernel, the step's dominant kernel) also sets two caller-created
 * hipEvent_t: attn_start when the kernel starts and attn_stop when it ends,
 * both from the dispatch's own timestamps (hipExtLaunchKernel), so no
 * marker is added to the stream and hipEventElapsedTime gives the kernel's
 * duration.  Either may be NULL.  For profiling a running decode loop; the
 * results are those of wedlm_decode_step.  Not for use under graph capture.
 */
int wedlm_decode_step_timed(const wedlm_shape *s, const wedlm_step_io *io, void *workspace, size_t ws_bytes,
                            void *stream, void *attn_start, void *attn_stop);

/*
 * wedlm_attn_plan -- the split-KV launch plan wedlm_step_attn uses for
 * this shape and bound: work-groups per (sequence, KV head, row tile)
 * (*nsplit) and keys per work-group (*split_keys).  Either may be NULL.
 */
int wedlm_attn_plan(const wedlm_shape *s, int32_t max_ctx_len, int32_t *nsplit,
                    int32_t *split_keys);

/*
 * wedlm_set_attn_split_keys -- process-wide override of the keys per
 * split-KV work-group (a multiple of 64, 64..32768), 0 restores the
 * automatic choice.  Affects later workspace queries and calls alike.
 */
int wedlm_set_attn_split_keys(int32_t keys);

/*
 * Tail splits (bf16).  When the plan has one split per (sequence, KV head)
 * and those work-groups fill between half and all of the CUs in one round,
 * the call is bound by its longest sequences, each streaming alone on one
 * CU once the short ones are done.  The plan then cuts the `tail` longest
 * sequences of the batch in two (ranked on the device from ctx_len at each
 * call, longest first, ties by index): one more work-group per KV head
 * takes the back part of each, and only their rows go through split
 * partials and the combine.  The cut is placed so both parts would end
 * together if every work-group streamed at one rate and the back part
 * started when a CU frees up (rounded up to 64 keys).  The result
 * is the same softmax attention; wedlm_attn_plan then reports nsplit = 2.
 *
 * wedlm_attn_tail -- the number of sequences the plan cuts for this shape
 * and bound (0: tail splits off), or -1 on a bad shape.
 * wedlm_set_attn_tail -- process-wide override: -1 automatic (3/8 of the
 * batch, rounded up, where the plan qualifies), 0 off, n > 0 the n longest
 * (at most B) wherever the plan has one split per group, one row tile, no
 * more groups than CUs and B <= 1024.  Affects later workspace queries and
 * calls alike.
 */
int32_t wedlm_attn_tail(const wedlm_shape *s, int32_t max_ctx_len);
int wedlm_set_attn_tail(int32_t n);

/*
 * Graph capture of decode steps -- the launch-latency remedy the pages
 * point to for a small causal prefill over the window ("Key claims",
 * sec. 5.2: the step stays a standard causal forward, so graph capture
 * applies unchanged).  Every entry point above only launches kernels and
 * device copies on its stream -- no allocation, no synchronisation, no
 * memset -- so any sequence of them (for example K whole steps of
 * reorder, attention and select) can be recorded once and replayed as one
 * launch:
 *
 *   wedlm_graph_begin(stream);            stream: a created stream, not 0
 *   ... library calls on `stream` ...     recorded, not run
 *   wedlm_graph_end(stream, &g);          instantiates; *g owned by caller
 *   wedlm_graph_launch(g, stream2);       replays on any stream, any times
 *   wedlm_graph_destroy(g);
 *
 * A replay reads and writes the buffers the recorded calls named, with the
 * scalars (shapes, alpha, tau, ...) fixed at capture; the caller restores
 * or advances the window state between replays as the recorded steps
 * expect.  Capture is thread-local (hipStreamCaptureModeThreadLocal).  If a
 * call fails validation during capture, call wedlm_graph_end anyway and
 * destroy what it returns.
 */
typedef struct wedlm_graph wedlm_graph;
int wedlm_graph_begin(void *stream);
int wedlm_graph_end(void *stream, wedlm_graph **out);
int wedlm_graph_launch(const wedlm_graph *g, void *stream);
/* Nodes of a captured graph: kernel launches, and all others (copies). */
int wedlm_graph_nodes(const wedlm_graph *g, size_t *kernels, size_t *others);
void wedlm_graph_destroy(wedlm_graph *g);

/* Thread-local message describing the last non-OK status ("" if none). */
const char *wedlm_last_error(void);

/* Library version string. */
const char *wedlm_version(void);

#ifdef __cplusplus
}
#endif
#endif /* WEDLM_H */
