/*
 * gdn.h -- libgdn: the Gated DeltaNet (GDN) recurrence of a speculative-decoding
 * verify pass, its GPU-resident commit, and its chunked prefill, for AMD MI355X
 * (gfx950).  Plain C ABI: device pointers, sizes and a HIP stream; no framework
 * types.
 *
 * The recurrence.  The lithos-metal README ("How it works", region table, "GDN
 * mixer" row) partitions a GDN layer's recurrent state by value columns and keeps
 * each slice on chip across a block of input tokens; the devdoido audit ("How does
 * lithos-metal fuse layer mixers on Metal?") says the state is fp32 with a key side
 * and a value side.  The update is the gated delta rule of Gated DeltaNet (Yang,
 * Kautz & Hatamizadeh, ICLR 2025), per (instance, head):
 *
 *     S_t = a_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,    o_t = S_t q_t
 *
 * with S in R^{dv x dk} (row i = value index i), a_t = exp(g_t) where g is the
 * log-decay, and no scaling of q inside the library.
 *
 * Layouts (row-major; every buffer is a caller-owned device allocation):
 *     S          fp32  [B][H][dv][dk]
 *     q, k       in_dt [B][T][H][dk]      (T = block rows, or L = prompt length)
 *     v          in_dt [B][T][H][dv]
 *     g, beta    fp32  [B][T][H]
 *     o          fp32  [B][T][H][dv]
 * B counts independent instances (GDN layers or sequences), H heads per instance.
 *
 * Conventions shared by every call:
 *   - Calls validate their host-visible arguments first and return a negative
 *     gdn_status without launching anything when one is bad.
 *   - Calls enqueue their kernels on `hip_stream` (a hipStream_t; NULL means the
 *     null stream) and return without synchronising the host, except
 *     gdn_record_status, which is a synchronising diagnostic.
 *   - The library allocates no device memory and keeps no global state; all
 *     scratch is in caller-provided buffers.
 *   - Device pointers must be 16-byte aligned (g, beta, n_accepted, pos: 4-byte).
 *   - NaN or Inf inputs propagate to outputs; nothing on the hot path checks them.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gdn_shape {
    int32_t B;   /* independent instances, >= 1 */
    int32_t H;   /* heads per instance, >= 1 */
    int32_t dk;  /* key head dimension: 64 or 128 */
    int32_t dv;  /* value head dimension: 64 or 128 */
} gdn_shape;

typedef enum gdn_in_dtype {
    GDN_IN_F32 = 0,   /* q, k, v are fp32 */
    GDN_IN_BF16 = 1   /* q, k, v are bf16 (the library never rounds them) */
} gdn_in_dtype;

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_EINVAL = -1,  /* null or misaligned pointer, unknown or unsupported dtype */
    GDN_EDIM = -2,    /* B or H < 1, dk or dv not in {64, 128}, sizes overflow */
    GDN_ERANGE = -3,  /* T not in [1, 16], L < 0, chunk not 64 */
    GDN_EWS = -4,     /* record or workspace smaller than required */
    GDN_EHIP = -5     /* the HIP runtime reported an error */
} gdn_status;

/* Error bits a commit leaves in the block record (read by gdn_record_status). */
enum {
    GDN_REC_NO_BLOCK = 1,  /* no verified block to commit: never verified, or already committed */
    GDN_REC_N_RANGE = 2,   /* n_accepted[b] outside [0, T] */
    GDN_REC_SHAPE = 4      /* the record was written for another shape */
};

/* Largest verify block. */
#define GDN_T_MAX 16
/* The only chunk length the prefill supports. */
#define GDN_PREFILL_CHUNK 64

/*
 * Bytes of the block record that gdn_verify_block writes and gdn_commit consumes,
 * for `T` rows of shape `shp` with inputs of dtype `in_dt`.  The record holds a
 * header, per-instance control words, the rows' log-decay prefix sums, the rows'
 * delta vectors (fp32) and a copy of the rows' keys (in_dt).  Returns 0 for an
 * invalid shape, T or dtype.
 */
size_t gdn_block_record_bytes(const gdn_shape *shp, int32_t T, gdn_in_dtype in_dt);

/*
 * Verify a speculative block: the outputs o_1..o_T of T consecutive tokens (the
 * anchor plus T-1 drafted tokens) from the checkpoint state S, without changing S.
 *
 * Source: the lithos-metal README, DSpark paragraph (the target verifies the
 * drafted block and then commits the accepted prefix) and its quick start (seven
 * drafted tokens verified together with one anchor); the devdoido audit, "How
 * does DSpark speculative decoding create more than one token per read?" (each
 * token is one row, eight rows in one pass).  T = 8 is that block.
 *
 *   S        fp32 [B][H][dv][dk], read only: S is the block's checkpoint.
 *   q, k, v  the block's rows, layouts above, dtype in_dt.
 *   g, beta  fp32 [B][T][H]: log-decay (a = exp(g)) and write strength.
 *   T        rows in the block, 1..GDN_T_MAX.
 *   o        fp32 [B][T][H][dv], written: o_t = S_t q_t for t = 1..T.
 *   record   device buffer of at least gdn_block_record_bytes(shp, T, in_dt)
 *            bytes; zero-filled once by the caller after allocation, then owned
 *            by the library's calls.  Overwritten: it becomes the pending block
 *            that gdn_commit consumes, replacing any block not yet committed.
 *
 * Returns GDN_OK or a negative gdn_status (nothing launched on a bad argument).
 */
int gdn_verify_block(const float *S, const void *q, const void *k, const void *v,
                     const float *g, const float *beta, int32_t T, gdn_in_dtype in_dt,
                     const gdn_shape *shp, float *o, void *record, size_t record_bytes,
                     void *hip_stream);

/*
 * Commit the accepted prefix of the pending block on the GPU: S <- S_n, the state
 * after the first n = n_accepted[b] rows of the block, for each instance b.
 *
 * Source: the lithos-metal README, "How it works" (GPU-resident state tracks token
 * positions, accepted tokens and recurrent-state commit/rollback with minimal CPU
 * involvement) and its DSpark paragraph (commit of the accepted prefix); the
 * devdoido audit, DSpark section (rewind brings the recurrent state in line with
 * the accepted tokens after every acceptance decision).
 *
 *   S           fp32 [B][H][dv][dk], the same checkpoint given to the verify;
 *               updated in place.  n = 0 leaves every byte of S untouched
 *               (full rollback); n = T keeps the whole block.
 *   record      the record written by the last gdn_verify_block of this shape.
 *   n_accepted  device int32 [B]: rows of the block to keep, anchor included,
 *               0..T.  Read on the device; the host never sees it.
 *   pos         device int32 [B] or NULL: advanced by n on success.
 *   shp         must equal the verify's shape (checked on the device).
 *
 * The pending block is consumed: a second commit without a new verify changes
 * nothing and sets GDN_REC_NO_BLOCK.  An n outside [0, T] or a shape mismatch
 * changes nothing for that instance and sets GDN_REC_N_RANGE / GDN_REC_SHAPE;
 * such an instance's block stays pending.  Returns GDN_OK or a negative gdn_status.
 */
int gdn_commit(float *S, void *record, const int32_t *n_accepted, int32_t *pos,
               const gdn_shape *shp, void *hip_stream);

/*
 * Commit, then verify, in one pass over the state: exactly gdn_commit(S,
 * record_prev, n_accepted, pos) followed by gdn_verify_block(S, q, k, v, g,
 * beta, T, in_dt, shp, o, record_next, record_next_bytes), with each (instance,
 * head) reading its state from memory once instead of twice.
 *
 * Source: the decode loop of the lithos-metal README, DSpark paragraph (each
 * pass commits the accepted prefix of the previous block, then verifies the next
 * drafted block) and "How it works" (a fused layer mixer keeps its state slice
 * on chip instead of making another round trip to memory); the devdoido audit,
 * DSpark section (the rewind follows every acceptance decision, before the next
 * block).
 *
 *   record_prev  the record of the block to commit (as for gdn_commit); its
 *                error bits, flags and pos are handled exactly as gdn_commit does.
 *   record_next  the record the new block is written to (as for
 *                gdn_verify_block); a different buffer from record_prev (the
 *                two records alternate between passes).
 *   other arguments as for gdn_commit and gdn_verify_block.
 *
 * The new block is verified from the committed state, or from the unchanged
 * state for instances whose commit failed (their error bits are set in
 * record_prev, as gdn_commit would set them).  Returns GDN_OK or a negative
 * gdn_status; GDN_EINVAL also when record_prev == record_next or the two
 * overlap.
 */
int gdn_commit_verify(float *S, void *record_prev, const int32_t *n_accepted, int32_t *pos,
                      const void *q, const void *k, const void *v, const float *g, const float *beta,
                      int32_t T, gdn_in_dtype in_dt, const gdn_shape *shp, float *o, void *record_next,
                      size_t record_next_bytes, void *hip_stream);

/*
 * Diagnostic: copy each instance's commit error bits (GDN_REC_*) into
 * host_err_bits[0..B-1].  Synchronises `hip_stream`.  Bits are cleared by the
 * next gdn_verify_block.
 */
int gdn_record_status(const void *record, const gdn_shape *shp, int32_t *host_err_bits,
                      void *hip_stream);

/*
 * Bytes of workspace with which gdn_prefill_chunked runs its two-phase schedule
 * for prompt length L: a parallel prep builds every chunk's state-independent
 * quantities into the workspace, so the sequential chunk scan carries only
 * state-coupled work.  The prompt's chunks are cut into segments; the prep of
 * each segment runs on the compute units the scan of the previous one leaves
 * idle (one launch per segment, on the caller's stream).  It pays off for few
 * (instance, head) pairs (long scans, idle compute units); 0 means the one-pass
 * schedule is used for this shape and no workspace helps.
 */
size_t gdn_prefill_workspace_bytes(const gdn_shape *shp, int32_t L, int32_t chunk);

/*
 * Chunked prefill: run the recurrence over an L-token prompt, writing every
 * output and advancing S from the initial to the final state.  q, k and v must be
 * bf16 (in_dt == GDN_IN_BF16; GDN_EINVAL otherwise).
 *
 * Source: the devdoido audit, "What does long-context prefill cost on Apple
 * silicon?" (prefill dominates long-context use), with the chunkwise UT/WY form of
 * the gated delta rule (Gated DeltaNet, ICLR 2025): within a chunk the products
 * are dense contractions, between chunks only the fp32 state is carried.
 *
 *   S        fp32 [B][H][dv][dk], in: initial state, out: state after L tokens.
 *   q, k, v, g, beta, o   as for the verify, with L rows.  L >= 0 (L = 0 is a
 *            no-op); the last chunk may be partial.
 *   chunk    GDN_PREFILL_CHUNK.
 *   ws       optional device workspace (16-byte aligned).  With at least
 *            gdn_prefill_workspace_bytes(...) bytes the two-phase schedule runs;
 *            with NULL or fewer bytes the one-pass schedule runs.  Results agree
 *            within rounding either way.
 *
 * Splitting a prompt is exact up to rounding: prefill(L1) then prefill(L2) on the
 * continued inputs equals prefill(L1 + L2).  Returns GDN_OK or a negative status.
 */
int gdn_prefill_chunked(float *S, const void *q, const void *k, const void *v,
                        const float *g, const float *beta, int32_t L, int32_t chunk,
                        gdn_in_dtype in_dt, const gdn_shape *shp, float *o, void *ws,
                        size_t ws_bytes, void *hip_stream);

/* ---------------------------------------------------------------------------
 * Acceptance and rewind, on the device.
 *
 * Source: the audited-numbers page ("Qwen 3.8 27B mac m5: 200 tok/s, audited"),
 * section "How does DSpark speculative decoding create more than one token per
 * read?": acceptance is exact speculative sampling -- greedy keeps a drafted
 * token only where it equals the target model's token, sampled keeps it with
 * probability min(1, p/q) -- and the pass emits a correction token at the first
 * rejection or a bonus token when every draft was kept; rewind then brings the
 * key-value cache, the short filter history and the recurrent state in line with
 * the kept tokens.  The README page ("How it works") keeps positions, accepted
 * tokens and commit/rollback on the GPU: here n_out feeds gdn_commit (or
 * gdn_commit_verify) directly, which rewinds the recurrent state and advances the
 * position (the key-value length) by n; gdn_history_rewind does the filter
 * history.  Nothing is read back to the host.
 *
 * A verify block's T rows are [anchor, d_1, .., d_{T-1}]: the last confirmed
 * token and T - 1 drafted tokens.  Target row t's logits give the distribution of
 * the token after row t; drafter row j (0 .. T-2) is the distribution d_{j+1} was
 * drawn from.  n_out[b] = 1 + (drafts kept) rows are confirmed, 1..T; the
 * emitted token (next_token[b]) is the next block's anchor.
 * ------------------------------------------------------------------------- */
#define GDN_HISTORY_MAX 16

/* B sequences, T rows per block (1..GDN_T_MAX), V vocabulary entries (1..2^26). */
typedef struct {
    int32_t B, T, V;
} gdn_accept_shape;

/* Workspace bytes of gdn_accept_greedy (sampled = 0) or gdn_accept_sampled
 * (sampled = 1); 0 for an invalid shape. */
size_t gdn_accept_workspace_bytes(const gdn_accept_shape *shp, int32_t sampled);

/*
 * Greedy acceptance.  Draft d_{j+1} is kept while it equals the argmax of target
 * row j (the lowest index among equal logits); n_out[b] = 1 + kept drafts and
 * next_token[b] = the argmax of target row n_out[b] - 1 (the correction, or the
 * bonus when all T - 1 drafts were kept).
 *
 *   target_logits  [B][T][V], dtype dt (bf16 or fp32), finite values.
 *   draft_tokens   int32 [B][T-1] (may be NULL when T = 1); a token outside
 *                  [0, V) is never kept.
 *   n_out, next_token   int32 [B], written.
 *   ws             device workspace of gdn_accept_workspace_bytes(shp, 0) bytes,
 *                  16-byte aligned; contents are scratch.
 * All pointers are device memory owned by the caller.  Returns GDN_OK, or a
 * negative status before anything is launched: GDN_EDIM (B < 1 or V out of
 * range), GDN_ERANGE (T out of range), GDN_EWS, GDN_EINVAL (null or misaligned
 * pointer, unknown dtype), GDN_EHIP.
 */
int gdn_accept_greedy(const void *target_logits, gdn_in_dtype dt, const int32_t *draft_tokens,
                      const gdn_accept_shape *shp, int32_t *n_out, int32_t *next_token, void *ws,
                      size_t ws_bytes, void *hip_stream);

/*
 * Sampled acceptance (exact speculative sampling).  With p = softmax(target row /
 * temperature) and q = softmax(drafter row / temperature), draft d_{j+1} is kept
 * while u_accept[b][j] * q(d) < p(d) (the event u < min(1, p/q)).  At the first
 * rejection, at row m, next_token[b] is drawn from max(0, p - q) normalised;
 * when every draft was kept, from p of target row T - 1.  A draw from weights w
 * with uniform u is the smallest x with w_0 + .. + w_x > u (w_0 + .. + w_{V-1});
 * it never returns a zero-weight entry (if the weights underflow to zero in
 * fp32, the row's argmax is returned).
 *
 *   target_logits  [B][T][V]; draft_logits [B][T-1][V] (may be NULL when T = 1);
 *                  both dtype dt, finite.
 *   draft_tokens   int32 [B][T-1]; a token outside [0, V) is rejected.
 *   u_accept       fp32 [B][T-1] in [0, 1); u_sample fp32 [B] in [0, 1): the
 *                  random numbers, drawn by the caller.
 *   temperature    > 0, finite.
 *   n_out, next_token, ws   as for the greedy call (ws of
 *                  gdn_accept_workspace_bytes(shp, 1) bytes).
 * Arithmetic is fp32; decisions within fp32 rounding of their threshold may
 * differ from an exact computation.  Errors as for the greedy call, plus
 * GDN_ERANGE for a temperature that is not positive and finite.
 */
int gdn_accept_sampled(const void *target_logits, const void *draft_logits, gdn_in_dtype dt,
                       const int32_t *draft_tokens, const float *u_accept, const float *u_sample,
                       float temperature, const gdn_accept_shape *shp, int32_t *n_out, int32_t *next_token,
                       void *ws, size_t ws_bytes, void *hip_stream);

/*
 * gdn_accept_sampled without a workspace argument, for callers that cannot
 * allocate device memory at call time (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the workspace is the
 * library's own scratch, a file-scope device array of
 * gdn_accept_noalloc_max_bytes() bytes (1 MiB) on each device the call runs on,
 * held until the process ends.  Same arguments, results and errors as
 * gdn_accept_sampled, except:
 *   - no ws / ws_bytes; a shape whose workspace
 *     (gdn_accept_workspace_bytes(shp, 1)) exceeds the scratch returns GDN_EWS
 *     before anything is launched (about 100 sequences at T = 8, V = 151,936);
 *   - the call runs on the stream's device (the current device for the null
 *     stream); the first call on a device resolves that device's scratch once
 *     (hipGetSymbolAddress), and no call allocates or frees memory;
 *   - every call on a device shares that device's scratch: calls that overlap
 *     on one device (on different streams, or from different threads) race and
 *     must be ordered by the caller.  Nothing in the scratch needs clearing
 *     between calls.
 */
int gdn_accept_sampled_noalloc(const void *target_logits, const void *draft_logits, gdn_in_dtype dt,
                               const int32_t *draft_tokens, const float *u_accept, const float *u_sample,
                               float temperature, const gdn_accept_shape *shp, int32_t *n_out,
                               int32_t *next_token, void *hip_stream);

/* Bytes of the per-device scratch that gdn_accept_sampled_noalloc uses. */
size_t gdn_accept_noalloc_max_bytes(void);

/*
 * Rewind of the filter history (the short causal filter before the mixer keeps
 * its last W inputs).  In place: history[b] becomes the last W rows of
 * [history[b]; rows[b][0 .. n[b]-1]], the history as if only the n[b] confirmed
 * rows of the block had been fed.
 *
 *   history  [B][W][C], dtype dt, updated in place;  rows [B][T][C], dtype dt:
 *            the block's filter inputs;  n  int32 [B] on the device (n_out of an
 *            acceptance call); an n outside [0, T] leaves that history unchanged.
 *   W in 1..GDN_HISTORY_MAX, T in 1..GDN_T_MAX, C >= 1.
 * Returns GDN_OK, GDN_EDIM, GDN_ERANGE, GDN_EINVAL or GDN_EHIP.
 */
int gdn_history_rewind(void *history, const void *rows, const int32_t *n, int32_t B, int32_t W, int32_t T,
                       int32_t C, gdn_in_dtype dt, void *hip_stream);

/* ---------------------------------------------------------------------------
 * The GDN mixer around the recurrence, fused into the verify.
 *
 * Source: the README page ("How it works", region table, "GDN mixer" row): one
 * megakernel runs the layer's projections, recurrence, gating and normalisation
 * in dependency order; the audited-numbers page (DSpark section): a filter
 * before the mixer holds its last few inputs, which a rewind restores.  The pages
 * give no formulas; these follow the published Gated DeltaNet layer (ICLR 2025)
 * as deployed in the Qwen3-Next hybrid.  Per token, from the layer's raw
 * in-projection row x (conv_dim = 2 Hk dk + H dv channels: q heads | k heads |
 * v heads):
 *   c = SiLU(sum_j w[c][j] x_{t-3+j}[c])      width-4 causal filter over the
 *                                             3-row history and the block
 *   q = c_q / |c_q| / sqrt(dk), k = c_k / |c_k|   per q/k head (eps 1e-6 under
 *                                             the root); value head h reads q/k
 *                                             head h / (H / Hk)
 *   v = c_v;  q, k, v rounded to bf16
 *   beta = sigmoid(b), g = -exp(A_log) softplus(a + dt_bias)
 * then the verify (or commit + verify) of gdn_verify_block / gdn_commit_verify,
 * and per token and value head
 *   y = o / sqrt(mean(o^2) + 1e-6) * norm_w * SiLU(z).
 * The block record holds the normalised keys, so gdn_commit and
 * gdn_commit_verify consume it as any other; gdn_history_rewind updates the
 * filter history with the rows x and the accepted n.
 * ------------------------------------------------------------------------- */
typedef struct {
    const void *x;           /* bf16 [B][T][conv_dim]: raw in-projection rows of the block */
    const void *history;     /* bf16 [B][3][conv_dim]: the filter's last 3 inputs, oldest first */
    const float *conv_w;     /* fp32 [conv_dim][4]: filter taps, tap 3 on the current row */
    const float *a, *b;      /* fp32 [B][T][H]: decay and beta pre-activations */
    const float *A_log;      /* fp32 [H] */
    const float *dt_bias;    /* fp32 [H] */
    const void *z;           /* bf16 [B][T][H][dv]: output gate pre-activation */
    const float *norm_w;     /* fp32 [dv]: RMS-norm weight */
    int32_t Hk;              /* q/k heads, H a multiple of Hk */
} gdn_mixer_inputs;

/*
 * gdn_verify_block with the mixer: S fp32 [B][H][128][128] (read only), inputs
 * as above, 1 <= T <= GDN_T_MAX, shp with dk = dv = 128; y fp32 [B][T][H][128]
 * (the gated, normalised outputs); record as for gdn_verify_block with bf16
 * inputs.  All pointers device memory owned by the caller, 16-byte aligned
 * (4-byte for the fp32 vectors).  Returns GDN_OK, or before any launch
 * GDN_EINVAL, GDN_EDIM (not dk = dv = 128, or H not a multiple of Hk),
 * GDN_ERANGE (T), GDN_EWS (record too small), GDN_EHIP.
 */
int gdn_mixer_verify(const float *S, const gdn_mixer_inputs *in, int32_t T, const gdn_shape *shp, float *y,
                     void *record, size_t record_bytes, void *hip_stream);

/* gdn_commit_verify with the mixer: commit record_prev at n_accepted[b] rows,
 * then the mixer verify of the next block into record_next (errors and device
 * behaviour as for gdn_commit_verify and gdn_mixer_verify). */
int gdn_mixer_commit_verify(float *S, void *record_prev, const int32_t *n_accepted, int32_t *pos,
                            const gdn_mixer_inputs *in, int32_t T, const gdn_shape *shp, float *y,
                            void *record_next, size_t record_next_bytes, void *hip_stream);

/* ---------------------------------------------------------------------------
 * The full-attention mixer of the verify pass.
 *
 * Source: the README page ("How it works", region table): the full-attention
 * mixer partitions the K/V context, accumulates online-softmax statistics
 * locally and merges the partial results before the output projection; the
 * audited-numbers page ("How does lithos-metal fuse layer mixers on Metal?"): 16
 * of the 64 layers are full attention, and workers keep small running softmax
 * totals in fp32 so the full score table is never written.
 * ------------------------------------------------------------------------- */

/* B instances (layers x sequences), Hq query heads, Hkv key/value heads (Hq a
 * multiple of Hkv; query head h reads key/value head h / (Hq / Hkv)), head size
 * d in {128, 256}, cache capacity Lmax positions. */
typedef struct {
    int32_t B, Hq, Hkv, d, Lmax;
} gdn_attn_shape;

/* Workspace bytes of gdn_attn_verify for blocks of T rows (the split partials:
 * per query row and split, a running max, a sum and d accumulators, fp32); 0
 * for an invalid shape. */
size_t gdn_attn_workspace_bytes(const gdn_attn_shape *shp, int32_t T);

/*
 * Attention of a T-row verify block.  Query row (t, h) attends to cache
 * positions 0 .. ctx[b]-1 and to the block's rows 0 .. t:
 *   o[b][t][h] = sum_p softmax_p(scale * q[b][t][h] . key_p) value_p.
 * The block's key/value rows are also written into the cache at positions
 * ctx[b] .. ctx[b]+T-1; rewinding the cache is then setting its length (the
 * position gdn_commit advances by n).
 *
 *   q        bf16 [B][T][Hq][d];  k_new, v_new  bf16 [B][T][Hkv][d]: the block's
 *            keys and values.
 *   k_cache, v_cache   bf16 [B][Lmax][Hkv][d], in/out (rows ctx .. ctx+T-1
 *            written).
 *   ctx      int32 [B] on the device: cached positions, 0 <= ctx <= Lmax - T; an
 *            instance outside that range gets NaN outputs and no cache write.
 *   scale    the score scale (1/sqrt(d) in the usual form), finite.
 *   o        fp32 [B][T][Hq][d], written.
 *   ws       device workspace of gdn_attn_workspace_bytes(shp, T) bytes, 16-byte
 *            aligned; contents are scratch.
 * Constraints: 1 <= T <= GDN_T_MAX, T * (Hq / Hkv) <= 256, Lmax >= T.  Returns
 * GDN_OK, or before any launch GDN_EINVAL (null or misaligned pointer), GDN_EDIM
 * (shape), GDN_ERANGE (T, scale), GDN_EWS, or GDN_EHIP.
 */
int gdn_attn_verify(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                    const int32_t *ctx, int32_t T, float scale, const gdn_attn_shape *shp, float *o, void *ws,
                    size_t ws_bytes, void *hip_stream);

/* Static description of a gdn_status value; never NULL. */
const char *gdn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
