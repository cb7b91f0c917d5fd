/*
 * looped_kv.h -- C ABI of the MI355X (gfx950) library for lazy looped-Transformer
 * inference.
 *
 * A looped Transformer runs P prelude layers, a block of R shared layers K times
 * (a learned loop embedding added to the state before each loop), Q coda layers
 * and a final RMSNorm; effective depth P + R*K + Q ("FlashLoop" walk-through,
 * discosf.com, sections 3.1, 3.2, 4.1).  Each extra loop costs one more pass and,
 * with a per-loop KV cache, one more KV set (FlashLoop abstract, arxivdaily.com;
 * per_loop / last_loop modes: Looped Transformer tutorial, aiboss88.com, step 4).
 * The lazy mode applies the three reductions named in the FlashLoop abstract:
 * token-sparse loop updates, sparse attention over a stable subset of key
 * columns, and low-bit quantized KV residuals between adjacent loops.  The
 * abstract gives no exact rules; the rules implemented are:
 *
 *   loop 1 is dense and writes the base KV (bf16, or int8 group-32 codes with
 *   float16 scales); its causal attention probabilities, summed over all
 *   prompt queries and over the query heads of each KV head, rank the key
 *   columns, and the top_s columns (ties to the lower index) form the stable
 *   set S of that (sequence, shared layer, KV head);
 *   at loop k >= 2 the n = clamp(ceil(rho*T - 1e-9), 1, T) tokens with the
 *   largest ||h_{k-1} - h_{k-2}||^2 (h_0 = prelude output; ties to the lower
 *   index) are recomputed and the others carry forward; a recomputed query at
 *   position i attends over (S intersect [0, i]) union [i-window+1, i];
 *   the loop-k KV of a recomputed row is stored as the quantized residual
 *   against the loop-(k-1) reconstruction (int4 or int8 codes, one float16
 *   scale per 32 elements, scale = fp16_rne(amax / qmax), code =
 *   rint_half_even(r / scale) clamped to +-qmax); 16 bits stores the row.
 *   A decode token runs every loop and is always stored.
 *
 * Memory: the caller owns all device memory (weights, ids, outputs, the KV-store
 * buffer and the workspace); the library never allocates device memory.  All
 * work is enqueued on the caller's HIP stream (passed as void*; NULL means the
 * default stream) with no host synchronisation (except the snapshot copies,
 * which wait for their stream).  Every call returns LK_OK (0) or
 * a negative LK_ERR_* code and leaves a message for lk_last_error() (thread
 * local); errors detected on the host are reported before anything is launched.
 * Calls that share a store or workspace must be ordered on one stream.
 */
#ifndef LOOPED_KV_H
#define LOOPED_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LK_OK 0
#define LK_ERR_INVALID_ARG (-1)  /* null pointer, bad size, inconsistent config */
#define LK_ERR_UNSUPPORTED (-2)  /* valid but not implemented (e.g. head_dim 96) */
#define LK_ERR_CAPACITY (-3)     /* store or workspace too small, decode past max */
#define LK_ERR_HIP (-4)          /* a HIP runtime call or launch failed */
#define LK_ERR_STATE (-5)        /* call out of order (decode before prefill, ...) */

#define LK_MODE_PER_LOOP 0
#define LK_MODE_LAST_LOOP 1
#define LK_MODE_LAZY 2

#define LK_ACT_GELU 0   /* exact erf GELU, FFN = W_down gelu(W_up x) */
#define LK_ACT_SWIGLU 1 /* FFN = W_down (silu(W_gate x) * W_up x) */

/* Model shape.  head_dim must be 32, 64 or 128; n_heads a multiple of
 * n_kv_heads with n_heads / n_kv_heads in {1, 2, 4, 8}; d_model and ffn_dim
 * multiples of 64.  RMSNorm epsilon and RoPE base (rotate-half) as given. */
typedef struct {
    int32_t vocab, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, ffn_act;
    int32_t n_prelude, n_shared, n_loops, n_coda;
    float rms_eps, rope_theta;
    /* 1: input re-injection variant (aiboss88.com tutorial, step 3: the input
     * representation is passed into every loop): the prelude output e is added to
     * the state before every loop k >= 2, as (state + e) + loop_emb[k-1]; in lazy
     * mode only the recomputed rows receive it.  0: no re-injection. */
    int32_t input_reinject;
} lk_model_cfg;

/* Cache/update policy.  mode LK_MODE_*; rho in (0, 1] (kept-token fraction at
 * loops >= 2), top_s >= 1 stable columns, window >= 1, base_bits 16 | 8,
 * res_bits 16 | 8 | 4, group must be 32.  Only mode LK_MODE_LAZY reads the
 * other fields.  stale_keys (0 | 1): 0 ranks a token carried through loop k-1 by
 * its change there, which is zero, so loop k >= 3 picks within the tokens loop
 * k-1 recomputed; 1 lets a carried token keep the change measured when it was
 * last recomputed (loop 2 measures every token), so tokens left out by one loop
 * can be picked again later (the FlashLoop abstract, arxivdaily.com: state
 * changes concentrate on a small subset of tokens as the loops proceed). */
typedef struct {
    int32_t mode;
    double rho;
    int32_t top_s, window, base_bits, res_bits, group;
    int32_t stale_keys;
    /* refresh_every = p > 0: every loop k >= 2 with (k - 1) % p == 0 recomputes every
     * token instead of the top n (the token set is refreshed periodically; attention
     * stays sparse and the residual rows of all tokens are stored); 0: never. */
    int32_t refresh_every;
    /* diff_attn (0 | 1): 1 takes the difference reading of sparse attention (the
     * FlashLoop abstract, arxivdaily.com: the attention-output differences between
     * loops come from a sparse, stable set of key columns).  A row recomputed at loop
     * k >= 2 outputs its previous output plus the change of its sparse term, which is
     * its sparse output a_k plus o_1 - a_1, o_1 its dense loop-1 output and a_1 its
     * loop-1 sparse output (same column set, loop-1 reconstruction).  Prefill keeps
     * o_1 - a_1 for every prompt row and shared layer in the workspace (float16,
     * R * batch * tokens * n_heads * head_dim * 2 bytes); a decode token computes its
     * own at its loop 1 (float32).  The store is unchanged.  0: a_k alone. */
    int32_t diff_attn;
    /* skip_tau >= 0: decode-time loop skipping (the FlashLoop abstract: state changes
     * concentrate on fewer tokens as the loops proceed, carried into decode).  A decode
     * token enters loop k >= 2 only if ||h_{k-1} - h_{k-2}||^2 >= skip_tau (h_0 the
     * prelude output); otherwise it leaves the loops with h_{k-1}, and for loops k..K
     * stores no residual row (slot map entry -1: its reconstruction stays the
     * previous loop's; its slot stays reserved).  In a batched step the sequences that
     * left are masked: every launch still runs.  0: never skipped. */
    float skip_tau;
} lk_lazy_cfg;

/* Device pointers of one layer, all bfloat16 row-major:
 *   attn_norm, ffn_norm  [d]
 *   wqkv  [(H + 2 Hkv) * hd, d]  rows: q heads, then k heads, then v heads
 *   wo    [d, H * hd]
 *   w_in  SwiGLU: [2F, d] (gate rows 0..F-1, up rows F..2F-1); GELU: [F, d]
 *   w_down [d, F] */
typedef struct {
    const void *attn_norm, *wqkv, *wo, *ffn_norm, *w_in, *w_down;
} lk_layer_weights;

/* tok_emb bf16 [vocab, d]; loop_emb bf16 [n_loops, d]; final_norm bf16 [d];
 * layers: HOST array of P + R + Q entries (prelude, shared block, coda). */
typedef struct {
    const void *tok_emb, *loop_emb, *final_norm;
    const lk_layer_weights *layers;
} lk_weights;

typedef struct lk_handle lk_handle;
typedef struct lk_kv_store lk_kv_store;

/* Validate the configuration and bind the weights (pointers are kept, not
 * copied: they must stay valid until lk_destroy). */
int lk_create(const lk_model_cfg *cfg, const lk_lazy_cfg *lazy, const lk_weights *w,
              lk_handle **out);
void lk_destroy(lk_handle *h);

/* KV store for `batch` sequences: one prefill of `prompt_tokens` tokens, then
 * decode steps up to `max_tokens` tokens per sequence.  Layout of the caller's
 * device buffer (all regions 256-byte aligned), per mode:
 *   dense prelude/coda layers: bf16 [P+Q][K|V][batch][Hkv][max_tokens][hd];
 *   per_loop: bf16 [n_loops][R][K|V][batch][Hkv][max_tokens][hd];
 *   last_loop: bf16 [R][K|V][batch][Hkv][max_tokens][hd];
 *   lazy: base [R][K|V][batch][Hkv][max_tokens][hd] as bf16, or int8 codes plus
 *   float16 scales [...][hd/32]; residuals [n_loops-1][R][K|V][batch][Hkv][slots]
 *   rows (int4 packed two per byte low nibble first, int8, or bf16) plus float16
 *   scales; slot maps int32 [n_loops-1][batch][max_tokens] (-1 = not stored);
 *   column sets int32 [R][batch][Hkv][min(top_s, prompt_tokens)];
 *   slots = the most prompt tokens a loop stores (n_selected(prompt_tokens), or
 *   prompt_tokens when some loop k <= n_loops refreshes) + max_tokens - prompt_tokens.
 * With dev_buf == NULL only *need_bytes is written (size query).  Otherwise
 * buf_bytes must be >= *need_bytes; the slot maps are cleared on `stream`
 * (void*, may be NULL) and *out receives a host handle. */
int lk_kv_store_alloc(lk_handle *h, int32_t batch, int32_t prompt_tokens, int32_t max_tokens,
                      void *dev_buf, size_t buf_bytes, void *stream, lk_kv_store **out,
                      size_t *need_bytes);
void lk_kv_store_release(lk_kv_store *s);

/* Bytes the store holds for its current length t (prompt + decoded tokens):
 * *shared = shared-block KV (base, residual rows, slot maps, column sets, or
 * the dense per-loop / last-loop rows); *total adds the prelude/coda rows.
 * Per-token figures divide by batch * t. */
int lk_kv_store_bytes_used(const lk_kv_store *s, size_t *shared, size_t *total);
/* Bytes of the lazy store's decode cache (0 in the other modes): for every loop
 * k >= 2 (k >= 1 with diff_attn) and shared layer, the float16 loop-k
 * reconstruction of (1) the stable
 * columns S, written at the end of prefill (S and those reconstructions do not
 * change afterwards), and (2) a ring of the last window + 16 positions (rounded up
 * to 128), filled at the end of prefill and extended by every decode step.  The
 * token-sparse decode attention reads these instead of reconstructing its
 * columns from base + residuals every step.  It is derived data, allocated with
 * the store (included in need_bytes) and not counted by lk_kv_store_bytes_used. */
int lk_kv_store_cache_bytes(const lk_kv_store *s, size_t *bytes);
/* Current tokens per sequence (0 before prefill). */
int lk_kv_store_length(const lk_kv_store *s, int32_t *tokens);
/* Float16 range check of the lazy store.  The pages fix no number format for the
 * attention operands (FlashLoop abstract: KV stored as low-bit residuals); this
 * library keeps the shared block's int8-base operands (code x scale), its loop-k
 * decode caches and q in float16.  The writer raises a flag on the device when an
 * element it handles -- a rotated q, a rotated K or a V element of a shared layer, as
 * the projections produced it -- is not finite or has |x| > 65504: those forms would
 * hold inf for it, and the outputs that depend on them are then not to be trusted
 * (codes and scales in the store stay finite; scales saturate at 65504).
 * *out_of_range receives 1 if the flag was raised since lk_kv_store_alloc or the
 * last call with clear != 0, else 0; clear != 0 then lowers it.  The call orders
 * itself after the work already on `stream` and waits for it (a device-to-host copy
 * of 4 bytes).  Snapshots carry the flag.  Dense prelude/coda layers (bf16 rows)
 * and the per_loop / last_loop modes never raise it.  LK_ERR_INVALID_ARG for a
 * null argument; LK_ERR_HIP when the copy fails. */
int lk_kv_store_range_check(lk_kv_store *s, int32_t clear, int32_t *out_of_range, void *stream);

/* Workspace bytes for a prefill of batch x tokens (tokens = 1 for decode). */
int lk_workspace_bytes(lk_handle *h, int32_t batch, int32_t tokens, size_t *bytes);

/* Prefill.  d_ids int32 [B, T] (device), B = store batch, T = store
 * prompt_tokens; d_out float32 [B, T, d] receives the final-normed hidden
 * states.  Runs embed, prelude, the K loops (lazy: dense loop 1 with column
 * selection, then token-sparse loops 2..K), coda and the final norm. */
int lk_looped_prefill(lk_handle *h, lk_kv_store *s, const int32_t *d_ids, int32_t B, int32_t T,
                      float *d_out, void *d_ws, size_t ws_bytes, void *stream);

/* One decode step: d_ids int32 [B] (device, the next token of every sequence),
 * d_out float32 [B, d].  Appends one token per sequence at position t = current
 * length; LK_ERR_CAPACITY once t == max_tokens, LK_ERR_STATE before prefill.
 * The step's launches read t from the store's device counter and the ids/output
 * through fixed workspace rows, so on a non-null stream the step is captured
 * once as a HIP graph (per store, workspace, stream and timing class) and
 * replayed on later calls; the results equal those of the launched kernels. */
int lk_looped_decode_step(lk_handle *h, lk_kv_store *s, const int32_t *d_ids, float *d_out,
                          void *d_ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory or call allocating routines (code
 * that a caller records into its own HIP graph, tight serving loops, harnesses that
 * forbid hipMalloc): lk_looped_decode_step with the workspace taken from a static
 * device array of 64 MiB per GPU that the library holds until the process ends, and
 * with the step's kernels launched on `stream` one by one (no graph of its own, so a
 * caller's capture records them).  Same arguments and results as
 * lk_looped_decode_step otherwise.  LK_ERR_CAPACITY when the decode workspace of this
 * model and batch (lk_workspace_bytes(batch, 1)) exceeds 64 MiB.  Every call on one
 * GPU uses that GPU's one array: calls that overlap on a GPU (other streams, other
 * threads, other handles) race and must be ordered by the caller; the array keeps
 * the last call's contents, and a step writes every part of it that it reads. */
int lk_looped_decode_step_static(lk_handle *h, lk_kv_store *s, const int32_t *d_ids, float *d_out,
                                 void *stream);

/* Graph replay of decode steps on (enable != 0, the default) or off (every
 * step launches its kernels one by one).  Drops any captured step. */
int lk_set_decode_graphs(lk_handle *h, int32_t enable);

/* Device bytes of the decode copy of the layer projections (0 if the shapes do
 * not take it: it needs d_model, heads*head_dim and ffn_dim multiples of 64).
 * Decode steps with at most 8 sequences multiply by this copy: the weights as
 * float16 (converted from bf16: exact for magnitudes in [2^-17, 65504], smaller ones
 * rounded to 2^-24 steps), in an operand order packed for the MFMA lanes (every wave
 * load reads 1 KB contiguous), with float16 activations. */
int lk_decode_weight_bytes(const lk_handle *h, size_t *bytes);

/* Give the handle a caller-owned device buffer of at least lk_decode_weight_bytes
 * bytes (16-byte aligned) and fill it with the packed copy of the caller's weights
 * on `stream`.  The buffer must stay allocated, and the weights unchanged, while
 * the handle decodes; several handles over the same weights may share one buffer
 * (each call rewrites the same contents).  d_buf == NULL detaches the buffer:
 * decode then multiplies by the row-major weights.  Either way the captured decode
 * step is dropped.  LK_ERR_UNSUPPORTED when the size query gives 0, LK_ERR_CAPACITY
 * when buf_bytes is too small.  The library allocates no device memory for this. */
int lk_set_decode_weights(lk_handle *h, void *d_buf, size_t buf_bytes, void *stream);

/* Loops the store runs (the tutorial's n_recurrent_loops, picked by the caller with
 * the same weights; default: the model's n_loops).  Set between allocation and
 * prefill: the prefill and every decode step of the store then run loops
 * 1..n_loops, and the byte counts cover those loops; the layout stays the one for
 * the model's n_loops.  LK_ERR_STATE after prefill, LK_ERR_INVALID_ARG outside
 * [1, model n_loops]. */
int lk_kv_store_set_loops(lk_kv_store *s, int32_t n_loops);

/* Decode-state snapshots: checkpoint and resume of a decode session, and a way to
 * start decode from a store filled on the host.  The pages define no snapshot;
 * this one holds exactly the method's stored state: a header, then `body_bytes`
 * bytes that are the start of the store buffer, laid out as lk_kv_store_alloc
 * describes (offsets from the buffer start as lk_kv_store_view reports them):
 * the dense prelude/coda rows, the per-loop / last-loop rows or the lazy base,
 * residuals, slot maps and column sets, and the device copy of the length.  The
 * lazy decode caches (lk_kv_store_cache_bytes) are derived data and are not in
 * it: import rebuilds them from the base and residuals, with the same values the
 * prefill and decode steps wrote. */
#define LK_SNAPSHOT_MAGIC 0x313050414e534b4cull /* bytes "LKSNAP01" */
#define LK_SNAPSHOT_VERSION 2
typedef struct {
    uint64_t magic;          /* LK_SNAPSHOT_MAGIC */
    uint32_t header_bytes;   /* sizeof(lk_store_snapshot); the body follows */
    uint32_t version;        /* LK_SNAPSHOT_VERSION */
    lk_model_cfg cfg;        /* model config of the handle that wrote it */
    lk_lazy_cfg lazy;        /* cache policy of that handle */
    int32_t batch, prompt_tokens, max_tokens;  /* the store's allocation */
    int32_t loops;           /* the store's loop count (lk_kv_store_set_loops) */
    int32_t tokens;          /* tokens held per sequence */
    int32_t prefilled;       /* 1 after prefill (then prompt_tokens <= tokens) */
    uint64_t body_bytes;     /* bytes of the store buffer that follow */
} lk_store_snapshot;

/* Copy the store's state into host memory: header, then body.  host_buf == NULL
 * is a size query (*need_bytes only).  Enqueues the copy on `stream` and waits
 * for that stream; work on other streams that writes the store must be finished
 * by the caller.  LK_ERR_CAPACITY if buf_bytes < *need_bytes. */
int lk_kv_store_export(const lk_kv_store *s, void *host_buf, size_t buf_bytes, size_t *need_bytes,
                       void *stream);

/* Replace the store's state with a snapshot (host memory, `bytes` long).  The
 * model config, cache policy, batch, prompt_tokens and max_tokens must equal the
 * store's (any handle with the same config may have written it), loops must be
 * in [1, model n_loops], tokens in [prompt_tokens, max_tokens] when prefilled and
 * 0 otherwise, body_bytes the store's state size.  Uploads the body on `stream`,
 * rebuilds the lazy decode caches there (positions up to tokens - 1), sets the
 * length and loop count, drops a captured decode step of this store, and waits
 * for the stream, so host_buf may be freed on return.  Errors other than
 * LK_ERR_HIP leave the store unchanged.  The store's selection overrides and
 * keep-codes setting are not part of the state and are kept. */
int lk_kv_store_import(lk_kv_store *s, const void *host_buf, size_t bytes, void *stream);

/* Layer applications one prefill/decode pass runs per token: P + R*K + Q. */
int lk_effective_depth(const lk_handle *h, int32_t *depth);

const char *lk_last_error(void);

/* Instrumentation: bracket every launch of the given kernel classes with HIP events
 * on the stream of the call that launches it.  kernel_class is one class name or a
 * comma-separated list of them: "attn_decode_dense" (decode attention over dense /
 * base rows), "attn_decode_sparse", "attn_prefill", "column_mass",
 * "attn_prefill_sparse", "gemm_decode", "gemm_prefill"; NULL disables.  Enabling
 * clears the record.  Not thread-safe per handle. */
int lk_timing_enable(lk_handle *h, const char *kernel_class);
/* Time only the first per_call launches of each class in each prefill or decode
 * call (0, the default: all of them).  Fewer timed launches cut the decode step
 * into fewer replayed graphs. */
int lk_timing_sample(lk_handle *h, int32_t per_call);
/* Launches recorded since lk_timing_enable or the previous read, and their
 * summed event time in ms (waits for the recorded events; clears the record).
 * A replayed decode step launches its timed-class kernels directly between two
 * events and the rest of the step from captured graphs. */
int lk_timing_read(lk_handle *h, int32_t *launches, double *total_ms);
/* The same for one of the enabled classes, without clearing the record. */
int lk_timing_read_class(lk_handle *h, const char *kernel_class, int32_t *launches, double *total_ms);

/* ---------------------------------------------------------------------------
 * Test and inspection entry points (same error conventions).
 * ------------------------------------------------------------------------- */

/* Device addresses of a store's regions (NULL where the mode has none). */
typedef struct {
    void *dense;            /* prelude/coda rows */
    void *loop_rows;        /* per_loop or last_loop rows */
    void *base_codes;       /* lazy base: bf16 rows or int8 codes */
    void *base_scales;      /* lazy base scales (int8 base only) */
    void *res_codes;        /* residual rows/codes */
    void *res_scales;       /* residual scales (4/8-bit residuals) */
    int32_t *slot_maps;     /* [n_loops-1][batch][max_tokens] */
    int32_t *columns;       /* [R][batch][Hkv][n_columns] */
    int64_t slots;          /* residual slots per (loop, layer, K|V, seq, head) */
    int32_t n_selected;     /* kept tokens per sequence at loops >= 2 */
    int32_t n_columns;      /* min(top_s, prompt_tokens) */
    int64_t res_row_bytes;  /* bytes of one residual row (hd elements) */
    int32_t row_stride;     /* Tp: positions per (sequence, KV head), max_tokens padded to 8 */
    /* lazy decode caches (lk_kv_store_cache_bytes; NULL when there are none), float16:
     * for loops k = first_cached_loop..n_loops and shared layers r (index (k -
     * first_cached_loop) * R + r), the stable-column reconstruction, K rows
     * [batch][Hkv][cache_rows][hd] then V rows 8-key interleaved
     * [batch][Hkv][cache_rows/8][hd][8] (row i = column i of the column set); after all
     * of those, in the same order, the window rings with ring_rows rows per (sequence,
     * KV head) in the same two layouts (position p at row p % ring_rows). */
    void *decode_cache;
    int32_t cache_rows, ring_rows, first_cached_loop;
} lk_store_view;
int lk_kv_store_view(const lk_kv_store *s, lk_store_view *v);

/* Override the selections of the next prefill with caller data (device
 * pointers read during lk_looped_prefill; NULL restores natural selection):
 * tokens int32 [L-1][batch][n_selected] ascending per row, L the store's loop
 * count (lk_kv_store_set_loops; refresh loops take every token and ignore theirs);
 * columns int32 [R][batch][Hkv][n_columns] ascending per row. */
int lk_kv_store_force_selection(lk_kv_store *s, const int32_t *d_tokens, const int32_t *d_columns);

/* When enabled, prefill and decode leave the int8 base codes and the 4/8-bit
 * residual codes, with their float16 scales, that the caller wrote into the
 * store (through lk_kv_store_view) in place instead of quantizing; 16-bit rows
 * are still written.  Lets a test inject another implementation's integer
 * quantization decisions, as lk_kv_store_force_selection does for indices. */
int lk_kv_store_keep_codes(lk_kv_store *s, int32_t enable);

/* Top-n selector: for each of `rows` rows of `cols` float32 keys, the n largest
 * (ties to the lower index) as ascending int32 indices [rows, n]. */
int lk_dbg_topk(const float *d_keys, int32_t rows, int32_t cols, int32_t n, int32_t *d_idx,
                void *stream);

/* Residual quantizer on float32 rows [rows, hd] (hd multiple of 32):
 * codes uint8 [rows, hd*bits/8] (int4 packed low nibble first, or int8) and
 * float16 scales [rows, hd/32] (raw bits as uint16). */
int lk_dbg_quantize(const float *d_x, int32_t rows, int32_t hd, int32_t bits, uint8_t *d_codes,
                    uint16_t *d_scales, void *stream);

/* Delta keys: d_key[m] = sum_j (a[m, j] - b[m, j])^2 over float32 rows [rows, d]. */
int lk_dbg_delta(const float *d_a, const float *d_b, int32_t rows, int32_t d, float *d_key,
                 void *stream);

/* C[M, N] = A[M, K] * W[N, K]^T with bf16 A and W and float32 C (row-major). */
int lk_dbg_gemm(const void *d_a, const void *d_w, float *d_c, int32_t M, int32_t N, int32_t K,
                void *stream);

/* The same product with one of the fused epilogues of the projections:
 *   epi 0 (store):  d_c float32 [M, N] = A W^T;
 *   epi 1 (add):    d_c float32 [M, N] += A W^T (the residual-stream update);
 *   epi 2 (SwiGLU): W bf16 [2N, K] = [gate rows; up rows],
 *                   d_out bf16 [M, N] = silu(A Wg^T) * (A Wu^T);
 *   epi 3 (GELU):   d_out bf16 [M, N] = gelu(A W^T) with the exact erf form.
 * d_c is used by epi 0 and 1, d_out by epi 2 and 3 (the other may be NULL).
 * Same size rules as lk_dbg_gemm. */
int lk_dbg_gemm_epi(const void *d_a, const void *d_w, int32_t epi, float *d_c, void *d_out,
                    int32_t M, int32_t N, int32_t K, void *stream);

/* Attention kernels on caller data (test entry point): each kind runs the kernels,
 * launch shapes and split counts that prefill or decode run for that step, on K/V
 * rows the caller lays out as the store does.  Softmax of q.k / sqrt(hd) over each
 * query's key set; query head h reads KV head h / (H / Hkv) (the FlashLoop abstract,
 * arxivdaily.com: loops k >= 2 attend over a sparse, stable subset of key columns;
 * the loop-1 attention that ranks those columns is the dense causal one).
 *
 * Row layouts (positions per (sequence, KV head) padded to `tmax`, a multiple of 8):
 *   K rows [B][Hkv][tmax][hd]; V rows 8-key interleaved [B][Hkv][tmax/8][hd][8]
 *   (element (pos, e) at ((b*Hkv + g)*tmax/8 + pos/8)*hd*8 + e*8 + pos%8);
 *   kv_format 0: bfloat16 rows; 1: int8 codes with float16 scales per 32 elements,
 *   K scales [B][Hkv][tmax][hd/32], V scales [B][Hkv][tmax/8][hd/32][8] (value =
 *   code * scale); 2: float16 rows.
 *
 * Kinds:
 *   LK_DBG_ATTN_DECODE: one query per sequence at position t over keys [0, t]
 *     (kv_format 0 or 1; t < tmax), split over the context and merged, as a decode
 *     step's loop-1 attention; q [B][H*hd] (float16 bits when q_half, which the
 *     int8 kernel takes as is; else bf16).  out bf16 [B][H*hd], out32 float32 (same).
 *   LK_DBG_ATTN_DECODE_SEG: one query per sequence at position t over
 *     (S intersect [0, t - window]) union [max(0, t - window + 1), t], S = cols
 *     [B][Hkv][n_cols] ascending, as a decode step's loop k >= 2 (split into
 *     128-row pieces, then merged): the stable columns are read from a float16
 *     cache (s_k / s_v: row i holds column cols[i], s_cap rows per (b, g), a
 *     multiple of 128, >= n_cols) and the window from a float16 ring (r_k / r_v:
 *     position p at row p % r_cap, r_cap a multiple of 128, >= window + 8).  q and
 *     outputs as LK_DBG_ATTN_DECODE.
 *   LK_DBG_ATTN_PREFILL: causal attention of T prompt tokens (query i over keys
 *     [0, i]; kv_format 0 or 1, T <= tmax); q bf16 [B][T][H*hd]; out bf16
 *     [B][T][H*hd]; lse float32 [B][H][T], the log2 of each row's softmax
 *     denominator in units of the log2-scaled scores (q.k * log2(e) / sqrt(hd)).
 *   LK_DBG_ATTN_MASS: column mass of that attention, mass float32 [B][Hkv][T]:
 *     mass[b][g][j] = sum over queries i >= j and the query heads of g of the
 *     probability of key j, with lse (as LK_DBG_ATTN_PREFILL writes it) as input.
 *   LK_DBG_ATTN_PREFILL_SPARSE: n_rows kept prompt rows per sequence (positions
 *     qpos [B][n_rows], ascending), row at position i over (S intersect [0, i -
 *     window]) union [max(0, i - window + 1), i], hd 128: stable columns from the
 *     float16 cache s_k / s_v (as above, s_cap a multiple of 8), the window from
 *     float16 rows at every position r_k / r_v (r_cap = positions, a multiple of 8);
 *     q bf16 [B][n_rows][H*hd]; out bf16 [B][n_rows][H*hd].
 * ws: device scratch of ws_bytes (the split partials of the two decode kinds; the
 * other kinds need none).  With ws == NULL and ws_need != NULL, lk_dbg_attention writes the
 * bytes the call needs to *ws_need and launches nothing.  head_dim 32, 64
 * or 128 (128 only for PREFILL_SPARSE); H / Hkv in {1, 2, 4, 8}. */
#define LK_DBG_ATTN_DECODE 0
#define LK_DBG_ATTN_DECODE_SEG 1
#define LK_DBG_ATTN_PREFILL 2
#define LK_DBG_ATTN_MASS 3
#define LK_DBG_ATTN_PREFILL_SPARSE 4
typedef struct {
    int32_t kind;
    int32_t B, H, Hkv, hd;
    int32_t kv_format;           /* 0 bf16, 1 int8 + float16 scales, 2 float16 */
    int32_t t;                   /* DECODE*: the query position */
    int32_t T;                   /* PREFILL, MASS, PREFILL_SPARSE: prompt tokens */
    int32_t tmax;                /* positions per (sequence, KV head) of k / v */
    const void *q;
    int32_t q_half;              /* DECODE*: q holds float16 bits */
    const void *k, *v;           /* rows (DECODE, PREFILL, MASS) */
    const uint16_t *k_scales, *v_scales;  /* kv_format 1 */
    const int32_t *cols;         /* DECODE_SEG, PREFILL_SPARSE: [B][Hkv][n_cols] */
    int32_t n_cols, window;
    const void *s_k, *s_v;       /* float16 stable-column cache */
    int32_t s_cap;
    const void *r_k, *r_v;       /* float16 window ring (DECODE_SEG) or rows (PREFILL_SPARSE) */
    int32_t r_cap;
    const int32_t *qpos;         /* PREFILL_SPARSE: [B][n_rows] */
    int32_t n_rows;
    void *out;                   /* bf16 outputs as above */
    float *out32;                /* DECODE*: float32 [B][H*hd] (may be NULL) */
    float *lse;                  /* PREFILL: output; MASS: input */
    float *mass;                 /* MASS: output */
    void *ws;
    size_t ws_bytes;
} lk_dbg_attn_args;
int lk_dbg_attention(const lk_dbg_attn_args *a, size_t *ws_need, void *stream);

/* Store writer on caller projections (test entry point).  d_qkv float32 [rows][(H +
 * 2 Hkv) hd], the QKV projection of each row (q heads, k heads, v heads).  q and K are
 * rotated at the row's position, q into d_q_out (bf16 [rows][H hd], float16 bits when
 * q_half), and K/V go into shared layer `layer` of lazy store s as loop `loop` writes
 * them (the FlashLoop abstract: loop-k KV kept as the loop-(k-1) KV plus a low-bit
 * residual; the quantizer and layouts as lk_kv_store_alloc describes):
 *   d_pos != NULL (prefill): rows = batch * rows_per_seq, row r of sequence r /
 *     rows_per_seq at position d_pos[r]; loop 1 writes the base rows; loop k >= 2
 *     quantizes the difference to the store's loop-(k-1) reconstruction of that
 *     position into slot r % rows_per_seq and sets the loop-k slot-map entry;
 *   d_pos == NULL (decode): one row per sequence at position t = the store length,
 *     exactly as a decode step's loop `loop` writes it: the slot is the loop's first
 *     decode slot plus t - prompt_tokens, the previous loop's reconstruction of the
 *     row is the float32 one the step carries in the decode workspace d_ws (so a
 *     token's loops are written in the order 1, 2, ..), and loops k >= 2 also write
 *     the row's float16 reconstruction into the window ring.  The store length is
 *     not changed.
 * d_ws: a decode workspace (lk_workspace_bytes(batch, 1)) in decode mode, else unused. */
int lk_dbg_kv_write(lk_kv_store *s, int32_t layer, int32_t loop, const float *d_qkv, int32_t rows_per_seq,
                    const int32_t *d_pos, void *d_q_out, int32_t q_half, void *d_ws, size_t ws_bytes,
                    void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LOOPED_KV_H */
