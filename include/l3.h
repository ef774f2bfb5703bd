/*
 * l3.h -- C ABI of the MI355X (gfx950) Large Lookup Layer (L^3) forward pass.
 *
 * The layer ("L^3: Large Lookup Layers", Tseng & De Sa, ICML 2026; the layer
 * equation on the papernotes.org page, section 整体框架, and on the
 * kimjy99.github.io page, section "Method") maps a hidden state x (d_in) and
 * a token ID t to
 *
 *     L3(x, t) = W_mix [ LN( W_up( V_t^T softmax(K_t x) ) ) ; x ]    (d_out)
 *
 * where K_t (d_t x d_in) and V_t (d_t x d_emb) are the d_t rows of the
 * concatenated tables W_K (v x d_in) and W_V (v x d_emb) that the token ID
 * selects statically (kimjy99.github.io page, section "2. Efficient Training
 * and Inference": the per-token key and value matrices concatenated into one
 * table each).  Row ranges come from the allocation D = (d_t), 1 <= d_t <= k,
 * sum d_t = v (papernotes.org page, section 关键设计 item 2), given here as
 * CSR offsets: token t owns rows [off[t], off[t+1]).
 *
 * Shape readings (the pages print inconsistent shapes): W_up is d_up x d_emb;
 * W_mix is d_out x (d_up + d_in) with columns [0, d_up) acting on the
 * LayerNorm output and [d_up, d_up + d_in) on x.  No biases, no softmax
 * temperature.  LayerNorm normalises the d_up features of one token with the
 * biased variance, then applies gamma and beta (fp32, d_up each) with the
 * plan's eps.  Token IDs are 0-based.
 *
 * Conventions for every call:
 *  - Matrices are dense, row-major, contiguous.  Row j of W_K / W_V is
 *    embedding j.  W_up and W_mix use the (out x in) layout.
 *  - Float tensors (x, W_K, W_V, W_up, W_mix, out) are all fp32 or all bf16
 *    (plan dtype); gamma and beta are always fp32; accumulation is fp32.
 *  - "dev" pointers are HIP device memory (or host memory the device can
 *    read, where stated); "host" pointers are ordinary host memory.  The
 *    caller owns every buffer it passes; the library owns only what it
 *    creates (plans, staging objects) and frees it in the matching destroy.
 *  - `stream` is a hipStream_t (NULL = the null stream), `event` a hipEvent_t.
 *    Calls only enqueue work on the stream; they do not synchronise, except
 *    l3_status (documented below).
 *  - Errors found on the host (bad arguments, offsets, sizes, capacities)
 *    are returned before anything is enqueued.  Token IDs outside
 *    [0, vocab) found on the device set a flag in the workspace; the output
 *    rows of those tokens are unspecified and l3_status reports the flag.
 *  - Device tensors and the workspace are at least 16-byte aligned (kernels
 *    use 16-byte vector accesses), token ID arrays 4-byte aligned; a
 *    misaligned pointer is rejected with L3_ERR_INVALID_ARG.
 *  - n = 0 is a no-op returning L3_OK.
 *  - Plans are immutable after creation and may be shared across threads and
 *    streams; a workspace serves one call at a time.  A bf16 plan owns one
 *    stream of its own (default priority) for the weight-only part of large
 *    forwards (l3_forward): calls on different streams that share the plan
 *    take turns on it for that part.
 */
#ifndef L3_H
#define L3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct l3_plan_s *l3_plan_t;
typedef struct l3_staging_s *l3_staging_t;

enum {
    L3_OK = 0,
    L3_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad enum        */
    L3_ERR_BAD_OFFSETS = -2, /* off[0] != 0, d_t < 1, d_t > k, off[vocab]!=v */
    L3_ERR_TOKEN_RANGE = -3, /* a token ID outside [0, vocab)                */
    L3_ERR_UNSUPPORTED = -4, /* dims the library does not handle            */
    L3_ERR_CAPACITY = -5,    /* n or rows above what a buffer was sized for  */
    L3_ERR_NOMEM = -6,       /* host or device allocation failed             */
    L3_ERR_HIP = -7          /* a HIP runtime call failed                    */
};

enum { L3_F32 = 0, L3_BF16 = 1 };

typedef struct {
    int64_t d_in, d_emb, d_up, d_out;
    int32_t dtype;  /* L3_F32 or L3_BF16 */
    float ln_eps;   /* LayerNorm epsilon (e.g. 1e-5) */
} l3_dims_t;

/* Text of a status code (static storage). */
const char *l3_strerror(int status);

/*
 * l3_plan -- validate an allocation and upload its CSR offsets (the allocation D
 * is fixed, each token ID owning between 1 and k embeddings and v in all:
 * papernotes.org page, section 关键设计 item 2).
 * offsets: host, vocab + 1 int64 entries; off[0] = 0, 1 <= off[t+1]-off[t] <= k,
 *          off[vocab] = v (the allocation bounds of the pages: every token gets
 *          at least one and at most k embeddings, budget v = sum d_t).
 *          v and vocab must be below 2^31 (UNSUPPORTED otherwise).
 * dims:    host; bf16 needs d_in, d_up, d_out multiples of 64, d_in <= 4096
 *          and d_emb one of 64, 128, 256, 512, or d_emb = d_in = 1024 or 2048 for
 *          tied tables only (l3_forward then needs W_V to be the W_K buffer;
 *          l3_backward and the decode stagings refuse such plans with
 *          UNSUPPORTED); fp32 takes any positive dims.
 * plan:    out; the handle owns a device copy of the offsets (allocated on the
 *          current HIP device).  Errors: INVALID_ARG, BAD_OFFSETS, UNSUPPORTED,
 *          NOMEM, HIP.
 */
int l3_plan(const int64_t *offsets, int64_t vocab, int64_t v, int32_t k,
            const l3_dims_t *dims, l3_plan_t *plan);

/* Frees a plan (NULL is accepted). */
int l3_plan_destroy(l3_plan_t plan);

/*
 * l3_allocate_lzw -- the allocation D itself, from a token corpus (host code, no
 * GPU): the pages' LZW-style rule (kimjy99.github.io page, section "1. Embedding
 * Allocation"; papernotes.org page, section 关键设计 item 2).  The corpus is
 * parsed LZW-style into codewords with frequencies (a new codeword counts 1, the
 * codeword without its first token +1); every token gets one embedding, then the
 * codewords by decreasing frequency (ties: shorter, then by token sequence) each
 * give one to the token they end with, up to k per token, in passes until v.
 * corpus: host int32 [n] in [0, vocab); offsets: host int64 [vocab + 1], written
 * (off[0] = 0, off[t+1] - off[t] = d_t), ready for l3_plan.
 * Errors: INVALID_ARG (also v outside [vocab, vocab * k]), TOKEN_RANGE (a corpus
 * token outside [0, vocab)), CAPACITY (the codewords cannot place all of v:
 * every token they end with is already at k).
 */
int l3_allocate_lzw(const int32_t *corpus, int64_t n, int64_t vocab, int64_t v, int32_t k,
                    int64_t *offsets);

/* Plan facts: vocab, v, k and the largest d_t (any pointer may be NULL). */
int l3_plan_info(l3_plan_t plan, int64_t *vocab, int64_t *v, int32_t *k,
                 int32_t *max_d);

/* Which distinct IDs of a batch the matrix-core gather-attention takes (the rest
 * go one wavefront per item): those with at least *min_tokens tokens in the
 * batch or at least *min_rows rows (d_t); both are INT32_MAX when the plan's
 * dims have no matrix-core path.  Either pointer may be NULL.  The rule applies
 * to batches of more than 512 tokens: smaller bf16 batches whose partials fit
 * (see l3_profile_enable) take the split-row gather for every ID. */
int l3_worklist_rule(l3_plan_t plan, int32_t *min_tokens, int32_t *min_rows);

/* Bytes of device workspace l3_forward / l3_route need for up to n_max tokens
 * (0 on a bad argument): enough for every batch size from 1 to n_max.  The
 * workspace is caller-allocated device memory, 256-byte aligned; its contents
 * need no initialisation.
 * l3_workspace_size_dims -- the same figure before any plan exists (host only, no
 * device needed): for a plan with these dims whose largest d_t is max_d. */
size_t l3_workspace_size(l3_plan_t plan, int64_t n_max);
size_t l3_workspace_size_dims(const l3_dims_t *dims, int32_t max_d, int64_t n_max);

/*
 * l3_forward -- out = L3(x, token_ids) for n tokens.
 * x:         dev [n x d_in]        token_ids: dev int32 [n]
 * W_K:       dev [v x d_in]        W_V:       dev [v x d_emb]
 * W_up:      dev [d_up x d_emb]    ln_gamma, ln_beta: dev fp32 [d_up]
 * W_mix:     dev [d_out x (d_up + d_in)]
 * out:       dev [n x d_out], rows in the input token order.
 * workspace: dev, >= l3_workspace_size(plan, n) bytes (workspace_bytes).
 * The batch is sorted by token ID so each distinct ID's K_t / V_t rows are
 * read once per call (the pages' batch sort: sciencestack.ai page, Fig. 3
 * caption); the result does not depend on the batch order.  W_V may be the same
 * buffer as W_K when d_emb == d_in (the pages' tied variant, papernotes.org page,
 * ablation table): the wavefront gather kernel then copies each row once for both
 * roles, and the matrix-core one finds the second read mostly in the caches.  bf16
 * plans with d_emb 1024 or 2048 take tied tables only (UNSUPPORTED when W_V is not
 * the W_K buffer) and gather every block in the wavefront kernel.
 * bf16 batches of more than 512 tokens evaluate W_mix [LN(h) ; x] in factored
 * form (the same function: with W_c the column-centred W_up, h - mean(h) = W_c o,
 * so W_mix [LN(h) ; x] = rstd (F o) + W1 beta + W2 x with F = W1 diag(gamma) W_c,
 * and var(h) = o^T G o / d_up with G = W_c^T W_c); F and G depend on the weights
 * only and are formed on the plan's own stream, forked from `stream` when the
 * call starts and joined before the first kernel that reads them, so they run
 * beside the sort and the gather.
 * Errors: INVALID_ARG, CAPACITY (workspace too small), HIP.
 */
int l3_forward(l3_plan_t plan, const void *x, const int32_t *token_ids, int64_t n,
               const void *W_K, const void *W_V, const void *W_up,
               const float *ln_gamma, const float *ln_beta, const void *W_mix,
               void *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * l3_forward_noalloc -- l3_forward for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and result bits as l3_forward, with the workspace
 * in a device array the library holds (64 MiB on every GPU it runs on, kept until
 * the process ends) instead of a caller buffer.  Nothing is allocated per call
 * (with stage timing, l3_profile_enable, off).  Arguments as for l3_forward, minus
 * the workspace.  Errors: INVALID_ARG, UNSUPPORTED, CAPACITY (this batch's
 * workspace would exceed 64 MiB; nothing is enqueued), HIP.  A batch of n tokens
 * always fits when l3_workspace_size(plan, n) <= 64 MiB: up to 146 tokens at d_in
 * 2048, d_emb 512, d_up = d_out = 2048 with d_t up to 512, 31 at d_in = d_up =
 * d_out = 4096, and batches of thousands at d_in 1024, d_emb 256, d_t up to 128.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (two streams, two threads) race and must be serialised by the caller.  The
 * out-of-range flag lands in that array, where l3_status cannot read it: callers
 * that need it use l3_forward.
 */
int l3_forward_noalloc(l3_plan_t plan, const void *x, const int32_t *token_ids, int64_t n,
                       const void *W_K, const void *W_V, const void *W_up,
                       const float *ln_gamma, const float *ln_beta, const void *W_mix,
                       void *out, void *stream);

/*
 * Backward pass (training).  The pages train the layer end to end, the batch
 * sorted by token ID so attention is block diagonal and the sort undone after
 * (sciencestack.ai page, Fig. 3 caption; kimjy99.github.io page, section "2.
 * Efficient Training and Inference"); the gradients are the derivatives of the
 * forward equation (papernotes.org page, section 整体框架).
 *
 * l3_backward_workspace_size -- device workspace bytes for up to n_max tokens
 * (0 on a bad argument); 256-byte aligned, no initialisation needed.
 *
 * l3_backward -- gradients of sum(dout * L3(x, token_ids)) for n tokens.
 * Inputs as for l3_forward (plan dtype), plus dout: dev [n x d_out] (plan dtype).
 * Outputs, all dev fp32, 16-byte aligned:
 *   dx [n x d_in]                 written (rows in the input token order);
 *   dW_K [v x d_in], dW_V [v x d_emb]   ADDED TO, on the rows of the IDs present
 *                                 in the batch (other rows untouched);
 *   dW_up [d_up x d_emb], dln_gamma, dln_beta [d_up],
 *   dW_mix [d_out x (d_up + d_in)]     ADDED TO.
 * The caller zeroes the accumulated gradients when a new accumulation starts.
 * The forward is recomputed inside (nothing is saved from l3_forward).  Every sum
 * over tokens runs in a fixed order (no atomics): results are bit-for-bit
 * reproducible.  Operands of the dense products are bf16 for bf16 plans
 * (fp32 accumulation), fp32 otherwise.  Supports d_in <= 4096, d_emb <= 1024
 * (bf16: d_emb <= 512; plans of the tied-only widths return UNSUPPORTED).
 * Errors: INVALID_ARG, CAPACITY, UNSUPPORTED, HIP.  IDs outside [0, vocab) set
 * the status flag (l3_status) and contribute no attention gradient.
 */
size_t l3_backward_workspace_size(l3_plan_t plan, int64_t n_max);
int l3_backward(l3_plan_t plan, const void *x, const int32_t *token_ids, int64_t n,
                const void *W_K, const void *W_V, const void *W_up, const float *ln_gamma,
                const float *ln_beta, const void *W_mix, const void *dout, float *dx,
                float *dW_K, float *dW_V, float *dW_up, float *dln_gamma, float *dln_beta,
                float *dW_mix, void *workspace, size_t workspace_bytes, void *stream);

/*
 * l3_route -- the batch sort alone (what l3_forward does first): the batch sorted
 * by token ID so that each ID's tokens form one block and the attention pattern is
 * block diagonal (sciencestack.ai page, Fig. 3 caption).
 * Sorting is stable: tokens with equal IDs keep their batch order.  IDs outside
 * [0, vocab) sort as the key `vocab` after every valid ID and set the flag.
 * Outputs (dev int32, caller-allocated; any may be NULL to skip):
 *   perm[n]        sorted position -> batch index
 *   sorted_ids[n]  keys in sorted order
 *   inv_perm[n]    batch index -> sorted position
 *   uniq[n]        the m distinct keys, ascending (first m entries written)
 *   counts[n]      tokens per distinct key (first m entries)
 *   seg_start[n+1] start of each key's block (first m+1 entries, last = n)
 *   num_segments   dev int32 scalar: m
 * Errors: INVALID_ARG, CAPACITY, HIP.
 */
int l3_route(l3_plan_t plan, const int32_t *token_ids, int64_t n, void *workspace,
             size_t workspace_bytes, void *stream, int32_t *perm, int32_t *sorted_ids,
             int32_t *inv_perm, int32_t *uniq, int32_t *counts, int32_t *seg_start,
             int32_t *num_segments);

/*
 * l3_status -- synchronises `stream`, then reports the device-side flag of the
 * last l3_forward / l3_route that used `workspace`: L3_ERR_TOKEN_RANGE if an ID
 * was outside [0, vocab), else L3_OK (or L3_ERR_HIP).
 */
int l3_status(void *workspace, void *stream);

/*
 * Decode path: the tables live in pinned host memory; only the rows of the
 * tokens being decoded cross to the device, copied on a side stream while the
 * main stream runs earlier layers (the pages' offloaded inference:
 * sciencestack.ai page, Fig. 4 caption; papernotes.org page, section 关键设计
 * item 3).
 *
 * l3_staging_create -- device staging for up to max_rows table rows and
 * max_tokens tokens per step (rows: K and V of the distinct IDs of one step).
 * Allocates device memory (owned by the staging object) on the current device.
 * Errors: INVALID_ARG, NOMEM, HIP; UNSUPPORTED for the tied-only bf16 plans
 * (d_emb 1024, 2048), whose K and V rows a staging would hold apart.
 */
int l3_staging_create(l3_plan_t plan, int64_t max_rows, int64_t max_tokens,
                      l3_staging_t *staging);
int l3_staging_destroy(l3_staging_t staging);

/*
 * l3_prefetch -- enqueue the copy of the K / V rows that `token_ids_host` need.
 * token_ids_host: host int32 [n] (the IDs just sampled).
 * W_K_host, W_V_host: the full tables in pinned host memory (hipHostMalloc, or
 *          torch's pin_memory), 16-byte aligned, same dtype and layout as the
 *          device tables of l3_forward; read-only while the staging is in use.
 * The distinct IDs are found on the host; their compact offsets, first table
 * rows and the remapped IDs go to the device in one hipMemcpyAsync on
 * `side_stream`, then one kernel on the same stream reads every row of those
 * IDs through the tables' device mapping (over PCIe) into the staging buffers.
 * `ready_event` (may be NULL) is recorded on `side_stream` after the kernel.
 * The caller orders the staged forward after it (hipStreamWaitEvent).  The next
 * prefetch into the same staging is ordered after the last l3_forward_staged that
 * read it by the library itself (an event recorded after that forward, waited on
 * by `side_stream` before anything is overwritten), so decode steps may be issued
 * back to back without host synchronisation; the host blocks only while the
 * previous step's index block is still being copied out of its pinned mirror.
 * The host arrays are read before the call returns (token_ids_host may be reused
 * at once); the pinned tables must stay valid until the kernel finishes.
 * Errors: INVALID_ARG (also tables without a device mapping, e.g. pageable
 * memory), TOKEN_RANGE (an ID outside [0, vocab); nothing is enqueued),
 * CAPACITY (more than max_tokens tokens or max_rows rows), HIP.
 */
int l3_prefetch(l3_plan_t plan, const int32_t *token_ids_host, int64_t n,
                const void *W_K_host, const void *W_V_host, l3_staging_t staging,
                void *side_stream, void *ready_event);

/*
 * l3_staging_set_cache -- keep the rows of hot_ids (host int32 [n_hot], the IDs
 * whose rows should stay on the device, e.g. the most frequent ones) in a
 * device-resident cache owned by the staging: later prefetches copy those IDs'
 * rows from the cache (HBM) and only the others over PCIe.  Fills the cache from
 * the pinned tables on `stream` and returns when it is filled; replaces any
 * previous cache (after waiting for the device to go idle); n_hot = 0 drops it.
 * Allocates device memory.  Errors: INVALID_ARG (also tables without a device
 * mapping), TOKEN_RANGE, HIP.
 *
 * l3_staging_stats -- rows staged by the last prefetch, and how many of them the
 * cache served (either pointer may be NULL).
 */
int l3_staging_set_cache(l3_staging_t staging, const int32_t *hot_ids, int64_t n_hot,
                         const void *W_K_host, const void *W_V_host, void *stream);
int l3_staging_stats(l3_staging_t staging, int64_t *rows, int64_t *cached_rows);

/*
 * l3_forward_staged -- l3_forward over the rows the last l3_prefetch staged,
 * for the same n tokens in the same order.  workspace: >= l3_workspace_size
 * (plan, n) bytes.  Records the staging's "consumed" event on `stream` after its
 * kernels (the next l3_prefetch into this staging waits for it).
 * Errors: INVALID_ARG, CAPACITY, HIP.
 */
int l3_forward_staged(l3_staging_t staging, const void *x, int64_t n, const void *W_up,
                      const float *ln_gamma, const float *ln_beta, const void *W_mix,
                      void *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Dense bf16 GEMM on the library's MFMA kernels: C[M x N] = A[M x K] * B[N x K]^T
 * (both operands k-contiguous, torch Linear layout), fp32 accumulate, bf16 out.
 * Used as the decode workload's stand-in for the layers before L^3.
 * K and N must be multiples of 64.  Batches of up to 512 rows take a split-K
 * kernel whose fp32 partial sums need a device workspace of
 * l3_gemm_workspace_size(M, N, K) bytes (0 for larger M: workspace may then be
 * NULL); the workspace is overwritten.  Errors: INVALID_ARG (also a pointer not
 * 16-byte aligned), CAPACITY (workspace too small), UNSUPPORTED, HIP.
 */
size_t l3_gemm_workspace_size(int64_t M, int64_t N, int64_t K);
int l3_gemm_bf16(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K,
                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * Per-kernel timing for measurement.  While enabled, l3_forward and
 * l3_backward record a pair of HIP events on their stream around each of their
 * kernel stages and accumulate their elapsed time; l3_profile_read synchronises
 * those events.  Stages: 0 route (sort + blocks + work lists), 1 gather-attention
 * on the matrix cores (heavy work list), 2 gather-attention, one wavefront per
 * item (light work list), 3 LayerNorm row statistics (the W_up GEMM for bf16
 * batches of at most 512 tokens and fp32 plans; o^T G o above), 4 the factors F
 * and G of larger bf16 batches (recorded on the plan's stream), 5 W_mix GEMM;
 * backward (which also runs
 * stages 0-2): 6 recompute of h and its LayerNorm statistics, 7 dense products
 * and the LayerNorm backward, 8 attention backward, 9 key / value gradients.
 * bf16 batches of at most 512 tokens run one split-row gather-attention (row
 * chunks, then a merge per token) recorded as stage 2, with no stage 1.
 * max_stages <= 10.  Not thread-safe; for benchmarking only.
 */
int l3_profile_enable(int enable);
int l3_profile_read(double *ms_total, int64_t *launches, int max_stages);

#ifdef __cplusplus
}
#endif

#endif /* L3_H */
