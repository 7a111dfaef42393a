/*
 * ngpt.h -- C ABI of the MI355X (gfx950) GPT-2 decoder library (libngpt.so).
 *
 * The library runs the forward pass that nanoGPT's generate() uses, with a
 * KV cache, entirely in hand-written HIP kernels on one GPU:
 *
 *   prefill:  x = wte[id] + wpe[pos]; per block x += c_proj(attn(ln_1(x)));
 *             x += mlp_proj(GELU(c_fc(ln_2(x)))); logits = ln_f(x_last) wte^T
 *   decode:   sample the next id from the current logits (temperature, top-k,
 *             inverse CDF on a caller uniform), then run that one token
 *             against the cached K/V and refresh the logits.
 *
 * Sources (page title, section):
 *   - serving page "原生 nanoGPT 模型服务首选": section 1 (LayerNorm with an
 *     optional bias), section 2 (generate(): last-position logits / T,
 *     top-k filter, softmax, multinomial, append), and the KV-cache section
 *     "一个值得做的改进" (c_attn split into q, k, v; past K/V concatenated
 *     along time; only the newest token is fed; causal masking only without
 *     a past).
 *   - SDK guide "极速上手nanoGPT", "模型架构解析" (GPTConfig fields and defaults,
 *     scaled masked softmax attention).
 *   - architecture analysis "nanoGPT 架构分析", section 4.1 (pre-LN blocks,
 *     4x GELU MLP, wte/lm_head tying, lm_head on the last position only).
 *   - model-building chapter "第 4 章 模型构建", section 4.5 (learned absolute
 *     position embeddings, lower-triangular causal mask, bias-free lm_head).
 *
 * Conventions
 *   - Every call returns an int status (NGPT_OK = 0, negative on error); no
 *     exception crosses the ABI.  ngpt_last_error() gives a message.
 *   - Work is enqueued asynchronously on the stream given to ngpt_create().
 *     No call synchronises the stream except ngpt_destroy(); the only host
 *     waits are the ones stated (ngpt_prefill reusing its pinned staging).
 *   - All device memory is caller-owned and borrowed: weights, the KV cache
 *     and the workspace (sized by ngpt_workspace_bytes()) must stay alive and
 *     unmodified by others while the model uses them.  The library never
 *     allocates device memory (ngpt_create_static() takes its workspace
 *     from a fixed array of the library instead of the caller).
 *   - A handle is bound to one stream and is not thread-safe.
 *   - Element type of every weight, bias, LayerNorm parameter and KV entry is
 *     the config dtype (fp32, bf16 or fp16).  The residual stream, LayerNorm
 *     statistics, attention softmax and logits are fp32 in every mode.
 */
#ifndef NGPT_H
#define NGPT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define NGPT_OK           0
#define NGPT_E_ARG       -1  /* NULL pointer, inconsistent argument        */
#define NGPT_E_CONFIG    -2  /* unsupported model shape or dtype           */
#define NGPT_E_RANGE     -3  /* a token id or a length outside its range   */
#define NGPT_E_SIZE      -4  /* batch, token count or buffer size out of bounds */
#define NGPT_E_CONTEXT   -5  /* no sequence can take another token          */
#define NGPT_E_HIP       -6  /* a HIP runtime call failed                   */
#define NGPT_E_DEVICE    -7  /* a kernel saw invalid input (id out of range,
                                or a logits row with no finite maximum)    */
#define NGPT_E_TIMEOUT   -8  /* a wait in the one-launch decode kernel gave up */
#define NGPT_E_PAGE      -9  /* a paged cache position to be written has no
                                page mapped (reported by ngpt_device_status) */

/* Element types (the fp16 model: SDK guide "极速上手nanoGPT", section
 * "性能优化技巧", mixed precision with float16). */
#define NGPT_F32   0
#define NGPT_BF16  1
#define NGPT_F16   2

/*
 * Model shape: the GPTConfig of the SDK guide ("模型架构解析"): block_size,
 * vocab_size, n_layer, n_head, n_embd, bias.  dropout is absent (inference).
 * Supported: n_embd % n_head == 0; head_dim = n_embd / n_head in {32, 64};
 * n_embd % 64 == 0 (bf16, fp16) or n_embd % 4 == 0 (fp32); n_embd <= 2048;
 * 1 <= block_size <= 4096;
 * vocab_size >= 1; max_batch in [1, NGPT_MAX_BATCH];
 * max_prefill_tokens >= 1 bounds the sum of prompt lengths of one prefill.
 * Every matrix stays below 2 GiB (the kernels use 32-bit buffer offsets):
 * vocab_size * n_embd * sizeof(dtype) < 2^31 and
 * max(max_prefill_tokens, max_batch) * 4 * n_embd * sizeof(dtype) < 2^31.
 */
#define NGPT_MAX_BATCH 256
typedef struct {
  int32_t n_layer;
  int32_t n_head;
  int32_t n_embd;
  int32_t block_size;
  int32_t vocab_size;
  int32_t bias;               /* 1: LayerNorm and Linear layers have biases */
  int32_t dtype;              /* NGPT_F32, NGPT_BF16 or NGPT_F16 */
  int32_t max_batch;
  int32_t max_prefill_tokens;
} ngpt_config;

/*
 * Weights of one block (SDK guide "模型架构解析": the Block of ln_1, attn
 * (c_attn, c_proj), ln_2, mlp (c_fc, GELU, c_proj)), device pointers in
 * nn.Linear layout [out_features][in_features], row-major, elements of the
 * config dtype.  attn_w is c_attn, [3C][C]: rows [0,C) give q, [C,2C) k,
 * [2C,3C) v; head j of each is the row slice [j*hs, (j+1)*hs) (serving
 * page, KV-cache section).  attnproj_w is the attention c_proj [C][C]; fc_w
 * is [4C][C]; mlpproj_w is [C][4C].  LayerNorm weights are [C].  Bias
 * pointers must all be NULL when bias == 0 and all non-NULL when bias == 1
 * (serving page, section 1).  Every pointer must be 16-byte aligned.
 */
typedef struct {
  const void *ln1_w, *ln1_b;
  const void *attn_w, *attn_b;
  const void *attnproj_w, *attnproj_b;
  const void *ln2_w, *ln2_b;
  const void *fc_w, *fc_b;
  const void *mlpproj_w, *mlpproj_b;
} ngpt_layer_weights;

/*
 * Whole-model weights.  wte [vocab][C] is also the lm_head (weight tying,
 * architecture analysis section 4.1), so there is no lm_head pointer and no
 * lm_head bias.  wpe is [block_size][C] (model-building chapter, section
 * 4.5: learned absolute positions).  `layers` is a HOST array of n_layer
 * entries; it is copied at create time.
 */
typedef struct {
  const void *wte, *wpe;
  const void *lnf_w, *lnf_b;
  const ngpt_layer_weights *layers;
} ngpt_weights;

/*
 * KV cache (serving page, KV-cache section: per layer the past K and V,
 * extended by one row per new token), caller-owned device memory.
 *
 * Contiguous (block_table == NULL): k and v are each laid out
 * [n_layer][batch][n_head][block_size][head_dim] in the config dtype
 * (ngpt_kv_bytes() bytes each).
 *
 * Paged (the paged KV memory of vLLM that the serving page's section
 * "HF 在哪些情况下实际上会更好" names): k and v are pools of num_pages pages,
 * each laid out [n_layer][num_pages][n_head][NGPT_PAGE_TOKENS][head_dim]
 * (ngpt_kv_pool_bytes() bytes each).  Positions 64j .. 64j+63 of sequence b
 * live in page block_table[b * ceil(block_size / 64) + j] (device int32
 * [batch][ceil(block_size / 64)]); an entry outside [0, num_pages) is an
 * unmapped block.  Sequences can share no page they both write.  The table
 * is the caller's memory, written by the caller or with ngpt_kv_map();
 * kernels read unmapped blocks as zeros and skip writes into them, which
 * ngpt_device_status() reports as NGPT_E_PAGE.  The one-launch batch-1
 * decode kernel takes contiguous caches only; a paged batch-1 cache decodes
 * through the per-layer graph.
 *
 * lens[b] is the number of positions of sequence b held in the cache;
 * limit[b] (<= block_size) is the total length at which sequence b stops
 * taking tokens.  Both are device int32 [batch], written by ngpt_prefill()
 * and advanced by the decode calls.  A sequence is active while lens[b] <
 * limit[b].  k and v must be 16-byte aligned.
 */
#define NGPT_PAGE_TOKENS 64

typedef struct {
  void *k;
  void *v;
  int32_t *lens;
  int32_t *limit;
  int32_t batch;
  int32_t num_pages;       /* pages per pool (paged), ignored otherwise */
  int32_t *block_table;    /* NULL: contiguous layout */
} ngpt_kv;

typedef struct ngpt_model ngpt_model;

/* Bytes of ONE of the two KV arrays for `batch` sequences (the KV-cache
 * section's per-layer K and V, block_size positions each); 0 if the config
 * is invalid or batch < 1.  Host-only, needs no GPU. */
size_t ngpt_kv_bytes(const ngpt_config *cfg, int32_t batch);

/* Bytes of ONE of the two paged KV pools of num_pages pages (each page
 * NGPT_PAGE_TOKENS positions of every layer and head); 0 if the config is
 * invalid or num_pages < 1.  Host-only, needs no GPU. */
size_t ngpt_kv_pool_bytes(const ngpt_config *cfg, int32_t num_pages);

/* Bytes of the workspace a model of this config needs (activations of up
 * to max(max_prefill_tokens, max_batch) rows of the forward of the SDK
 * guide's GPT class, split-K attention partials, fp32 logits
 * [max_batch][vocab], the one-launch decode exchange buffers, counters);
 * 0 if the config is invalid.  Host-only, needs no GPU. */
size_t ngpt_workspace_bytes(const ngpt_config *cfg);

/* Validate a config (GPTConfig fields of the SDK guide, "模型架构解析")
 * without creating anything: NGPT_OK or NGPT_E_CONFIG / NGPT_E_ARG.
 * Host-only. */
int ngpt_check_config(const ngpt_config *cfg);

/*
 * Create a model (the GPT class of the SDK guide, "模型架构解析", with its
 * weights) on the current HIP device.  `stream` is a hipStream_t (NULL =
 * the default stream) on which every later call enqueues its work.
 * `workspace` is caller-owned device memory of ws_bytes >=
 * ngpt_workspace_bytes(cfg) bytes, 256-byte aligned; the library zeroes it
 * (asynchronously, on the stream) and keeps using it until destroy.
 * Sampling defaults: greedy.  Every weight and bias pointer must be 16-byte
 * aligned (the kernels read parameter rows with 8- and 16-byte accesses).
 * Errors: NGPT_E_ARG (NULL pointers, bias pointers inconsistent with
 * cfg->bias, misaligned pointers), NGPT_E_CONFIG, NGPT_E_SIZE (ws_bytes too
 * small), NGPT_E_HIP.  *out is NULL on error.
 */
int ngpt_create(const ngpt_config *cfg, const ngpt_weights *w,
                void *workspace, size_t ws_bytes, void *stream,
                ngpt_model **out);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops or harnesses that forbid hipMalloc): ngpt_create()
 * with the workspace taken from a fixed array inside the library, one per
 * GPU, of NGPT_STATIC_WORKSPACE_BYTES bytes, held until the process ends.
 * Calls no hipMalloc, hipFree or other allocating routine; the array is
 * zeroed on the stream at creation.  Every model created this way on a
 * device shares that device's array, so at most one may be alive per device
 * at a time: a second create on the same device fails with NGPT_E_ARG until
 * the first is destroyed (calls that overlapped on one array would race).
 * Errors: as ngpt_create, and NGPT_E_SIZE when ngpt_workspace_bytes(cfg)
 * exceeds the array.
 */
#define NGPT_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
int ngpt_create_static(const ngpt_config *cfg, const ngpt_weights *w,
                       void *stream, ngpt_model **out);

/* Wait for the stream, then release the handle (the caller still owns the
 * workspace, weights and KV memory).  The only call that synchronises. */
int ngpt_destroy(ngpt_model *m);

/*
 * Sampling parameters of the decode step (serving page, section 2):
 * logits are divided by `temperature` (> 0, fp32 correctly rounded), values
 * below the k-th largest with k = min(top_k, vocab) are dropped (top_k <= 0:
 * no filter; ties with the k-th value are kept), softmax in fp64 over the
 * kept ids, and the id is the smallest kept id (ascending) whose running
 * probability sum exceeds u * total for the caller's uniform u in [0,1).
 * greedy != 0 replaces all of this by the argmax (lowest id on ties) and
 * ignores the uniforms.  The values are written to device memory by a small
 * kernel on the stream (no host copy, no wait); later calls see them, and no
 * graph is captured again.  Errors: NGPT_E_ARG (temperature <= 0 unless
 * greedy), NGPT_E_HIP.
 */
int ngpt_set_sampling(ngpt_model *m, float temperature, int32_t top_k,
                      int32_t greedy);

/*
 * Prefill (the first forward of generate(), serving page section 2, over
 * each whole prompt; model-building chapter section 4.5 for positions 0..):
 * run each prompt through the model from an empty cache.
 *   ids    HOST int32 [B][Tmax], right-padded (entries past lens[b] ignored)
 *   lens   HOST int32 [B], 1 <= lens[b] <= block_size
 *   limit  HOST int32 [B] or NULL (NULL: every limit = block_size);
 *          lens[b] <= limit[b] <= block_size
 * Every id is checked on the host (0 <= id < vocab) before anything is
 * enqueued; the valid ids are packed into a pinned staging buffer of the
 * handle (allocated on first use) and copied asynchronously.  Reusing that
 * staging waits only for the copy enqueued by the previous prefill.
 * Requires B <= kv->batch <= cfg.max_batch and sum(lens) <=
 * cfg.max_prefill_tokens.  Writes K/V rows [0, lens[b]) of every layer, sets
 * kv->lens and kv->limit (rows B..kv->batch-1 get lens = limit = 0, i.e.
 * inactive), and leaves the logits of position lens[b]-1 of each sequence in
 * the logits buffer.  Errors: NGPT_E_ARG, NGPT_E_RANGE (an id, a length or a
 * limit out of range), NGPT_E_SIZE, NGPT_E_HIP.
 */
int ngpt_prefill(ngpt_model *m, ngpt_kv *kv, const int32_t *ids,
                 const int32_t *lens, const int32_t *limit, int32_t B,
                 int32_t Tmax);

/*
 * ngpt_prefill() with the ids already in device memory (device int32
 * [B][Tmax]), for callers whose tokens are produced on the GPU; no host copy.
 * The ids cannot be checked on the host: an id outside [0, vocab) is used as
 * 0 by the kernel and reported by ngpt_device_status() as NGPT_E_DEVICE.
 */
int ngpt_prefill_device(ngpt_model *m, ngpt_kv *kv, const int32_t *ids,
                        const int32_t *lens, const int32_t *limit, int32_t B,
                        int32_t Tmax);

/*
 * Admit prompts into chosen rows of a live batch (continuous batching: new
 * sequences take the rows of finished ones while the others keep their
 * state; serving page, section "HF 在哪些情况下实际上会更好" on batched
 * serving, and the KV-cache section for the per-row cache).  Like
 * ngpt_prefill for n prompts (host ids [n][Tmax], lens, limit), but prompt b
 * goes to kv row slots[b] (distinct, < kv->batch) from an empty cache, and
 * every other row keeps its cache, lens, limit and logits.  When kv is not
 * the cache of the last prefill on this model, every other row is made
 * inactive instead.  Errors: as ngpt_prefill; NGPT_E_RANGE for a slot out
 * of range, NGPT_E_ARG for a repeated slot.
 */
int ngpt_prefill_slots(ngpt_model *m, ngpt_kv *kv, const int32_t *slots,
                       const int32_t *ids, const int32_t *lens,
                       const int32_t *limit, int32_t n, int32_t Tmax);

/*
 * Chunked prefill into a live cache: append counts[b] tokens (host ids
 * [n][Tmax], row b) to live row slots[b] of the cache of the last prefill,
 * at positions lens .. lens + counts[b] - 1.  Each new token attends to every
 * cached position and to the new tokens up to itself: the causal mask offset
 * by the past length, which the serving page's KV-cache sketch leaves out
 * (it masks only when there is no past).  Leaves the logits of each row's
 * last new token.  Requires lens + counts[b] <= limit of the row.
 * Errors: NGPT_E_ARG, NGPT_E_RANGE (ids, slots, counts), NGPT_E_CONTEXT (the
 * row's limit), NGPT_E_SIZE (sum(counts) > max_prefill_tokens), NGPT_E_HIP.
 */
int ngpt_extend(ngpt_model *m, ngpt_kv *kv, const int32_t *slots,
                const int32_t *ids, const int32_t *counts, int32_t n,
                int32_t Tmax);

/*
 * Retire rows of the cache of the last prefill: each listed row stops taking
 * tokens (its limit becomes its length; cache and logits are kept), so its
 * row can be admitted again with ngpt_prefill_slots.  Errors: NGPT_E_ARG,
 * NGPT_E_RANGE, NGPT_E_HIP.
 */
int ngpt_retire(ngpt_model *m, ngpt_kv *kv, const int32_t *slots, int32_t n);

/*
 * Map blocks first_block .. first_block + count - 1 of row `slot` of a
 * paged cache to the pages pages[0 .. count-1] (HOST int32; -1 unmaps a
 * block), in stream order: a later prefill, extend or decode call on the
 * model's stream sees the new table.  This is the page bookkeeping of a
 * paged cache (serving page, section "HF 在哪些情况下实际上会更好": vLLM's
 * paged KV memory with continuous batching): the caller keeps the free list,
 * maps a row's blocks before positions in them are written, and may hand a
 * retired row's pages to another row.  Errors: NGPT_E_ARG (NULL pointers, kv
 * not paged), NGPT_E_RANGE (slot, block range or a page id outside
 * [-1, num_pages)), NGPT_E_HIP.
 */
int ngpt_kv_map(ngpt_model *m, ngpt_kv *kv, int32_t slot, int32_t first_block,
                int32_t count, const int32_t *pages);

/*
 * Generation past block_size (generate() crops its input to the last
 * block_size tokens, serving page section 2): for each listed row whose cache
 * holds block_size positions, the window of its cached tokens 1 .. Tb-1
 * followed by next_ids[row] (device int32 [kv->batch], e.g. drawn by
 * ngpt_sample from the row's logits) is run again from position 0 (the
 * positions are absolute, so the cache cannot be shifted), which refreshes
 * the row's cache and leaves the logits of the window's last token.  The
 * row's tokens come from the library's token history, written by every
 * prefill and decode call.  Requires n * block_size <= max_prefill_tokens.
 * Errors: NGPT_E_ARG (a row that is not full, kv not the recorded cache),
 * NGPT_E_RANGE, NGPT_E_SIZE, NGPT_E_HIP.
 */
int ngpt_slide(ngpt_model *m, ngpt_kv *kv, const int32_t *slots, int32_t n,
               const int32_t *next_ids);

/*
 * Evaluation forward with labels (model-building chapter "第 4 章 模型构建",
 * section 4.6: logits at every position; the last position is dropped and
 * the labels, the ids themselves, are shifted by one; the loss is the mean
 * cross-entropy).  For B sequences (host ids [B][Tmax], lens[b] in [1,
 * block_size], sum(lens) <= max_prefill_tokens) the forward runs over every
 * position from an empty cache (kv holds their K/V afterwards), then ln_f and
 * the tied lm_head on every row:
 *   logits     device fp32 [sum(lens)][vocab], packed rows (sequence b's
 *              rows follow sequence b-1's), output
 *   losses     device fp32 [sum(lens)], output: row t of a sequence gets
 *              log(sum_j exp(l_j)) - l[id at t+1]; its last row gets 0
 *   mean_loss  device fp32 [1], output: the mean over the sum(lens) - B
 *              scored rows (0 if there are none)
 * The model's own logits buffer is not refreshed, so decoding needs a new
 * prefill afterwards.  Errors: as ngpt_prefill.
 */
int ngpt_eval_loss(ngpt_model *m, ngpt_kv *kv, const int32_t *ids,
                   const int32_t *lens, int32_t B, int32_t Tmax, float *logits,
                   float *losses, float *mean_loss);

/*
 * One decode step for all kv->batch sequences (the loop body of generate()
 * in the serving page, section 2, with the KV cache of its "一个值得做的改进"
 * section: only the newest token is run, against the cached K/V): for every
 * active b (lens[b] < limit[b]):
 *   1. sample next_ids[b] from the current logits row with uniforms[b];
 *   2. run that token at position lens[b], append its K/V, refresh logits[b];
 *   3. lens[b] += 1.
 * Inactive rows get next_ids[b] = -1; their cache and logits are untouched.
 *   next_ids  device int32 [kv->batch], output
 *   uniforms  device double [kv->batch], in [0,1) (unused when greedy)
 * kv must be the cache of the last prefill on this model (its pointers and
 * batch); the host keeps a record of its lengths.  The step is one HIP graph
 * launch or, for greedy batch-1 bf16 steps, one kernel launch; the graph is
 * captured on first use; uniforms/next_ids pointers may change freely.
 * Errors: NGPT_E_ARG, NGPT_E_CONTEXT (no active row, known from the host's
 * record of lens and limits), NGPT_E_HIP.
 */
int ngpt_decode_step(ngpt_model *m, ngpt_kv *kv, int32_t *next_ids,
                     const double *uniforms);

/*
 * Teacher-forced decode step (the same KV-cached step of the serving page,
 * with the appended token given rather than drawn): like ngpt_decode_step()
 * but the token of each active row is given (device int32 [kv->batch]).
 * Out-of-range ids are used as 0 and reported by ngpt_device_status().
 */
int ngpt_decode_feed(ngpt_model *m, ngpt_kv *kv, const int32_t *ids);

/*
 * The sampler of generate() (serving page, section 2; rule as in
 * ngpt_set_sampling) alone, on caller logits (device fp32 [B][ld], ld >=
 * vocab), with the model's sampling parameters; writes next_ids (device
 * int32 [B]).  uniforms is device double [B] (may be NULL when greedy).  No
 * model state changes.  Taking the logits as an argument (instead of the
 * model's own logits) lets a caller replay the draw on any row, e.g. for a
 * bit-exact check; the model's logits are one such input (ngpt_logits).
 * Errors: NGPT_E_ARG, NGPT_E_SIZE (B > max_batch), NGPT_E_HIP.
 */
int ngpt_sample(ngpt_model *m, const float *logits, int32_t ld, int32_t B,
                const double *uniforms, int32_t *next_ids);

/*
 * Borrow the logits buffer (the last-position logits that generate() reads,
 * serving page section 2): device fp32 [max_batch][ld] with ld = vocab.  Row
 * b holds the logits of sequence b's last processed position.  Valid until
 * the next prefill/decode call on this model.
 */
int ngpt_logits(ngpt_model *m, const float **logits, int32_t *ld);

/* Copy rows [0, B) of the logits (as ngpt_logits) to dst (device fp32
 * [B][ld_dst]), asynchronously on the model's stream. */
int ngpt_copy_logits(ngpt_model *m, float *dst, int32_t ld_dst, int32_t B);

/*
 * Report kernel-side input errors since the last call, without waiting:
 * enqueues a small kernel that writes one int32 to *status (device memory,
 * or host memory the device can write, e.g. pinned) and clears the flags.
 * After the stream reaches it, *status is NGPT_OK, NGPT_E_DEVICE (an id
 * outside [0, vocab), or a greedy logits row with no finite maximum, was
 * seen; such an id is used as 0) or NGPT_E_TIMEOUT (a wait inside the
 * one-launch decode kernel gave up, see ngpt_set_wait_limit: that step's
 * ids, logits and cache rows are invalid, and the sequence must be
 * prefilled again).  A timeout is reported ahead of an id error.  This is
 * the status path of the generate() loop (serving page, section 2), which
 * has no error channel of its own.
 */
int ngpt_device_status(ngpt_model *m, int32_t *status);

/*
 * Poll passes after which a wait inside the one-launch decode kernel (batch
 * 1, bf16) gives up and sets the timeout flag; passes <= 0 restores the
 * default, 2^20 passes (tens of milliseconds).  Every wait in that kernel is
 * bounded this way, so a launch whose partners never answer ends instead of
 * hanging.  A small limit is a test hook that makes the timeout path run
 * (1: give up after the second pass that finds a word missing).  Takes
 * effect for later calls (a captured decode graph is captured again).
 * (Not a step of the pages' method: a guard of this implementation's
 * one-launch form of the KV-cached decode step.)  Errors: NGPT_E_ARG.
 */
int ngpt_set_wait_limit(ngpt_model *m, int32_t passes);

/* Message of the last error on this handle (static storage if m is NULL). */
const char *ngpt_last_error(const ngpt_model *m);

/* Name of a status code. */
const char *ngpt_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* NGPT_H */
