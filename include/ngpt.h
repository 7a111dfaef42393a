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
 *     (c_attn split into q, k, v; past K/V concatenated along time; only the
 *     newest token is fed; causal masking only without a past).
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
 *   - Work is enqueued asynchronously on the stream given to ngpt_create();
 *     calls do not synchronise unless stated.
 *   - Weights and KV buffers are caller-owned device memory and are borrowed:
 *     they must stay alive and unmodified while the model uses them.  The
 *     library owns only its workspace (allocated in ngpt_create, freed in
 *     ngpt_destroy).
 *   - A handle is bound to one stream and is not thread-safe.
 *   - Element type of every weight, bias, LayerNorm parameter and KV entry is
 *     the config dtype (fp32 or bf16).  The residual stream, LayerNorm
 *     statistics, attention softmax and logits are fp32 in both modes.
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
#define NGPT_E_SIZE      -4  /* batch or token count above the create-time bound */
#define NGPT_E_CONTEXT   -5  /* no sequence can take another token          */
#define NGPT_E_HIP       -6  /* a HIP runtime call failed                   */
#define NGPT_E_DEVICE    -7  /* a kernel reported an out-of-range id        */
#define NGPT_E_TIMEOUT   -8  /* a wait in the one-launch decode kernel gave up */

/* Element types. */
#define NGPT_F32   0
#define NGPT_BF16  1

/*
 * Model shape, the GPTConfig of the SDK guide ("模型架构解析"): block_size,
 * vocab_size, n_layer, n_head, n_embd, bias.  dropout is absent (inference).
 * Supported: n_embd % n_head == 0; head_dim = n_embd / n_head in {32, 64};
 * n_embd % 64 == 0 (bf16) or n_embd % 4 == 0 (fp32); n_embd <= 2048;
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
  int32_t dtype;              /* NGPT_F32 or NGPT_BF16 */
  int32_t max_batch;
  int32_t max_prefill_tokens;
} ngpt_config;

/*
 * Weights of one block, device pointers in nn.Linear layout
 * [out_features][in_features], row-major, elements of the config dtype.
 * attn_w is c_attn, [3C][C]: rows [0,C) give q, [C,2C) k, [2C,3C) v; head j
 * of each is the row slice [j*hs, (j+1)*hs) (serving page, KV-cache section).
 * attnproj_w is the attention c_proj [C][C]; fc_w is [4C][C]; mlpproj_w is
 * [C][4C].  LayerNorm weights are [C].  Bias pointers must all be NULL when
 * bias == 0 and all non-NULL when bias == 1 (serving page, section 1).
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
 * lm_head bias.  wpe is [block_size][C].  `layers` is a HOST array of
 * n_layer entries; it is copied at create time.
 */
typedef struct {
  const void *wte, *wpe;
  const void *lnf_w, *lnf_b;
  const ngpt_layer_weights *layers;
} ngpt_weights;

/*
 * KV cache, caller-owned device memory.  k and v are each laid out
 * [n_layer][batch][n_head][block_size][head_dim] in the config dtype
 * (ngpt_kv_bytes() bytes each).  lens[b] is the number of positions of
 * sequence b held in the cache; limit[b] (<= block_size) is the total length
 * at which sequence b stops taking tokens.  Both are device int32 [batch],
 * written by ngpt_prefill() and advanced by the decode calls.  A sequence is
 * active while lens[b] < limit[b].
 */
typedef struct {
  void *k;
  void *v;
  int32_t *lens;
  int32_t *limit;
  int32_t batch;
} ngpt_kv;

typedef struct ngpt_model ngpt_model;

/* Bytes of ONE of the two KV arrays for `batch` sequences; 0 if the config is
 * invalid.  Host-only, needs no GPU. */
size_t ngpt_kv_bytes(const ngpt_config *cfg, int32_t batch);

/* Validate a config without creating anything: NGPT_OK or NGPT_E_CONFIG /
 * NGPT_E_ARG.  Host-only. */
int ngpt_check_config(const ngpt_config *cfg);

/*
 * Create a model on the current HIP device.  `stream` is a hipStream_t
 * (NULL = the default stream) on which every later call enqueues its work.
 * Allocates the workspace (activations, split-K partials, fp32 logits
 * [max_batch][vocab]).  Sampling defaults: greedy.
 * Every weight and bias pointer must be 16-byte aligned (the kernels read
 * parameter rows with 8- and 16-byte accesses); fresh device allocations and
 * framework tensors are.
 * Errors: NGPT_E_ARG (NULL pointers, bias pointers inconsistent with
 * cfg->bias, misaligned pointers), NGPT_E_CONFIG, NGPT_E_HIP.  *out is NULL
 * on error.
 */
int ngpt_create(const ngpt_config *cfg, const ngpt_weights *w, void *stream,
                ngpt_model **out);

/* Wait for the stream, then free the workspace and the handle. */
int ngpt_destroy(ngpt_model *m);

/*
 * Sampling parameters of the decode step (serving page, section 2):
 * logits are divided by `temperature` (> 0, fp32 correctly rounded), values
 * below the k-th largest with k = min(top_k, vocab) are dropped (top_k <= 0:
 * no filter; ties with the k-th value are kept), softmax in fp64 over the
 * kept ids, and the id is the smallest kept id (ascending) whose running
 * probability sum exceeds u * total for the caller's uniform u in [0,1).
 * greedy != 0 replaces all of this by the argmax (lowest id on ties) and
 * ignores the uniforms.  Takes effect for later calls; no re-capture.
 */
int ngpt_set_sampling(ngpt_model *m, float temperature, int32_t top_k,
                      int32_t greedy);

/*
 * Prefill: run each prompt through the model from an empty cache.
 *   ids    device int32 [B][Tmax], right-padded (entries past lens[b] ignored)
 *   lens   HOST int32 [B], 1 <= lens[b] <= block_size
 *   limit  HOST int32 [B] or NULL (NULL: every limit = block_size);
 *          lens[b] <= limit[b] <= block_size
 * Requires B <= kv->batch <= cfg.max_batch and sum(lens) <=
 * cfg.max_prefill_tokens.  Writes K/V rows [0, lens[b]) of every layer, sets
 * kv->lens and kv->limit, and leaves the logits of position lens[b]-1 of
 * each sequence in the logits buffer.  Ids outside [0, vocab) are treated as
 * 0 by the kernel and reported by ngpt_device_status() as NGPT_E_DEVICE.
 * Errors: NGPT_E_ARG, NGPT_E_RANGE (lens/limit), NGPT_E_SIZE, NGPT_E_HIP.
 */
int ngpt_prefill(ngpt_model *m, ngpt_kv *kv, const int32_t *ids,
                 const int32_t *lens, const int32_t *limit, int32_t B,
                 int32_t Tmax);

/*
 * One decode step for all kv->batch sequences (the loop body of generate()
 * with a KV cache): for every active b (lens[b] < limit[b]):
 *   1. sample next_ids[b] from the current logits row with uniforms[b];
 *   2. run that token at position lens[b], append its K/V, refresh logits[b];
 *   3. lens[b] += 1.
 * Inactive rows get next_ids[b] = -1; their cache and logits are untouched.
 *   next_ids  device int32 [kv->batch], output
 *   uniforms  device double [kv->batch], in [0,1) (unused when greedy)
 * The step is one HIP graph launch (captured on first use for this kv;
 * re-captured if kv's pointers change; uniforms/next_ids pointers may change
 * freely).  Errors: NGPT_E_ARG, NGPT_E_CONTEXT (no active row, known from the
 * host's record of lens and limits), NGPT_E_HIP.
 */
int ngpt_decode_step(ngpt_model *m, ngpt_kv *kv, int32_t *next_ids,
                     const double *uniforms);

/*
 * Teacher-forced decode step: like ngpt_decode_step() but the token of each
 * active row is given (device int32 [kv->batch]) instead of sampled.
 * Out-of-range ids are treated as 0 and reported by ngpt_device_status().
 */
int ngpt_decode_feed(ngpt_model *m, ngpt_kv *kv, const int32_t *ids);

/*
 * Run the sampler alone on caller logits (device fp32 [B][ld], ld >= vocab)
 * with the model's sampling parameters; writes next_ids (device int32 [B]).
 * uniforms is device double [B] (may be NULL when greedy).  No model state
 * changes.  Errors: NGPT_E_ARG, NGPT_E_SIZE (B > max_batch), NGPT_E_HIP.
 */
int ngpt_sample(ngpt_model *m, const float *logits, int32_t ld, int32_t B,
                const double *uniforms, int32_t *next_ids);

/*
 * Borrow the logits buffer: device fp32 [max_batch][ld] with ld = vocab.
 * Row b holds the logits of sequence b's last processed position.  Valid
 * until the next prefill/decode call on this model.
 */
int ngpt_logits(ngpt_model *m, const float **logits, int32_t *ld);

/* Copy rows [0, B) of the logits to dst (device fp32 [B][ld_dst]),
 * asynchronously on the model's stream. */
int ngpt_copy_logits(ngpt_model *m, float *dst, int32_t ld_dst, int32_t B);

/*
 * Synchronise the stream and report kernel-side input errors since the last
 * call: *status = NGPT_OK, NGPT_E_DEVICE (an id outside [0, vocab) was
 * seen) or NGPT_E_TIMEOUT (a wait inside the one-launch decode kernel gave
 * up, see ngpt_set_wait_limit: that step's ids, logits and cache rows are
 * invalid, and the sequence must be prefilled again).  A timeout is reported
 * ahead of an id error.  Clears the flags.
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
 * Errors: NGPT_E_ARG.
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
