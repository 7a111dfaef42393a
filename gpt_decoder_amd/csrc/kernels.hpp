// Host-side launchers of the libngpt kernels and their argument records.
// Every launcher enqueues on the given stream and returns immediately.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ngpt.h"

namespace ngpt {
typedef uint16_t bf16_t;
}

namespace ngpt {

// Packed prefill rows: sequence b owns rows [off[b], off[b+1]).
struct RowMap {
  int32_t B;
  int32_t off[NGPT_MAX_BATCH + 1];
};

// Linear-layer epilogues (what happens to acc = A W^T for row r, column n).
enum Epi {
  EPI_GELU = 1,    // out[r][n] = GELU(acc + bias)                (dtype)
  EPI_RESID = 2,   // out[r][n] += acc + bias                      (fp32 residual)
  EPI_QKV = 3,     // split into q (out, dtype) and the K/V cache rows
  EPI_LOGITS = 4,  // out[r][n] = acc                             (fp32)
};

struct EpiArgs {
  const void* bias = nullptr;     // [N] dtype or null
  void* out = nullptr;
  int ldo = 0;
  // EPI_QKV: this layer's cache, each [batch][H][Tb][hs]
  void* kc = nullptr;
  void* vc = nullptr;
  const int32_t* row_b = nullptr;    // row -> sequence (null: identity)
  const int32_t* row_pos = nullptr;  // row -> position; < 0 => inactive row
  int C = 0, H = 0, hs = 0, Tb = 0;
};

// Sampling parameters, resident in device memory so that a captured decode
// graph picks up changes.
struct SampleParams {
  float temperature;
  int32_t top_k;
  int32_t greedy;
  int32_t pad;
};

enum SampleMode {
  SAMPLE_ONLY = 0,  // write next_ids only
  SAMPLE_STEP = 1,  // decode step: also tok/pos, advance lens
  FEED_STEP = 2,    // teacher forcing: ids given, set tok/pos, advance lens
};

void launch_embed_prefill(int dtype, const int32_t* ids, int Tmax,
                          const RowMap& map, int M, const void* wte,
                          const void* wpe, int C, int V, float* x,
                          int32_t* row_b, int32_t* row_pos, int32_t* last_rows,
                          int32_t* status, hipStream_t s);

void launch_embed_decode(int dtype, const int32_t* tok, const int32_t* pos,
                         int B, const void* wte, const void* wpe, int C, int V,
                         float* x, int32_t* status, hipStream_t s);

// out[i] = LN(x[rows ? rows[i] : i]) over C columns, fp32 statistics.
void launch_layernorm(int dtype, const float* x, int ldx, const int32_t* rows,
                      int M, const void* w, const void* b, void* out, int ldo,
                      int C, hipStream_t s);

// Optional LayerNorm of the A operand: A = LN(x) with x fp32 [M][ldx] and
// K = C features.  Paths that need a materialised LN output write it to h
// ([M][K], dtype) first.
struct LnArgs {
  const float* x = nullptr;
  int ldx = 0;
  const void* w = nullptr;
  const void* b = nullptr;
  void* h = nullptr;
};

// acc = A[M][K] W[N][K]^T, then the epilogue.  A and W are dtype.  With
// ln != null the A operand is LN(ln->x) and `A` is ignored.
void launch_linear(int dtype, int epi, const void* A, int lda,
                   const LnArgs* ln, const void* W, int M, int N, int K,
                   const EpiArgs& e, hipStream_t s);

// Causal attention of each packed prefill row against its own sequence's
// keys in the cache (positions 0..pos).  q is [M][ldq] (head j at columns
// j*hs), the output y [M][ldy] likewise.
void launch_attn_prefill(int dtype, const void* q, int ldq, const void* kc,
                         const void* vc, const RowMap& map, int maxlen, int H,
                         int hs, int Tb, void* y, int ldy, float* part, hipStream_t s);
// chunks per (row, head) of the prefill key split: the partial buffer holds
// [H][Tb][chunks][hs + 4] floats (one sequence)
int attn_prefill_split_chunks(int Tb);

// One query per active sequence (pos[b] >= 0) against cache rows
// 0..pos[b], split over key chunks: each chunk leaves a record (max, sum,
// o[hs]) in `part` [B][H][nchunk][hs+2].  With merge_into_y the records are
// merged (in chunk order) into y [B][C] by a second launch; otherwise the
// consumer merges them (launch_attn_proj).
int attn_decode_chunks(int Tb);
int attn_decode_chunk_keys();
void launch_attn_decode(int dtype, const void* q, const void* kc,
                        const void* vc, const int32_t* pos, int B, int H,
                        int hs, int Tb, float* part, void* y,
                        bool merge_into_y, hipStream_t s);

// Decode output projection fed directly by the attention records:
// x[m] += merge(part[m]) W^T + b for M <= 4 rows (see decode_fused_proj).
bool decode_fused_proj(int M);
void launch_attn_proj(int dtype, const float* part, const int32_t* pos, int H,
                      int hs, int nchunk, int chunk_keys, const void* W, int M,
                      int C, const EpiArgs& e, hipStream_t s);

// Argument pack of the sampler kernel, used to (re)write its graph node.
struct SamplerArgs {
  int mode = 0;
  const float* logits = nullptr;
  int ld = 0;
  int V = 0;
  const double* uniforms = nullptr;
  const SampleParams* params = nullptr;
  const int32_t* feed_ids = nullptr;
  int32_t* next_ids = nullptr;
  int32_t* tok = nullptr;
  int32_t* pos = nullptr;
  int32_t* lens = nullptr;
  const int32_t* limit = nullptr;
  int32_t* status = nullptr;
  // decode steps also write the embedding x = wte[id] + wpe[pos] (fp32 [B][C])
  const void* wte = nullptr;
  const void* wpe = nullptr;
  int C = 0;
  int dtype = 0;
  float* x = nullptr;
  void* ptrs[18] = {};
};
// Fill a kernel-node description for B rows; `a` must outlive its use.
void sampler_node_params(SamplerArgs& a, int B, hipKernelNodeParams* p);

// Sampler / feed head node: picks each row's next id and, in the step modes,
// sets tok/pos, advances lens and writes the row's embedding.
void launch_sampler(const SamplerArgs& a, int B, hipStream_t s);

// ---------------------------------------------------------------------------
// One-launch decode step for batch 1 (bf16, head size 64, n_embd <= 768).
struct PersistLayer {
  const bf16_t *ln1_w, *ln1_b, *attn_w, *attn_b, *proj_w, *proj_b;
  const bf16_t *ln2_w, *ln2_b, *fc_w, *fc_b, *mp_w, *mp_b;
};

struct PersistArgs {
  int L, H, C, V, Tb, nchunk;
  const bf16_t *wte, *wpe, *lnf_w, *lnf_b;
  const PersistLayer* layers;   // device array [L]
  int32_t* pos;                 // [1]: set by the head node (< 0: inactive),
                                // or written here in a fused greedy step
  int fused;                    // 1: greedy step without a head node
  int32_t* lens;                // kv lens [1] (fused: read, then advanced)
  int32_t* tok;                 // fused: the chosen id ...
  int32_t* next_ids;            // ... and the caller's copy
  uint64_t* e_cand;             // greedy candidates, 2 words per workgroup
  const float* x0;              // [C] embedding written by the head node
  bf16_t* kc;                   // cache bases and per-layer stride (elements)
  bf16_t* vc;
  size_t layer_stride;
  float* logits;                // [V]
  // exchange words (fp32 value | epoch << 32), per layer
  uint64_t *e_qkv, *e_rec, *e_y, *e_x1, *e_f, *e_x2;
  uint32_t* epoch;              // advanced once per launch
  int32_t* status;              // bit 2: a wait timed out
  int wait_limit;                // poll passes before a wait gives up (0: default)
};

bool persistent_decode_supported(int dtype, int C, int H, int L, int Tb,
                                 int batch, int grid);
size_t persistent_lds_bytes(int C, int L);
// words of slack past the end of each exchange buffer (polls read ahead)
int persistent_exchange_slack();
void launch_decode_persistent(const PersistArgs& a, int grid, hipStream_t s);

}  // namespace ngpt
