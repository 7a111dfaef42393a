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

// Packed prefill rows: sequence b owns rows [off[b], off[b+1]); they go to
// cache row (slot) slot[b] at positions past[b] .. past[b] + (its row count)
// - 1, after the past[b] positions already cached there.
struct RowMap {
  int32_t B;
  int32_t off[NGPT_MAX_BATCH + 1];
  int32_t slot[NGPT_MAX_BATCH];
  int32_t past[NGPT_MAX_BATCH];
};

// Where one layer's cache keeps position t of sequence b, head h: the row
// (of hs elements) block_base(b, t / 64) + h * hstride + t % 64.
//  * contiguous layout [batch][H][Tb][hs] (table == null):
//    block_base = b * H * Tb + 64 * (t / 64), hstride = Tb;
//  * paged layout [pages][H][64][hs]: block t / 64 of sequence b lives in
//    page table[b * nblk + t / 64], block_base = page * H * 64, hstride = 64.
//    A page id outside [0, npages) is an unmapped block.
struct KvMap {
  const int32_t* table = nullptr;
  int nblk = 0;     // table row stride: blocks per sequence, ceil(Tb / 64)
  int npages = 0;
  int H = 0, Tb = 0;
};

constexpr int kPageTokens = NGPT_PAGE_TOKENS;

// First row of block `blk` of sequence b (head 0); -1 when unmapped.
__device__ __forceinline__ int64_t kv_block_base(const KvMap& k, int b, int blk) {
  if (!k.table) return (int64_t)b * k.H * k.Tb + (int64_t)blk * kPageTokens;
  const int pg = k.table[b * k.nblk + blk];
  return (uint32_t)pg < (uint32_t)k.npages ? (int64_t)pg * k.H * kPageTokens : -1;
}
__device__ __forceinline__ int kv_hstride(const KvMap& k) {
  return k.table ? kPageTokens : k.Tb;
}

// Linear-layer epilogues (what happens to acc = A W^T for row r, column n).
enum Epi {
  EPI_GELU = 1,    // out[r][n] = GELU(acc + bias)                (dtype)
  EPI_RESID = 2,   // out[r][n] += acc + bias                      (fp32 residual)
  EPI_QKV = 3,     // split into q (out, dtype) and the K/V cache rows
  EPI_LOGITS = 4,  // out[row_b ? row_b[r] : r][n] = acc          (fp32)
};

struct EpiArgs {
  const void* bias = nullptr;     // [N] dtype or null
  void* out = nullptr;
  int ldo = 0;
  // EPI_QKV: this layer's cache (addressed through kv); a position whose
  // block is unmapped is not written and sets bit 4 of *status
  void* kc = nullptr;
  void* vc = nullptr;
  KvMap kv;
  int32_t* status = nullptr;
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

// ids: [B][Tmax] right-padded (Tmax > 0) or packed by row (Tmax == 0).
// Writes x, the row -> (slot, position) maps, each sequence's last row and
// its slot (last_rows[b], last_slot[b]), and the ids into the token history
// hist [max_batch][Tb] (slot, position).
void launch_embed_prefill(int dtype, const int32_t* ids, int Tmax,
                          const RowMap& map, int M, const void* wte,
                          const void* wpe, int C, int V, float* x,
                          int32_t* row_b, int32_t* row_pos, int32_t* last_rows,
                          int32_t* last_slot, int32_t* hist, int Tb,
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

// Skinny 16-bit linear layer for 1 <= M <= 64 rows (K a multiple of 32 and
// at most 13 * 16 steps of 32); false (nothing launched) for other shapes.
bool launch_skinny(int dtype, int epi, const void* A, int lda, const void* W, int M, int N,
                   int K, const EpiArgs& e, hipStream_t s);

// Causal attention of each packed prefill row against its own sequence's
// keys in the cache (positions 0..pos).  q is [M][ldq] (head j at columns
// j*hs), the output y [M][ldy] likewise.
// kc / vc: this layer's cache, addressed through kv.
void launch_attn_prefill(int dtype, const void* q, int ldq, const void* kc,
                         const void* vc, const KvMap& kv, const RowMap& map, int maxlen, int H,
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
                        const void* vc, const KvMap& kv, const int32_t* pos, int B, int H,
                        int hs, int Tb, float* part, void* y,
                        bool merge_into_y, hipStream_t s);

// Decode output projection fed directly by the attention records:
// x[m] += merge(part[m]) W^T + b for M <= 4 rows (see decode_fused_proj).
bool decode_fused_proj(int M);
void launch_attn_proj(int dtype, const float* part, const int32_t* pos, int H,
                      int hs, int nchunk, int chunk_keys, const void* W, int M,
                      int C, const EpiArgs& e, hipStream_t s);

// Cross-entropy of packed rows against the next id of the same sequence
// (none for a sequence's last row, whose loss is 0), and the mean over the
// nscored scored rows.  logits [M][ld] fp32; ids packed [M].
void launch_cross_entropy(const float* logits, int ld, int V, int M, int nscored,
                          const int32_t* ids, const int32_t* row_b,
                          const int32_t* last_rows, float* losses, float* mean,
                          hipStream_t s);

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
  int32_t* hist = nullptr;   // token history [B][Tb]: the step's id at pos
  int Tb = 0;
  // decode steps also write the embedding x = wte[id] + wpe[pos] (fp32 [B][C])
  const void* wte = nullptr;
  const void* wpe = nullptr;
  int C = 0;
  int dtype = 0;
  float* x = nullptr;
  uint32_t* epoch = nullptr;  // advanced by one when the forward is the one-launch kernel
  void* ptrs[21] = {};
};
// Fill a kernel-node description for B rows; `a` must outlive its use.
void sampler_node_params(SamplerArgs& a, int B, hipKernelNodeParams* p);

// Sampler / feed head node: picks each row's next id and, in the step modes,
// sets tok/pos, advances lens and writes the row's embedding.
void launch_sampler(const SamplerArgs& a, int B, hipStream_t s);

}  // namespace ngpt

#include "k_persist.hpp"
