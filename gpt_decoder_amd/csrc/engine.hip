// libngpt host engine: argument validation, workspace carving, the prefill
// launch sequence and the HIP-graph decode step.  All arithmetic runs in the
// kernels declared in kernels.hpp; this file only orders launches.
//
// Forward pass (SDK guide "极速上手nanoGPT", "模型架构解析"; architecture
// analysis "nanoGPT 架构分析", section 4.1):
//   x = wte[id] + wpe[pos]
//   per block: x += c_proj(attn(ln_1(x)));  x += mlp_proj(GELU(c_fc(ln_2(x))))
//   logits = ln_f(x_last) wte^T
// generate() loop with a KV cache (serving page "原生 nanoGPT 模型服务首选",
// sections 2 and "一个值得做的改进"): sample from the last logits, append the
// token, run only that token against the cached K/V.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "ngpt.h"

using namespace ngpt;

namespace {

struct LensArgs {
  int32_t n;        // rows of the kv batch to set
  int32_t lens[NGPT_MAX_BATCH];
  int32_t limit[NGPT_MAX_BATCH];
};

__global__ void set_lens_kernel(LensArgs a, int32_t* lens, int32_t* limit) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < a.n) {
    lens[b] = a.lens[b];
    limit[b] = a.limit[b];
  }
}

__global__ void clear_status_kernel(int32_t* status) {
  if (threadIdx.x == 0) status[0] = 0;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct GraphSlot {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  hipGraphNode_t head = nullptr;  // the sampler / feed node
  // what the graph was captured for
  void* k = nullptr;
  void* v = nullptr;
  int32_t* lens = nullptr;
  int32_t* limit = nullptr;
  int32_t batch = 0;
  int32_t wait_limit = 0;
  const void* arg_in = nullptr;   // uniforms (step) or feed ids (feed)
  int32_t* arg_out = nullptr;     // next_ids (step)
  SamplerArgs head_args;          // arguments of the head node
};

const char* status_name(int s) {
  switch (s) {
    case NGPT_OK: return "NGPT_OK";
    case NGPT_E_ARG: return "NGPT_E_ARG";
    case NGPT_E_CONFIG: return "NGPT_E_CONFIG";
    case NGPT_E_RANGE: return "NGPT_E_RANGE";
    case NGPT_E_SIZE: return "NGPT_E_SIZE";
    case NGPT_E_CONTEXT: return "NGPT_E_CONTEXT";
    case NGPT_E_HIP: return "NGPT_E_HIP";
    case NGPT_E_DEVICE: return "NGPT_E_DEVICE";
    case NGPT_E_TIMEOUT: return "NGPT_E_TIMEOUT";
    default: return "NGPT_E_UNKNOWN";
  }
}

std::string g_static_error;

}  // namespace

struct ngpt_model {
  ngpt_config cfg{};
  int L = 0, H = 0, C = 0, hs = 0, Tb = 0, V = 0, Mmax = 0, nchunk = 0;
  size_t esz = 0;
  const void *wte = nullptr, *wpe = nullptr, *lnf_w = nullptr, *lnf_b = nullptr;
  std::vector<ngpt_layer_weights> layers;
  hipStream_t stream = nullptr;
  hipStream_t cap = nullptr;
  // workspace
  void* ws = nullptr;
  float* x = nullptr;
  void *h = nullptr, *q = nullptr, *y = nullptr, *f = nullptr, *z = nullptr;
  float* logits = nullptr;
  int32_t *row_b = nullptr, *row_pos = nullptr, *last_rows = nullptr;
  float* part = nullptr;
  float* ppart = nullptr;   // prefill attention key-split partials (one sequence)
  int32_t *tok = nullptr, *pos = nullptr, *status = nullptr;
  int32_t h_wait_limit = 0;        // one-launch decode poll limit (0: default)
  SampleParams* params = nullptr;
  SampleParams h_params{1.0f, 0, 1, 0};  // host copy of *params
  // one-launch batch-1 decode (see k_persist.hip)
  int persist_grid = 0;   // workgroups of the one-launch decode kernel
  bool persist = false;
  PersistLayer* d_layers = nullptr;
  uint64_t *e_qkv = nullptr, *e_rec = nullptr, *e_y = nullptr, *e_x1 = nullptr,
           *e_f = nullptr, *e_x2 = nullptr;
  uint32_t* epoch = nullptr;
  uint64_t* e_cand = nullptr;   // greedy candidates left by the last launch
  bool cand_ok = false;         // the current logits came from that launch
  // host record of the KV batch state
  std::vector<int32_t> h_lens, h_limit;
  GraphSlot g_step, g_feed;
  std::string err;
};

static int fail(ngpt_model* m, int code, const std::string& msg) {
  if (m) m->err = msg; else g_static_error = msg;
  return code;
}

#define HIP_TRY(m, expr)                                                   \
  do {                                                                     \
    hipError_t e_ = (expr);                                                \
    if (e_ != hipSuccess)                                                  \
      return fail((m), NGPT_E_HIP, std::string(#expr) + ": " +             \
                                       hipGetErrorString(e_));             \
  } while (0)

static int check_config(const ngpt_config* c, std::string* why) {
  auto bad = [&](const char* s) { if (why) *why = s; return NGPT_E_CONFIG; };
  if (!c) { if (why) *why = "config is NULL"; return NGPT_E_ARG; }
  if (c->n_layer < 0) return bad("n_layer < 0");
  if (c->n_head < 1 || c->n_embd < 1) return bad("n_head and n_embd must be >= 1");
  if (c->n_embd % c->n_head != 0) return bad("n_embd % n_head != 0");
  const int hs = c->n_embd / c->n_head;
  if (hs != 32 && hs != 64) return bad("head_dim must be 32 or 64");
  if (c->dtype != NGPT_F32 && c->dtype != NGPT_BF16) return bad("unknown dtype");
  if (c->dtype == NGPT_BF16 && c->n_embd % 64 != 0) return bad("bf16 needs n_embd % 64 == 0");
  if (c->dtype == NGPT_F32 && c->n_embd % 4 != 0) return bad("fp32 needs n_embd % 4 == 0");
  if (c->n_embd > 2048) return bad("n_embd must be <= 2048");
  if (c->block_size < 1 || c->block_size > 4096) return bad("block_size must be in [1, 4096]");
  if (c->vocab_size < 1) return bad("vocab_size must be >= 1");
  if (c->bias != 0 && c->bias != 1) return bad("bias must be 0 or 1");
  if (c->max_batch < 1 || c->max_batch > NGPT_MAX_BATCH) return bad("max_batch must be in [1, NGPT_MAX_BATCH]");
  if (c->max_prefill_tokens < 1) return bad("max_prefill_tokens must be >= 1");
  // The kernels address each matrix with 32-bit buffer offsets and use
  // offset 2^31 as "past the end" (reads zeros), so every weight matrix and
  // every activation buffer must stay below 2 GiB.
  const size_t esz = c->dtype == NGPT_BF16 ? 2 : 4;
  const size_t kMaxBytes = (size_t)1 << 31;
  if ((size_t)c->vocab_size * c->n_embd * esz >= kMaxBytes)
    return bad("vocab_size * n_embd too large (the embedding matrix must be < 2 GiB)");
  const size_t rows = (size_t)std::max(c->max_prefill_tokens, c->max_batch);
  if (rows * 4 * c->n_embd * esz >= kMaxBytes)
    return bad("max_prefill_tokens * 4 * n_embd too large (activations must be < 2 GiB)");
  return NGPT_OK;
}

static bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

extern "C" {

const char* ngpt_status_string(int status) { return status_name(status); }

const char* ngpt_last_error(const ngpt_model* m) {
  return m ? m->err.c_str() : g_static_error.c_str();
}

int ngpt_check_config(const ngpt_config* cfg) {
  std::string why;
  const int rc = check_config(cfg, &why);
  if (rc != NGPT_OK) g_static_error = why;
  return rc;
}

size_t ngpt_kv_bytes(const ngpt_config* cfg, int32_t batch) {
  if (check_config(cfg, nullptr) != NGPT_OK || batch < 1) return 0;
  const size_t es = cfg->dtype == NGPT_BF16 ? 2 : 4;
  return (size_t)cfg->n_layer * batch * cfg->n_head * cfg->block_size *
         (cfg->n_embd / cfg->n_head) * es;
}

int ngpt_create(const ngpt_config* cfg, const ngpt_weights* w, void* stream,
                ngpt_model** out) {
  if (!out) return fail(nullptr, NGPT_E_ARG, "out is NULL");
  *out = nullptr;
  std::string why;
  int rc = check_config(cfg, &why);
  if (rc != NGPT_OK) return fail(nullptr, rc, why);
  if (!w || !w->wte || !w->wpe || !w->lnf_w || (cfg->n_layer > 0 && !w->layers))
    return fail(nullptr, NGPT_E_ARG, "missing weight pointer");
  const bool bias = cfg->bias != 0;
  if ((w->lnf_b != nullptr) != bias)
    return fail(nullptr, NGPT_E_ARG, "lnf_b must be non-NULL iff bias");
  if (misaligned(w->wte) || misaligned(w->wpe) || misaligned(w->lnf_w) || misaligned(w->lnf_b))
    return fail(nullptr, NGPT_E_ARG, "weights must be 16-byte aligned");
  for (int l = 0; l < cfg->n_layer; ++l) {
    const ngpt_layer_weights& lw = w->layers[l];
    const void* req[] = {lw.ln1_w, lw.attn_w, lw.attnproj_w, lw.ln2_w, lw.fc_w, lw.mlpproj_w};
    const void* opt[] = {lw.ln1_b, lw.attn_b, lw.attnproj_b, lw.ln2_b, lw.fc_b, lw.mlpproj_b};
    for (const void* p : req) {
      if (!p) return fail(nullptr, NGPT_E_ARG, "missing layer weight pointer");
      if (misaligned(p)) return fail(nullptr, NGPT_E_ARG, "weights must be 16-byte aligned");
    }
    for (const void* p : opt) {
      if ((p != nullptr) != bias)
        return fail(nullptr, NGPT_E_ARG, "bias pointers must be non-NULL iff bias");
      if (misaligned(p)) return fail(nullptr, NGPT_E_ARG, "weights must be 16-byte aligned");
    }
  }

  ngpt_model* m = new ngpt_model();
  m->cfg = *cfg;
  m->L = cfg->n_layer; m->H = cfg->n_head; m->C = cfg->n_embd;
  m->hs = m->C / m->H; m->Tb = cfg->block_size; m->V = cfg->vocab_size;
  m->esz = cfg->dtype == NGPT_BF16 ? 2 : 4;
  m->Mmax = std::max(cfg->max_prefill_tokens, cfg->max_batch);
  m->nchunk = attn_decode_chunks(m->Tb);
  m->wte = w->wte; m->wpe = w->wpe; m->lnf_w = w->lnf_w; m->lnf_b = w->lnf_b;
  m->layers.assign(w->layers, w->layers + m->L);
  m->stream = static_cast<hipStream_t>(stream);

  const size_t Mm = m->Mmax, Bm = cfg->max_batch, C = m->C, es = m->esz;
  size_t off = 0;
  auto carve = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  const size_t o_x = carve(Mm * C * 4), o_h = carve(Mm * C * es),
               o_q = carve(Mm * C * es), o_y = carve(Mm * C * es),
               o_f = carve(Mm * 4 * C * es), o_z = carve(Bm * C * es),
               o_lg = carve(Bm * (size_t)m->V * 4), o_rb = carve(Mm * 4),
               o_rp = carve(Mm * 4), o_lr = carve(Bm * 4),
               o_part = carve(Bm * m->H * (size_t)m->nchunk * (m->hs + 2) * 4),
               o_ppart = carve((size_t)m->H * m->Tb * attn_prefill_split_chunks(m->Tb) *
                               (m->hs + 4) * 4),
               o_tok = carve(Bm * 4),
               o_pos = carve(Bm * 4), o_st = carve(16),
               o_prm = carve(sizeof(SampleParams));
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0) != hipSuccess) cus = 0;
  {
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess)
      (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  }
  // One-launch decode grid: the fewest workgroups (a multiple of 8, at most
  // one per CU) whose register slabs hold every phase's rows.  Each exchange
  // waits for words from all workgroups, and that wait shortens with fewer
  // participants (measured: 245 us per GPT-2-small step at 192 workgroups,
  // 260 at 224, 265 at 256).
  int pgrid = 0;
  for (int g = 64; g <= cus && pgrid == 0; g += 8)
    if (persistent_decode_supported(cfg->dtype, m->C, m->H, m->L, m->Tb, 1, g)) pgrid = g;
  m->persist_grid = pgrid;
  m->persist = pgrid > 0;
  const size_t L = m->L, SL = (size_t)persistent_exchange_slack();
  const size_t o_eq = m->persist ? carve((L * 3 * C + SL) * 8) : 0,
               o_er = m->persist ? carve((L * m->H * (size_t)m->nchunk * (m->hs + 2) + SL) * 8) : 0,
               o_ey = m->persist ? carve((L * C + SL) * 8) : 0,
               o_e1 = m->persist ? carve((L * C + SL) * 8) : 0,
               o_ef = m->persist ? carve((L * 4 * C + SL) * 8) : 0,
               o_e2 = m->persist ? carve((L * C + SL) * 8) : 0,
               o_ep = m->persist ? carve(16) : 0,
               o_ec = m->persist ? carve((2 * (size_t)pgrid + SL) * 8) : 0,
               o_dl = m->persist ? carve(L * sizeof(PersistLayer)) : 0;
  hipError_t e = hipMalloc(&m->ws, off);
  if (e != hipSuccess) {
    delete m;
    return fail(nullptr, NGPT_E_HIP, std::string("hipMalloc workspace: ") + hipGetErrorString(e));
  }
  char* base = static_cast<char*>(m->ws);
  m->x = (float*)(base + o_x); m->h = base + o_h; m->q = base + o_q;
  m->y = base + o_y; m->f = base + o_f; m->z = base + o_z;
  m->logits = (float*)(base + o_lg);
  m->row_b = (int32_t*)(base + o_rb); m->row_pos = (int32_t*)(base + o_rp);
  m->last_rows = (int32_t*)(base + o_lr); m->part = (float*)(base + o_part);
  m->ppart = (float*)(base + o_ppart);
  m->tok = (int32_t*)(base + o_tok);
  m->pos = (int32_t*)(base + o_pos); m->status = (int32_t*)(base + o_st);
  m->params = (SampleParams*)(base + o_prm);
  std::vector<PersistLayer> hl;
  if (m->persist) {
    m->e_qkv = (uint64_t*)(base + o_eq); m->e_rec = (uint64_t*)(base + o_er);
    m->e_y = (uint64_t*)(base + o_ey); m->e_x1 = (uint64_t*)(base + o_e1);
    m->e_f = (uint64_t*)(base + o_ef); m->e_x2 = (uint64_t*)(base + o_e2);
    m->epoch = (uint32_t*)(base + o_ep);
    m->e_cand = (uint64_t*)(base + o_ec);
    m->d_layers = (PersistLayer*)(base + o_dl);
    for (const ngpt_layer_weights& lw : m->layers)
      hl.push_back(PersistLayer{(const bf16_t*)lw.ln1_w, (const bf16_t*)lw.ln1_b,
                                (const bf16_t*)lw.attn_w, (const bf16_t*)lw.attn_b,
                                (const bf16_t*)lw.attnproj_w, (const bf16_t*)lw.attnproj_b,
                                (const bf16_t*)lw.ln2_w, (const bf16_t*)lw.ln2_b,
                                (const bf16_t*)lw.fc_w, (const bf16_t*)lw.fc_b,
                                (const bf16_t*)lw.mlpproj_w, (const bf16_t*)lw.mlpproj_b});
  }
  e = hipStreamCreateWithFlags(&m->cap, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipMemsetAsync(m->ws, 0, off, m->stream);
  SampleParams p{1.0f, 0, 1, 0};
  if (e == hipSuccess)
    e = hipMemcpyAsync(m->params, &p, sizeof(p), hipMemcpyHostToDevice, m->stream);
  if (e == hipSuccess && m->persist)
    e = hipMemcpyAsync(m->d_layers, hl.data(), hl.size() * sizeof(PersistLayer),
                       hipMemcpyHostToDevice, m->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(m->stream);
  if (e != hipSuccess) {
    std::string msg = std::string("workspace init: ") + hipGetErrorString(e);
    if (m->cap) (void)hipStreamDestroy(m->cap);
    (void)hipFree(m->ws);
    delete m;
    return fail(nullptr, NGPT_E_HIP, msg);
  }
  *out = m;
  return NGPT_OK;
}

static void drop_graph(GraphSlot& g) {
  if (g.exec) (void)hipGraphExecDestroy(g.exec);
  if (g.graph) (void)hipGraphDestroy(g.graph);
  g = GraphSlot();
}

int ngpt_destroy(ngpt_model* m) {
  if (!m) return fail(nullptr, NGPT_E_ARG, "model is NULL");
  hipError_t e = hipStreamSynchronize(m->stream);
  drop_graph(m->g_step);
  drop_graph(m->g_feed);
  if (m->cap) (void)hipStreamDestroy(m->cap);
  if (m->ws) (void)hipFree(m->ws);
  delete m;
  if (e != hipSuccess)
    return fail(nullptr, NGPT_E_HIP, std::string("destroy: ") + hipGetErrorString(e));
  return NGPT_OK;
}

int ngpt_set_wait_limit(ngpt_model* m, int32_t passes) {
  if (!m) return fail(nullptr, NGPT_E_ARG, "model is NULL");
  // a kernel argument of the one-launch decode kernel (0: its default); a
  // captured graph records the value it was captured with and is captured
  // again when it changes
  m->h_wait_limit = passes > 0 ? passes : 0;
  return NGPT_OK;
}

int ngpt_set_sampling(ngpt_model* m, float temperature, int32_t top_k, int32_t greedy) {
  if (!m) return fail(nullptr, NGPT_E_ARG, "model is NULL");
  if (!greedy && !(temperature > 0.f))
    return fail(m, NGPT_E_ARG, "temperature must be > 0 unless greedy");
  // The parameters live in device memory read by the sampler kernel; the
  // copy is ordered on the stream and waited for, so the host value can go.
  SampleParams p{temperature, top_k, greedy ? 1 : 0, 0};
  HIP_TRY(m, hipMemcpyAsync(m->params, &p, sizeof(p), hipMemcpyHostToDevice, m->stream));
  HIP_TRY(m, hipStreamSynchronize(m->stream));
  m->h_params = p;
  return NGPT_OK;
}

static int check_kv(ngpt_model* m, const ngpt_kv* kv) {
  if (!kv || !kv->k || !kv->v || !kv->lens || !kv->limit)
    return fail(m, NGPT_E_ARG, "kv has a NULL pointer");
  if (kv->batch < 1) return fail(m, NGPT_E_ARG, "kv batch < 1");
  if (kv->batch > m->cfg.max_batch) return fail(m, NGPT_E_SIZE, "kv batch > max_batch");
  if (misaligned(kv->k) || misaligned(kv->v))
    return fail(m, NGPT_E_ARG, "kv arrays must be 16-byte aligned");
  return NGPT_OK;
}

static void* layer_cache(const ngpt_model* m, void* base, int l, int kvB) {
  return static_cast<char*>(base) +
         (size_t)l * kvB * m->H * m->Tb * m->hs * m->esz;
}

int ngpt_prefill(ngpt_model* m, ngpt_kv* kv, const int32_t* ids,
                 const int32_t* lens, const int32_t* limit, int32_t B,
                 int32_t Tmax) {
  if (!m) return fail(nullptr, NGPT_E_ARG, "model is NULL");
  int rc = check_kv(m, kv);
  if (rc != NGPT_OK) return rc;
  if (!ids || !lens) return fail(m, NGPT_E_ARG, "ids or lens is NULL");
  if (B < 1 || B > kv->batch) return fail(m, NGPT_E_ARG, "B must be in [1, kv->batch]");
  RowMap map{};
  map.B = B;
  LensArgs la{};
  la.n = kv->batch;
  long total = 0;
  int maxlen = 0;
  for (int b = 0; b < B; ++b) {
    const int lb = lens[b];
    const int lim = limit ? limit[b] : m->Tb;
    if (lb < 1 || lb > m->Tb) return fail(m, NGPT_E_RANGE, "lens[b] must be in [1, block_size]");
    if (lim < lb || lim > m->Tb) return fail(m, NGPT_E_RANGE, "limit[b] must be in [lens[b], block_size]");
    if (lb > Tmax) return fail(m, NGPT_E_ARG, "lens[b] > Tmax");
    map.off[b] = (int32_t)total;
    total += lb;
    maxlen = std::max(maxlen, lb);
    la.lens[b] = lb;
    la.limit[b] = lim;
  }
  map.off[B] = (int32_t)total;
  if (total > m->cfg.max_prefill_tokens)
    return fail(m, NGPT_E_SIZE, "sum(lens) > max_prefill_tokens");
  for (int b = B; b < kv->batch; ++b) { la.lens[b] = 0; la.limit[b] = 0; }

  const int M = (int)total, C = m->C, dt = m->cfg.dtype;
  hipStream_t s = m->stream;
  m->cand_ok = false;   // the logits are about to come from this prefill
  set_lens_kernel<<<(kv->batch + 63) / 64, 64, 0, s>>>(la, kv->lens, kv->limit);
  launch_embed_prefill(dt, ids, Tmax, map, M, m->wte, m->wpe, C, m->V, m->x,
                       m->row_b, m->row_pos, m->last_rows, m->status, s);
  for (int l = 0; l < m->L; ++l) {
    const ngpt_layer_weights& w = m->layers[l];
    void* kl = layer_cache(m, kv->k, l, kv->batch);
    void* vl = layer_cache(m, kv->v, l, kv->batch);
    const LnArgs ln1{m->x, C, w.ln1_w, w.ln1_b, m->h};
    EpiArgs eq;
    eq.bias = w.attn_b; eq.out = m->q; eq.ldo = C; eq.kc = kl; eq.vc = vl;
    eq.row_b = m->row_b; eq.row_pos = m->row_pos;
    eq.C = C; eq.H = m->H; eq.hs = m->hs; eq.Tb = m->Tb;
    launch_linear(dt, EPI_QKV, nullptr, C, &ln1, w.attn_w, M, 3 * C, C, eq, s);
    launch_attn_prefill(dt, m->q, C, kl, vl, map, maxlen, m->H, m->hs, m->Tb,
                        m->y, C, m->ppart, s);
    EpiArgs ep;
    ep.bias = w.attnproj_b; ep.out = m->x; ep.ldo = C;
    launch_linear(dt, EPI_RESID, m->y, C, nullptr, w.attnproj_w, M, C, C, ep, s);
    const LnArgs ln2{m->x, C, w.ln2_w, w.ln2_b, m->h};
    EpiArgs ef;
    ef.bias = w.fc_b; ef.out = m->f; ef.ldo = 4 * C;
    launch_linear(dt, EPI_GELU, nullptr, C, &ln2, w.fc_w, M, 4 * C, C, ef, s);
    EpiArgs em;
    em.bias = w.mlpproj_b; em.out = m->x; em.ldo = C;
    launch_linear(dt, EPI_RESID, m->f, 4 * C, nullptr, w.mlpproj_w, M, C, 4 * C, em, s);
  }
  // ln_f and the tied lm_head on each sequence's last row only
  launch_layernorm(dt, m->x, C, m->last_rows, B, m->lnf_w, m->lnf_b, m->z, C, C, s);
  EpiArgs el;
  el.out = m->logits; el.ldo = m->V;
  launch_linear(dt, EPI_LOGITS, m->z, C, nullptr, m->wte, B, m->V, C, el, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(m, NGPT_E_HIP, std::string("prefill launch: ") + hipGetErrorString(e));

  m->h_lens.assign(kv->batch, 0);
  m->h_limit.assign(kv->batch, 0);
  for (int b = 0; b < B; ++b) { m->h_lens[b] = la.lens[b]; m->h_limit[b] = la.limit[b]; }
  return NGPT_OK;
}

// The one-token forward shared by the step and feed graphs.  The head node
// (sampler or feed) has already set tok/pos, advanced lens and written the
// embedding x = wte[tok] + wpe[pos] of every row.
static PersistArgs persist_args(ngpt_model* m, const ngpt_kv* kv) {
  PersistArgs a{};
  a.L = m->L; a.H = m->H; a.C = m->C; a.V = m->V; a.Tb = m->Tb;
  a.nchunk = m->nchunk;
  a.wte = (const bf16_t*)m->wte; a.wpe = (const bf16_t*)m->wpe;
  a.lnf_w = (const bf16_t*)m->lnf_w; a.lnf_b = (const bf16_t*)m->lnf_b;
  a.layers = m->d_layers;
  a.pos = m->pos;
  a.fused = 0;
  a.lens = kv->lens; a.tok = m->tok; a.next_ids = nullptr;
  a.e_cand = m->e_cand;
  a.x0 = m->x;
  a.kc = (bf16_t*)kv->k; a.vc = (bf16_t*)kv->v;
  a.layer_stride = (size_t)m->H * m->Tb * m->hs;
  a.logits = m->logits;
  a.e_qkv = m->e_qkv; a.e_rec = m->e_rec; a.e_y = m->e_y;
  a.e_x1 = m->e_x1; a.e_f = m->e_f; a.e_x2 = m->e_x2;
  a.epoch = m->epoch; a.status = m->status; a.wait_limit = m->h_wait_limit;
  return a;
}

static void enqueue_decode_forward(ngpt_model* m, const ngpt_kv* kv, hipStream_t s) {
  const int Bk = kv->batch, C = m->C, dt = m->cfg.dtype;
  if (m->persist && Bk == 1) {
    launch_decode_persistent(persist_args(m, kv), m->persist_grid, s);
    return;
  }
  for (int l = 0; l < m->L; ++l) {
    const ngpt_layer_weights& w = m->layers[l];
    void* kl = layer_cache(m, kv->k, l, Bk);
    void* vl = layer_cache(m, kv->v, l, Bk);
    const LnArgs ln1{m->x, C, w.ln1_w, w.ln1_b, m->h};
    EpiArgs eq;
    eq.bias = w.attn_b; eq.out = m->q; eq.ldo = C; eq.kc = kl; eq.vc = vl;
    eq.row_b = nullptr; eq.row_pos = m->pos;
    eq.C = C; eq.H = m->H; eq.hs = m->hs; eq.Tb = m->Tb;
    launch_linear(dt, EPI_QKV, nullptr, C, &ln1, w.attn_w, Bk, 3 * C, C, eq, s);
    const bool fused = decode_fused_proj(Bk);
    launch_attn_decode(dt, m->q, kl, vl, m->pos, Bk, m->H, m->hs, m->Tb,
                       m->part, m->y, !fused, s);
    EpiArgs ep;
    ep.bias = w.attnproj_b; ep.out = m->x; ep.ldo = C;
    if (fused)
      launch_attn_proj(dt, m->part, m->pos, m->H, m->hs, m->nchunk,
                       attn_decode_chunk_keys(), w.attnproj_w, Bk, C, ep, s);
    else
      launch_linear(dt, EPI_RESID, m->y, C, nullptr, w.attnproj_w, Bk, C, C, ep, s);
    const LnArgs ln2{m->x, C, w.ln2_w, w.ln2_b, m->h};
    EpiArgs ef;
    ef.bias = w.fc_b; ef.out = m->f; ef.ldo = 4 * C;
    launch_linear(dt, EPI_GELU, nullptr, C, &ln2, w.fc_w, Bk, 4 * C, C, ef, s);
    EpiArgs em;
    em.bias = w.mlpproj_b; em.out = m->x; em.ldo = C;
    launch_linear(dt, EPI_RESID, m->f, 4 * C, nullptr, w.mlpproj_w, Bk, C, 4 * C, em, s);
  }
  const LnArgs lnf{m->x, C, m->lnf_w, m->lnf_b, m->z};
  EpiArgs el;
  el.out = m->logits; el.ldo = m->V; el.row_pos = m->pos;
  launch_linear(dt, EPI_LOGITS, nullptr, C, &lnf, m->wte, Bk, m->V, C, el, s);
}

static SamplerArgs head_args(ngpt_model* m, const ngpt_kv* kv, int mode,
                             const void* arg_in, int32_t* arg_out) {
  SamplerArgs a;
  a.mode = mode;
  a.logits = m->logits;
  a.ld = m->V;
  a.V = m->V;
  a.uniforms = mode == SAMPLE_STEP ? static_cast<const double*>(arg_in) : nullptr;
  a.params = m->params;
  a.feed_ids = mode == FEED_STEP ? static_cast<const int32_t*>(arg_in) : nullptr;
  a.next_ids = arg_out;
  a.tok = m->tok;
  a.pos = m->pos;
  a.lens = kv->lens;
  a.limit = kv->limit;
  a.status = m->status;
  a.wte = m->wte;
  a.wpe = m->wpe;
  a.C = m->C;
  a.dtype = m->cfg.dtype;
  a.x = m->x;
  return a;
}

static int capture(ngpt_model* m, GraphSlot& g, const ngpt_kv* kv, int mode,
                   const void* arg_in, int32_t* arg_out) {
  drop_graph(g);
  hipStream_t s = m->cap;
  HIP_TRY(m, hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
  const SamplerArgs a = head_args(m, kv, mode, arg_in, arg_out);
  launch_sampler(a, kv->batch, s);
  enqueue_decode_forward(m, kv, s);
  hipError_t le = hipGetLastError();
  hipGraph_t graph = nullptr;
  hipError_t ce = hipStreamEndCapture(s, &graph);
  if (le != hipSuccess || ce != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    return fail(m, NGPT_E_HIP, std::string("decode capture: ") +
                                   hipGetErrorString(le != hipSuccess ? le : ce));
  }
  size_t nroot = 1;
  hipGraphNode_t root = nullptr;
  hipError_t e = hipGraphGetRootNodes(graph, &root, &nroot);
  if (e == hipSuccess && nroot != 1) e = hipErrorUnknown;
  hipGraphExec_t exec = nullptr;
  if (e == hipSuccess) e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return fail(m, NGPT_E_HIP, std::string("decode graph: ") + hipGetErrorString(e));
  }
  g.graph = graph; g.exec = exec; g.head = root;
  g.k = kv->k; g.v = kv->v; g.lens = kv->lens; g.limit = kv->limit;
  g.batch = kv->batch; g.arg_in = arg_in; g.arg_out = arg_out;
  g.wait_limit = m->h_wait_limit;
  g.head_args = a;
  return NGPT_OK;
}

static int run_step(ngpt_model* m, ngpt_kv* kv, GraphSlot& g, int mode,
                    const void* arg_in, int32_t* arg_out) {
  int rc = check_kv(m, kv);
  if (rc != NGPT_OK) return rc;
  if ((int)m->h_lens.size() != kv->batch)
    return fail(m, NGPT_E_ARG, "kv batch differs from the last prefill");
  bool any = false;
  for (int b = 0; b < kv->batch; ++b) any |= m->h_lens[b] < m->h_limit[b];
  if (!any) return fail(m, NGPT_E_CONTEXT, "no sequence can take another token");
  // Greedy batch-1 step after a one-launch forward: the launch picks its own
  // token from the candidates the previous one left, no head node.
  if (mode == SAMPLE_STEP && m->h_params.greedy && m->persist && kv->batch == 1 &&
      m->cand_ok) {
    PersistArgs a = persist_args(m, kv);
    a.fused = 1;
    a.next_ids = arg_out;
    launch_decode_persistent(a, m->persist_grid, m->stream);
    HIP_TRY(m, hipGetLastError());
    if (m->h_lens[0] < m->h_limit[0]) ++m->h_lens[0];
    return NGPT_OK;
  }
  const bool same_kv = g.exec && g.k == kv->k && g.v == kv->v &&
                       g.lens == kv->lens && g.limit == kv->limit &&
                       g.batch == kv->batch && g.wait_limit == m->h_wait_limit;
  if (!same_kv) {
    rc = capture(m, g, kv, mode, arg_in, arg_out);
    if (rc != NGPT_OK) return rc;
  } else if (g.arg_in != arg_in || g.arg_out != arg_out) {
    // only the head node reads caller pointers: rewrite its arguments
    g.head_args = head_args(m, kv, mode, arg_in, arg_out);
    hipKernelNodeParams p{};
    sampler_node_params(g.head_args, kv->batch, &p);
    HIP_TRY(m, hipGraphExecKernelNodeSetParams(g.exec, g.head, &p));
    g.arg_in = arg_in;
    g.arg_out = arg_out;
  }
  HIP_TRY(m, hipGraphLaunch(g.exec, m->stream));
  m->cand_ok = m->persist && kv->batch == 1;
  for (int b = 0; b < kv->batch; ++b)
    if (m->h_lens[b] < m->h_limit[b]) ++m->h_lens[b];
  return NGPT_OK;
}

int ngpt_decode_step(ngpt_model* m, ngpt_kv* kv, int32_t* next_ids,
                     const double* uniforms) {
  if (!m) return fail(nullptr, NGPT_E_ARG, "model is NULL");
  if (!next_ids) return fail(m, NGPT_E_ARG, "next_ids is NULL");
  if (!uniforms && !m->h_params.greedy)
    return fail(m, NGPT_E_ARG, "uniforms is NULL and sampling is not greedy");
  return run_step(m, kv, m->g_step, SAMPLE_STEP, uniforms, next_ids);
}

int ngpt_decode_feed(ngpt_model* m, ngpt_kv* kv, const int32_t* ids) {
  if (!m) return fail(nullptr, NGPT_E_ARG, "model is NULL");
  if (!ids) return fail(m, NGPT_E_ARG, "ids is NULL");
  return run_step(m, kv, m->g_feed, FEED_STEP, ids, nullptr);
}

int ngpt_sample(ngpt_model* m, const float* logits, int32_t ld, int32_t B,
                const double* uniforms, int32_t* next_ids) {
  if (!m) return fail(nullptr, NGPT_E_ARG, "model is NULL");
  if (!logits || !next_ids) return fail(m, NGPT_E_ARG, "logits or next_ids is NULL");
  if (ld < m->V) return fail(m, NGPT_E_ARG, "ld < vocab");
  if (B < 1) return fail(m, NGPT_E_ARG, "B < 1");
  if (B > m->cfg.max_batch) return fail(m, NGPT_E_SIZE, "B > max_batch");
  if (!uniforms && !m->h_params.greedy)
    return fail(m, NGPT_E_ARG, "uniforms is NULL and sampling is not greedy");
  SamplerArgs a;
  a.mode = SAMPLE_ONLY;
  a.logits = logits;
  a.ld = ld;
  a.V = m->V;
  a.uniforms = uniforms;
  a.params = m->params;
  a.next_ids = next_ids;
  a.status = m->status;
  launch_sampler(a, B, m->stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(m, NGPT_E_HIP, std::string("sample: ") + hipGetErrorString(e));
  return NGPT_OK;
}

int ngpt_logits(ngpt_model* m, const float** logits, int32_t* ld) {
  if (!m || !logits || !ld) return fail(m, NGPT_E_ARG, "NULL argument");
  *logits = m->logits;
  *ld = m->V;
  return NGPT_OK;
}

int ngpt_copy_logits(ngpt_model* m, float* dst, int32_t ld_dst, int32_t B) {
  if (!m || !dst) return fail(m, NGPT_E_ARG, "NULL argument");
  if (B < 1 || B > m->cfg.max_batch) return fail(m, NGPT_E_SIZE, "B out of range");
  if (ld_dst < m->V) return fail(m, NGPT_E_ARG, "ld_dst < vocab");
  HIP_TRY(m, hipMemcpy2DAsync(dst, (size_t)ld_dst * 4, m->logits, (size_t)m->V * 4,
                              (size_t)m->V * 4, B, hipMemcpyDeviceToDevice, m->stream));
  return NGPT_OK;
}

int ngpt_device_status(ngpt_model* m, int32_t* status) {
  if (!m || !status) return fail(m, NGPT_E_ARG, "NULL argument");
  int32_t v = 0;
  HIP_TRY(m, hipStreamSynchronize(m->stream));
  HIP_TRY(m, hipMemcpy(&v, m->status, sizeof(v), hipMemcpyDeviceToHost));
  clear_status_kernel<<<1, 64, 0, m->stream>>>(m->status);
  HIP_TRY(m, hipGetLastError());
  HIP_TRY(m, hipStreamSynchronize(m->stream));
  // bit 2: a one-launch decode wait gave up; bit 1: an id out of range
  *status = (v & 2) ? NGPT_E_TIMEOUT : v ? NGPT_E_DEVICE : NGPT_OK;
  return NGPT_OK;
}

}  // extern "C"
