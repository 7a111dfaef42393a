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
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "ngpt.h"

using namespace ngpt;

namespace {

// New lens / limit of the rows of a kv batch; -1 leaves a value unchanged.
struct LensArgs {
  int32_t n;        // rows of the kv batch
  int32_t lens[NGPT_MAX_BATCH];
  int32_t limit[NGPT_MAX_BATCH];
};

__global__ void set_lens_kernel(LensArgs a, int32_t* lens, int32_t* limit) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < a.n) {
    if (a.lens[b] >= 0) lens[b] = a.lens[b];
    if (a.limit[b] >= 0) limit[b] = a.limit[b];
  }
}

// Ids of a cropped window (generate() beyond block_size): for each listed
// row, its cached tokens 1 .. Tb-1 (from the token history) followed by the
// row's new token; packed, Tb ids per row.
struct SlotList {
  int32_t n;
  int32_t slot[NGPT_MAX_BATCH];
};
__global__ void window_ids_kernel(SlotList sl, const int32_t* hist, int Tb,
                                  const int32_t* next, int32_t* out) {
  const int i = blockIdx.y, p = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= sl.n || p >= Tb) return;
  const int b = sl.slot[i];
  out[(size_t)i * Tb + p] = p + 1 < Tb ? hist[(size_t)b * Tb + p + 1] : next[b];
}

// Report and clear the kernel-side flags: bit 2 a one-launch decode wait
// gave up, bit 4 a cache write into an unmapped block of a paged cache, bit
// 1 invalid input (an id out of range, or a greedy row with no finite
// maximum).  `out` is device memory or device-writable host memory.
__global__ void read_status_kernel(int32_t* status, int32_t* out) {
  if (threadIdx.x == 0) {
    const int32_t v = status[0];
    out[0] = (v & 2) ? NGPT_E_TIMEOUT : (v & 4) ? NGPT_E_PAGE : v ? NGPT_E_DEVICE : NGPT_OK;
    status[0] = 0;
  }
}

// Block-table entries of one row of a paged cache, from a kernel argument
// (so the call needs no host staging and no wait).
constexpr int kMaxMapBlocks = (4096 + NGPT_PAGE_TOKENS - 1) / NGPT_PAGE_TOKENS;
struct PageArgs {
  int32_t count;
  int32_t pages[kMaxMapBlocks];
};
__global__ void set_pages_kernel(int32_t* dst, PageArgs a) {
  const int i = threadIdx.x;
  if (i < a.count) dst[i] = a.pages[i];
}

// Sampling parameters written on the stream from a kernel argument, so that
// setting them needs no host copy and no wait.
__global__ void set_params_kernel(SampleParams* dst, SampleParams p) {
  if (threadIdx.x == 0) *dst = p;
}

// Zero the workspace (a fill kernel rather than a memset node, so the same
// code is safe to record in a graph).
__global__ void zero_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

// The one-launch decode kernel's table of block weight pointers, written
// from kernel arguments in chunks (no host staging to keep alive).
constexpr int kTableChunk = 16;
struct LayerTableChunk {
  int32_t first, n;
  PersistLayer l[kTableChunk];
};
__global__ void set_layer_table_kernel(PersistLayer* dst, LayerTableChunk c) {
  const int i = threadIdx.x;
  if (i < c.n) dst[c.first + i] = c.l[i];
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
  int32_t* table = nullptr;
  int32_t num_pages = 0;
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
    case NGPT_E_PAGE: return "NGPT_E_PAGE";
    default: return "NGPT_E_UNKNOWN";
  }
}

std::string g_static_error;

// The workspace of ngpt_create_static(): a fixed array of the library, one
// copy per GPU at that GPU's own address.  Host code never uses the array's
// name as an address: each device's address comes from hipGetSymbolAddress
// (taken once per device, with the device current) and is what the kernels
// receive.
constexpr size_t kStaticWorkspaceBytes = NGPT_STATIC_WORKSPACE_BYTES;
struct StaticSlot {
  void* ptr = nullptr;   // device address of `scratch` on this device
  bool live = false;     // a model currently uses it
};
std::mutex g_static_mu;
std::map<int, StaticSlot> g_static_slots;

}  // namespace

// Byte offsets of the workspace regions (every region 256-byte aligned).
struct WsLayout {
  size_t x, h, q, y, f, z, logits, row_b, row_pos, last_rows, last_slot, hist,
      part, ppart, ids, tok, pos, status, params;
  // one-launch decode exchange buffers (absent: persist_shape == false)
  bool persist_shape = false;
  size_t eq, er, ey, e1, ef, e2, epoch, ecand, dlayers;
  size_t total = 0;
};

static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

struct ngpt_model {
  ngpt_config cfg{};
  int L = 0, H = 0, C = 0, hs = 0, Tb = 0, V = 0, Mmax = 0, nchunk = 0;
  size_t esz = 0;
  const void *wte = nullptr, *wpe = nullptr, *lnf_w = nullptr, *lnf_b = nullptr;
  std::vector<ngpt_layer_weights> layers;
  hipStream_t stream = nullptr;
  hipStream_t cap = nullptr;       // graph capture stream (created on first use)
  // workspace (caller-owned)
  void* ws = nullptr;
  size_t ws_bytes = 0;
  float* x = nullptr;
  void *h = nullptr, *q = nullptr, *y = nullptr, *f = nullptr, *z = nullptr;
  float* logits = nullptr;
  int32_t *row_b = nullptr, *row_pos = nullptr, *last_rows = nullptr;
  int32_t* last_slot = nullptr;  // cache row of each prefilled sequence
  int32_t* hist = nullptr;       // token history [max_batch][Tb]
  float* part = nullptr;
  float* ppart = nullptr;   // prefill attention key-split partials (one sequence)
  int32_t* d_ids = nullptr; // packed prompt ids copied from the host
  int32_t *tok = nullptr, *pos = nullptr, *status = nullptr;
  int32_t h_wait_limit = 0;        // one-launch decode poll limit (0: default)
  SampleParams* params = nullptr;
  SampleParams h_params{1.0f, 0, 1, 0};  // host copy of *params
  // pinned staging of host prompt ids: two halves, each reused only after
  // the copy that last read it has completed (created on first use)
  int32_t* pinned = nullptr;
  hipEvent_t pinned_ev[2] = {nullptr, nullptr};
  bool pinned_used[2] = {false, false};
  int pinned_half = 0;
  // one-launch batch-1 decode (see k_persist.hip)
  int persist_grid = 0;   // workgroups of the one-launch decode kernel
  bool persist = false;
  PersistLayer* d_layers = nullptr;
  uint64_t *e_qkv = nullptr, *e_rec = nullptr, *e_y = nullptr, *e_x1 = nullptr,
           *e_f = nullptr, *e_x2 = nullptr;
  uint32_t* epoch = nullptr;     // the last one-launch forward's exchange epoch
  uint32_t h_epoch = 0;          // launches of that kernel so far (== *epoch)
  uint64_t* e_cand = nullptr;   // greedy candidates left by the last launch
  bool cand_ok = false;         // the current logits came from that launch
  // the KV cache of the last prefill and the host record of its lengths
  ngpt_kv rec_kv{};
  std::vector<int32_t> h_lens, h_limit;
  int static_dev = -1;          // device whose static workspace this model uses
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
  if (c->dtype != NGPT_F32 && c->dtype != NGPT_BF16 && c->dtype != NGPT_F16)
    return bad("unknown dtype");
  if (c->dtype != NGPT_F32 && c->n_embd % 64 != 0) return bad("bf16 / fp16 need n_embd % 64 == 0");
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
  const size_t esz = c->dtype == NGPT_F32 ? 4 : 2;
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
  const size_t es = cfg->dtype == NGPT_F32 ? 4 : 2;
  return (size_t)cfg->n_layer * batch * cfg->n_head * cfg->block_size *
         (cfg->n_embd / cfg->n_head) * es;
}

size_t ngpt_kv_pool_bytes(const ngpt_config* cfg, int32_t num_pages) {
  if (check_config(cfg, nullptr) != NGPT_OK || num_pages < 1) return 0;
  const size_t es = cfg->dtype == NGPT_F32 ? 4 : 2;
  return (size_t)cfg->n_layer * num_pages * cfg->n_head * NGPT_PAGE_TOKENS *
         (cfg->n_embd / cfg->n_head) * es;
}

}  // extern "C"

// The workspace regions of a config.  Host-only: the one-launch decode
// buffers are sized for the largest grid the kernel supports, so the layout
// does not depend on the device.
static WsLayout ws_layout(const ngpt_config* cfg) {
  WsLayout o;
  const size_t Mm = std::max(cfg->max_prefill_tokens, cfg->max_batch);
  const size_t Bm = cfg->max_batch, C = cfg->n_embd;
  const size_t es = cfg->dtype == NGPT_F32 ? 4 : 2;
  const int H = cfg->n_head, hs = cfg->n_embd / cfg->n_head, Tb = cfg->block_size;
  const int nchunk = attn_decode_chunks(Tb);
  size_t off = 0;
  auto carve = [&](size_t bytes) { size_t r = off; off += align_up(bytes); return r; };
  o.x = carve(Mm * C * 4); o.h = carve(Mm * C * es); o.q = carve(Mm * C * es);
  o.y = carve(Mm * C * es); o.f = carve(Mm * 4 * C * es); o.z = carve(Bm * C * es);
  o.logits = carve(Bm * (size_t)cfg->vocab_size * 4);
  o.row_b = carve(Mm * 4); o.row_pos = carve(Mm * 4); o.last_rows = carve(Bm * 4);
  o.last_slot = carve(Bm * 4); o.hist = carve(Bm * (size_t)Tb * 4);
  o.part = carve(Bm * H * (size_t)nchunk * (hs + 2) * 4);
  o.ppart = carve((size_t)H * Tb * attn_prefill_split_chunks(Tb) * (hs + 4) * 4);
  o.ids = carve((size_t)cfg->max_prefill_tokens * 4);
  o.tok = carve(Bm * 4); o.pos = carve(Bm * 4); o.status = carve(16);
  o.params = carve(sizeof(SampleParams));
  for (int g = 64; g <= persistent_max_grid() && !o.persist_shape; g += 8)
    o.persist_shape = persistent_decode_supported(cfg->dtype, cfg->n_embd, H,
                                                  cfg->n_layer, Tb, 1, g);
  if (o.persist_shape) {
    const size_t L = cfg->n_layer, SL = (size_t)persistent_exchange_slack();
    o.eq = carve((L * 3 * C + SL) * 8);
    o.er = carve((L * H * (size_t)nchunk * (hs + 2) + SL) * 8);
    o.ey = carve((L * C + SL) * 8);
    o.e1 = carve((L * C + SL) * 8);
    o.ef = carve((L * 4 * C + SL) * 8);
    o.e2 = carve((L * C + SL) * 8);
    o.epoch = carve(16);
    o.ecand = carve((2 * (size_t)persistent_max_grid() + SL) * 8);
    o.dlayers = carve(L * sizeof(PersistLayer));
  }
  o.total = off;
  return o;
}

static int check_weights(const ngpt_config* cfg, const ngpt_weights* w) {
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
  return NGPT_OK;
}

// Build a handle over a workspace the caller (or the library's static
// array) provides.  Enqueues the zero fill and the layer-table writes; no
// allocation, no wait.
static int create_on(const ngpt_config* cfg, const ngpt_weights* w, void* ws,
                     size_t ws_bytes, void* stream, ngpt_model** out) {
  *out = nullptr;
  const WsLayout o = ws_layout(cfg);
  if (!ws) return fail(nullptr, NGPT_E_ARG, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
    return fail(nullptr, NGPT_E_ARG, "workspace must be 256-byte aligned");
  if (ws_bytes < o.total)
    return fail(nullptr, NGPT_E_SIZE, "workspace smaller than ngpt_workspace_bytes(cfg)");

  ngpt_model* m = new ngpt_model();
  m->cfg = *cfg;
  m->L = cfg->n_layer; m->H = cfg->n_head; m->C = cfg->n_embd;
  m->hs = m->C / m->H; m->Tb = cfg->block_size; m->V = cfg->vocab_size;
  m->esz = cfg->dtype == NGPT_F32 ? 4 : 2;
  m->Mmax = std::max(cfg->max_prefill_tokens, cfg->max_batch);
  m->nchunk = attn_decode_chunks(m->Tb);
  m->wte = w->wte; m->wpe = w->wpe; m->lnf_w = w->lnf_w; m->lnf_b = w->lnf_b;
  m->layers.assign(w->layers, w->layers + m->L);
  m->stream = static_cast<hipStream_t>(stream);
  m->ws = ws;
  m->ws_bytes = o.total;

  char* base = static_cast<char*>(ws);
  m->x = (float*)(base + o.x); m->h = base + o.h; m->q = base + o.q;
  m->y = base + o.y; m->f = base + o.f; m->z = base + o.z;
  m->logits = (float*)(base + o.logits);
  m->row_b = (int32_t*)(base + o.row_b); m->row_pos = (int32_t*)(base + o.row_pos);
  m->last_rows = (int32_t*)(base + o.last_rows); m->part = (float*)(base + o.part);
  m->last_slot = (int32_t*)(base + o.last_slot); m->hist = (int32_t*)(base + o.hist);
  m->ppart = (float*)(base + o.ppart);
  m->d_ids = (int32_t*)(base + o.ids);
  m->tok = (int32_t*)(base + o.tok);
  m->pos = (int32_t*)(base + o.pos); m->status = (int32_t*)(base + o.status);
  m->params = (SampleParams*)(base + o.params);

  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 0;
  const int pgrid = o.persist_shape
                        ? persistent_pick_grid(cfg->dtype, m->C, m->H, m->L, m->Tb, cus)
                        : 0;
  m->persist_grid = pgrid;
  m->persist = pgrid > 0;
  if (o.persist_shape) {
    m->e_qkv = (uint64_t*)(base + o.eq); m->e_rec = (uint64_t*)(base + o.er);
    m->e_y = (uint64_t*)(base + o.ey); m->e_x1 = (uint64_t*)(base + o.e1);
    m->e_f = (uint64_t*)(base + o.ef); m->e_x2 = (uint64_t*)(base + o.e2);
    m->epoch = (uint32_t*)(base + o.epoch);
    m->e_cand = (uint64_t*)(base + o.ecand);
    m->d_layers = (PersistLayer*)(base + o.dlayers);
  }

  hipStream_t s = m->stream;
  zero_kernel<<<1024, 256, 0, s>>>(static_cast<uint4*>(ws), o.total / 16);
  set_params_kernel<<<1, 64, 0, s>>>(m->params, m->h_params);
  if (m->persist) {
    for (int l0 = 0; l0 < m->L; l0 += kTableChunk) {
      LayerTableChunk c{};
      c.first = l0;
      c.n = std::min(kTableChunk, m->L - l0);
      for (int i = 0; i < c.n; ++i) {
        const ngpt_layer_weights& lw = m->layers[l0 + i];
        c.l[i] = PersistLayer{(const bf16_t*)lw.ln1_w, (const bf16_t*)lw.ln1_b,
                              (const bf16_t*)lw.attn_w, (const bf16_t*)lw.attn_b,
                              (const bf16_t*)lw.attnproj_w, (const bf16_t*)lw.attnproj_b,
                              (const bf16_t*)lw.ln2_w, (const bf16_t*)lw.ln2_b,
                              (const bf16_t*)lw.fc_w, (const bf16_t*)lw.fc_b,
                              (const bf16_t*)lw.mlpproj_w, (const bf16_t*)lw.mlpproj_b};
      }
      set_layer_table_kernel<<<1, 64, 0, s>>>(m->d_layers, c);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    delete m;
    return fail(nullptr, NGPT_E_HIP, std::string("workspace init: ") + hipGetErrorString(e));
  }
  *out = m;
  return NGPT_OK;
}

static void drop_graph(GraphSlot& g) {
  if (g.exec) (void)hipGraphExecDestroy(g.exec);
  if (g.graph) (void)hipGraphDestroy(g.graph);
  g = GraphSlot();
}

static int release(ngpt_model* m) {
  hipError_t e = hipStreamSynchronize(m->stream);
  if (m->static_dev >= 0) {
    std::lock_guard<std::mutex> lk(g_static_mu);
    g_static_slots[m->static_dev].live = false;
  }
  drop_graph(m->g_step);
  drop_graph(m->g_feed);
  if (m->cap) (void)hipStreamDestroy(m->cap);
  for (hipEvent_t ev : m->pinned_ev)
    if (ev) (void)hipEventDestroy(ev);
  if (m->pinned) (void)hipHostFree(m->pinned);
  delete m;
  if (e != hipSuccess)
    return fail(nullptr, NGPT_E_HIP, std::string("destroy: ") + hipGetErrorString(e));
  return NGPT_OK;
}

extern "C" {

size_t ngpt_workspace_bytes(const ngpt_config* cfg) {
  if (check_config(cfg, nullptr) != NGPT_OK) return 0;
  return ws_layout(cfg).total;
}

int ngpt_create(const ngpt_config* cfg, const ngpt_weights* w, void* workspace,
                size_t ws_bytes, void* stream, ngpt_model** out) {
  if (!out) return fail(nullptr, NGPT_E_ARG, "out is NULL");
  *out = nullptr;
  std::string why;
  int rc = check_config(cfg, &why);
  if (rc != NGPT_OK) return fail(nullptr, rc, why);
  rc = check_weights(cfg, w);
  if (rc != NGPT_OK) return rc;
  return create_on(cfg, w, workspace, ws_bytes, stream, out);
}

int ngpt_create_static(const ngpt_config* cfg, const ngpt_weights* w, void* stream,
                       ngpt_model** out) {
  if (!out) return fail(nullptr, NGPT_E_ARG, "out is NULL");
  *out = nullptr;
  std::string why;
  int rc = check_config(cfg, &why);
  if (rc != NGPT_OK) return fail(nullptr, rc, why);
  rc = check_weights(cfg, w);
  if (rc != NGPT_OK) return rc;
  if (ws_layout(cfg).total > kStaticWorkspaceBytes)
    return fail(nullptr, NGPT_E_SIZE, "config needs more workspace than the static array holds");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(nullptr, NGPT_E_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_static_mu);
  StaticSlot& slot = g_static_slots[dev];
  if (slot.live)
    return fail(nullptr, NGPT_E_ARG, "a model already uses this device's static workspace");
  if (!slot.ptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(nullptr, NGPT_E_HIP, std::string("hipGetSymbolAddress(static workspace): ") +
                                           hipGetErrorString(e));
    slot.ptr = p;
  }
  rc = create_on(cfg, w, slot.ptr, kStaticWorkspaceBytes, stream, out);
  if (rc != NGPT_OK) return rc;
  (*out)->static_dev = dev;
  slot.live = true;
  return NGPT_OK;
}

int ngpt_destroy(ngpt_model* m) {
  if (!m) return fail(nullptr, NGPT_E_ARG, "model is NULL");
  return release(m);
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
  // The parameters live in device memory read by the sampler kernel; they
  // are written by a kernel on the stream, ordered after earlier work.
  SampleParams p{temperature, top_k, greedy ? 1 : 0, 0};
  set_params_kernel<<<1, 64, 0, m->stream>>>(m->params, p);
  HIP_TRY(m, hipGetLastError());
  m->h_params = p;
  return NGPT_OK;
}

}  // extern "C"

static int check_kv(ngpt_model* m, const ngpt_kv* kv) {
  if (!kv || !kv->k || !kv->v || !kv->lens || !kv->limit)
    return fail(m, NGPT_E_ARG, "kv has a NULL pointer");
  if (kv->batch < 1) return fail(m, NGPT_E_ARG, "kv batch < 1");
  if (kv->batch > m->cfg.max_batch) return fail(m, NGPT_E_SIZE, "kv batch > max_batch");
  if (misaligned(kv->k) || misaligned(kv->v))
    return fail(m, NGPT_E_ARG, "kv arrays must be 16-byte aligned");
  if (kv->block_table && kv->num_pages < 1)
    return fail(m, NGPT_E_ARG, "a paged kv needs num_pages >= 1");
  return NGPT_OK;
}

static bool same_kv(const ngpt_kv& a, const ngpt_kv& b) {
  return a.k == b.k && a.v == b.v && a.lens == b.lens && a.limit == b.limit &&
         a.batch == b.batch && a.block_table == b.block_table &&
         (!a.block_table || a.num_pages == b.num_pages);
}

// One layer of the K or V array: [batch][H][Tb][hs] contiguous, or
// [num_pages][H][64][hs] paged.
static void* layer_cache(const ngpt_model* m, void* base, int l, const ngpt_kv* kv) {
  const size_t rows = kv->block_table ? (size_t)kv->num_pages * m->H * NGPT_PAGE_TOKENS
                                      : (size_t)kv->batch * m->H * m->Tb;
  return static_cast<char*>(base) + (size_t)l * rows * m->hs * m->esz;
}

static KvMap kv_map(const ngpt_model* m, const ngpt_kv* kv) {
  KvMap k;
  k.table = kv->block_table;
  k.nblk = (m->Tb + NGPT_PAGE_TOKENS - 1) / NGPT_PAGE_TOKENS;
  k.npages = kv->block_table ? kv->num_pages : 0;
  k.H = m->H;
  k.Tb = m->Tb;
  return k;
}

// Whether a decode step of this cache runs as the one-launch kernel (batch
// 1, contiguous cache, a supported shape).
static bool one_launch(const ngpt_model* m, const ngpt_kv* kv) {
  return m->persist && kv->batch == 1 && !kv->block_table;
}

// Which rows a launch of the prefill sequence processes, and how the host
// record and the device lens / limit change.
struct RowPlan {
  RowMap map{};
  LensArgs la{};
  int maxlen = 0;        // most new rows of one sequence
  bool reset = false;    // the kv becomes the recorded cache; other rows inactive
};

// Prompts of B sequences into kv rows `slots` (NULL: 0 .. B-1) from an empty
// cache.  With reset, every other row of the kv becomes inactive.
static int plan_prompts(ngpt_model* m, const ngpt_kv* kv, const int32_t* slots,
                        const int32_t* lens, const int32_t* limit, int32_t B,
                        int32_t Tmax, bool reset, RowPlan& pl) {
  int rc = check_kv(m, kv);
  if (rc != NGPT_OK) return rc;
  if (!lens) return fail(m, NGPT_E_ARG, "lens is NULL");
  if (B < 1 || B > kv->batch) return fail(m, NGPT_E_ARG, "B must be in [1, kv->batch]");
  pl.map.B = B;
  pl.la.n = kv->batch;
  pl.reset = reset;
  for (int b = 0; b < kv->batch; ++b) {
    pl.la.lens[b] = reset ? 0 : -1;
    pl.la.limit[b] = reset ? 0 : -1;
  }
  std::vector<char> seen(kv->batch, 0);
  long total = 0;
  for (int b = 0; b < B; ++b) {
    const int sl = slots ? slots[b] : b;
    if (sl < 0 || sl >= kv->batch) return fail(m, NGPT_E_RANGE, "slot outside [0, kv->batch)");
    if (seen[sl]) return fail(m, NGPT_E_ARG, "a slot is listed twice");
    seen[sl] = 1;
    const int lb = lens[b];
    const int lim = limit ? limit[b] : m->Tb;
    if (lb < 1 || lb > m->Tb) return fail(m, NGPT_E_RANGE, "lens[b] must be in [1, block_size]");
    if (lim < lb || lim > m->Tb) return fail(m, NGPT_E_RANGE, "limit[b] must be in [lens[b], block_size]");
    if (lb > Tmax) return fail(m, NGPT_E_ARG, "lens[b] > Tmax");
    pl.map.off[b] = (int32_t)total;
    pl.map.slot[b] = sl;
    pl.map.past[b] = 0;
    total += lb;
    pl.maxlen = std::max(pl.maxlen, lb);
    pl.la.lens[sl] = lb;
    pl.la.limit[sl] = lim;
  }
  pl.map.off[B] = (int32_t)total;
  if (total > m->cfg.max_prefill_tokens)
    return fail(m, NGPT_E_SIZE, "sum(lens) > max_prefill_tokens");
  return NGPT_OK;
}

// counts[b] new tokens appended to live rows slots[b] of the recorded cache.
static int plan_extend(ngpt_model* m, const ngpt_kv* kv, const int32_t* slots,
                       const int32_t* counts, int32_t n, int32_t Tmax, RowPlan& pl) {
  int rc = check_kv(m, kv);
  if (rc != NGPT_OK) return rc;
  if (m->h_lens.empty() || !same_kv(*kv, m->rec_kv))
    return fail(m, NGPT_E_ARG, "kv is not the cache of the last prefill on this model");
  if (!slots || !counts) return fail(m, NGPT_E_ARG, "slots or counts is NULL");
  if (n < 1 || n > kv->batch) return fail(m, NGPT_E_ARG, "n must be in [1, kv->batch]");
  pl.map.B = n;
  pl.la.n = kv->batch;
  for (int b = 0; b < kv->batch; ++b) pl.la.lens[b] = pl.la.limit[b] = -1;
  std::vector<char> seen(kv->batch, 0);
  long total = 0;
  for (int b = 0; b < n; ++b) {
    const int sl = slots[b];
    if (sl < 0 || sl >= kv->batch) return fail(m, NGPT_E_RANGE, "slot outside [0, kv->batch)");
    if (seen[sl]) return fail(m, NGPT_E_ARG, "a slot is listed twice");
    seen[sl] = 1;
    const int c = counts[b];
    if (c < 1 || c > Tmax) return fail(m, NGPT_E_RANGE, "counts[b] must be in [1, Tmax]");
    if (m->h_lens[sl] + c > m->h_limit[sl])
      return fail(m, NGPT_E_CONTEXT, "the row cannot take that many tokens (limit)");
    pl.map.off[b] = (int32_t)total;
    pl.map.slot[b] = sl;
    pl.map.past[b] = m->h_lens[sl];
    total += c;
    pl.maxlen = std::max(pl.maxlen, c);
    pl.la.lens[sl] = m->h_lens[sl] + c;
  }
  pl.map.off[n] = (int32_t)total;
  if (total > m->cfg.max_prefill_tokens)
    return fail(m, NGPT_E_SIZE, "sum(counts) > max_prefill_tokens");
  return NGPT_OK;
}

// Every id of the plan's sequences on the host, then a packed asynchronous
// copy through the pinned staging into the workspace.
static int stage_host_ids(ngpt_model* m, const RowPlan& pl, const int32_t* ids, int Tmax) {
  const RowMap& map = pl.map;
  for (int b = 0; b < map.B; ++b) {
    const int cnt = map.off[b + 1] - map.off[b];
    for (int p = 0; p < cnt; ++p) {
      const int32_t id = ids[(size_t)b * Tmax + p];
      if (id < 0 || id >= m->V)
        return fail(m, NGPT_E_RANGE, "token id outside [0, vocab_size)");
    }
  }
  const size_t half = (size_t)m->cfg.max_prefill_tokens;
  if (!m->pinned) {
    HIP_TRY(m, hipHostMalloc(reinterpret_cast<void**>(&m->pinned), 2 * half * sizeof(int32_t),
                             hipHostMallocDefault));
    HIP_TRY(m, hipEventCreateWithFlags(&m->pinned_ev[0], hipEventDisableTiming));
    HIP_TRY(m, hipEventCreateWithFlags(&m->pinned_ev[1], hipEventDisableTiming));
  }
  const int hf = m->pinned_half;
  if (m->pinned_used[hf]) HIP_TRY(m, hipEventSynchronize(m->pinned_ev[hf]));
  int32_t* stage = m->pinned + hf * half;
  for (int b = 0; b < map.B; ++b)
    memcpy(stage + map.off[b], ids + (size_t)b * Tmax,
           sizeof(int32_t) * (map.off[b + 1] - map.off[b]));
  const int M = map.off[map.B];
  HIP_TRY(m, hipMemcpyAsync(m->d_ids, stage, sizeof(int32_t) * M, hipMemcpyHostToDevice,
                            m->stream));
  HIP_TRY(m, hipEventRecord(m->pinned_ev[hf], m->stream));
  m->pinned_used[hf] = true;
  m->pinned_half = hf ^ 1;
  return NGPT_OK;
}

// The blocks of the prefill launch sequence over the plan's rows: x holds
// the final residual stream of every row afterwards.  ids: device; Tmax > 0
// gives the [B][Tmax] right-padded layout, Tmax == 0 the packed layout.
static void enqueue_blocks(ngpt_model* m, ngpt_kv* kv, const int32_t* ids, int Tmax,
                           const RowPlan& pl) {
  const RowMap& map = pl.map;
  const int M = map.off[map.B], C = m->C, dt = m->cfg.dtype;
  hipStream_t s = m->stream;
  m->cand_ok = false;   // the logits are about to come from this prefill
  set_lens_kernel<<<(kv->batch + 63) / 64, 64, 0, s>>>(pl.la, kv->lens, kv->limit);
  launch_embed_prefill(dt, ids, Tmax, map, M, m->wte, m->wpe, C, m->V, m->x,
                       m->row_b, m->row_pos, m->last_rows, m->last_slot, m->hist,
                       m->Tb, m->status, s);
  const KvMap kvm = kv_map(m, kv);
  for (int l = 0; l < m->L; ++l) {
    const ngpt_layer_weights& w = m->layers[l];
    void* kl = layer_cache(m, kv->k, l, kv);
    void* vl = layer_cache(m, kv->v, l, kv);
    const LnArgs ln1{m->x, C, w.ln1_w, w.ln1_b, m->h};
    EpiArgs eq;
    eq.bias = w.attn_b; eq.out = m->q; eq.ldo = C; eq.kc = kl; eq.vc = vl;
    eq.row_b = m->row_b; eq.row_pos = m->row_pos;
    eq.kv = kvm; eq.status = m->status;
    eq.C = C; eq.H = m->H; eq.hs = m->hs; eq.Tb = m->Tb;
    launch_linear(dt, EPI_QKV, nullptr, C, &ln1, w.attn_w, M, 3 * C, C, eq, s);
    launch_attn_prefill(dt, m->q, C, kl, vl, kvm, map, pl.maxlen, m->H, m->hs, m->Tb,
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
}

// Record the plan's lens / limit on the host.
static void record_plan(ngpt_model* m, const ngpt_kv* kv, const RowPlan& pl) {
  if (pl.reset || m->h_lens.empty() || !same_kv(*kv, m->rec_kv)) {
    m->rec_kv = *kv;
    m->h_lens.assign(kv->batch, 0);
    m->h_limit.assign(kv->batch, 0);
  }
  for (int b = 0; b < kv->batch; ++b) {
    if (pl.la.lens[b] >= 0) m->h_lens[b] = pl.la.lens[b];
    if (pl.la.limit[b] >= 0) m->h_limit[b] = pl.la.limit[b];
  }
}

// The prefill launch sequence: the blocks, then ln_f and the tied lm_head on
// each sequence's last new row, into the logits row of its slot.
static int enqueue_rows(ngpt_model* m, ngpt_kv* kv, const int32_t* ids, int Tmax,
                        const RowPlan& pl) {
  const int C = m->C, dt = m->cfg.dtype, B = pl.map.B;
  hipStream_t s = m->stream;
  enqueue_blocks(m, kv, ids, Tmax, pl);
  launch_layernorm(dt, m->x, C, m->last_rows, B, m->lnf_w, m->lnf_b, m->z, C, C, s);
  EpiArgs el;
  el.out = m->logits; el.ldo = m->V; el.row_b = m->last_slot;
  launch_linear(dt, EPI_LOGITS, m->z, C, nullptr, m->wte, B, m->V, C, el, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(m, NGPT_E_HIP, std::string("prefill launch: ") + hipGetErrorString(e));
  record_plan(m, kv, pl);
  return NGPT_OK;
}

extern "C" {

int ngpt_prefill(ngpt_model* m, ngpt_kv* kv, const int32_t* ids,
                 const int32_t* lens, const int32_t* limit, int32_t B,
                 int32_t Tmax) {
  if (!m) return fail(nullptr, NGPT_E_ARG, "model is NULL");
  if (!ids) return fail(m, NGPT_E_ARG, "ids is NULL");
  RowPlan pl;
  int rc = plan_prompts(m, kv, nullptr, lens, limit, B, Tmax, true, pl);
  if (rc == NGPT_OK) rc = stage_host_ids(m, pl, ids, Tmax);
  if (rc != NGPT_OK) return rc;
  return enqueue_rows(m, kv, m->d_ids, 0, pl);
}

int ngpt_prefill_device(ngpt_model* m, ngpt_kv* kv, const int32_t* ids,
                        const int32_t* lens, const int32_t* limit, int32_t B,
                        int32_t Tmax) {
  if (!m) return fail(nullptr, NGPT_E_ARG, "model is NULL");
  if (!ids) return fail(m, NGPT_E_ARG, "ids is NULL");
  if (Tmax < 1) return fail(m, NGPT_E_ARG, "Tmax must be >= 1");
  RowPlan pl;
  int rc = plan_prompts(m, kv, nullptr, lens, limit, B, Tmax, true, pl);
  if (rc != NGPT_OK) return rc;
  return enqueue_rows(m, kv, ids, Tmax, pl);
}

int ngpt_prefill_slots(ngpt_model* m, ngpt_kv* kv, const int32_t* slots,
                       const int32_t* ids, const int32_t* lens, const int32_t* limit,
                       int32_t n, int32_t Tmax) {
  if (!m) return fail(nullptr, NGPT_E_ARG, "model is NULL");
  if (!ids || !slots) return fail(m, NGPT_E_ARG, "ids or slots is NULL");
  // a cache other than the recorded one starts with every row inactive
  const bool fresh = m->h_lens.empty() || !kv || !same_kv(*kv, m->rec_kv);
  RowPlan pl;
  int rc = plan_prompts(m, kv, slots, lens, limit, n, Tmax, fresh, pl);
  if (rc == NGPT_OK) rc = stage_host_ids(m, pl, ids, Tmax);
  if (rc != NGPT_OK) return rc;
  return enqueue_rows(m, kv, m->d_ids, 0, pl);
}

int ngpt_extend(ngpt_model* m, ngpt_kv* kv, const int32_t* slots, const int32_t* ids,
                const int32_t* counts, int32_t n, int32_t Tmax) {
  if (!m) return fail(nullptr, NGPT_E_ARG, "model is NULL");
  if (!ids) return fail(m, NGPT_E_ARG, "ids is NULL");
  RowPlan pl;
  int rc = plan_extend(m, kv, slots, counts, n, Tmax, pl);
  if (rc == NGPT_OK) rc = stage_host_ids(m, pl, ids, Tmax);
  if (rc != NGPT_OK) return rc;
  return enqueue_rows(m, kv, m->d_ids, 0, pl);
}

int ngpt_eval_loss(ngpt_model* m, ngpt_kv* kv, const int32_t* ids, const int32_t* lens,
                   int32_t B, int32_t Tmax, float* logits, float* losses, float* mean_loss) {
  if (!m) return fail(nullptr, NGPT_E_ARG, "model is NULL");
  if (!ids || !logits || !losses || !mean_loss)
    return fail(m, NGPT_E_ARG, "ids, logits, losses or mean_loss is NULL");
  RowPlan pl;
  int rc = plan_prompts(m, kv, nullptr, lens, nullptr, B, Tmax, true, pl);
  if (rc == NGPT_OK) rc = stage_host_ids(m, pl, ids, Tmax);
  if (rc != NGPT_OK) return rc;
  const int M = pl.map.off[B], C = m->C, dt = m->cfg.dtype;
  hipStream_t s = m->stream;
  m->cand_ok = false;
  enqueue_blocks(m, kv, m->d_ids, 0, pl);
  // ln_f and the tied lm_head on every row (the h rows hold M x C)
  launch_layernorm(dt, m->x, C, nullptr, M, m->lnf_w, m->lnf_b, m->h, C, C, s);
  EpiArgs el;
  el.out = logits; el.ldo = m->V;
  launch_linear(dt, EPI_LOGITS, m->h, C, nullptr, m->wte, M, m->V, C, el, s);
  launch_cross_entropy(logits, m->V, m->V, M, M - B, m->d_ids, m->row_b, m->last_rows,
                       losses, mean_loss, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(m, NGPT_E_HIP, std::string("eval launch: ") + hipGetErrorString(e));
  // the cache holds the sequences, but the model's own logits rows were not
  // refreshed: a decode step needs a prefill first
  m->h_lens.clear();
  m->h_limit.clear();
  return NGPT_OK;
}

int ngpt_retire(ngpt_model* m, ngpt_kv* kv, const int32_t* slots, int32_t n) {
  if (!m) return fail(nullptr, NGPT_E_ARG, "model is NULL");
  int rc = check_kv(m, kv);
  if (rc != NGPT_OK) return rc;
  if (m->h_lens.empty() || !same_kv(*kv, m->rec_kv))
    return fail(m, NGPT_E_ARG, "kv is not the cache of the last prefill on this model");
  if (!slots || n < 1 || n > kv->batch) return fail(m, NGPT_E_ARG, "slots / n");
  LensArgs la{};
  la.n = kv->batch;
  for (int b = 0; b < kv->batch; ++b) la.lens[b] = la.limit[b] = -1;
  for (int i = 0; i < n; ++i) {
    const int sl = slots[i];
    if (sl < 0 || sl >= kv->batch) return fail(m, NGPT_E_RANGE, "slot outside [0, kv->batch)");
    la.limit[sl] = m->h_lens[sl];   // no further tokens; the cache is kept
  }
  set_lens_kernel<<<(kv->batch + 63) / 64, 64, 0, m->stream>>>(la, kv->lens, kv->limit);
  HIP_TRY(m, hipGetLastError());
  for (int b = 0; b < kv->batch; ++b)
    if (la.limit[b] >= 0) m->h_limit[b] = la.limit[b];
  return NGPT_OK;
}

int ngpt_kv_map(ngpt_model* m, ngpt_kv* kv, int32_t slot, int32_t first_block,
                int32_t count, const int32_t* pages) {
  if (!m) return fail(nullptr, NGPT_E_ARG, "model is NULL");
  int rc = check_kv(m, kv);
  if (rc != NGPT_OK) return rc;
  if (!kv->block_table) return fail(m, NGPT_E_ARG, "kv is not paged (block_table is NULL)");
  if (!pages) return fail(m, NGPT_E_ARG, "pages is NULL");
  const int nblk = (m->Tb + NGPT_PAGE_TOKENS - 1) / NGPT_PAGE_TOKENS;
  if (slot < 0 || slot >= kv->batch) return fail(m, NGPT_E_RANGE, "slot outside [0, kv->batch)");
  if (first_block < 0 || count < 1 || first_block + count > nblk)
    return fail(m, NGPT_E_RANGE, "blocks outside [0, ceil(block_size / 64))");
  PageArgs a{};
  a.count = count;
  for (int i = 0; i < count; ++i) {
    if (pages[i] < -1 || pages[i] >= kv->num_pages)
      return fail(m, NGPT_E_RANGE, "page id outside [-1, num_pages)");
    a.pages[i] = pages[i];
  }
  set_pages_kernel<<<1, kMaxMapBlocks, 0, m->stream>>>(
      kv->block_table + (size_t)slot * nblk + first_block, a);
  HIP_TRY(m, hipGetLastError());
  return NGPT_OK;
}

int ngpt_slide(ngpt_model* m, ngpt_kv* kv, const int32_t* slots, int32_t n,
               const int32_t* next_ids) {
  if (!m) return fail(nullptr, NGPT_E_ARG, "model is NULL");
  int rc = check_kv(m, kv);
  if (rc != NGPT_OK) return rc;
  if (m->h_lens.empty() || !same_kv(*kv, m->rec_kv))
    return fail(m, NGPT_E_ARG, "kv is not the cache of the last prefill on this model");
  if (!slots || !next_ids || n < 1 || n > kv->batch) return fail(m, NGPT_E_ARG, "slots / ids / n");
  if ((long)n * m->Tb > m->cfg.max_prefill_tokens)
    return fail(m, NGPT_E_SIZE, "n * block_size > max_prefill_tokens");
  RowPlan pl;
  pl.map.B = n;
  pl.la.n = kv->batch;
  for (int b = 0; b < kv->batch; ++b) pl.la.lens[b] = pl.la.limit[b] = -1;
  SlotList sl{};
  sl.n = n;
  std::vector<char> seen(kv->batch, 0);
  for (int i = 0; i < n; ++i) {
    const int b = slots[i];
    if (b < 0 || b >= kv->batch) return fail(m, NGPT_E_RANGE, "slot outside [0, kv->batch)");
    if (seen[b]) return fail(m, NGPT_E_ARG, "a slot is listed twice");
    seen[b] = 1;
    if (m->h_lens[b] != m->Tb)
      return fail(m, NGPT_E_ARG, "slide needs a row whose cache holds block_size positions");
    sl.slot[i] = b;
    pl.map.off[i] = i * m->Tb;
    pl.map.slot[i] = b;
    pl.map.past[i] = 0;
    pl.la.lens[b] = m->Tb;
  }
  pl.map.off[n] = n * m->Tb;
  pl.maxlen = m->Tb;
  const dim3 g((m->Tb + 255) / 256, n);
  window_ids_kernel<<<g, 256, 0, m->stream>>>(sl, m->hist, m->Tb, next_ids, m->d_ids);
  HIP_TRY(m, hipGetLastError());
  return enqueue_rows(m, kv, m->d_ids, 0, pl);
}

}  // extern "C"

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
  a.lens = kv->lens; a.limit = kv->limit; a.tok = m->tok; a.next_ids = nullptr;
  a.e_cand = m->e_cand;
  a.x0 = m->x;
  a.kc = (bf16_t*)kv->k; a.vc = (bf16_t*)kv->v;
  a.layer_stride = (size_t)m->H * m->Tb * m->hs;
  a.logits = m->logits;
  a.e_qkv = m->e_qkv; a.e_rec = m->e_rec; a.e_y = m->e_y;
  a.e_x1 = m->e_x1; a.e_f = m->e_f; a.e_x2 = m->e_x2;
  a.epoch = m->epoch; a.status = m->status;
  a.hist = m->hist;
  a.wait_limit = m->h_wait_limit;
  return a;
}

static void enqueue_decode_forward(ngpt_model* m, const ngpt_kv* kv, hipStream_t s) {
  const int Bk = kv->batch, C = m->C, dt = m->cfg.dtype;
  if (one_launch(m, kv)) {
    launch_decode_persistent(persist_args(m, kv), m->persist_grid, s);
    return;
  }
  const KvMap kvm = kv_map(m, kv);
  for (int l = 0; l < m->L; ++l) {
    const ngpt_layer_weights& w = m->layers[l];
    void* kl = layer_cache(m, kv->k, l, kv);
    void* vl = layer_cache(m, kv->v, l, kv);
    const LnArgs ln1{m->x, C, w.ln1_w, w.ln1_b, m->h};
    EpiArgs eq;
    eq.bias = w.attn_b; eq.out = m->q; eq.ldo = C; eq.kc = kl; eq.vc = vl;
    eq.row_b = nullptr; eq.row_pos = m->pos;
    eq.kv = kvm; eq.status = m->status;
    eq.C = C; eq.H = m->H; eq.hs = m->hs; eq.Tb = m->Tb;
    launch_linear(dt, EPI_QKV, nullptr, C, &ln1, w.attn_w, Bk, 3 * C, C, eq, s);
    const bool fused = decode_fused_proj(Bk);
    launch_attn_decode(dt, m->q, kl, vl, kvm, m->pos, Bk, m->H, m->hs, m->Tb,
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
  a.hist = m->hist;
  a.Tb = m->Tb;
  a.wte = m->wte;
  a.wpe = m->wpe;
  a.C = m->C;
  a.dtype = m->cfg.dtype;
  a.x = m->x;
  a.epoch = one_launch(m, kv) ? m->epoch : nullptr;
  return a;
}

static int capture(ngpt_model* m, GraphSlot& g, const ngpt_kv* kv, int mode,
                   const void* arg_in, int32_t* arg_out) {
  drop_graph(g);
  if (!m->cap) HIP_TRY(m, hipStreamCreateWithFlags(&m->cap, hipStreamNonBlocking));
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
  g.table = kv->block_table; g.num_pages = kv->num_pages;
  g.batch = kv->batch; g.arg_in = arg_in; g.arg_out = arg_out;
  g.wait_limit = m->h_wait_limit;
  g.head_args = a;
  return NGPT_OK;
}

static int run_step(ngpt_model* m, ngpt_kv* kv, GraphSlot& g, int mode,
                    const void* arg_in, int32_t* arg_out) {
  int rc = check_kv(m, kv);
  if (rc != NGPT_OK) return rc;
  // the host record of lens / limit and the greedy candidates belong to the
  // cache of the last prefill
  if (m->h_lens.empty() || !same_kv(*kv, m->rec_kv))
    return fail(m, NGPT_E_ARG, "kv is not the cache of the last prefill on this model");
  bool any = false;
  for (int b = 0; b < kv->batch; ++b) any |= m->h_lens[b] < m->h_limit[b];
  if (!any) return fail(m, NGPT_E_CONTEXT, "no sequence can take another token");
  // Greedy batch-1 step after a one-launch forward: the launch picks its own
  // token from the candidates the previous one left, no head node.
  if (mode == SAMPLE_STEP && m->h_params.greedy && one_launch(m, kv) && m->cand_ok) {
    PersistArgs a = persist_args(m, kv);
    a.fused = 1;
    a.ep = ++m->h_epoch;
    a.next_ids = arg_out;
    launch_decode_persistent(a, m->persist_grid, m->stream);
    HIP_TRY(m, hipGetLastError());
    if (m->h_lens[0] < m->h_limit[0]) ++m->h_lens[0];
    return NGPT_OK;
  }
  const bool same = g.exec && g.k == kv->k && g.v == kv->v &&
                    g.lens == kv->lens && g.limit == kv->limit &&
                    g.table == kv->block_table && g.num_pages == kv->num_pages &&
                    g.batch == kv->batch && g.wait_limit == m->h_wait_limit;
  if (!same) {
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
  m->cand_ok = one_launch(m, kv);
  if (m->cand_ok) ++m->h_epoch;   // the head node advanced the word
  for (int b = 0; b < kv->batch; ++b)
    if (m->h_lens[b] < m->h_limit[b]) ++m->h_lens[b];
  return NGPT_OK;
}

extern "C" {

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
  read_status_kernel<<<1, 64, 0, m->stream>>>(m->status, status);
  HIP_TRY(m, hipGetLastError());
  return NGPT_OK;
}

}  // extern "C"
