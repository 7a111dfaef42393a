// One-launch decode step for batch 1 (bf16, head size 64, n_embd <= 768):
// argument records and host entry points of decode_persistent_kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ngpt {
typedef uint16_t bf16_t;

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
  const int32_t* limit;         // kv limit [1] (fused: lens >= limit => inactive)
  int32_t* tok;                 // fused: the chosen id ...
  int32_t* next_ids;            // ... and the caller's copy
  int32_t* hist;                // fused: token history [1][Tb] (id at p)
  uint64_t* e_cand;             // greedy candidates, 2 words per workgroup
  const float* x0;              // [C] embedding written by the head node
  bf16_t* kc;                   // cache bases and per-layer stride (elements)
  bf16_t* vc;
  size_t layer_stride;
  float* logits;                // [V]
  // exchange words (fp32 value | epoch << 32), per layer
  uint64_t *e_qkv, *e_rec, *e_y, *e_x1, *e_f, *e_x2;
  uint32_t* epoch;              // the last launch's epoch
  uint32_t ep;                  // fused: this launch's epoch (the host counts
                                // launches); otherwise the head node has
                                // already advanced *epoch and it is read
  int32_t* status;              // bit 2: a wait timed out; bit 1: bad input
  int wait_limit;                // poll passes before a wait gives up (0: default)
};

bool persistent_decode_supported(int dtype, int C, int H, int L, int Tb,
                                 int batch, int grid);
size_t persistent_lds_bytes(int C, int L);
// the largest grid the kernel supports, and how many of its workgroups one
// CU can hold at once (0 if the query fails)
int persistent_max_grid();
int persistent_blocks_per_cu(int C, int L);
// words of slack past the end of each exchange buffer (polls read ahead)
int persistent_exchange_slack();
void launch_decode_persistent(const PersistArgs& a, int grid, hipStream_t s);

// The launch grid at this shape on a device with `cus` compute units: the
// fewest workgroups (a multiple of 8) whose register slabs hold every
// phase's rows, provided that many can be resident at once; 0 if none.
int persistent_pick_grid(int dtype, int C, int H, int L, int Tb, int cus);

}  // namespace ngpt
