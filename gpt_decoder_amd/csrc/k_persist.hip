// One-launch decode step for a single sequence (batch 1, bf16, head size
// 64): the whole one-token forward of every block plus ln_f and the tied
// lm_head, in one persistent kernel with one workgroup per CU.
//
// The arithmetic is the same as the per-layer kernels' (pre-LN block of the
// architecture analysis "nanoGPT 架构分析", section 4.1; KV-cached attention of
// the serving page "原生 nanoGPT 模型服务首选", KV-cache section: the new query
// attends to every cached key and itself).  What changes is how the
// dependent phases of one step meet:
//
//   per block: A  LN1 + c_attn rows (q, k, v; k/v also appended to the cache)
//              B  attention: a work item is up to four 32-key chunks of one
//                 head (one per compute wavefront); item 0 of each head
//                 merges the items' records into y
//              C  c_proj rows + residual      -> x1
//              D  LN2 + c_fc rows + GELU      -> f
//              E  MLP c_proj rows + residual  -> x2
//   then:      ln_f + lm_head rows (fp32 logits)
//
// A workgroup is four compute wavefronts and one sync wavefront.  Weight
// rows and cached K/V do not depend on the step's data, so the compute
// wavefronts issue their loads two or three phases before they are used.
// Vector loads of one wavefront complete in issue order, so the waiting for
// inputs is left to the sync wavefront, which issues no weight loads: its
// polls return as soon as the data is there.
//
// Phase outputs are exchanged as 64-bit words: fp32 value in the low half,
// the launch's epoch in the high half, stored and loaded with device-scope
// relaxed atomics (cache-bypassing; no cache-wide fences).  A consumer
// accepts a word only when it carries the current epoch, so a word is its
// own ready flag.  Every wait is bounded: on timeout the kernel sets a status
// bit and leaves, and every other workgroup then times out too.
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace ngpt {

namespace {

constexpr int kCompute = 4;                 // compute wavefronts
constexpr int kThreads = 64 * (kCompute + 1);
constexpr int kSyncWave = kCompute;
constexpr int kSpinLimit = 1 << 20;
constexpr float kLog2eP = 1.4426950408889634f;
constexpr int kHs = 64;          // head size
constexpr int kChunk = 32;       // keys per attention chunk (one wavefront)
constexpr int kRec = kHs + 2;    // record: m, l, o[64]

__device__ __forceinline__ void tag_store(uint64_t* p, float v, uint32_t ep) {
  const uint64_t w = (static_cast<uint64_t>(ep) << 32) | __float_as_uint(v);
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t tag_load(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Called by the whole sync wavefront: wait until src[0..n) all carry epoch
// ep and copy the values to dst (LDS).  n <= 64 * NJ; the words up to
// src[64 * NJ) are read too (the exchange buffers carry that much slack) and
// ignored.  Every pass issues all NJ loads before inspecting any, and copies
// every word that carries ep (a word does not change once tagged, so copying
// it again is harmless); the wait ends on the first pass with nothing
// missing.  No per-word bookkeeping is carried between passes.  False after
// kSpinLimit passes (status bit 2).
template <int NJ>
__device__ __forceinline__ bool sync_wave_wait(const uint64_t* src, int n,
                                               uint32_t ep, float* dst,
                                               int32_t* status) {
  const int lane = threadIdx.x & 63;
  for (int spin = 0;; ++spin) {
    uint64_t v[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) v[j] = tag_load(src + lane + 64 * j);
    bool miss = false;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const bool in = lane + 64 * j < n;
      const bool got = static_cast<uint32_t>(v[j] >> 32) == ep;
      if (in && got) dst[lane + 64 * j] = __uint_as_float(static_cast<uint32_t>(v[j]));
      miss |= in && !got;
    }
    if (!__any(miss)) return true;
    if (spin >= kSpinLimit) {
      if (lane == 0) atomicOr(status, 2);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// The waits of one launch, by the size of what they read; each picks the
// smallest load count that covers n.  Reads past n stay below 1024 words,
// the exchange buffers' slack.
enum WaitKind { kWaitHead, kWaitRec, kWaitC, kWait4C };

template <int KIND>
__device__ __forceinline__ bool sync_wave_wait_n(const uint64_t* src, int n,
                                                 uint32_t ep, float* dst,
                                                 int32_t* status) {
  if constexpr (KIND == kWaitHead) {           // n == 64
    return sync_wave_wait<1>(src, n, ep, dst, status);
  } else if constexpr (KIND == kWaitRec) {     // n <= 512
    if (n <= 128) return sync_wave_wait<2>(src, n, ep, dst, status);
    if (n <= 256) return sync_wave_wait<4>(src, n, ep, dst, status);
    return sync_wave_wait<8>(src, n, ep, dst, status);
  } else if constexpr (KIND == kWaitC) {       // 64 <= n <= 768
    if (n <= 256) return sync_wave_wait<4>(src, n, ep, dst, status);
    if (n <= 512) return sync_wave_wait<8>(src, n, ep, dst, status);
    return sync_wave_wait<12>(src, n, ep, dst, status);
  } else {                                     // 256 <= n <= 3072
    if (n <= 1024) return sync_wave_wait<16>(src, n, ep, dst, status);
    if (n <= 2048) return sync_wave_wait<32>(src, n, ep, dst, status);
    return sync_wave_wait<48>(src, n, ep, dst, status);
  }
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i <= kCompute; ++i) t += red[i];
  return t;
}

// out = bf16-rounded LN(x) over C features (two-pass fp32 statistics).
__device__ void block_layernorm(const float* x, float* out, int C,
                                const bf16_t* w, const bf16_t* b, float* red) {
  float s = 0.f;
  for (int i = threadIdx.x; i < C; i += kThreads) s += x[i];
  const float mean = block_sum(s, red) / (float)C;
  float q = 0.f;
  for (int i = threadIdx.x; i < C; i += kThreads) {
    const float d = x[i] - mean;
    q += d * d;
  }
  const float rstd = 1.0f / sqrtf(block_sum(q, red) / (float)C + 1e-5f);
  for (int i = threadIdx.x; i < C; i += kThreads) {
    float y = (x[i] - mean) * rstd * to_f32(w[i]);
    if (b) y += to_f32(b[i]);
    out[i] = to_f32(f32_to_bf16(y));
  }
  __syncthreads();
}

// Weight rows of one phase held in registers of the compute wavefronts:
// wavefront v owns rows r0 + v + 4i (i < RPW) of [r0, r1); lane l holds
// K-elements j*512 + 8l .. +7 of each row (chunk j < NCH).
template <int RPW, int NCH>
struct RowSlab {
  uint4 w[RPW][NCH];

  __device__ __forceinline__ void load(const bf16_t* W, int K, int r0, int r1) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int r = r0 + wave + kCompute * i;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int k = j * 512 + lane * 8;
        w[i][j] = (r < r1 && k < K)
                      ? *reinterpret_cast<const uint4*>(W + (size_t)r * K + k)
                      : make_uint4(0, 0, 0, 0);
      }
    }
  }

  // Dot products with the LDS vector a[K]; calls f(row, value) once per row
  // of this wavefront (from one lane).
  template <class F>
  __device__ __forceinline__ void dots(const float* a, int K, int r0, int r1,
                                       F&& f) const {
    constexpr int LG = (RPW == 1) ? 0 : (RPW == 2) ? 1 : (RPW == 4) ? 2 : 3;
    static_assert((1 << LG) == RPW, "RPW must be 1, 2, 4 or 8");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float acc[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int k = j * 512 + lane * 8;
      if (k < K) {
        const float4 a0 = *reinterpret_cast<const float4*>(a + k);
        const float4 a1 = *reinterpret_cast<const float4*>(a + k + 4);
        const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          float wf[8];
          bf16x8_to_f32(w[i][j], wf);
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[i] = fmaf(av[q], wf[q], acc[i]);
        }
      }
    }
    // multi-value wavefront reduction: value i ends in lane i << (6 - LG)
#pragma unroll
    for (int st = 0; st < LG; ++st) {
      const int o = 32 >> st;
      const int cnt = RPW >> st;
      const bool hi = (lane & o) != 0;
#pragma unroll
      for (int i = 0; i < cnt / 2; ++i) {
        const float send = hi ? acc[i] : acc[i + cnt / 2];
        const float keep = hi ? acc[i + cnt / 2] : acc[i];
        acc[i] = keep + __shfl_xor(send, o, 64);
      }
    }
    float r = acc[0];
#pragma unroll
    for (int o = 32 >> LG; o > 0; o >>= 1) r += __shfl_xor(r, o, 64);
    if ((lane & ((1 << (6 - LG)) - 1)) == 0) {
      const int i = lane >> (6 - LG);
      const int row = r0 + wave + kCompute * i;
      if (row < r1) f(row, r);
    }
  }
};

// Cached K/V of one wavefront's 32-key chunk: 4 passes of 8 keys, 8 lanes
// per key (8 dims each).  Keys at or past the new position p are not loaded.
constexpr int kPasses = kChunk / 8;
struct KvSlab {
  uint4 k[kPasses], v[kPasses];

  __device__ __forceinline__ void load(const bf16_t* kb, const bf16_t* vb,
                                       int key0, int p) {
    const int lane = threadIdx.x & 63, sub = lane & 7, kgrp = lane >> 3;
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
      const int u = key0 + ps * 8 + kgrp;
      const bool cached = key0 >= 0 && u < p;
      k[ps] = cached ? *reinterpret_cast<const uint4*>(kb + (size_t)u * kHs + sub * 8)
                     : make_uint4(0, 0, 0, 0);
      v[ps] = cached ? *reinterpret_cast<const uint4*>(vb + (size_t)u * kHs + sub * 8)
                     : make_uint4(0, 0, 0, 0);
    }
  }
};

__device__ __forceinline__ int split_lo(int n, int parts, int i) {
  return (int)(((long long)n * i) / parts);
}

}  // namespace

struct PShared {
  float part[kCompute][kRec];
  int ok;
};

// One workgroup's schedule for one launch, instantiated once per role:
// SYNC = the polling wavefront, otherwise the compute wavefronts.  Both
// instantiations run the same sequence of barriers (every wait is two
// barriers; LayerNorm and the record merge are executed by both), and both
// read the shared ok flag right after each wait, so a timeout takes every
// wavefront out of the loop at the same barrier.
template <bool SYNC>
__device__ __forceinline__ void run_role(const PersistArgs& a, float* smem,
                                         PShared& S, uint32_t ep, int p) {
  const int C = a.C, H = a.H, L = a.L, G = gridDim.x, w = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* sx = smem;              // residual stream x, [C]
  float* sh = sx + C;            // LayerNorm output, [C]
  float* sv = sh + C;            // y [C], f [4C] or item records
  float* sq = sv + a.sv_floats;  // q, new k, new v of one head, [3][64]
  float* red = sq + 3 * kHs;     // reductions, [8]

  for (int i = tid; i < C; i += kThreads) sx[i] = a.x0[i];
  __syncthreads();
  const int nact = p / kChunk + 1;                       // chunks of keys 0..p
  const int nitem = (nact + kCompute - 1) / kCompute;    // items per head
  const float sl2 = rsqrtf((float)kHs) * kLog2eP;
  const int rA0 = split_lo(3 * C, G, w), rA1 = split_lo(3 * C, G, w + 1);
  const int rC0 = split_lo(C, G, w), rC1 = split_lo(C, G, w + 1);
  const int rD0 = split_lo(4 * C, G, w), rD1 = split_lo(4 * C, G, w + 1);

  auto wait_in = [&](auto kind, const uint64_t* src, int n, float* dst) -> bool {
    __syncthreads();
    if constexpr (SYNC) {
      if (!sync_wave_wait_n<decltype(kind)::value>(src, n, ep, dst, a.status) && lane == 0)
        S.ok = 0;
    }
    __syncthreads();
    // read as a scalar so every branch that encloses a barrier is uniform
    return __builtin_amdgcn_readfirstlane(S.ok) != 0;
  };
  using WH = std::integral_constant<int, kWaitHead>;
  using WR = std::integral_constant<int, kWaitRec>;
  using WC = std::integral_constant<int, kWaitC>;
  using W4 = std::integral_constant<int, kWait4C>;
  auto item_key0 = [&](int item) -> int {   // first key of this wavefront
    const int c = (item % nitem) * kCompute + wave;
    return (c < nact) ? c * kChunk : -1;
  };

  RowSlab<4, 2> sA, sD;
  RowSlab<1, 2> sC;
  RowSlab<1, 8> sE;
  KvSlab kv;
  if constexpr (!SYNC) {
    sA.load(a.layers[0].attn_w, C, rA0, rA1);
    sC.load(a.layers[0].proj_w, C, rC0, rC1);
  }

  bool ok = true;
  for (int l = 0; l < L && ok; ++l) {
    const PersistLayer* lw = a.layers + l;
    bf16_t* kl = a.kc + (size_t)l * a.layer_stride;
    bf16_t* vl = a.vc + (size_t)l * a.layer_stride;
    uint64_t* e_qkv = a.e_qkv + (size_t)l * 3 * C;
    uint64_t* e_rec = a.e_rec + (size_t)l * H * a.nchunk * kRec;
    uint64_t* e_y = a.e_y + (size_t)l * C;
    uint64_t* e_x1 = a.e_x1 + (size_t)l * C;
    uint64_t* e_f = a.e_f + (size_t)l * 4 * C;
    uint64_t* e_x2 = a.e_x2 + (size_t)l * C;

    // ---- A: LN1 + c_attn rows --------------------------------------
    if (l > 0) ok = wait_in(WC{}, a.e_x2 + (size_t)(l - 1) * C, C, sx);
    if (!ok) break;
    block_layernorm(sx, sh, C, lw->ln1_w, lw->ln1_b, red);
    if constexpr (!SYNC) {
      const bf16_t* bias = lw->attn_b;
      sA.dots(sh, C, rA0, rA1, [&](int r, float v) {
        if (bias) v += to_f32(bias[r]);
        const bf16_t vb = f32_to_bf16(v);
        tag_store(e_qkv + r, to_f32(vb), ep);
        if (r >= C) {  // k or v row: append at position p
          const int c = r - (r >= 2 * C ? 2 * C : C);
          const int h = c / kHs, d = c - h * kHs;
          bf16_t* cache = r >= 2 * C ? vl : kl;
          cache[((size_t)h * a.Tb + p) * kHs + d] = vb;
        }
      });
      // cached K/V of this workgroup's first attention item, then c_fc rows
      if (w < H * nitem) {
        const int h = w / nitem;
        kv.load(kl + (size_t)h * a.Tb * kHs, vl + (size_t)h * a.Tb * kHs,
                item_key0(w), p);
      }
      sD.load(lw->fc_w, C, rD0, rD1);
    }

    // ---- B: attention items; item 0 of each head merges ----------------
    for (int item = w; item < H * nitem && ok; item += G) {
      const int h = item / nitem, it = item - h * nitem;
      const bool last = (it == nitem - 1);  // holds the new key p
      if constexpr (!SYNC) {
        if (item != w)  // items beyond the first (grid smaller than items)
          kv.load(kl + (size_t)h * a.Tb * kHs, vl + (size_t)h * a.Tb * kHs,
                  item_key0(item), p);
      }
      ok = wait_in(WH{}, e_qkv + h * kHs, kHs, sq);
      if (ok && last) ok = wait_in(WH{}, e_qkv + C + h * kHs, kHs, sq + kHs);
      if (ok && last) ok = wait_in(WH{}, e_qkv + 2 * C + h * kHs, kHs, sq + 2 * kHs);
      if (!ok) break;
      if constexpr (!SYNC) {
        const int key0 = item_key0(item);
        const int sub = lane & 7, kgrp = lane >> 3;
        float m = -INFINITY, lsum = 0.f, o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = 0.f;
        if (key0 >= 0) {
          float qv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) qv[j] = sq[sub * 8 + j] * sl2;
          // scores of the keys this lane group meets (log2 domain)
          float sc[kPasses];
#pragma unroll
          for (int ps = 0; ps < kPasses; ++ps) {
            const int u = key0 + ps * 8 + kgrp;
            float kf[8];
            if (u == p) {
#pragma unroll
              for (int j = 0; j < 8; ++j) kf[j] = sq[kHs + sub * 8 + j];
            } else {
              bf16x8_to_f32(kv.k[ps], kf);
            }
            float t = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) t = fmaf(qv[j], kf[j], t);
#pragma unroll
            for (int o2 = 1; o2 < 8; o2 <<= 1) t += __shfl_xor(t, o2, 64);
            sc[ps] = (u <= p) ? t : -INFINITY;
          }
          float mx = -INFINITY;
#pragma unroll
          for (int ps = 0; ps < kPasses; ++ps) mx = fmaxf(mx, sc[ps]);
          if (mx != -INFINITY) {
            m = mx;
#pragma unroll
            for (int ps = 0; ps < kPasses; ++ps) {
              const int u = key0 + ps * 8 + kgrp;
              const float pr = (sc[ps] == -INFINITY) ? 0.f : exp2f(sc[ps] - mx);
              lsum += pr;
              float vf[8];
              if (u == p) {
#pragma unroll
                for (int j = 0; j < 8; ++j) vf[j] = sq[2 * kHs + sub * 8 + j];
              } else {
                bf16x8_to_f32(kv.v[ps], vf);
              }
#pragma unroll
              for (int j = 0; j < 8; ++j) o[j] = fmaf(pr, vf[j], o[j]);
            }
          }
#pragma unroll
          for (int off = 8; off < 64; off <<= 1) {
            const float m2 = __shfl_xor(m, off, 64);
            const float l2 = __shfl_xor(lsum, off, 64);
            float o2[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) o2[j] = __shfl_xor(o[j], off, 64);
            merge_state(m, lsum, o, m2, l2, o2, 8);
          }
        }
        if (lane < 8) {
          if (lane == 0) { S.part[wave][0] = m; S.part[wave][1] = lsum; }
#pragma unroll
          for (int j = 0; j < 8; ++j) S.part[wave][2 + sub * 8 + j] = o[j];
        }
      }
      __syncthreads();
      // this item's record: its wavefronts merged in chunk order (by the
      // first compute wavefront)
      float mm = -INFINITY, ll = 0.f, oo = 0.f;
      if (!SYNC && tid < kHs)
        for (int v4 = 0; v4 < kCompute; ++v4)
          merge_state(mm, ll, &oo, S.part[v4][0], S.part[v4][1], &S.part[v4][2 + tid], 1);
      if (it == 0) {
        // merger: this record, then the other items' records in order
        if (nitem > 1)
          ok = wait_in(WR{}, e_rec + ((size_t)h * a.nchunk + 1) * kRec, (nitem - 1) * kRec, sv);
        if (!ok) break;
        if (!SYNC && tid < kHs) {
          for (int i2 = 1; i2 < nitem; ++i2) {
            const float* r = sv + (i2 - 1) * kRec;
            merge_state(mm, ll, &oo, r[0], r[1], &r[2 + tid], 1);
          }
          tag_store(e_y + h * kHs + tid, to_f32(f32_to_bf16(oo / ll)), ep);
        }
      } else if (!SYNC && tid < kHs) {
        uint64_t* rec = e_rec + ((size_t)h * a.nchunk + it) * kRec;
        tag_store(rec + 2 + tid, oo, ep);
        if (tid == 0) {
          tag_store(rec, mm, ep);
          tag_store(rec + 1, ll, ep);
        }
      }
    }
    if (!ok) break;
    if constexpr (!SYNC) sE.load(lw->mp_w, 4 * C, rC0, rC1);

    // ---- C: c_proj rows + residual ------------------------------------
    ok = wait_in(WC{}, e_y, C, sv);
    if (!ok) break;
    if constexpr (!SYNC) {
      const bf16_t* bias = lw->proj_b;
      sC.dots(sv, C, rC0, rC1, [&](int r, float v) {
        if (bias) v += to_f32(bias[r]);
        tag_store(e_x1 + r, sx[r] + v, ep);
      });
      if (l + 1 < L) sA.load(a.layers[l + 1].attn_w, C, rA0, rA1);
    }

    // ---- D: LN2 + c_fc rows + GELU ------------------------------------
    ok = wait_in(WC{}, e_x1, C, sx);
    if (!ok) break;
    block_layernorm(sx, sh, C, lw->ln2_w, lw->ln2_b, red);
    if constexpr (!SYNC) {
      const bf16_t* bias = lw->fc_b;
      sD.dots(sh, C, rD0, rD1, [&](int r, float v) {
        if (bias) v += to_f32(bias[r]);
        tag_store(e_f + r, to_f32(f32_to_bf16(gelu_erf(v))), ep);
      });
      if (l + 1 < L) sC.load(a.layers[l + 1].proj_w, C, rC0, rC1);
    }

    // ---- E: MLP c_proj rows + residual --------------------------------
    ok = wait_in(W4{}, e_f, 4 * C, sv);
    if (!ok) break;
    if constexpr (!SYNC) {
      const bf16_t* bias = lw->mp_b;
      sE.dots(sv, 4 * C, rC0, rC1, [&](int r, float v) {
        if (bias) v += to_f32(bias[r]);
        tag_store(e_x2 + r, sx[r] + v, ep);
      });
    }
  }

  // ---- ln_f + tied lm_head rows ------------------------------------------
  if (ok) {
    const int r0 = split_lo(a.V, G, w), r1 = split_lo(a.V, G, w + 1);
    constexpr int GR = 4 * kCompute;  // rows per group
    RowSlab<4, 2> cur, nxt;
    if constexpr (!SYNC) cur.load(a.wte, C, r0, min(r1, r0 + GR));
    ok = wait_in(WC{}, a.e_x2 + (size_t)(L - 1) * C, C, sx);
    if (ok) {
      block_layernorm(sx, sh, C, a.lnf_w, a.lnf_b, red);
      if constexpr (!SYNC) {
        for (int g0 = r0; g0 < r1; g0 += 2 * GR) {
          const int g1 = min(r1, g0 + GR);
          if (g1 < r1) nxt.load(a.wte, C, g1, min(r1, g1 + GR));
          cur.dots(sh, C, g0, g1, [&](int r, float v) { a.logits[r] = v; });
          if (g1 >= r1) break;
          const int g2 = min(r1, g1 + GR);
          if (g2 < r1) cur.load(a.wte, C, g2, min(r1, g2 + GR));
          nxt.dots(sh, C, g1, g2, [&](int r, float v) { a.logits[r] = v; });
        }
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void decode_persistent_kernel(PersistArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ PShared S;
  const uint32_t ep = *a.epoch + 1u;
  const int p = a.pos[0];
  if (threadIdx.x == 0) S.ok = 1;
  __syncthreads();
  // The role test must compile to a scalar branch: as a per-lane (divergent)
  // branch both roles' code would be laid out for every wavefront under exec
  // masks, and a wavefront could then pass barriers of the role it does not
  // run, breaking the pairing of the roles' barriers.
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  if (p >= 0) {
    if (wv == kSyncWave)
      run_role<true>(a, smem, S, ep, p);
    else
      run_role<false>(a, smem, S, ep, p);
  }
  // the epoch advances once per launch; workgroup 0 finishes last among
  // the readers of the old value (its final phase waits for every block)
  __syncthreads();
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.epoch = ep;
}

bool persistent_decode_supported(int dtype, int C, int H, int L, int Tb,
                                 int batch, int grid) {
  if (dtype != NGPT_BF16 || batch != 1 || L < 1 || H * kHs != C) return false;
  if (C > 768 || C % 64 != 0 || grid < 64) return false;
  // rows per workgroup must fit the register slabs: 4 per compute
  // wavefront for c_attn and c_fc, 1 for the two projections
  if ((3 * C + grid - 1) / grid > 4 * kCompute) return false;
  if ((4 * C + grid - 1) / grid > 4 * kCompute) return false;
  if ((C + grid - 1) / grid > kCompute) return false;
  // a head's attention items must sit in distinct workgroups
  // and the merger polls at most (nitem - 1) records (<= 512 words)
  const int nitem_max = ((Tb + kChunk - 1) / kChunk + kCompute - 1) / kCompute;
  return Tb >= 1 && nitem_max <= grid && (nitem_max - 1) * kRec <= 512 &&
         nitem_max <= (Tb + 63) / 64;
}

size_t persistent_lds_bytes(int C, int nchunk) {
  return (size_t)(2 * C + persistent_sv_floats(C, nchunk) + 3 * kHs + 8) * sizeof(float);
}

int persistent_sv_floats(int C, int nchunk) { return max(4 * C, nchunk * kRec); }

int persistent_exchange_slack() { return 1024; }

void launch_decode_persistent(const PersistArgs& a, int grid, hipStream_t s) {
  const size_t lds = persistent_lds_bytes(a.C, a.nchunk);
  decode_persistent_kernel<<<grid, kThreads, lds, s>>>(a);
}

}  // namespace ngpt
