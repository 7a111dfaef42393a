// One-launch decode step for a single sequence (batch 1, bf16, head size
// 64): the whole one-token forward of every block plus ln_f and the tied
// lm_head, in one persistent kernel with at most one workgroup per CU (the
// host picks the fewest workgroups whose register slabs hold a phase's rows).
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
// inputs (and the LayerNorm rows) is left to the sync wavefront, which
// issues no weight loads: its polls return as soon as the data is there.
// Every phase input has an LDS buffer of its own, so the sync wavefront
// starts polling for the next phase while the compute wavefronts still work
// on the current one; each wait is one barrier.  LayerNorm statistics are
// computed by every compute wavefront on its own (no barrier), and the
// normalised vector lives in registers for the dot products.
//
// Phase outputs are exchanged as 64-bit words: the value in the low half
// (one fp32, or two bf16 for q/k/v, y and f), the launch's epoch in the high
// half, stored and loaded with device-scope relaxed atomics (cache-
// bypassing; no cache-wide fences).  A consumer accepts a word only when it
// carries the current epoch, so a word is its own ready flag.  Every wait is
// bounded: on timeout the kernel sets a status bit and leaves, and every
// other workgroup then times out too.
#include <limits.h>
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace ngpt {

namespace {

constexpr int kCompute = 4;                 // compute wavefronts
constexpr int kNSync = 2;                   // sync wavefronts (after the compute ones)
constexpr int kThreads = 64 * (kCompute + kNSync);
constexpr int kSyncLanes = 64 * kNSync;
constexpr int kSpinLimit = 1 << 20;         // default poll passes per wait

// Where a wait reports a timeout (status bit 2) and after how many passes.
struct WaitCtl {
  int32_t* status;
  int limit;
};
constexpr float kLog2eP = 1.4426950408889634f;
constexpr int kHs = 64;          // head size
constexpr int kChunk = 32;       // keys per attention chunk (one wavefront)
constexpr int kRec = kHs + 2;    // record: m, l, o[64]
constexpr int kRecWords = 512;   // most record words one merger reads
constexpr int kMaxC = 768;

// Range-checked buffer loads: a resource over [base, base + bytes); an offset
// past the end reads zeros.  Used for every prefetch so that no load sits
// behind a branch (each wavefront issues the same loads on every path, and
// the compiler's wait before a use then covers exactly the loads it needs).
constexpr uint32_t kOutOfRange = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ void tag_store(uint64_t* p, float v, uint32_t ep) {
  const uint64_t w = (static_cast<uint64_t>(ep) << 32) | __float_as_uint(v);
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Two bf16 values in one exchange word (lo = the even element).
__device__ __forceinline__ void tag_store2(uint64_t* p, bf16_t lo, bf16_t hi, uint32_t ep) {
  const uint64_t w = (static_cast<uint64_t>(ep) << 32) |
                     (static_cast<uint32_t>(hi) << 16) | static_cast<uint32_t>(lo);
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t tag_load(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Copy one accepted word to LDS: one fp32, or two bf16 (PACK, word k holds
// elements 2k in the low half and 2k+1 in the high half).
template <bool PACK>
__device__ __forceinline__ void put_word(float* dst, int k, uint64_t v) {
  const uint32_t x = static_cast<uint32_t>(v);
  if constexpr (PACK)
    *reinterpret_cast<float2*>(dst + 2 * k) =
        make_float2(__uint_as_float(x << 16), __uint_as_float(x & 0xFFFF0000u));
  else
    dst[k] = __uint_as_float(x);
}

// Called by every sync wavefront: wait until src[0..n) all carry epoch ep
// and copy the values to dst (LDS).  Sync lane s (of kSyncLanes) polls words
// s + kSyncLanes * j, j < NJ; n <= kSyncLanes * NJ, and the words up to
// src[kSyncLanes * NJ) are read too (the exchange buffers carry that much
// slack) and ignored.  Every pass issues all NJ loads before inspecting any, and copies
// every word that carries ep (a word does not change once tagged, so copying
// it again is harmless); the wait ends on the first pass with nothing
// missing.  No per-word bookkeeping is carried between passes.  False after
// wc.limit passes (status bit 2).
template <int NJ, bool PACK>
__device__ __forceinline__ bool sync_wave_wait(const uint64_t* src, int n,
                                               uint32_t ep, float* dst,
                                               WaitCtl wc) {
  const int sl = static_cast<int>(threadIdx.x) - 64 * kCompute;
  for (int spin = 0;; ++spin) {
    uint64_t v[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) v[j] = tag_load(src + sl + kSyncLanes * j);
    bool miss = false;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const bool in = sl + kSyncLanes * j < n;
      const bool got = static_cast<uint32_t>(v[j] >> 32) == ep;
      if (in && got) put_word<PACK>(dst, sl + kSyncLanes * j, v[j]);
      miss |= in && !got;
    }
    if (!__any(miss)) return true;
    if (spin >= wc.limit) {
      if ((sl & 63) == 0) atomicOr(wc.status, 2);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// q of one head (32 packed words at e + qo), and with kv also the new k and
// v (at e + ko, e + vo), into sq[0:64), sq[64:128), sq[128:192).
__device__ __forceinline__ bool sync_wave_wait_qkv(const uint64_t* e, int qo, int ko,
                                                   int vo, bool kv, uint32_t ep,
                                                   float* sq, WaitCtl wc) {
  const int lane = threadIdx.x & 63, hl = lane & 31;
  const bool lo = lane < 32;
  const uint64_t* a0 = e + (lo ? qo : ko) + hl;
  const uint64_t* a1 = e + vo + hl;
  float* d0 = sq + (lo ? 0 : kHs);
  const bool in0 = lo || kv, in1 = lo && kv;
  for (int spin = 0;; ++spin) {
    const uint64_t v0 = tag_load(a0);
    const uint64_t v1 = tag_load(a1);
    const bool g0 = static_cast<uint32_t>(v0 >> 32) == ep;
    const bool g1 = static_cast<uint32_t>(v1 >> 32) == ep;
    if (in0 && g0) put_word<true>(d0, hl, v0);
    if (in1 && g1) put_word<true>(sq + 2 * kHs, hl, v1);
    if (!__any((in0 && !g0) || (in1 && !g1))) return true;
    if (spin >= wc.limit) {
      if (lane == 0) atomicOr(wc.status, 2);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// The waits of one launch, by the number of words they read; each picks the
// smallest load count that covers n (in rounds of kSyncLanes words).  Reads
// past n stay below 512 words, the exchange buffers' slack.
//   kWaitRec   attention records of one head: n <= 512 fp32 words
//   kWaitY     y: C/2 packed words (32..384)
//   kWaitC     x1 or x2: C fp32 words (64..768)
//   kWaitF     f: 2C packed words (128..1536)
enum WaitKind { kWaitRec, kWaitY, kWaitC, kWaitF };
static_assert(kSyncLanes == 128, "the load counts below assume two sync wavefronts");

template <int KIND>
__device__ __forceinline__ bool sync_wave_wait_n(const uint64_t* src, int n,
                                                 uint32_t ep, float* dst,
                                                 WaitCtl wc) {
  if constexpr (KIND == kWaitRec) {
    if (n <= 128) return sync_wave_wait<1, false>(src, n, ep, dst, wc);
    if (n <= 256) return sync_wave_wait<2, false>(src, n, ep, dst, wc);
    return sync_wave_wait<4, false>(src, n, ep, dst, wc);
  } else if constexpr (KIND == kWaitY) {
    if (n <= 128) return sync_wave_wait<1, true>(src, n, ep, dst, wc);
    if (n <= 256) return sync_wave_wait<2, true>(src, n, ep, dst, wc);
    return sync_wave_wait<3, true>(src, n, ep, dst, wc);
  } else if constexpr (KIND == kWaitC) {
    if (n <= 256) return sync_wave_wait<2, false>(src, n, ep, dst, wc);
    if (n <= 512) return sync_wave_wait<4, false>(src, n, ep, dst, wc);
    return sync_wave_wait<6, false>(src, n, ep, dst, wc);
  } else {
    if (n <= 512) return sync_wave_wait<4, true>(src, n, ep, dst, wc);
    if (n <= 1024) return sync_wave_wait<8, true>(src, n, ep, dst, wc);
    return sync_wave_wait<12, true>(src, n, ep, dst, wc);
  }
}

// LayerNorm rows of one block (or ln_f), staged through the sync wavefront:
// up to four bf16 rows of C (gain, shift, gain, shift) -> LDS.  A missing
// row (bias-free LN, or only two rows for ln_f) reads as zeros.
constexpr int kLnRegs = 4 * kMaxC / (64 * 8);   // uint4 per lane
struct LnStage {
  uint4 r[kLnRegs];

  __device__ __forceinline__ void load(const bf16_t* const* rows, int nrows, int C) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < kLnRegs; ++k) {
      const int e = (lane + 64 * k) * 8;       // element of the [nrows][C] block
      const int seg = e / C, off = e - seg * C;
      const bf16_t* src = (seg < nrows) ? rows[seg] : nullptr;
      r[k] = (e < 4 * C && src) ? *reinterpret_cast<const uint4*>(src + off)
                                : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(bf16_t* sln, int C) const {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < kLnRegs; ++k) {
      const int e = (lane + 64 * k) * 8;
      if (e < 4 * C) *reinterpret_cast<uint4*>(sln + e) = r[k];
    }
  }
};

// LayerNorm of x[0..C) (LDS, fp32), computed by one wavefront on its own:
// two-pass fp32 statistics, then the bf16-rounded normalised values
// (x - mean) * rstd * g + b of this lane's dot-product chunks, elements
// j*512 + 8*lane .. +7 (zeros past C).  g, b: bf16 rows in LDS.
template <int NCH>
__device__ __forceinline__ void wave_layernorm(const float* x, int C, const bf16_t* g,
                                               const bf16_t* b, float (&h)[NCH][8]) {
  const int lane = threadIdx.x & 63;
  float v[kMaxC / 64];
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxC / 64; ++k) {
    v[k] = (lane + 64 * k < C) ? x[lane + 64 * k] : 0.f;
    s += v[k];
  }
  const float mean = wave_sum_all(s) / (float)C;
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxC / 64; ++k) {
    if (lane + 64 * k < C) {
      const float d = v[k] - mean;
      q += d * d;
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum_all(q) / (float)C + 1e-5f);
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int k0 = j * 512 + lane * 8;
    if (k0 < C) {
      const float4 x0 = *reinterpret_cast<const float4*>(x + k0);
      const float4 x1 = *reinterpret_cast<const float4*>(x + k0 + 4);
      const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      float gf[8], bf[8];
      bf16x8_to_f32(*reinterpret_cast<const uint4*>(g + k0), gf);
      bf16x8_to_f32(*reinterpret_cast<const uint4*>(b + k0), bf);
#pragma unroll
      for (int q2 = 0; q2 < 8; ++q2)
        h[j][q2] = to_f32(f32_to_bf16((xv[q2] - mean) * rstd * gf[q2] + bf[q2]));
    } else {
#pragma unroll
      for (int q2 = 0; q2 < 8; ++q2) h[j][q2] = 0.f;
    }
  }
}

// Weight rows of one phase held in registers of the compute wavefronts.
// Slot i of wavefront v holds row r0 + v + 4i, or with PAIR rows in pairs,
// r0 + 2v + 8(i/2) + i%2 (r0 even), so that both rows of a pair end in one
// wavefront.  Lane l holds K-elements j*512 + 8l .. +7 of each row (chunk
// j < NCH).
template <int RPW, int NCH, bool PAIR = false>
struct RowSlab {
  static_assert(RPW == 1 || RPW == 2 || RPW == 4, "RPW must be 1, 2 or 4");
  static constexpr int LG = (RPW == 1) ? 0 : (RPW == 2) ? 1 : 2;
  uint4 w[RPW][NCH];

  __device__ __forceinline__ static int row(int r0, int wave, int i) {
    return PAIR ? r0 + 2 * wave + 2 * kCompute * (i >> 1) + (i & 1)
                : r0 + wave + kCompute * i;
  }

  // W is [N][K] bf16.  Every load is issued (an unused slot reads past the
  // end of the range and gets zeros), so each wavefront issues the same
  // RPW * NCH loads on every path.
  __device__ __forceinline__ void load(const bf16_t* W, int N, int K, int r0, int r1) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(W, (uint32_t)N * (uint32_t)K * 2u);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int r = row(r0, wave, i);
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int k = j * 512 + lane * 8;
        const bool use = r < r1 && k < K;
        w[i][j] = buf_load16(rs, use ? ((uint32_t)r * (uint32_t)K + (uint32_t)k) * 2u : kOutOfRange);
      }
    }
  }

  // Dot products with a vector held in registers (h[j] = this lane's
  // elements of chunk j) or read from LDS (a[K]).  f(row, value) once per
  // row of this wavefront (from one lane), or with PAIR f(even row, value of
  // the even row, value of the odd row) once per pair.
  template <class F>
  __device__ __forceinline__ void dots_reg(const float (&h)[NCH][8], int K, int r0, int r1,
                                           F&& f) const {
    const int lane = threadIdx.x & 63;
    float acc[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      if (j * 512 + lane * 8 < K) {
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          float wf[8];
          bf16x8_to_f32(w[i][j], wf);
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[i] = fmaf(h[j][q], wf[q], acc[i]);
        }
      }
    }
    finish(acc, r0, r1, f);
  }

  template <class F>
  __device__ __forceinline__ void dots_lds(const float* a, int K, int r0, int r1, F&& f) const {
    const int lane = threadIdx.x & 63;
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
    finish(acc, r0, r1, f);
  }

  // Reduce the RPW per-lane partial sums over the wavefront: slot i ends in
  // the lanes i << (6 - LG) .. (each lane of that group holds it).
  template <class F>
  __device__ __forceinline__ void finish(float (&acc)[RPW], int r0, int r1, F&& f) const {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float r;
    if constexpr (RPW == 1) {
      r = wave_sum_all(acc[0]);
    } else if constexpr (RPW == 2) {
      r = halves_sum2(acc[0], acc[1]);
      r += lane_xor16(r);
      r = row_sum16(r);
    } else {
      r = row_sum16(rows_sum2(halves_sum2(acc[0], acc[2]), halves_sum2(acc[1], acc[3])));
    }
    if constexpr (PAIR) {
      static_assert(RPW >= 2, "pairs need two slots");
      const float r_odd = (LG == 2) ? lane_xor16(r) : lane_xor32(r);
      if ((lane & ((2 << (6 - LG)) - 1)) == 0) {
        const int rw = row(r0, wave, lane >> (6 - LG));
        if (rw < r1) f(rw, r, r_odd);
      }
    } else {
      if ((lane & ((1 << (6 - LG)) - 1)) == 0) {
        const int rw = row(r0, wave, lane >> (6 - LG));
        if (rw < r1) f(rw, r);
      }
    }
  }
};

// Cached K/V of one wavefront's 32-key chunk of one head (kb, vb: the
// head's [Tb][64] rows): 4 passes of 8 keys, 8 lanes per key (8 dims each).
// Keys at or past the new position p (or a chunk key0 < 0) read zeros;
// every load is issued.
constexpr int kPasses = kChunk / 8;
struct KvSlab {
  uint4 k[kPasses], v[kPasses];

  __device__ __forceinline__ void load(const bf16_t* kb, const bf16_t* vb, int Tb,
                                       int key0, int p) {
    const int lane = threadIdx.x & 63, sub = lane & 7, kgrp = lane >> 3;
    const uint32_t bytes = (uint32_t)Tb * kHs * 2u;
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kb, bytes), rv = buf_rsrc(vb, bytes);
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
      const int u = key0 + ps * 8 + kgrp;
      const bool cached = key0 >= 0 && u < p;
      const uint32_t off = cached ? ((uint32_t)u * kHs + sub * 8) * 2u : kOutOfRange;
      k[ps] = buf_load16(rk, off);
      v[ps] = buf_load16(rv, off);
    }
  }
};

__device__ __forceinline__ int split_lo(int n, int parts, int i) {
  return (int)(((long long)n * i) / parts);
}

// LDS layout (floats): x, x1, y [C] each, f [4C], records [kRecWords],
// q/k/v [3][64], the LayerNorm rows [2 parities][4][C] bf16, the greedy
// candidates of the previous launch [G][2], then the blocks' weight
// pointers [L][12] (uint64).
constexpr int kLayerPtrs = sizeof(PersistLayer) / sizeof(uint64_t);
constexpr int kMaxGrid = 256;   // candidates: 2 words per workgroup, <= 512 words
__host__ __device__ constexpr int lds_floats(int C, int L) {
  return 11 * C + kRecWords + 3 * kHs + 2 * kMaxGrid + 2 * kLayerPtrs * L;
}

// Greedy choice, the sampler's rule: the largest logit, lowest id among
// equal maxima; NaN and -inf never win (an all -inf/NaN row gives INT_MAX).
__device__ __forceinline__ void cand_take(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && v > -INFINITY && i < bi)) { bv = v; bi = i; }
}
// the best candidate over the wavefront, in every lane
__device__ __forceinline__ void cand_wave(float& bv, int& bi) {
  auto step = [&](float pv, float pib) { cand_take(bv, bi, pv, __float_as_int(pib)); };
  step(lane_xor1(bv), lane_xor1(__int_as_float(bi)));
  step(lane_xor2(bv), lane_xor2(__int_as_float(bi)));
  step(lane_mirror8(bv), lane_mirror8(__int_as_float(bi)));
  step(lane_xor8(bv), lane_xor8(__int_as_float(bi)));
  step(lane_xor16(bv), lane_xor16(__int_as_float(bi)));
  step(lane_xor32(bv), lane_xor32(__int_as_float(bi)));
}

}  // namespace

struct PShared {
  float part[kCompute][kRec];
  float cv[kCompute];   // greedy candidates of the compute wavefronts
  int ci[kCompute];
  int fail;   // sequence number of the first wait that timed out
};

// One workgroup's schedule for one launch, instantiated once per role:
// SYNC = the polling wavefront, otherwise the compute wavefronts.  Both
// instantiations run the same sequence of waits, each ending in one barrier,
// under the same (scalar) conditions; each wait has a sequence number and a
// timeout of the sync wavefront at wait k is seen by everyone after barrier
// k, so every wavefront leaves the loop at the same barrier.
template <bool SYNC>
__device__ __forceinline__ void run_role(const PersistArgs& a, float* smem,
                                         PShared& S, uint32_t ep, int p) {
  const int C = a.C, H = a.H, L = a.L, G = gridDim.x, w = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* bX = smem;                    // x: the block's input
  float* bX1 = bX + C;                 // x1
  float* bY = bX1 + C;                 // y
  float* bF = bY + C;                  // f [4C]
  float* bRec = bF + 4 * C;            // other items' records
  float* sq = bRec + kRecWords;        // q, new k, new v of one head
  bf16_t* sln = reinterpret_cast<bf16_t*>(sq + 3 * kHs);  // [2][4][C]
  float* bCand = sq + 3 * kHs + 4 * C;                  // [G][2]
  uint64_t* slay = reinterpret_cast<uint64_t*>(bCand + 2 * kMaxGrid);  // [L][12]

  const bool sync0 = SYNC && __builtin_amdgcn_readfirstlane(wave) == kCompute;  // first sync wavefront
  int seq = 0;
  // every wait gives up after the host-set number of passes (0: the default)
  const WaitCtl wc{a.status, a.wait_limit > 0 ? a.wait_limit : kSpinLimit};
  // n == 0: nothing to poll, the wait is just the barrier
  auto wait_in = [&](auto kind, const uint64_t* src, int n, float* dst) -> bool {
    ++seq;
    if constexpr (SYNC) {
      if (n > 0 && !sync_wave_wait_n<decltype(kind)::value>(src, n, ep, dst, wc) &&
          lane == 0)
        S.fail = seq;
    }
    __syncthreads();
    // read as a scalar so every branch that encloses a barrier is uniform
    return __builtin_amdgcn_readfirstlane(S.fail) > seq;
  };
  using WR = std::integral_constant<int, kWaitRec>;
  using WY = std::integral_constant<int, kWaitY>;
  using WC = std::integral_constant<int, kWaitC>;
  using WF = std::integral_constant<int, kWaitF>;

  LnStage lns;
  if (sync0) {
    const PersistLayer& q = a.layers[0];
    const bf16_t* rows[4] = {q.ln1_w, q.ln1_b, q.ln2_w, q.ln2_b};
    lns.load(rows, 4, C);
  }
  if (!a.fused)
    for (int i = tid; i < C; i += kThreads) bX[i] = a.x0[i];
  {
    const uint64_t* src = reinterpret_cast<const uint64_t*>(a.layers);
    for (int i = tid; i < L * kLayerPtrs; i += kThreads) slay[i] = src[i];
  }
  if (sync0) lns.store(sln, C);
  __syncthreads();
  // weight pointers of block l as scalars (the table in global memory could
  // only be read with vector loads, which would queue behind the prefetches)
  auto lptr = [&](int l, int field) -> const bf16_t* {
    const uint64_t v = slay[l * kLayerPtrs + field];
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    return reinterpret_cast<const bf16_t*>((static_cast<uint64_t>(hi) << 32) | lo);
  };
  enum { kLn1W, kLn1B, kAttnW, kAttnB, kProjW, kProjB, kLn2W, kLn2B, kFcW, kFcB, kMpW, kMpB };
  auto stage = [&](int l) {   // LayerNorm rows of block l, or ln_f for l == L
    if (l < L) {
      const bf16_t* rows[4] = {lptr(l, kLn1W), lptr(l, kLn1B), lptr(l, kLn2W), lptr(l, kLn2B)};
      lns.load(rows, 4, C);
    } else {
      const bf16_t* rows[2] = {a.lnf_w, a.lnf_b};
      lns.load(rows, 2, C);
    }
  };

  const int nact = p / kChunk + 1;                       // chunks of keys 0..p
  const int nitem = (nact + kCompute - 1) / kCompute;    // items per head
  const float sl2 = rsqrtf((float)kHs) * kLog2eP;
  // c_attn and c_fc rows go out in whole pairs (packed exchange words)
  const int rA0 = 2 * split_lo(3 * C / 2, G, w), rA1 = 2 * split_lo(3 * C / 2, G, w + 1);
  const int rC0 = split_lo(C, G, w), rC1 = split_lo(C, G, w + 1);
  const int rD0 = 2 * split_lo(2 * C, G, w), rD1 = 2 * split_lo(2 * C, G, w + 1);

  // Attention items, one per workgroup: workgroup w runs on XCD w % 8, and
  // all items of head h sit on XCD h % 8 (the support check guarantees the
  // room), so a head's records meet inside one L2.
  const int h0 = (w & 7) + 8 * ((w >> 3) / nitem);
  const int it0 = (w >> 3) - ((w >> 3) / nitem) * nitem;
  const bool has_item = h0 < H;
  auto key0_of = [&](int it) -> int {   // first key of this wavefront's chunk
    const int c = it * kCompute + wave;
    return (c < nact) ? c * kChunk : -1;
  };

  RowSlab<4, 2, true> sA, sD;
  RowSlab<1, 2> sC;
  RowSlab<1, 8> sE;
  KvSlab kv;
  if constexpr (!SYNC) {
    sA.load(lptr(0, kAttnW), 3 * C, C, rA0, rA1);
    sC.load(lptr(0, kProjW), C, C, rC0, rC1);
  }

  bool ok = true;
  if (a.fused) {
    // Greedy step: the token is the argmax of the logits the previous launch
    // produced, from its workgroups' candidates (tagged with its epoch);
    // the sync wavefronts pick it and write x = wte[tok] + wpe[p].
    ++seq;
    if constexpr (SYNC) {
      if (!sync_wave_wait<(2 * kMaxGrid) / kSyncLanes, false>(a.e_cand, 2 * G, ep - 1u, bCand, wc) &&
          lane == 0)
        S.fail = seq;
    }
    __syncthreads();
    ok = __builtin_amdgcn_readfirstlane(S.fail) > seq;
    if (ok) {
      if constexpr (SYNC) {
        float bv = -INFINITY;
        int bi = INT_MAX;
        for (int k = lane; k < G; k += 64) cand_take(bv, bi, bCand[2 * k], __float_as_int(bCand[2 * k + 1]));
        cand_wave(bv, bi);
        // a row with no finite maximum (bi == INT_MAX) gives id 0 and the
        // invalid-input flag, the sampler's rule
        const int sl = tid - 64 * kCompute;
        const bool bad = !(bi >= 0 && bi < a.V);
        const int tok = bad ? 0 : bi;
        if (bad && w == 0 && sl == 0) atomicOr(a.status, 1);
        {
          const bf16_t* te = a.wte + (size_t)tok * C;
          const bf16_t* pe = a.wpe + (size_t)p * C;
          for (int c = sl; c < C; c += kSyncLanes) bX[c] = to_f32(te[c]) + to_f32(pe[c]);
        }
        if (w == 0 && sl == 0) {
          a.next_ids[0] = tok;
          a.tok[0] = tok;
          a.pos[0] = p;
          a.hist[p] = tok;
        }
      }
      __syncthreads();
    }
  }
  for (int l = 0; l < L && ok; ++l) {
    const bf16_t* lnr = sln + (size_t)(l & 1) * 4 * C;
    bf16_t* kl = a.kc + (size_t)l * a.layer_stride;
    bf16_t* vl = a.vc + (size_t)l * a.layer_stride;
    uint64_t* e_qkv = a.e_qkv + (size_t)l * 3 * C;
    uint64_t* e_rec = a.e_rec + (size_t)l * H * a.nchunk * kRec;
    uint64_t* e_y = a.e_y + (size_t)l * C;
    uint64_t* e_x1 = a.e_x1 + (size_t)l * C;
    uint64_t* e_f = a.e_f + (size_t)l * 4 * C;
    uint64_t* e_x2 = a.e_x2 + (size_t)l * C;

    // ---- A: LN1 + c_attn rows --------------------------------------
    if (l > 0) ok = wait_in(WC{}, a.e_x2 + (size_t)(l - 1) * C, C, bX);
    if (!ok) break;
    if constexpr (!SYNC) {
      float hv[2][8];
      wave_layernorm<2>(bX, C, lnr, lnr + C, hv);
      const bf16_t* bias = lptr(l, kAttnB);
      sA.dots_reg(hv, C, rA0, rA1, [&](int r, float v0, float v1) {
        if (bias) { v0 += to_f32(bias[r]); v1 += to_f32(bias[r + 1]); }
        const bf16_t b0 = f32_to_bf16(v0), b1 = f32_to_bf16(v1);
        tag_store2(e_qkv + r / 2, b0, b1, ep);
        if (r >= C) {  // k or v rows: append at position p
          const int c = r - (r >= 2 * C ? 2 * C : C);
          const int h = c / kHs, d = c - h * kHs;
          bf16_t* cache = r >= 2 * C ? vl : kl;
          *reinterpret_cast<uint32_t*>(cache + ((size_t)h * a.Tb + p) * kHs + d) =
              static_cast<uint32_t>(b0) | (static_cast<uint32_t>(b1) << 16);
        }
      });
      // cached K/V of this workgroup's first attention item (issued also
      // without one, as key0 = -1), then c_fc rows
      kv.load(kl + (size_t)h0 * a.Tb * kHs, vl + (size_t)h0 * a.Tb * kHs, a.Tb,
              has_item ? key0_of(it0) : -1, p);
      sD.load(lptr(l, kFcW), 4 * C, C, rD0, rD1);
    }

    // ---- B: attention items; item 0 of each head merges ----------------
    if (has_item) {
      const int h = h0, it = it0;
      const bool last = (it == nitem - 1);  // holds the new key p
      ++seq;   // wait: q of head h (with the new k, v for the last item)
      if (sync0) {
        if (!sync_wave_wait_qkv(e_qkv, h * kHs / 2, (C + h * kHs) / 2, (2 * C + h * kHs) / 2,
                                last, ep, sq, wc) && lane == 0)
          S.fail = seq;
      }
      __syncthreads();
      ok = __builtin_amdgcn_readfirstlane(S.fail) > seq;
      if (!ok) break;
      if constexpr (!SYNC) {
        const int key0 = key0_of(it);
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
            t += lane_xor1(t);      // sum over the key's 8 lanes
            t += lane_xor2(t);
            t += lane_mirror8(t);
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
              const float pr = (sc[ps] == -INFINITY) ? 0.f : exp2_fast(sc[ps] - mx);
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
          // merge the 8 key groups' states (partners 8, 16, 32 lanes away)
#pragma unroll
          for (int stage = 0; stage < 3; ++stage) {
            auto partner = [&](float x) {
              return stage == 0 ? lane_xor8(x) : stage == 1 ? lane_xor16(x) : lane_xor32(x);
            };
            const float m2 = partner(m), l2 = partner(lsum);
            float o2[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) o2[j] = partner(o[j]);
            merge_state(m, lsum, o, m2, l2, o2, 8);
          }
        }
        if (lane < 8) {
          if (lane == 0) { S.part[wave][0] = m; S.part[wave][1] = lsum; }
#pragma unroll
          for (int j = 0; j < 8; ++j) S.part[wave][2 + sub * 8 + j] = o[j];
        }
      }
      // wait: the wavefronts' partial states, and for the merger the other
      // items' records (polled while the partials are computed)
      const bool merger = (it == 0 && nitem > 1);
      ok = wait_in(WR{}, e_rec + ((size_t)h * a.nchunk + 1) * kRec,
                   merger ? (nitem - 1) * kRec : 0, bRec);
      if (!ok) break;
      // this item's record: its wavefronts merged in chunk order (by the
      // first compute wavefront)
      if (!SYNC && tid < kHs) {
        float mm = -INFINITY, ll = 0.f, oo = 0.f;
        for (int v4 = 0; v4 < kCompute; ++v4)
          merge_state(mm, ll, &oo, S.part[v4][0], S.part[v4][1], &S.part[v4][2 + tid], 1);
        if (it == 0) {
          // merger: this record, then the other items' records in order
          for (int i2 = 1; i2 < nitem; ++i2) {
            const float* r = bRec + (i2 - 1) * kRec;
            merge_state(mm, ll, &oo, r[0], r[1], &r[2 + tid], 1);
          }
          const bf16_t yb = f32_to_bf16(oo / ll);
          const int yb1 = __builtin_amdgcn_update_dpp(0, static_cast<int>(yb), 0xB1, 0xf, 0xf, false);
          if ((tid & 1) == 0)
            tag_store2(e_y + (h * kHs + tid) / 2, yb, static_cast<bf16_t>(yb1), ep);
        } else {
          uint64_t* rec = e_rec + ((size_t)h * a.nchunk + it) * kRec;
          tag_store(rec + 2 + tid, oo, ep);
          if (tid == 0) {
            tag_store(rec, mm, ep);
            tag_store(rec + 1, ll, ep);
          }
        }
      }
    }
    if (!ok) break;
    if constexpr (!SYNC) sE.load(lptr(l, kMpW), C, 4 * C, rC0, rC1);

    // ---- C: c_proj rows + residual ------------------------------------
    // (the sync wavefront stages the next block's LayerNorm rows, or ln_f,
    // into the other parity's LDS rows, last read two blocks back)
    if (sync0) stage(l + 1);
    ok = wait_in(WY{}, e_y, C / 2, bY);
    if (sync0) lns.store(sln + (size_t)((l + 1) & 1) * 4 * C, C);
    if (!ok) break;
    if constexpr (!SYNC) {
      const bf16_t* bias = lptr(l, kProjB);
      sC.dots_lds(bY, C, rC0, rC1, [&](int r, float v) {
        if (bias) v += to_f32(bias[r]);
        tag_store(e_x1 + r, bX[r] + v, ep);
      });
      // (the last block reloads its own rows: a load on every path)
      sA.load(lptr(l + 1 < L ? l + 1 : l, kAttnW), 3 * C, C, rA0, rA1);
    }

    // ---- D: LN2 + c_fc rows + GELU ------------------------------------
    ok = wait_in(WC{}, e_x1, C, bX1);
    if (!ok) break;
    if constexpr (!SYNC) {
      float hv[2][8];
      wave_layernorm<2>(bX1, C, lnr + 2 * C, lnr + 3 * C, hv);
      const bf16_t* bias = lptr(l, kFcB);
      sD.dots_reg(hv, C, rD0, rD1, [&](int r, float v0, float v1) {
        if (bias) { v0 += to_f32(bias[r]); v1 += to_f32(bias[r + 1]); }
        tag_store2(e_f + r / 2, f32_to_bf16(gelu_erf(v0)), f32_to_bf16(gelu_erf(v1)), ep);
      });
      sC.load(lptr(l + 1 < L ? l + 1 : l, kProjW), C, C, rC0, rC1);
    }

    // ---- E: MLP c_proj rows + residual --------------------------------
    ok = wait_in(WF{}, e_f, 2 * C, bF);
    if (!ok) break;
    if constexpr (!SYNC) {
      const bf16_t* bias = lptr(l, kMpB);
      sE.dots_lds(bF, 4 * C, rC0, rC1, [&](int r, float v) {
        if (bias) v += to_f32(bias[r]);
        tag_store(e_x2 + r, bX1[r] + v, ep);
      });
    }
  }

  // ---- ln_f + tied lm_head rows ------------------------------------------
  if (ok) {
    const int r0 = split_lo(a.V, G, w), r1 = split_lo(a.V, G, w + 1);
    constexpr int GR = 4 * kCompute;  // rows per group
    RowSlab<4, 2> cur, nxt;
    // groups of GR rows, two per trip, each group's loads issued one group
    // ahead (rows past r1 read row 0 and are not stored)
    auto grp = [&](int g, int& g0, int& g1) { g0 = r0 + g * GR; g1 = min(r1, g0 + GR); };
    if constexpr (!SYNC) {
      int g0, g1;
      grp(0, g0, g1);
      cur.load(a.wte, a.V, C, g0, g1);
    }
    ok = wait_in(WC{}, a.e_x2 + (size_t)(L - 1) * C, C, bX);
    if (ok) {
      if constexpr (!SYNC) {
        float bv = -INFINITY;   // this lane's greedy candidate over its rows
        int bi = INT_MAX;
        const bf16_t* lnr = sln + (size_t)(L & 1) * 4 * C;
        float hv[2][8];
        wave_layernorm<2>(bX, C, lnr, lnr + C, hv);
        const int ngrp = (r1 - r0 + GR - 1) / GR;
        for (int g = 0; g < ngrp; g += 2) {
          int g0, g1;
          grp(g + 1, g0, g1);
          nxt.load(a.wte, a.V, C, g0, g1);
          grp(g, g0, g1);
          cur.dots_reg(hv, C, g0, g1, [&](int r, float v) { a.logits[r] = v; cand_take(bv, bi, v, r); });
          grp(g + 2, g0, g1);
          cur.load(a.wte, a.V, C, g0, g1);
          grp(g + 1, g0, g1);
          nxt.dots_reg(hv, C, g0, g1, [&](int r, float v) { a.logits[r] = v; cand_take(bv, bi, v, r); });
        }
        cand_wave(bv, bi);
        if (lane == 0) { S.cv[wave] = bv; S.ci[wave] = bi; }
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void decode_persistent_kernel(PersistArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ PShared S;
  // Every workgroup reads the same epoch: nothing writes *a.epoch while a
  // launch that reads it runs (the head node advanced it before), and a
  // fused launch takes its epoch as an argument.
  const uint32_t ep = a.fused ? a.ep : *a.epoch;
  // position of the new token: the sampler head node has set pos (< 0:
  // inactive), or, in a fused greedy step, the current length (advanced at
  // the end) while it is below the sequence's limit
  int p = a.pos[0];
  if (a.fused) {
    p = a.lens[0];
    if (p >= a.limit[0]) p = -1;
    if (p < 0 && blockIdx.x == 0 && threadIdx.x == 0) {
      a.next_ids[0] = -1;
      a.pos[0] = -1;
    }
  }
  if (threadIdx.x == 0) S.fail = INT_MAX;
  if (threadIdx.x < kCompute) { S.cv[threadIdx.x] = -INFINITY; S.ci[threadIdx.x] = INT_MAX; }
  __syncthreads();
  // The role test must compile to a scalar branch: as a per-lane (divergent)
  // branch both roles' code would be laid out for every wavefront under exec
  // masks, and a wavefront could then pass barriers of the role it does not
  // run, breaking the pairing of the roles' barriers.
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  if (p >= 0) {
    if (wv >= kCompute)
      run_role<true>(a, smem, S, ep, p);
    else
      run_role<false>(a, smem, S, ep, p);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    // this workgroup's greedy candidate for the next launch, only from a
    // launch whose waits all completed here
    if (p >= 0 && S.fail == INT_MAX) {
      float bv = -INFINITY;
      int bi = INT_MAX;
      for (int i = 0; i < kCompute; ++i) cand_take(bv, bi, S.cv[i], S.ci[i]);
      tag_store(a.e_cand + 2 * blockIdx.x, bv, ep);
      tag_store(a.e_cand + 2 * blockIdx.x + 1, __int_as_float(bi), ep);
    }
    if (blockIdx.x == 0 && a.fused && p >= 0 && S.fail == INT_MAX) a.lens[0] = p + 1;
    // a fused launch keeps the word in step with the host's count, for the
    // next head node; no workgroup of this launch reads it
    if (a.fused && blockIdx.x == 0)
      __hip_atomic_store(a.epoch, ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

bool persistent_decode_supported(int dtype, int C, int H, int L, int Tb,
                                 int batch, int grid) {
  if (dtype != NGPT_BF16 || batch != 1 || L < 1 || H * kHs != C) return false;
  if (C > kMaxC || C % 64 != 0 || grid < 64 || grid > kMaxGrid) return false;
  // rows per workgroup must fit the register slabs: 4 per compute
  // wavefront for c_attn and c_fc (handed out in pairs), 1 for the two
  // projections
  if (2 * ((3 * C / 2 + grid - 1) / grid) > 4 * kCompute) return false;
  if (2 * ((2 * C + grid - 1) / grid) > 4 * kCompute) return false;
  if ((C + grid - 1) / grid > kCompute) return false;
  // one attention item per workgroup, a head's items on one XCD (grid a
  // multiple of 8, workgroup w on XCD w % 8), and the merger reads at most
  // (nitem - 1) records (<= 512 words)
  const int nitem_max = ((Tb + kChunk - 1) / kChunk + kCompute - 1) / kCompute;
  if (grid % 8 != 0 || ((H + 7) / 8) * nitem_max > grid / 8) return false;
  if (L * (int)sizeof(PersistLayer) > 16384) return false;   // pointer table in LDS
  return Tb >= 1 && (nitem_max - 1) * kRec <= kRecWords && nitem_max <= (Tb + 63) / 64;
}

size_t persistent_lds_bytes(int C, int L) { return (size_t)lds_floats(C, L) * sizeof(float); }

int persistent_max_grid() { return kMaxGrid; }

int persistent_blocks_per_cu(int C, int L) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(decode_persistent_kernel), kThreads,
          persistent_lds_bytes(C, L)) != hipSuccess)
    return 0;
  return n;
}

// Each exchange waits for words from all workgroups, and that wait shortens
// with fewer participants (measured: 245 us per GPT-2-small step at 192
// workgroups, 260 at 224, 265 at 256), so the grid is the fewest workgroups
// that hold the rows.  Every workgroup must be resident at once (the phases
// wait on each other), which the occupancy query confirms.
int persistent_pick_grid(int dtype, int C, int H, int L, int Tb, int cus) {
  int g = 0;
  for (int t = 64; t <= (cus < kMaxGrid ? cus : kMaxGrid) && g == 0; t += 8)
    if (persistent_decode_supported(dtype, C, H, L, Tb, 1, t)) g = t;
  if (g > 0 && (long)persistent_blocks_per_cu(C, L) * cus < g) g = 0;
  return g;
}

int persistent_exchange_slack() { return 512; }

void launch_decode_persistent(const PersistArgs& a, int grid, hipStream_t s) {
  decode_persistent_kernel<<<grid, kThreads, persistent_lds_bytes(a.C, a.L), s>>>(a);
}

}  // namespace ngpt
