// Causal multi-head self-attention over the KV cache.
//
// Definition (SDK guide "极速上手nanoGPT", "模型架构解析", manual path): per
// head, scores q k^T * 1/sqrt(hs), entries above the diagonal set to -inf,
// softmax over keys, times v.  With a cache (serving page "原生 nanoGPT
// 模型服务首选", KV-cache section) the keys of a sequence are its cached
// rows 0..t; a decode query at position t sees every cached key and itself.
// The lower-triangular visibility rule is the model-building chapter's
// (section 4.5).  The K/V of the rows being processed have already been
// written into the cache by the c_attn epilogue.
//
// Cache layout: [batch][H][Tb][hs] for this layer, so one (sequence, head)
// is a contiguous [Tb][hs] block.
//
// Kernels:
//   attn_prefill_mfma   bf16 / fp16, one workgroup per (64-row query tile, head,
//                       sequence); K/V tiles of 64 keys staged in LDS;
//                       scores and P*V on MFMA; online (running max / sum)
//                       softmax in fp32; tiles above the diagonal skipped.
//   attn_prefill_simt   one thread per query row (fp32 model).
//   attn_decode         one query per sequence, split over 64-key chunks;
//                       each workgroup leaves (max, sum, o) for its chunk and
//                       a second small launch merges the chunks in order.
#include <math.h>

#include <utility>

#include "common.hpp"
#include "kernels.hpp"

namespace ngpt {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kPrefillKch = 8;   // key tiles per chunk when a prefill tile is split

// ---------------------------------------------------------------------------
// Prefill, bf16 MFMA.  Scores are formed transposed, S^T = K Q^T, so that a
// lane holds one query column: lane l owns query q0 + 16*wave + (l % 16) and
// keys 16*t + 4*(l/16) + i (i < 4) of each 16-key sub-tile t.  The running
// softmax statistics are then per lane.  The output is formed as
// O^T = V^T P^T; P^T is fed straight from the score registers, and the V^T
// fragments are read from a key-major LDS copy of V by the transposing LDS
// read (ds_read_b64_tr_b16) in the same key order.
// ---------------------------------------------------------------------------
//
// With a past (chunked prefill into a live cache) the new rows of a
// sequence sit at positions past .. past + len - 1 and each sees every key
// up to its own position (the offset causal mask); without one, past = 0.
//
// Key split (kch > 0, batch 1): a query tile that meets more than kch key
// tiles is split into chunks of kch key tiles, one workgroup each; such a
// chunk leaves its rows' unnormalised state (m, l, o) in part, and
// attn_prefill_merge combines the chunks in order.  Workgroup x takes query
// tile ntiles - 1 - x / nsplit (heavy tiles first) and chunk x % nsplit.
constexpr int kPrefillWaves = 8;   // two wavefronts per 16-row query sub-tile

// Work order of a split batch-1 prefill: the (query tile, chunk) pairs of
// one head, most key tiles first; workgroup x takes pair it[x / H] of head
// x % H, so the longest chunks of every head start in the first wave of
// workgroups and no workgroup is launched without work.  n == 0: the grid is
// (tiles x chunks, H, B) instead.
constexpr int kPrefillOrderMax = 128;
struct PrefillOrder {
  int n;
  uint16_t it[kPrefillOrderMax];   // query tile | chunk << 8
};

template <class T, int HS>
__global__ __launch_bounds__(64 * kPrefillWaves) void attn_prefill_mfma(
    const T* __restrict__ q, int ldq, const T* __restrict__ kc,
    const T* __restrict__ vc, KvMap kvm, RowMap map, int H, int Tb, float scale,
    T* __restrict__ y, int ldy, int kch, int nsplit, float* __restrict__ part,
    PrefillOrder ord) {
  typedef typename Half16<T>::vec8 vec8;
  constexpr int KT = 64;             // keys per tile
  constexpr int KS = HS + 8;         // sK row stride (elements)
  // sV row stride (elements): 16 more than a row, so that the four keys one
  // transposing read takes (32 bytes each) start 32 bytes apart modulo 128
  constexpr int VS = HS + 16;
  constexpr int NKK = HS / 32;       // MFMA steps over the head dimension
  constexpr int ND = HS / 16;        // 16-row output sub-tiles over hs
  constexpr int MS = ND * 4 + 4;     // merge record per lane: o, then m, l
  __shared__ __attribute__((aligned(16))) bf16_t sK[KT * KS];
  __shared__ __attribute__((aligned(16))) bf16_t sV[KT * VS];
  __shared__ __attribute__((aligned(16))) float sM[4 * 64 * MS];

  int b, h, qt, chunk;
  if (ord.n > 0) {
    const int x = blockIdx.x, r = x / H;
    b = 0;
    h = x - r * H;
    qt = ord.it[r] & 0xFF;
    chunk = ord.it[r] >> 8;
  } else {
    b = blockIdx.z;
    h = blockIdx.y;
    const int ntiles = (map.off[b + 1] - map.off[b] + 63) / 64;
    qt = ntiles - 1 - (kch > 0 ? (int)blockIdx.x / nsplit : (int)blockIdx.x);
    chunk = kch > 0 ? (int)blockIdx.x % nsplit : 0;
  }
  const int len = map.off[b + 1] - map.off[b];
  const int past = map.past[b];
  if (qt < 0) return;
  const int q0 = qt * 64;
  // key tiles this query tile meets: 0 .. (its last row's position) / 64
  const int nkt_all = (past + min(q0 + 63, len - 1)) / KT + 1;
  // key tiles [kt0, kt0 + nkt) of this workgroup
  const int nch = kch > 0 ? (nkt_all + kch - 1) / kch : 1;
  if (chunk >= nch) return;
  const int kt0 = kch > 0 ? chunk * kch : 0;
  const int tid = threadIdx.x, lane = tid & 63;
  // the wavefront index as a scalar, so that per-wavefront tests are scalar
  // branches.  Wavefront w takes query rows 16 (w % 4) .. + 15 of the tile
  // and keys 32 (w / 4) .. + 31 of every key tile.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qs = wave & 3, kh = wave >> 2;
  const int g = lane >> 4;                        // lane group 0..3
  const int qrow = q0 + qs * 16 + (lane & 15);    // this lane's query (new row)
  const int qpos = past + qrow;                   // ... and its position
  const int qpos_w = past + q0 + qs * 16;         // the wavefront's first position
  const int kend = past + len;                    // keys in the cache
  const size_t row0 = (size_t)map.off[b];
  const int slot = map.slot[b];
  const int64_t hoff = (int64_t)h * kv_hstride(kvm);

  // Q^T operand: column = this lane's query, K-values = dims 8g.. (+32 kk)
  vec8 qf[NKK];
  {
    const int qr = qrow < len ? qrow : len - 1;
    const T* qp = q + (row0 + qr) * ldq + h * HS;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[kk] = *reinterpret_cast<const vec8*>(qp + kk * 32 + g * 8);
  }

  const float sl2 = scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t o[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) o[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nkt = (nch > 1 ? min(kt0 + kch, nkt_all) : nkt_all) - kt0;
  // Staging work item: a pair of keys (2kp, 2kp+1) x 8 dims, of K for the
  // first four wavefronts and of V for the other four; both go to LDS
  // key-major.
  // S tiles are in flight in registers.  The loads are range-checked buffer
  // loads issued on every path, through a resource spanning the tile's 64
  // cache rows (one block): keys at or past len (whose cache rows may hold
  // anything), tiles past the last key and unmapped blocks read zeros.
  constexpr int ITEMS = (KT / 2) * (HS / 8);
  static_assert(ITEMS <= 256, "one staging item per thread of each half");
  constexpr int S = 4;
  constexpr uint32_t kOut = 0x80000000u;
  const bool vrole = wave >= 4;
  const int c = tid & 255;
  const int kp = c / (HS / 8), d0 = (c % (HS / 8)) * 8;
  const T* src = vrole ? vc : kc;
  uint4 rs[S][2];
  auto load_tile = [&](int st, int k0) {
    const int64_t bb = k0 < kend ? kv_block_base(kvm, slot, k0 / KT) : -1;
    const size_t r0 = bb < 0 ? 0 : (size_t)(bb + hoff) * HS;
    const int nrec = bb < 0 ? 0 : KT * HS * 2;
    const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(src + r0), (short)0, nrec, 0x00020000);
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
      const int key = k0 + 2 * kp + e2;
      const uint32_t off =
          (c < ITEMS && key < kend) ? ((uint32_t)(key - k0) * HS + d0) * 2u : kOut;
      rs[st][e2] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsc, off, 0, 0));
    }
  };
  auto store_tile = [&](int st) {
    if (c >= ITEMS) return;
    if (!vrole) {
      *reinterpret_cast<uint4*>(sK + (2 * kp) * KS + d0) = rs[st][0];
      *reinterpret_cast<uint4*>(sK + (2 * kp + 1) * KS + d0) = rs[st][1];
    } else {
      *reinterpret_cast<uint4*>(sV + (2 * kp) * VS + d0) = rs[st][0];
      *reinterpret_cast<uint4*>(sV + (2 * kp + 1) * VS + d0) = rs[st][1];
    }
  };
#pragma unroll
  for (int st = 0; st < S; ++st) load_tile(st, (kt0 + st) * KT);
  for (int t0 = 0; t0 < nkt; t0 += S) {
#pragma unroll
  for (int st = 0; st < S; ++st) {
    const int k0 = (kt0 + t0 + st) * KT;
    __syncthreads();
    store_tile(st);
    __syncthreads();
    load_tile(st, k0 + S * KT);
    if (t0 + st >= nkt) continue;       // padding of the last group (uniform)
    const int kb = k0 + kh * 32;        // this wavefront's first key
    if (kb > qpos_w + 15) continue;     // all 32 keys above the diagonal (uniform)

    // S^T for 2 sub-tiles of 16 keys
    f32x4_t s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const vec8 kf = *reinterpret_cast<const vec8*>(
            sK + (kh * 32 + t * 16 + (lane & 15)) * KS + kk * 32 + g * 8);
        s[t] = Half16<T>::mfma(kf, qf[kk], s[t]);
      }
    }
    float alpha, psum = 0.f;
    if (qpos_w >= kb + 31) {
      // every key is visible to all of the wavefront's queries: no mask,
      // and the running maximum is finite after this step
      float tmax = s[0][0];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, s[t][i]);
      tmax = fmaxf(tmax, lane_xor16(tmax));
      tmax = fmaxf(tmax, lane_xor32(tmax));
      // scaling by sl2 > 0 keeps the maximum where it is
      const float m_new = fmaxf(m_run, tmax * sl2);
      alpha = exp2_fast(m_run - m_new);   // 0 while m_run is -inf
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = exp2_fast(fmaf(s[t][i], sl2, -m_new));
          s[t][i] = p;
          psum += p;
        }
      m_run = m_new;
    } else {
      // mask and maximum (log2 domain)
      float tmax = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb + t * 16 + g * 4 + i;
          const float v = (key <= qpos) ? s[t][i] : -INFINITY;
          s[t][i] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, lane_xor16(tmax));
      tmax = fmaxf(tmax, lane_xor32(tmax));
      const float m_new = fmaxf(m_run, tmax * sl2);
      alpha = (m_new == -INFINITY) ? 1.f : exp2_fast(m_run - m_new);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = (s[t][i] == -INFINITY) ? 0.f : exp2_fast(fmaf(s[t][i], sl2, -m_new));
          s[t][i] = p;
          psum += p;
        }
      m_run = m_new;
    }
    psum += lane_xor16(psum);
    psum += lane_xor32(psum);
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] *= alpha;

    // O^T += V^T P^T over this wavefront's 32 keys (sub-tiles 0 and 1)
    vec8 pf;
    {
      const uint32_t w0 = Half16<T>::pack2(s[0][0], s[0][1]);
      const uint32_t w1 = Half16<T>::pack2(s[0][2], s[0][3]);
      const uint32_t w2 = Half16<T>::pack2(s[1][0], s[1][1]);
      const uint32_t w3 = Half16<T>::pack2(s[1][2], s[1][3]);
      pf = __builtin_bit_cast(vec8, make_uint4(w0, w1, w2, w3));
    }
    // V^T fragment of dims 16 d .. 16 d + 15: lane l needs dim 16 d + l % 16
    // at keys e .. e + 3 and e + 16 .. e + 19 (e = 32 kh + 4 g), the key
    // order of pf.  A transposing read hands lane j of a 16-lane group
    // element j % 4 of rows j / 4 + 4 i (i = 0..3) of the 16 rows of four
    // 16-bit values its lanes address; lane j addresses key e + j / 4,
    // dims 16 d + 4 (j % 4) .. + 3, so it receives dim 16 d + j of keys
    // e .. e + 3 in order.
    {
      const int jj = lane & 15, e = kh * 32 + g * 4;
      const bf16_t* vb = sV + (e + (jj >> 2)) * VS + (jj & 3) * 4;
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        typedef short v4s __attribute__((ext_vector_type(4)));
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(vb + d * 16));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(vb + 16 * VS + d * 16));
        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
        const vec8 vf = __builtin_bit_cast(vec8, make_uint4(l2.x, l2.y, h2.x, h2.y));
        o[d] = Half16<T>::mfma(vf, pf, o[d]);
      }
    }
  }
  }

  // The two wavefronts of a query sub-tile merge in key order: the second
  // leaves its state in LDS, the first folds it into its own and writes.
  float* mr = sM + ((size_t)qs * 64 + lane) * MS;
  if (kh == 1) {
#pragma unroll
    for (int d = 0; d < ND; ++d)
      *reinterpret_cast<float4*>(mr + 4 * d) = make_float4(o[d][0], o[d][1], o[d][2], o[d][3]);
    *reinterpret_cast<float2*>(mr + 4 * ND) = make_float2(m_run, l_run);
  }
  __syncthreads();
  if (kh == 1) return;
  {
    const float2 ml = *reinterpret_cast<const float2*>(mr + 4 * ND);
    const float mn = fmaxf(m_run, ml.x);
    if (mn != -INFINITY) {
      const float a = (m_run == -INFINITY) ? 0.f : exp2_fast(m_run - mn);
      const float c2 = (ml.x == -INFINITY) ? 0.f : exp2_fast(ml.x - mn);
      l_run = l_run * a + ml.y * c2;
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const float4 o2 = *reinterpret_cast<const float4*>(mr + 4 * d);
        o[d][0] = o[d][0] * a + o2.x * c2;
        o[d][1] = o[d][1] * a + o2.y * c2;
        o[d][2] = o[d][2] * a + o2.z * c2;
        o[d][3] = o[d][3] * a + o2.w * c2;
      }
      m_run = mn;
    }
  }

  if (nch > 1) {   // a chunk of a split tile: leave (m, l, o) for the merge
    if (qrow < len) {
      // record: m, l, 2 spare, o[HS] (16-byte aligned)
      float* pp = part + (((size_t)h * Tb + qrow) * nsplit + chunk) * (HS + 4);
      if (g == 0) { pp[0] = m_run; pp[1] = l_run; }
#pragma unroll
      for (int d = 0; d < ND; ++d)
        *reinterpret_cast<float4*>(pp + 4 + d * 16 + g * 4) =
            make_float4(o[d][0], o[d][1], o[d][2], o[d][3]);
    }
    return;
  }
  if (qrow < len) {
    const float inv = 1.f / l_run;
    T* yp = y + (row0 + qrow) * ldy + h * HS;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const uint32_t w0 = Half16<T>::pack2(o[d][0] * inv, o[d][1] * inv);
      const uint32_t w1 = Half16<T>::pack2(o[d][2] * inv, o[d][3] * inv);
      *reinterpret_cast<uint2*>(yp + d * 16 + g * 4) = make_uint2(w0, w1);
    }
  }
}

// Merge of a split query tile's chunks (batch 1): one wavefront per (row,
// head), four rows per workgroup; lane d merges dimension d over the chunks
// in chunk order.  Rows whose tile had a single chunk were written directly.
constexpr int kMergeRows = 4;
template <class T, int HS>
__global__ __launch_bounds__(64 * kMergeRows) void attn_prefill_merge(
    const float* __restrict__ part, int len, int past, int Tb, int kch, int nsplit,
    T* __restrict__ y, int ldy, int r0) {
  const int row = r0 + (int)blockIdx.x * kMergeRows + (int)(threadIdx.x >> 6);
  const int h = blockIdx.y, d = threadIdx.x & 63;
  if (row >= len || d >= HS) return;
  const int q0 = (row / 64) * 64;
  const int nkt_all = (past + min(q0 + 63, len - 1)) / 64 + 1;
  const int nch = (nkt_all + kch - 1) / kch;
  if (nch <= 1) return;
  const float* pp = part + ((size_t)h * Tb + row) * nsplit * (HS + 4);
  float m = pp[0], l = pp[1], o = pp[4 + d];
  for (int c = 1; c < nch; ++c) {
    const float* pc = pp + c * (HS + 4);
    merge_state(m, l, &o, pc[0], pc[1], &pc[4 + d], 1);
  }
  y[(size_t)row * ldy + h * HS + d] = from_f32<T>(o / l);
}

// ---------------------------------------------------------------------------
// Prefill, one thread per query row (any dtype; used for the fp32 model).
// ---------------------------------------------------------------------------
template <class T, int HS>
__global__ __launch_bounds__(64) void attn_prefill_simt(
    const T* __restrict__ q, int ldq, const T* __restrict__ kc,
    const T* __restrict__ vc, KvMap kvm, RowMap map, int H, int Tb, float scale,
    T* __restrict__ y, int ldy) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int len = map.off[b + 1] - map.off[b];
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= len) return;
  const int t = map.past[b] + i;        // position: sees keys 0 .. t
  const size_t row = (size_t)map.off[b] + i;
  const int slot = map.slot[b];
  const int64_t hoff = (int64_t)h * kv_hstride(kvm);
  float qv[HS], acc[HS];
#pragma unroll
  for (int d = 0; d < HS; ++d) {
    qv[d] = to_f32(q[row * ldq + h * HS + d]) * scale;
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  int64_t bb = -1;
  for (int u = 0; u <= t; ++u) {
    if (u % kPageTokens == 0) bb = kv_block_base(kvm, slot, u / kPageTokens);
    // an unmapped block reads as zeros
    const bool ok = bb >= 0;
    const size_t kr0 = ok ? (size_t)(bb + hoff + u % kPageTokens) * HS : 0;
    const T* kr = kc + kr0;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < HS; ++d) s = fmaf(qv[d], ok ? to_f32(kr[d]) : 0.f, s);
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);
    const float p = expf(s - m_new);
    l = l * alpha + p;
    const T* vr = vc + kr0;
#pragma unroll
    for (int d = 0; d < HS; ++d) acc[d] = acc[d] * alpha + p * (ok ? to_f32(vr[d]) : 0.f);
    m = m_new;
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int d = 0; d < HS; ++d) y[row * ldy + h * HS + d] = from_f32<T>(acc[d] * inv);
}

// ---------------------------------------------------------------------------
// Decode, split over key chunks.  256 threads = 4 wavefronts; a chunk has
// 64 keys, 16 per wavefront.  LPK = HS/8 lanes share one key (8 dims each),
// so a wavefront covers 64/LPK keys per pass.  Every lane group keeps its own
// running (max, sum, o[8]) and the groups, wavefronts and chunks are merged
// afterwards.
// ---------------------------------------------------------------------------
constexpr int kDecChunk = 64;

template <class T, int HS>
__global__ __launch_bounds__(256) void attn_decode_kernel(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
    KvMap kvm, const int32_t* __restrict__ pos, int H, int Tb, int nchunk, float scale,
    float* __restrict__ part) {
  constexpr int LPK = HS / 8;          // lanes per key
  constexpr int KPP = 64 / LPK;        // keys per wavefront pass
  constexpr int KPW = kDecChunk / 4;   // keys per wavefront
  constexpr int PS = HS + 2;           // partial record: m, l, o[HS]
  static_assert(kPageTokens % KPW == 0, "a wavefront's keys must lie in one cache block");
  __shared__ float sw[4][PS];

  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int C = H * HS;
  const int p = pos[b];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (p < 0 || chunk > p / kDecChunk) return;  // inactive row / empty chunk

  const int sub = lane % LPK;   // which 8 dims
  const int kgrp = lane / LPK;  // key slot within a pass
  const float sl2 = scale * kLog2e;
  // the wavefront's keys kw .. kw + KPW - 1 lie in one cache block (KPW
  // divides the block's 64 positions); an unmapped block reads as zeros
  const int kw = chunk * kDecChunk + wave * KPW;
  const int64_t bb = kw <= p ? kv_block_base(kvm, b, kw / kPageTokens) : -1;
  const size_t r0 = bb < 0 ? 0 : (size_t)(bb + (int64_t)h * kv_hstride(kvm)) * HS;
  const T* kbase = kc + r0;
  const T* vbase = vc + r0;

  // issue every K/V load of this lane first, then the query
  float kf[KPW / KPP][8], vf[KPW / KPP][8];
#pragma unroll
  for (int pass = 0; pass < KPW / KPP; ++pass) {
    const int u = kw + pass * KPP + kgrp;
    if (u <= p && bb >= 0) {
      if constexpr (sizeof(T) == 2) {
        Half16<T>::unpack8(*reinterpret_cast<const uint4*>(kbase + (size_t)(u % kPageTokens) * HS + sub * 8), kf[pass]);
        Half16<T>::unpack8(*reinterpret_cast<const uint4*>(vbase + (size_t)(u % kPageTokens) * HS + sub * 8), vf[pass]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          kf[pass][j] = to_f32(kbase[(size_t)(u % kPageTokens) * HS + sub * 8 + j]);
          vf[pass][j] = to_f32(vbase[(size_t)(u % kPageTokens) * HS + sub * 8 + j]);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) kf[pass][j] = vf[pass][j] = 0.f;
    }
  }
  float qv[8];
  {
    const T* qp = q + (size_t)b * C + h * HS + sub * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) qv[j] = to_f32(qp[j]) * sl2;
  }

  float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = 0.f;
#pragma unroll
  for (int pass = 0; pass < KPW / KPP; ++pass) {
    const int u = kw + pass * KPP + kgrp;
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s = fmaf(qv[j], kf[pass][j], s);
#pragma unroll
    for (int o2 = 1; o2 < LPK; o2 <<= 1) s += __shfl_xor(s, o2, 64);
    if (u <= p) {
      const float mn = fmaxf(m, s);
      const float a = exp2_fast(m - mn);  // m = -inf gives 0
      const float pr = exp2_fast(s - mn);
      l = l * a + pr;
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = o[j] * a + pr * vf[pass][j];
      m = mn;
    }
  }
  // merge the key slots of the wavefront (lanes differing in bits >= LPK)
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    const float l2 = __shfl_xor(l, off, 64);
    float o2[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o2[j] = __shfl_xor(o[j], off, 64);
    merge_state(m, l, o, m2, l2, o2, 8);
  }
  if (lane < LPK) {
    if (lane == 0) {
      sw[wave][0] = m;
      sw[wave][1] = l;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) sw[wave][2 + sub * 8 + j] = o[j];
  }
  __syncthreads();
  float* rec = part + (((size_t)b * H + h) * nchunk + chunk) * PS;
  if (tid < HS) {
    float mm = -INFINITY, ll = 0.f, oo = 0.f;
    for (int w = 0; w < 4; ++w) merge_state(mm, ll, &oo, sw[w][0], sw[w][1], &sw[w][2 + tid], 1);
    rec[2 + tid] = oo;
    if (tid == 0) {
      rec[0] = mm;
      rec[1] = ll;
    }
  }
}

// Merge the chunk records of one (sequence, head) in chunk order.  Runs as
// its own launch, so the records of every chunk are visible without fences.
template <class T, int HS>
__global__ __launch_bounds__(64) void attn_decode_combine(
    const float* __restrict__ part, const int32_t* __restrict__ pos, int H,
    int nchunk, T* __restrict__ y) {
  constexpr int PS = HS + 2;
  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int C = H * HS;
  const int p = pos[b];
  if (t >= HS) return;
  if (p < 0) {  // inactive sequence: a zero row keeps later layers finite
    y[(size_t)b * C + h * HS + t] = from_f32<T>(0.f);
    return;
  }
  const int nact = p / kDecChunk + 1;
  const float* base = part + ((size_t)b * H + h) * nchunk * PS;
  float mm = -INFINITY, ll = 0.f, oo = 0.f;
  for (int c0 = 0; c0 < nact; c0 += 8) {
    float rm[8], rl[8], ro[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float* r = base + (size_t)(c0 + u) * PS;
      const bool ok = c0 + u < nact;
      rm[u] = ok ? r[0] : -INFINITY;
      rl[u] = ok ? r[1] : 0.f;
      ro[u] = ok ? r[2 + t] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) merge_state(mm, ll, &oo, rm[u], rl[u], &ro[u], 1);
  }
  y[(size_t)b * C + h * HS + t] = from_f32<T>(oo / ll);
}

// ---------------------------------------------------------------------------
// Decode with many (sequence, head) pairs (batched steps): one workgroup per
// pair streams every key of its sequence and writes y itself, so the grid
// holds no empty chunks and no merge launch follows.  Keys go in groups of
// GK = 2 * (64 / LPK) (16 at hs 64): wavefront w takes groups w, w + 4, ...,
// four groups in flight, each lane group keeping its own running (max, sum,
// o[8]); lanes, then wavefronts (in order) are merged at the end.  A group
// lies in one 64-position cache block; an unmapped block reads as zeros.
// ---------------------------------------------------------------------------
// One group of GK keys: the K and V rows of this lane's two passes.
struct DecGroup {
  uint4 k0, k1, v0, v1;
};

template <class T, int HS>
__global__ __launch_bounds__(256) void attn_decode_rows_kernel(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
    KvMap kvm, const int32_t* __restrict__ pos, int H, float scale, T* __restrict__ y) {
  static_assert(sizeof(T) == 2, "16-bit caches only");
  constexpr int LPK = HS / 8;          // lanes per key
  constexpr int KPP = 64 / LPK;        // keys per wavefront pass
  constexpr int GK = 2 * KPP;          // keys per group (two passes)
  static_assert(kPageTokens % GK == 0, "a group must lie in one cache block");
  __shared__ float sw[4][HS + 2];

  const int h = blockIdx.x, b = blockIdx.y;
  const int C = H * HS;
  const int p = pos[b];
  // (the wavefront index as a uniform value, so that the block-table reads
  // are scalar loads, which do not wait behind the K/V loads in flight)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  T* yo = y + (size_t)b * C + h * HS;
  if (p < 0) {   // inactive sequence: a zero row keeps later layers finite
    if (tid < HS) yo[tid] = from_f32<T>(0.f);
    return;
  }
  const int sub = lane % LPK, kgrp = lane / LPK;
  const int ng = p / GK + 1;                        // groups holding keys 0..p
  const int nmine = ng > wave ? (ng - wave + 3) / 4 : 0;
  const int64_t hoff = (int64_t)h * kv_hstride(kvm);
  const float sl2 = scale * kLog2e;

  // this wavefront's i-th group (zeros past the last one), through
  // range-checked buffer loads over the group's 64-position cache block:
  // keys past p, groups past the last and unmapped blocks read zeros, and
  // every load is issued on every path (guarded loads were each waited for
  // before the next was issued, which emptied the four-group pipeline)
  constexpr uint32_t kOut = 0x80000000u;
  auto load = [&](int i) {
    DecGroup g;
    const int g0 = (wave + 4 * i) * GK;
    const int64_t bb = i < nmine ? kv_block_base(kvm, b, g0 / kPageTokens) : -1;
    const size_t r0 = bb < 0 ? 0 : (size_t)(bb + hoff) * HS;
    const int nrec = bb < 0 ? 0 : kPageTokens * HS * 2;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(kc + r0), (short)0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(vc + r0), (short)0, nrec, 0x00020000);
    const int u0 = g0 + kgrp, u1 = g0 + KPP + kgrp;
    const uint32_t o0 = u0 <= p ? ((uint32_t)(u0 % kPageTokens) * HS + sub * 8) * 2u : kOut;
    const uint32_t o1 = u1 <= p ? ((uint32_t)(u1 % kPageTokens) * HS + sub * 8) * 2u : kOut;
    g.k0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, o0, 0, 0));
    g.v0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, o0, 0, 0));
    g.k1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, o1, 0, 0));
    g.v1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, o1, 0, 0));
    return g;
  };
  // the query first: waiting for it then does not wait for the groups
  const uint4 qraw = *reinterpret_cast<const uint4*>(q + (size_t)b * C + h * HS + sub * 8);
  DecGroup g0 = load(0), g1 = load(1), g2 = load(2), g3 = load(3);
  float qv[8];
  Half16<T>::unpack8(qraw, qv);
#pragma unroll
  for (int j = 0; j < 8; ++j) qv[j] *= sl2;
  float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = 0.f;
  auto pass = [&](const uint4& kraw, const uint4& vraw, int u) {
    float kf[8];
    Half16<T>::unpack8(kraw, kf);
    float sc = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) sc = fmaf(qv[j], kf[j], sc);
    // sum over the key's LPK lanes (DPP; every lane of the group gets the
    // same bits: each step adds a symmetric partner)
    sc += lane_xor1(sc);
    sc += lane_xor2(sc);
    if constexpr (LPK == 8) sc += lane_mirror8(sc);
    if (u <= p) {
      float vf[8];
      Half16<T>::unpack8(vraw, vf);
      const float mn = fmaxf(m, sc);
      const float a = exp2_fast(m - mn);  // m = -inf gives 0
      const float pr = exp2_fast(sc - mn);
      l = l * a + pr;
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = o[j] * a + pr * vf[j];
      m = mn;
    }
  };
  auto group = [&](const DecGroup& g, int i) {
    const int gk = (wave + 4 * i) * GK;
    pass(g.k0, g.v0, gk + kgrp);
    pass(g.k1, g.v1, gk + KPP + kgrp);
  };
  // four groups in flight: process one, then fetch the one four ahead, in
  // whole rounds of four (groups past the last hold no key at or below p
  // and change nothing), so the loop has one exit and the wait before each
  // group leaves the three younger groups in flight
  const int nround = (nmine + 3) / 4;
  for (int r = 0; r < nround; ++r) {
    const int i = 4 * r;
    group(g0, i);
    g0 = load(i + 4);
    group(g1, i + 1);
    g1 = load(i + 5);
    group(g2, i + 2);
    g2 = load(i + 6);
    group(g3, i + 3);
    g3 = load(i + 7);
  }
  // merge the key slots of the wavefront (lanes differing in bits >= LPK),
  // through DPP / permlane moves
  auto xlane = [](float v, int off) {
    return off == 4 ? __shfl_xor(v, 4, 64)   // (head size 32 only)
                    : off == 8 ? lane_xor8(v) : off == 16 ? lane_xor16(v) : lane_xor32(v);
  };
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    const float m2 = xlane(m, off);
    const float l2 = xlane(l, off);
    float o2[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o2[j] = xlane(o[j], off);
    merge_state(m, l, o, m2, l2, o2, 8);
  }
  if (lane < LPK) {
    if (lane == 0) {
      sw[wave][0] = m;
      sw[wave][1] = l;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) sw[wave][2 + sub * 8 + j] = o[j];
  }
  __syncthreads();
  if (tid < HS) {
    float mm = -INFINITY, ll = 0.f, oo = 0.f;
    for (int w = 0; w < 4; ++w) merge_state(mm, ll, &oo, sw[w][0], sw[w][1], &sw[w][2 + tid], 1);
    yo[tid] = from_f32<T>(oo / ll);
  }
}

// ---------------------------------------------------------------------------
int attn_prefill_split_chunks(int Tb) { return ((Tb + 63) / 64 + kPrefillKch - 1) / kPrefillKch; }

template <class T>
static void launch_attn_prefill_h(const T* q, int ldq, const T* kc, const T* vc,
                                  const KvMap& kv, const RowMap& map, int maxlen, int H,
                                  int hs, int Tb,
                                  T* y, int ldy, float* part, hipStream_t s) {
  const float scale = 1.0f / sqrtf((float)hs);
  const int ntiles = (maxlen + 63) / 64;
  // one sequence with few workgroups: split the long query tiles' keys
  const int past = map.past[0];
  const int nkt_max = (past + maxlen - 1) / 64 + 1;
  const bool split = part && map.B == 1 && nkt_max > kPrefillKch && ntiles * H < 256;
  const int kch = split ? kPrefillKch : 0;
  const int nsplit = split ? (nkt_max + kPrefillKch - 1) / kPrefillKch : 1;
  dim3 grid(ntiles * nsplit, H, map.B);
  PrefillOrder ord;
  ord.n = 0;
  if (split) {
    // every (query tile, chunk) pair of a head with its key-tile count,
    // longest first (ties: later tiles first); the heads interleave
    int size[kPrefillOrderMax];
    int n = 0;
    for (int qt = ntiles - 1; qt >= 0 && n >= 0; --qt) {
      const int nkt_all = (past + min(qt * 64 + 63, maxlen - 1)) / 64 + 1;
      for (int c = 0; c * kch < nkt_all; ++c) {
        if (n == kPrefillOrderMax || qt > 0xFF || c > 0xFF) { n = -1; break; }
        size[n] = min(kch, nkt_all - c * kch);
        ord.it[n++] = (uint16_t)(qt | (c << 8));
      }
    }
    if (n > 0) {
      for (int i = 1; i < n; ++i)   // stable insertion sort, size descending
        for (int j = i; j > 0 && size[j] > size[j - 1]; --j) {
          std::swap(size[j], size[j - 1]);
          std::swap(ord.it[j], ord.it[j - 1]);
        }
      ord.n = n;
      grid = dim3(n * H, 1, 1);
    }
  }
  if (hs == 64)
    attn_prefill_mfma<T, 64><<<grid, 64 * kPrefillWaves, 0, s>>>(q, ldq, kc, vc, kv, map, H, Tb, scale, y, ldy,
                                                   kch, nsplit, part, ord);
  else
    attn_prefill_mfma<T, 32><<<grid, 64 * kPrefillWaves, 0, s>>>(q, ldq, kc, vc, kv, map, H, Tb, scale, y, ldy,
                                                   kch, nsplit, part, ord);
  if (split) {
    // rows of single-chunk tiles need no merge: start at the first tile
    // with more than one chunk
    int first = 0;
    while (first < ntiles && (past + min(first * 64 + 63, maxlen - 1)) / 64 + 1 <= kch) ++first;
    const int r0 = first * 64;
    const dim3 mgrid((maxlen - r0 + kMergeRows - 1) / kMergeRows, H);
    if (hs == 64)
      attn_prefill_merge<T, 64><<<mgrid, 64 * kMergeRows, 0, s>>>(part, maxlen, past, Tb, kch,
                                                                  nsplit, y, ldy, r0);
    else
      attn_prefill_merge<T, 32><<<mgrid, 64 * kMergeRows, 0, s>>>(part, maxlen, past, Tb, kch,
                                                                  nsplit, y, ldy, r0);
  }
}

void launch_attn_prefill(int dtype, const void* q, int ldq, const void* kc,
                         const void* vc, const KvMap& kv, const RowMap& map, int maxlen,
                         int H, int hs, int Tb, void* y, int ldy, float* part,
                         hipStream_t s) {
  if (dtype == NGPT_BF16) {
    launch_attn_prefill_h<bf16_t>((const bf16_t*)q, ldq, (const bf16_t*)kc, (const bf16_t*)vc,
                                  kv, map, maxlen, H, hs, Tb, (bf16_t*)y, ldy, part, s);
  } else if (dtype == NGPT_F16) {
    launch_attn_prefill_h<f16_t>((const f16_t*)q, ldq, (const f16_t*)kc, (const f16_t*)vc,
                                 kv, map, maxlen, H, hs, Tb, (f16_t*)y, ldy, part, s);
  } else {
    const float scale = 1.0f / sqrtf((float)hs);
    const int ntiles = (maxlen + 63) / 64;
    const dim3 grid(ntiles, H, map.B);
    const float* qq = (const float*)q;
    if (hs == 64)
      attn_prefill_simt<float, 64><<<grid, 64, 0, s>>>(qq, ldq, (const float*)kc,
          (const float*)vc, kv, map, H, Tb, scale, (float*)y, ldy);
    else
      attn_prefill_simt<float, 32><<<grid, 64, 0, s>>>(qq, ldq, (const float*)kc,
          (const float*)vc, kv, map, H, Tb, scale, (float*)y, ldy);
  }
}

int attn_decode_chunks(int Tb) { return (Tb + kDecChunk - 1) / kDecChunk; }

// (sequence, head) pairs from which a merged decode step takes one
// workgroup per pair rather than one per 64-key chunk
constexpr int kDecodeRowsMinPairs = 256;

int attn_decode_chunk_keys() { return kDecChunk; }

template <class T>
static void launch_attn_decode_t(const T* q, const T* kc, const T* vc, const KvMap& kv,
                                 const int32_t* pos, int B, int H, int hs, int Tb,
                                 float* part, T* y, bool merge_into_y, hipStream_t s) {
  const float scale = 1.0f / sqrtf((float)hs);
  if constexpr (sizeof(T) == 2) {
    // enough (sequence, head) pairs to fill the chip: one workgroup each
    if (merge_into_y && B * H >= kDecodeRowsMinPairs) {
      const dim3 rgrid(H, B);
      if (hs == 64)
        attn_decode_rows_kernel<T, 64><<<rgrid, 256, 0, s>>>(q, kc, vc, kv, pos, H, scale, y);
      else
        attn_decode_rows_kernel<T, 32><<<rgrid, 256, 0, s>>>(q, kc, vc, kv, pos, H, scale, y);
      return;
    }
  }
  const int nchunk = attn_decode_chunks(Tb);
  const dim3 grid(nchunk, H, B), cgrid(H, B);
  if (hs == 64) {
    attn_decode_kernel<T, 64><<<grid, 256, 0, s>>>(q, kc, vc, kv, pos, H, Tb, nchunk, scale, part);
    if (merge_into_y) attn_decode_combine<T, 64><<<cgrid, 64, 0, s>>>(part, pos, H, nchunk, y);
  } else {
    attn_decode_kernel<T, 32><<<grid, 256, 0, s>>>(q, kc, vc, kv, pos, H, Tb, nchunk, scale, part);
    if (merge_into_y) attn_decode_combine<T, 32><<<cgrid, 64, 0, s>>>(part, pos, H, nchunk, y);
  }
}

void launch_attn_decode(int dtype, const void* q, const void* kc,
                        const void* vc, const KvMap& kv, const int32_t* pos, int B, int H,
                        int hs, int Tb, float* part, void* y,
                        bool merge_into_y, hipStream_t s) {
  if (dtype == NGPT_BF16) {
    launch_attn_decode_t<bf16_t>((const bf16_t*)q, (const bf16_t*)kc, (const bf16_t*)vc, kv,
                                 pos, B, H, hs, Tb, part, (bf16_t*)y, merge_into_y, s);
  } else if (dtype == NGPT_F16) {
    launch_attn_decode_t<f16_t>((const f16_t*)q, (const f16_t*)kc, (const f16_t*)vc, kv,
                                pos, B, H, hs, Tb, part, (f16_t*)y, merge_into_y, s);
  } else {
    launch_attn_decode_t<float>((const float*)q, (const float*)kc, (const float*)vc, kv,
                                pos, B, H, hs, Tb, part, (float*)y, merge_into_y, s);
  }
}

}  // namespace ngpt
