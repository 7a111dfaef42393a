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
//   attn_prefill_mfma   bf16, one workgroup per (64-row query tile, head,
//                       sequence); K/V tiles of 64 keys staged in LDS;
//                       scores and P*V on MFMA; online (running max / sum)
//                       softmax in fp32; tiles above the diagonal skipped.
//   attn_prefill_simt   one thread per query row (fp32 model).
//   attn_decode         one query per sequence, split over 64-key chunks;
//                       each workgroup leaves (max, sum, o) for its chunk and
//                       a second small launch merges the chunks in order.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace ngpt {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kPrefillKch = 4;   // key tiles per chunk when a prefill tile is split

// ---------------------------------------------------------------------------
// Prefill, bf16 MFMA.  Scores are formed transposed, S^T = K Q^T, so that a
// lane holds one query column: lane l owns query q0 + 16*wave + (l % 16) and
// keys 16*t + 4*(l/16) + i (i < 4) of each 16-key sub-tile t.  The running
// softmax statistics are then per lane.  The output is formed as
// O^T = V^T P^T; P^T is fed straight from the score registers, with V^T read
// from a transposed LDS copy in the same key order.
// ---------------------------------------------------------------------------
//
// Key split (kch > 0, batch 1): a query tile that meets more than kch key
// tiles is split into chunks of kch key tiles, one workgroup each; such a
// chunk leaves its rows' unnormalised state (m, l, o) in part, and
// attn_prefill_merge combines the chunks in order.  Workgroup x takes query
// tile ntiles - 1 - x / nsplit (heavy tiles first) and chunk x % nsplit.
template <int HS>
__global__ __launch_bounds__(256) void attn_prefill_mfma(
    const bf16_t* __restrict__ q, int ldq, const bf16_t* __restrict__ kc,
    const bf16_t* __restrict__ vc, RowMap map, int H, int Tb, float scale,
    bf16_t* __restrict__ y, int ldy, int kch, int nsplit, float* __restrict__ part) {
  constexpr int KT = 64;             // keys per tile
  constexpr int KS = HS + 8;         // sK row stride (elements)
  constexpr int VS = KT + 8;         // sVt row stride (elements)
  constexpr int NKK = HS / 32;       // MFMA steps over the head dimension
  constexpr int ND = HS / 16;        // 16-row output sub-tiles over hs
  __shared__ __attribute__((aligned(16))) bf16_t sK[KT * KS];
  __shared__ __attribute__((aligned(16))) bf16_t sVt[HS * VS];

  const int b = blockIdx.z, h = blockIdx.y;
  const int len = map.off[b + 1] - map.off[b];
  const int ntiles = (len + 63) / 64;
  const int qt = ntiles - 1 - (kch > 0 ? (int)blockIdx.x / nsplit : (int)blockIdx.x);
  if (qt < 0) return;
  // key tiles [kt0, kt1) of this workgroup
  const int nch = kch > 0 ? (qt + kch) / kch : 1;
  const int chunk = kch > 0 ? (int)blockIdx.x % nsplit : 0;
  if (chunk >= nch) return;
  const int kt0 = kch > 0 ? chunk * kch : 0;
  const int q0 = qt * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4;                       // lane group 0..3
  const int qrow = q0 + wave * 16 + (lane & 15);  // this lane's query
  const size_t row0 = (size_t)map.off[b];
  const bf16_t* kbase = kc + ((size_t)b * H + h) * Tb * HS;
  const bf16_t* vbase = vc + ((size_t)b * H + h) * Tb * HS;

  // Q^T operand: column = this lane's query, K-values = dims 8g.. (+32 kk)
  bf16x8_t qf[NKK];
  {
    const int qr = qrow < len ? qrow : len - 1;
    const bf16_t* qp = q + (row0 + qr) * ldq + h * HS;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[kk] = *reinterpret_cast<const bf16x8_t*>(qp + kk * 32 + g * 8);
  }

  const float sl2 = scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t o[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) o[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int last_key = min(q0 + 63, len - 1);
  const int nkt = (nch > 1 ? min(kt0 + kch, qt + 1) : last_key / KT + 1) - kt0;
  // Staging work item: a pair of keys (2kp, 2kp+1) x 8 dims; K goes to LDS
  // key-major, V transposed (dim-major) with the two keys packed in 32 bits.
  // S tiles are in flight in registers.  The loads are range-checked buffer
  // loads issued on every path: keys at or past len (whose cache rows may
  // hold anything) and tiles past the block read zeros.
  constexpr int ITEMS = (KT / 2) * (HS / 8);
  constexpr int IPT = (ITEMS + 255) / 256;
  constexpr int S = 4;
  constexpr uint32_t kOut = 0x80000000u;
  const uint32_t blk = (uint32_t)Tb * HS * 2u;
  const __amdgpu_buffer_rsrc_t rks = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(kbase), (short)0, (int)blk, 0x00020000);
  const __amdgpu_buffer_rsrc_t rvs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(vbase), (short)0, (int)blk, 0x00020000);
  uint4 rk[S][IPT][2], rv[S][IPT][2];
  auto load_tile = [&](int st, int k0) {
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int c = tid + it * 256;
      const int kp = c / (HS / 8), d0 = (c % (HS / 8)) * 8;
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        const int key = k0 + 2 * kp + e2;
        const uint32_t off = (c < ITEMS && key < len) ? ((uint32_t)key * HS + d0) * 2u : kOut;
        rk[st][it][e2] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rks, off, 0, 0));
        rv[st][it][e2] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rvs, off, 0, 0));
      }
    }
  };
  auto store_tile = [&](int st) {
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int c = tid + it * 256;
      if (c >= ITEMS) break;
      const int kp = c / (HS / 8), d0 = (c % (HS / 8)) * 8;
      *reinterpret_cast<uint4*>(sK + (2 * kp) * KS + d0) = rk[st][it][0];
      *reinterpret_cast<uint4*>(sK + (2 * kp + 1) * KS + d0) = rk[st][it][1];
      const uint32_t a[4] = {rv[st][it][0].x, rv[st][it][0].y, rv[st][it][0].z, rv[st][it][0].w};
      const uint32_t b2[4] = {rv[st][it][1].x, rv[st][it][1].y, rv[st][it][1].z, rv[st][it][1].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // dims d0+2j (low halves) and d0+2j+1 (high halves) of the two keys
        *reinterpret_cast<uint32_t*>(sVt + (d0 + 2 * j) * VS + 2 * kp) =
            (a[j] & 0xFFFFu) | (b2[j] << 16);
        *reinterpret_cast<uint32_t*>(sVt + (d0 + 2 * j + 1) * VS + 2 * kp) =
            (a[j] >> 16) | (b2[j] & 0xFFFF0000u);
      }
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
    if (t0 + st >= nkt) continue;   // padding of the last group (uniform)

    // S^T for 4 sub-tiles of 16 keys
    f32x4_t s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      s[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(
            sK + (t * 16 + (lane & 15)) * KS + kk * 32 + g * 8);
        s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[kk], s[t], 0, 0, 0);
      }
    }
    // mask and tile maximum (log2 domain)
    float tmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + t * 16 + g * 4 + i;
        const float v = (key <= qrow) ? s[t][i] * sl2 : -INFINITY;
        s[t][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, lane_xor16(tmax));
    tmax = fmaxf(tmax, lane_xor32(tmax));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : exp2_fast(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = (s[t][i] == -INFINITY) ? 0.f : exp2_fast(s[t][i] - m_new);
        s[t][i] = p;
        psum += p;
      }
    psum += lane_xor16(psum);
    psum += lane_xor32(psum);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] *= alpha;

    // O^T += V^T P^T, 32 keys per MFMA: sub-tiles 2u and 2u+1
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x8_t pf;
      {
        const uint32_t w0 = pack_bf16x2(s[2 * u][0], s[2 * u][1]);
        const uint32_t w1 = pack_bf16x2(s[2 * u][2], s[2 * u][3]);
        const uint32_t w2 = pack_bf16x2(s[2 * u + 1][0], s[2 * u + 1][1]);
        const uint32_t w3 = pack_bf16x2(s[2 * u + 1][2], s[2 * u + 1][3]);
        pf = __builtin_bit_cast(bf16x8_t, make_uint4(w0, w1, w2, w3));
      }
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const bf16_t* vr = sVt + (d * 16 + (lane & 15)) * VS + u * 32 + g * 4;
        const uint2 lo = *reinterpret_cast<const uint2*>(vr);
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + 16);
        const bf16x8_t vf =
            __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
        o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, o[d], 0, 0, 0);
      }
    }
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
    bf16_t* yp = y + (row0 + qrow) * ldy + h * HS;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const uint32_t w0 = pack_bf16x2(o[d][0] * inv, o[d][1] * inv);
      const uint32_t w1 = pack_bf16x2(o[d][2] * inv, o[d][3] * inv);
      *reinterpret_cast<uint2*>(yp + d * 16 + g * 4) = make_uint2(w0, w1);
    }
  }
}

// Merge of a split query tile's chunks (batch 1): one wavefront per (row,
// head), four rows per workgroup; lane d merges dimension d over the chunks
// in chunk order.
constexpr int kMergeRows = 4;
template <int HS>
__global__ __launch_bounds__(64 * kMergeRows) void attn_prefill_merge(
    const float* __restrict__ part, int len, int Tb, int kch, int nsplit,
    bf16_t* __restrict__ y, int ldy) {
  const int row = kch * 64 + (int)blockIdx.x * kMergeRows + (int)(threadIdx.x >> 6);
  const int h = blockIdx.y, d = threadIdx.x & 63;
  if (row >= len || d >= HS) return;
  const int nch = (row / 64 + kch) / kch;
  const float* pp = part + ((size_t)h * Tb + row) * nsplit * (HS + 4);
  float m = pp[0], l = pp[1], o = pp[4 + d];
  for (int c = 1; c < nch; ++c) {
    const float* pc = pp + c * (HS + 4);
    merge_state(m, l, &o, pc[0], pc[1], &pc[4 + d], 1);
  }
  y[(size_t)row * ldy + h * HS + d] = f32_to_bf16(o / l);
}

// ---------------------------------------------------------------------------
// Prefill, one thread per query row (any dtype; used for the fp32 model).
// ---------------------------------------------------------------------------
template <class T, int HS>
__global__ __launch_bounds__(64) void attn_prefill_simt(
    const T* __restrict__ q, int ldq, const T* __restrict__ kc,
    const T* __restrict__ vc, RowMap map, int H, int Tb, float scale,
    T* __restrict__ y, int ldy) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int len = map.off[b + 1] - map.off[b];
  const int t = blockIdx.x * 64 + threadIdx.x;
  if (t >= len) return;
  const size_t row = (size_t)map.off[b] + t;
  const T* kbase = kc + ((size_t)b * H + h) * Tb * HS;
  const T* vbase = vc + ((size_t)b * H + h) * Tb * HS;
  float qv[HS], acc[HS];
#pragma unroll
  for (int d = 0; d < HS; ++d) {
    qv[d] = to_f32(q[row * ldq + h * HS + d]) * scale;
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int u = 0; u <= t; ++u) {
    const T* kr = kbase + (size_t)u * HS;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < HS; ++d) s = fmaf(qv[d], to_f32(kr[d]), s);
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);
    const float p = expf(s - m_new);
    l = l * alpha + p;
    const T* vr = vbase + (size_t)u * HS;
#pragma unroll
    for (int d = 0; d < HS; ++d) acc[d] = acc[d] * alpha + p * to_f32(vr[d]);
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
    const int32_t* __restrict__ pos, int H, int Tb, int nchunk, float scale,
    float* __restrict__ part) {
  constexpr int LPK = HS / 8;          // lanes per key
  constexpr int KPP = 64 / LPK;        // keys per wavefront pass
  constexpr int KPW = kDecChunk / 4;   // keys per wavefront
  constexpr int PS = HS + 2;           // partial record: m, l, o[HS]
  __shared__ float sw[4][PS];

  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int C = H * HS;
  const int p = pos[b];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (p < 0 || chunk > p / kDecChunk) return;  // inactive row / empty chunk

  const int sub = lane % LPK;   // which 8 dims
  const int kgrp = lane / LPK;  // key slot within a pass
  const float sl2 = scale * kLog2e;
  const T* kbase = kc + ((size_t)b * H + h) * Tb * HS;
  const T* vbase = vc + ((size_t)b * H + h) * Tb * HS;

  // issue every K/V load of this lane first, then the query
  const int kw = chunk * kDecChunk + wave * KPW;
  float kf[KPW / KPP][8], vf[KPW / KPP][8];
#pragma unroll
  for (int pass = 0; pass < KPW / KPP; ++pass) {
    const int u = kw + pass * KPP + kgrp;
    if (u <= p) {
      if constexpr (sizeof(T) == 2) {
        bf16x8_to_f32(*reinterpret_cast<const uint4*>(kbase + (size_t)u * HS + sub * 8), kf[pass]);
        bf16x8_to_f32(*reinterpret_cast<const uint4*>(vbase + (size_t)u * HS + sub * 8), vf[pass]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          kf[pass][j] = to_f32(kbase[(size_t)u * HS + sub * 8 + j]);
          vf[pass][j] = to_f32(vbase[(size_t)u * HS + sub * 8 + j]);
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
int attn_prefill_split_chunks(int Tb) { return ((Tb + 63) / 64 + kPrefillKch - 1) / kPrefillKch; }

void launch_attn_prefill(int dtype, const void* q, int ldq, const void* kc,
                         const void* vc, const RowMap& map, int maxlen, int H,
                         int hs, int Tb, void* y, int ldy, float* part, hipStream_t s) {
  const float scale = 1.0f / sqrtf((float)hs);
  const int ntiles = (maxlen + 63) / 64;
  if (dtype == NGPT_BF16) {
    const bf16_t* qq = (const bf16_t*)q;
    // one sequence with few workgroups: split the long query tiles' keys
    const bool split = part && map.B == 1 && ntiles > kPrefillKch && ntiles * H < 256;
    const int kch = split ? kPrefillKch : 0;
    const int nsplit = split ? (ntiles + kPrefillKch - 1) / kPrefillKch : 1;
    const dim3 grid(ntiles * nsplit, H, map.B);
    if (hs == 64)
      attn_prefill_mfma<64><<<grid, 256, 0, s>>>(qq, ldq, (const bf16_t*)kc,
          (const bf16_t*)vc, map, H, Tb, scale, (bf16_t*)y, ldy, kch, nsplit, part);
    else
      attn_prefill_mfma<32><<<grid, 256, 0, s>>>(qq, ldq, (const bf16_t*)kc,
          (const bf16_t*)vc, map, H, Tb, scale, (bf16_t*)y, ldy, kch, nsplit, part);
    if (split) {
      const dim3 mgrid((maxlen - kch * 64 + kMergeRows - 1) / kMergeRows, H);
      if (hs == 64)
        attn_prefill_merge<64><<<mgrid, 64 * kMergeRows, 0, s>>>(part, maxlen, Tb, kch, nsplit,
                                                                (bf16_t*)y, ldy);
      else
        attn_prefill_merge<32><<<mgrid, 64 * kMergeRows, 0, s>>>(part, maxlen, Tb, kch, nsplit,
                                                                (bf16_t*)y, ldy);
    }
  } else {
    const dim3 grid(ntiles, H, map.B);
    const float* qq = (const float*)q;
    if (hs == 64)
      attn_prefill_simt<float, 64><<<grid, 64, 0, s>>>(qq, ldq, (const float*)kc,
          (const float*)vc, map, H, Tb, scale, (float*)y, ldy);
    else
      attn_prefill_simt<float, 32><<<grid, 64, 0, s>>>(qq, ldq, (const float*)kc,
          (const float*)vc, map, H, Tb, scale, (float*)y, ldy);
  }
}

int attn_decode_chunks(int Tb) { return (Tb + kDecChunk - 1) / kDecChunk; }

int attn_decode_chunk_keys() { return kDecChunk; }

void launch_attn_decode(int dtype, const void* q, const void* kc,
                        const void* vc, const int32_t* pos, int B, int H,
                        int hs, int Tb, float* part, void* y,
                        bool merge_into_y, hipStream_t s) {
  const float scale = 1.0f / sqrtf((float)hs);
  const int nchunk = attn_decode_chunks(Tb);
  const dim3 grid(nchunk, H, B), cgrid(H, B);
  if (dtype == NGPT_BF16) {
    if (hs == 64) {
      attn_decode_kernel<bf16_t, 64><<<grid, 256, 0, s>>>((const bf16_t*)q,
          (const bf16_t*)kc, (const bf16_t*)vc, pos, H, Tb, nchunk, scale, part);
      if (merge_into_y) attn_decode_combine<bf16_t, 64><<<cgrid, 64, 0, s>>>(part, pos, H, nchunk, (bf16_t*)y);
    } else {
      attn_decode_kernel<bf16_t, 32><<<grid, 256, 0, s>>>((const bf16_t*)q,
          (const bf16_t*)kc, (const bf16_t*)vc, pos, H, Tb, nchunk, scale, part);
      if (merge_into_y) attn_decode_combine<bf16_t, 32><<<cgrid, 64, 0, s>>>(part, pos, H, nchunk, (bf16_t*)y);
    }
  } else {
    if (hs == 64) {
      attn_decode_kernel<float, 64><<<grid, 256, 0, s>>>((const float*)q,
          (const float*)kc, (const float*)vc, pos, H, Tb, nchunk, scale, part);
      if (merge_into_y) attn_decode_combine<float, 64><<<cgrid, 64, 0, s>>>(part, pos, H, nchunk, (float*)y);
    } else {
      attn_decode_kernel<float, 32><<<grid, 256, 0, s>>>((const float*)q,
          (const float*)kc, (const float*)vc, pos, H, Tb, nchunk, scale, part);
      if (merge_into_y) attn_decode_combine<float, 32><<<cgrid, 64, 0, s>>>(part, pos, H, nchunk, (float*)y);
    }
  }
}

}  // namespace ngpt
