// Sampler: temperature, top-k, softmax, inverse-CDF draw on caller uniforms.
//
// generate() on the serving page "原生 nanoGPT 模型服务首选" (section 2) takes
// the last-position logits, divides them by the temperature, replaces every
// value below the k-th largest (k = min(top_k, vocab)) by -inf, applies a
// softmax and draws one id with torch.multinomial.  Here the draw is the
// inverse CDF of the caller's uniform u in [0, 1):
//   s_i = float32(logit_i / T), correctly rounded (IEEE fp32 division; the
//         same value as the quotient formed in double and then rounded, since
//         53 >= 2 * 24 + 2 makes that double rounding innocuous);
//   kept set K = {i : s_i >= v}, v the k-th largest s (ties kept);
//   w_i = exp(double(s_i) - max s), S = sum over K;
//   id  = smallest i in K whose running sum (ascending ids) exceeds u * S,
//         or the largest id in K if rounding leaves none.
// Greedy mode is the argmax of the logits with the lowest id among ties.
//
// One 1024-thread workgroup per row.  The k-th largest value is found by a
// radix select over order-preserving 32-bit keys, most significant byte
// first.  Rows of up to 1024 * 50 ids keep their keys in registers
// (row_sample_regs: the first digit from counts below the row maximum, the
// running sum chunk by chunk); longer rows stream from memory (row_sample:
// each thread owns a contiguous run of ids, the per-thread totals are
// prefix-summed across the workgroup, then the owning thread walks its run).
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace ngpt {

constexpr int kSampThreads = 1024;
constexpr int kSampMaxRun = 50;    // register-resident chunks per wavefront

// logit / T rounded once to fp32: the fp32 division here is IEEE
// correctly rounded (the compiler's default division, no fast-math), so it
// equals the quotient formed in fp64 and then rounded.
__device__ __forceinline__ float scaled(float logit, float T) {
  return logit / T;
}

// Order-preserving key: larger float <=> larger key; -0 is folded into +0.
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

struct SampShared {
  uint32_t hist[256];
  double dred[kSampThreads / 64];
  float fred[kSampThreads / 64];
  int ired[kSampThreads / 64];
  double scan[1];
  double wsum[kSampThreads / 64];
  unsigned long long kmask[kSampThreads / 64][kSampMaxRun];   // kept lanes per chunk
  float wcnt[kSampThreads / 64][4];   // per-wavefront counts of the top digits
  uint32_t prefix;
  uint32_t remaining;
  int found;
  int last_kept;
  int done;
};

__device__ __forceinline__ double block_sum_d(double v, SampShared& sh) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.dred[w] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < kSampThreads / 64; ++i) t += sh.dred[i];
  return t;
}

__device__ __forceinline__ float block_max_f(float v, SampShared& sh) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.fred[w] = v;
  __syncthreads();
  float t = -INFINITY;
  for (int i = 0; i < kSampThreads / 64; ++i) t = fmaxf(t, sh.fred[i]);
  return t;
}

// Greedy: argmax of the raw logits, lowest id among equal maxima.  Each
// thread scans its ids in ascending order, so a strict comparison keeps the
// first of equal values.
__device__ __forceinline__ int row_argmax(const float* lg, int V, SampShared& sh) {
  float best = -INFINITY;
  int bi = 0x7FFFFFFF;
  int tail = 0;
  if ((reinterpret_cast<uintptr_t>(lg) & 15u) == 0) {
    const float4* l4 = reinterpret_cast<const float4*>(lg);
    const int V4 = V >> 2;
    constexpr int U = 8;  // loads in flight per thread
    for (int i0 = threadIdx.x; i0 < V4; i0 += U * kSampThreads) {
      float4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * kSampThreads;
        v[u] = i < V4 ? l4[i] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * kSampThreads;
        if (v[u].x > best) { best = v[u].x; bi = 4 * i; }
        if (v[u].y > best) { best = v[u].y; bi = 4 * i + 1; }
        if (v[u].z > best) { best = v[u].z; bi = 4 * i + 2; }
        if (v[u].w > best) { best = v[u].w; bi = 4 * i + 3; }
      }
    }
    tail = V4 << 2;
  }
  for (int i = tail + threadIdx.x; i < V; i += kSampThreads) {
    const float v = lg[i];
    if (v > best) { best = v; bi = i; }
  }
  const float gmax = block_max_f(best, sh);
  int cand = (best == gmax) ? bi : 0x7FFFFFFF;
  for (int o = 32; o > 0; o >>= 1) cand = min(cand, __shfl_xor(cand, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.ired[threadIdx.x >> 6] = cand;
  __syncthreads();
  int r = 0x7FFFFFFF;
  for (int i = 0; i < kSampThreads / 64; ++i) r = min(r, sh.ired[i]);
  return r;   // 0x7FFFFFFF: no finite maximum (all -inf or NaN)
}

// Wavefront-aggregated histogram add: the lanes with `match` add 1 to
// hist[bin]; lanes sharing a bin are counted with one atomic (logits crowd
// into a few top-byte bins, where per-lane atomics would serialise).  The
// leader's bin is read with a scalar lane read, not an LDS permute.
__device__ __forceinline__ void hist_add(uint32_t* hist, bool match, uint32_t bin) {
  const int lane = threadIdx.x & 63;
  unsigned long long act = __ballot(match);
  while (act) {
    const int leader = __ffsll(act) - 1;
    const uint32_t lbin = (uint32_t)__builtin_amdgcn_readlane((int)bin, leader);
    const unsigned long long same = __ballot(match && bin == lbin);
    if (lane == leader) atomicAdd(&hist[lbin], (uint32_t)__popcll(same));
    act &= ~same;
  }
}

// Inclusive prefix sums of one double per thread over the workgroup, in a
// fixed order (shuffles within each wavefront, then the wavefront totals).
__device__ __forceinline__ double block_scan_incl(double v, SampShared& sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  __syncthreads();
  if (lane == 63) sh.dred[w] = v;
  __syncthreads();
  double before = 0.0;
  for (int i = 0; i < w; ++i) before += sh.dred[i];
  return before + v;
}

// One radix level of the top-k threshold search, after the histogram of
// the level's digit (over the keys matching the prefix so far) is in
// sh.hist: the digit d is the highest bin where the count of keys in bins
// >= d reaches the number still wanted, S(d) >= rem with S the suffix sums;
// the keys in bins above d are kept, and rem - S(d + 1) are still wanted
// from bin d.  Wavefront 0 does it: lane l holds bins 4l .. 4l + 3, the
// suffix sums run over the lanes from the top, and d is the largest bin with
// S(d) >= rem (S never grows with d).  Sets sh.prefix, sh.remaining and
// sh.done (the bin holds exactly the keys still wanted).  Integer sums:
// exact, so the same digit as a serial walk from the top.
__device__ __forceinline__ void radix_pick(SampShared& sh, uint32_t prefix, int shift) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const uint32_t rem = sh.remaining;
  uint32_t h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = sh.hist[4 * lane + i];
  const uint32_t ls = (h[0] + h[1]) + (h[2] + h[3]);
  uint32_t t = ls;   // sum over lanes >= this one
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_down(t, o, 64);
    if (lane + o < 64) t += u;
  }
  // suffix sums of this lane's bins, from its top bin down
  uint32_t sfx[4];
  sfx[3] = t - ls + h[3];
  sfx[2] = sfx[3] + h[2];
  sfx[1] = sfx[2] + h[1];
  sfx[0] = sfx[1] + h[0];
  int best = -1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (sfx[i] >= rem) best = 4 * lane + i;
  int d = best;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) d = max(d, __shfl_xor(d, o, 64));
  // (bin 0 always qualifies: the keys matching the prefix number >= rem)
  if (d < 0) d = 0;
  if (lane == d / 4) {
    const int i = d % 4;
    const uint32_t above = sfx[i] - h[i];
    sh.remaining = rem - above;
    sh.prefix = prefix | ((uint32_t)d << shift);
    sh.done = sfx[i] == rem;
  }
}

__device__ __forceinline__ int row_sample(const float* lg, int V, float T, int top_k, double u,
                          SampShared& sh) {
  const int tid = threadIdx.x;
  // -- threshold: the k'-th largest scaled logit, k' = min(top_k, V)
  uint32_t thr_key = 0;  // keep everything
  if (top_k > 0 && top_k < V) {
    if (tid == 0) { sh.prefix = 0; sh.remaining = (uint32_t)top_k; }
    uint32_t mask = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
      __syncthreads();
      for (int i = tid; i < 256; i += kSampThreads) sh.hist[i] = 0;
      __syncthreads();
      const uint32_t prefix = sh.prefix;
      constexpr int U = 4;   // loads issued before their histogram adds
      for (int i0 = 0; i0 < V; i0 += U * kSampThreads) {   // uniform trip count
        uint32_t k[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u * kSampThreads + tid;
          k[u] = i < V ? fkey(scaled(lg[i], T)) : 0u;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u * kSampThreads + tid;
          hist_add(sh.hist, i < V && (k[u] & mask) == prefix, (k[u] >> shift) & 0xFFu);
        }
      }
      __syncthreads();
      radix_pick(sh, prefix, shift);
      mask |= 0xFFu << shift;
    }
    __syncthreads();
    thr_key = sh.prefix;
  }
  // -- max of the kept values (the overall max is always kept)
  float lmax = -INFINITY;
  for (int i = tid; i < V; i += kSampThreads) lmax = fmaxf(lmax, scaled(lg[i], T));
  const double m = (double)block_max_f(lmax, sh);

  // -- per-thread contiguous runs, ascending ids
  const int run = (V + kSampThreads - 1) / kSampThreads;
  const int i0 = tid * run;
  const int i1 = min(V, i0 + run);
  double local = 0.0;
  int last_kept = -1;
  for (int i = i0; i < i1; ++i) {
    const float sv = scaled(lg[i], T);
    if (fkey(sv) >= thr_key) {
      local += exp((double)sv - m);
      last_kept = i;
    }
  }
  const double incl = block_scan_incl(local, sh);
  __syncthreads();
  if (tid == kSampThreads - 1) sh.scan[0] = incl;   // total S
  if (tid == 0) {
    sh.found = 0x7FFFFFFF;
    sh.last_kept = -1;
  }
  __syncthreads();
  const double target = u * sh.scan[0];
  double c = incl - local;   // exclusive prefix
  int hit = 0x7FFFFFFF;
  if (i0 < i1 && c + local > target) {
    for (int i = i0; i < i1; ++i) {
      const float sv = scaled(lg[i], T);
      if (fkey(sv) >= thr_key) {
        c += exp((double)sv - m);
        if (c > target) { hit = i; break; }
      }
    }
  }
  if (hit != 0x7FFFFFFF) atomicMin(&sh.found, hit);
  if (last_kept >= 0) atomicMax(&sh.last_kept, last_kept);
  __syncthreads();
  return sh.found != 0x7FFFFFFF ? sh.found : sh.last_kept;
}

// Sum of a double over the wavefront with the DPP and permlane moves of
// common.hpp applied to both 32-bit halves (no LDS permutes): every lane
// gets the same bits, as each step adds a symmetric pair of partial sums.
template <class F>
__device__ __forceinline__ double move_d(double v, F mov) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __float_as_uint(mov(__uint_as_float((uint32_t)u)));
  const uint32_t hi = __float_as_uint(mov(__uint_as_float((uint32_t)(u >> 32))));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double wave_sum_d(double v) {
  v += move_d(v, lane_xor1);
  v += move_d(v, lane_xor2);
  v += move_d(v, lane_mirror8);
  v += move_d(v, lane_xor8);
  v += move_d(v, lane_xor16);
  v += move_d(v, lane_xor32);
  return v;
}

// The draw with the row's scaled logits held in registers as order keys,
// read and divided once for the threshold and the maximum.  Wavefront w
// owns ids [64 RUN w, 64 RUN (w + 1)) as RUN chunks of 64 consecutive ids,
// lane l holding id 64 RUN w + 64 j + l of chunk j (coalesced loads).
// Requires V <= 1024 RUN.  Each chunk's kept lanes go to LDS as a mask; the
// weights are then formed for kept ids only, re-reading their logits (the
// same division gives the same value), in a plain loop over the chunks.
// Running sums go chunk by chunk: a chunk's kept weights are summed over the
// wavefront, the wavefront totals in wavefront order, and the chunk holding
// u * S is scanned lane by lane; chunks without a kept id are skipped.
template <int RUN>
__device__ __forceinline__ int row_sample_regs(const float* lg, int V, float T, int top_k, double u,
                               SampShared& sh) {
  static_assert(RUN <= kSampMaxRun, "chunk masks are sized for kSampMaxRun");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int base = wave * 64 * RUN;
  // Range-checked buffer loads (an id past V reads 0): every load is issued
  // on every path, all before the first use, where loads under a per-lane
  // branch would each be waited for in turn.
  constexpr uint32_t kOut = 0x80000000u;
  const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(lg), (short)0, V * 4, 0x00020000);
  auto ld = [&](int i, bool on) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
        rl, on ? (uint32_t)i * 4u : kOut, 0, 0));
  };
  uint32_t key[RUN];
#pragma unroll
  for (int j = 0; j < RUN; ++j) {
    const int i = base + 64 * j + lane;
    key[j] = __float_as_uint(ld(i, i < V));
  }
  auto valid = [&](int j) { return base + 64 * j + lane < V; };
#pragma unroll
  for (int j = 0; j < RUN; ++j)
    key[j] = valid(j) ? fkey(scaled(__uint_as_float(key[j]), T)) : 0u;

  // -- the maximum (it is always kept, and it bounds the threshold's top digit)
  float lmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < RUN; ++j)
    if (valid(j)) lmax = fmaxf(lmax, key_to_float(key[j]));
  const float mx = block_max_f(lmax, sh);
  const double m = (double)mx;

  // -- threshold key: the k'-th largest, k' = min(top_k, V); 0 keeps all
  uint32_t thr = 0;
  if (top_k > 0 && top_k < V) {
    if (tid == 0) { sh.prefix = 0; sh.remaining = (uint32_t)top_k; sh.done = 0; }
    // First digit from counts of the four top digits at and below the
    // maximum's, kept in registers (the logits crowd into a few top-byte
    // bins, where histogram atomics would collide); the histogram pass runs
    // only if the k'-th largest lies lower.
    const int mb = (int)(fkey(mx) >> 24);
    float c[4] = {0.f, 0.f, 0.f, 0.f};   // counts below 2^24: exact
#pragma unroll
    for (int j = 0; j < RUN; ++j) {
      const int d = (int)(key[j] >> 24);
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] += (valid(j) && d == mb - i) ? 1.f : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = wave_sum_all(c[i]);
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sh.wcnt[wave][i] = c[i];
    }
    __syncthreads();
    int shift0 = 24;
    {
      uint32_t cum = 0;
      for (int i = 0; i < 4 && mb - i >= 0; ++i) {
        uint32_t ci = 0;
        for (int w = 0; w < kSampThreads / 64; ++w) ci += (uint32_t)sh.wcnt[w][i];
        if (cum + ci >= (uint32_t)top_k) {   // the k'-th largest has digit mb - i
          shift0 = 16;
          if (tid == 0) {
            sh.prefix = (uint32_t)(mb - i) << 24;
            sh.remaining = (uint32_t)top_k - cum;
            sh.done = cum + ci == (uint32_t)top_k;
          }
          break;
        }
        cum += ci;
      }
    }
    __syncthreads();
    uint32_t mask = shift0 == 24 ? 0u : 0xFF000000u;
    for (int shift = shift0; shift >= 0 && !sh.done; shift -= 8) {
      __syncthreads();
      for (int i = tid; i < 256; i += kSampThreads) sh.hist[i] = 0;
      __syncthreads();
      const uint32_t prefix = sh.prefix;
#pragma unroll
      for (int j = 0; j < RUN; ++j)
        if (valid(j) && (key[j] & mask) == prefix) atomicAdd(&sh.hist[(key[j] >> shift) & 0xFFu], 1u);
      __syncthreads();
      // (done: the bin holds exactly the ids still wanted, so every key at
      // or above the bin's lowest possible key is kept and the search stops)
      radix_pick(sh, prefix, shift);
      __syncthreads();
      mask |= 0xFFu << shift;
      if (sh.done) break;
    }
    thr = sh.prefix;
  }

  // -- kept masks (lane l collects the masks of chunks l and l + 64, then
  // stores them)
  unsigned long long my0 = 0, my1 = 0;
#pragma unroll
  for (int j = 0; j < RUN; ++j) {
    const unsigned long long km = __ballot(valid(j) && key[j] >= thr);
    if (j < 64) my0 = lane == j ? km : my0;
    else my1 = lane == j - 64 ? km : my1;
  }
  if (lane < RUN) sh.kmask[wave][lane] = my0;
  if (lane + 64 < RUN) sh.kmask[wave][lane + 64] = my1;
  __syncthreads();

  // -- this wavefront's total, chunk by chunk, and its last kept id; the
  // kept logits of 8 chunks are fetched together (one memory latency per 8
  // chunks rather than per chunk)
  constexpr int CB = 8;
  unsigned long long km[CB];
  float lv[CB];
  // (returns whether any of the 8 chunks has a kept id; none: nothing fetched)
  auto fetch = [&](int j0) {
    unsigned long long any = 0;
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      km[u] = j0 + u < RUN ? sh.kmask[wave][j0 + u] : 0ull;
      any |= km[u];
    }
    if (any == 0) return false;
#pragma unroll
    for (int u = 0; u < CB; ++u)
      lv[u] = ld(base + 64 * (j0 + u) + lane, (km[u] >> lane) & 1);
    return true;
  };
  auto weight = [&](int u) {
    return ((km[u] >> lane) & 1) ? exp((double)scaled(lv[u], T) - m) : 0.0;
  };
  double wt = 0.0;
  int lk = -1;
  for (int j0 = 0; j0 < RUN; j0 += CB) {
    if (!fetch(j0)) continue;
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      if (km[u] == 0) continue;
      wt += wave_sum_d(weight(u));
      lk = base + 64 * (j0 + u) + 63 - __clzll(km[u]);
    }
  }
  if (lane == 0) sh.wsum[wave] = wt;
  if (tid == 0) { sh.found = 0x7FFFFFFF; sh.last_kept = -1; }
  __syncthreads();
  if (lane == 0 && lk >= 0) atomicMax(&sh.last_kept, lk);
  double S = 0.0, C = 0.0;
  for (int w = 0; w < kSampThreads / 64; ++w) {
    if (w == wave) C = S;
    S += sh.wsum[w];
  }
  const double target = u * S;
  if (C <= target && C + wt > target) {   // the wavefront holding the draw
    double c = C;
    int hit = -1;
    for (int j0 = 0; j0 < RUN && hit < 0; j0 += CB) {
      if (!fetch(j0)) continue;
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        if (km[u] == 0 || hit >= 0) continue;
        const double w = weight(u);
        const double cs = wave_sum_d(w);
        if (c + cs > target) {
          // running sum over the lanes of this chunk, ascending ids
          double incl = w;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const double t = __shfl_up(incl, o, 64);
            if (lane >= o) incl += t;
          }
          const unsigned long long over = __ballot(((km[u] >> lane) & 1) && c + incl > target);
          // rounding may leave no lane above u * S: the chunk's last kept id
          const int l = over ? __ffsll(over) - 1 : 63 - __clzll(km[u]);
          hit = base + 64 * (j0 + u) + l;
        } else {
          c += cs;
        }
      }
    }
    if (lane == 0) sh.found = hit >= 0 ? hit : 0x7FFFFFFF;
  }
  __syncthreads();
  return sh.found != 0x7FFFFFFF ? sh.found : sh.last_kept;
}

template <class T>
__device__ void write_embedding(const T* wte, const T* wpe, int id, int p,
                                int C, float* xr) {
  const T* te = wte + (size_t)id * C;
  const T* pe = wpe + (size_t)p * C;
  for (int c = threadIdx.x; c < C; c += blockDim.x)
    xr[c] = to_f32(te[c]) + to_f32(pe[c]);
}

__global__ __launch_bounds__(kSampThreads) void sampler_kernel(
    int mode, const float* __restrict__ logits, int ld, int V,
    const double* __restrict__ uniforms, const SampleParams* __restrict__ prm,
    const int32_t* __restrict__ feed_ids, int32_t* __restrict__ next_ids,
    int32_t* __restrict__ tok, int32_t* __restrict__ pos,
    int32_t* __restrict__ lens, const int32_t* __restrict__ limit,
    int32_t* __restrict__ status, int32_t* __restrict__ hist, int Tb,
    const void* __restrict__ wte,
    const void* __restrict__ wpe, int C, int dtype, float* __restrict__ x,
    uint32_t* __restrict__ epoch) {
  __shared__ SampShared sh;
  const int b = blockIdx.x;
  // ahead of a one-launch forward: advance its exchange epoch (that kernel
  // starts after this one ends, so all its workgroups read the new value)
  if (epoch && b == 0 && threadIdx.x == 0)
    __hip_atomic_store(epoch, *epoch + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  bool active = true;
  int len = 0;
  if (mode != SAMPLE_ONLY) {
    len = lens[b];
    active = len < limit[b];
  }
  if (!active) {
    if (threadIdx.x == 0) {
      if (next_ids) next_ids[b] = -1;
      pos[b] = -1;
    }
    // inactive row: keep its residual finite; nothing of it is stored
    for (int c = threadIdx.x; c < C; c += blockDim.x) x[(size_t)b * C + c] = 0.f;
    return;
  }
  int id;
  if (mode == FEED_STEP) {
    id = feed_ids[b];
    if (id < 0 || id >= V) {
      if (threadIdx.x == 0) atomicOr(status, 1);
      id = 0;
    }
  } else {
    const SampleParams p = *prm;
    const float* lg = logits + (size_t)b * ld;
    if (p.greedy) {
      // a row with no finite maximum gives id 0 and the invalid-input flag
      // (the same rule as the one-launch decode kernel's greedy pick)
      id = row_argmax(lg, V, sh);
      if (id == 0x7FFFFFFF) {
        if (threadIdx.x == 0) atomicOr(status, 1);
        id = 0;
      }
    } else {
      const int run = (V + kSampThreads - 1) / kSampThreads;
      const double u = uniforms[b];
      if (run <= 1) id = row_sample_regs<1>(lg, V, p.temperature, p.top_k, u, sh);
      else if (run <= 4) id = row_sample_regs<4>(lg, V, p.temperature, p.top_k, u, sh);
      else if (run <= 16) id = row_sample_regs<16>(lg, V, p.temperature, p.top_k, u, sh);
      else if (run <= 50) id = row_sample_regs<50>(lg, V, p.temperature, p.top_k, u, sh);
      else id = row_sample(lg, V, p.temperature, p.top_k, u, sh);
    }
  }
  if (threadIdx.x == 0) {
    if (next_ids) next_ids[b] = id;
    if (mode != SAMPLE_ONLY) {
      tok[b] = id;
      pos[b] = len;
      lens[b] = len + 1;
      hist[(size_t)b * Tb + len] = id;
    }
  }
  if (mode != SAMPLE_ONLY) {
    float* xr = x + (size_t)b * C;
    if (dtype == NGPT_BF16)
      write_embedding((const bf16_t*)wte, (const bf16_t*)wpe, id, len, C, xr);
    else if (dtype == NGPT_F16)
      write_embedding((const f16_t*)wte, (const f16_t*)wpe, id, len, C, xr);
    else
      write_embedding((const float*)wte, (const float*)wpe, id, len, C, xr);
  }
}

void sampler_node_params(SamplerArgs& a, int B, hipKernelNodeParams* p) {
  void* vals[21] = {&a.mode, &a.logits, &a.ld, &a.V, &a.uniforms, &a.params,
                    &a.feed_ids, &a.next_ids, &a.tok, &a.pos, &a.lens,
                    &a.limit, &a.status, &a.hist, &a.Tb, &a.wte, &a.wpe, &a.C,
                    &a.dtype, &a.x, &a.epoch};
  for (int i = 0; i < 21; ++i) a.ptrs[i] = vals[i];
  p->func = reinterpret_cast<void*>(sampler_kernel);
  p->gridDim = dim3(B);
  p->blockDim = dim3(a.mode == FEED_STEP ? 256 : kSampThreads);
  p->sharedMemBytes = 0;
  p->kernelParams = a.ptrs;
  p->extra = nullptr;
}

void launch_sampler(const SamplerArgs& a, int B, hipStream_t s) {
  if (B <= 0) return;
  const int threads = (a.mode == FEED_STEP) ? 256 : kSampThreads;
  sampler_kernel<<<B, threads, 0, s>>>(a.mode, a.logits, a.ld, a.V, a.uniforms,
                                       a.params, a.feed_ids, a.next_ids, a.tok,
                                       a.pos, a.lens, a.limit, a.status,
                                       a.hist, a.Tb, a.wte, a.wpe, a.C,
                                       a.dtype, a.x, a.epoch);
}

}  // namespace ngpt
