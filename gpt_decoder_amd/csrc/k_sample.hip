// Sampler: temperature, top-k, softmax, inverse-CDF draw on caller uniforms.
//
// generate() on the serving page "原生 nanoGPT 模型服务首选" (section 2) takes
// the last-position logits, divides them by the temperature, replaces every
// value below the k-th largest (k = min(top_k, vocab)) by -inf, applies a
// softmax and draws one id with torch.multinomial.  Here the draw is the
// inverse CDF of the caller's uniform u in [0, 1):
//   s_i = float32(logit_i / T), correctly rounded (the quotient is formed in
//         double, whose 53-bit significand makes the final rounding to
//         float32 exact);
//   kept set K = {i : s_i >= v}, v the k-th largest s (ties kept);
//   w_i = exp(double(s_i) - max s), S = sum over K;
//   id  = smallest i in K whose running sum (ascending ids) exceeds u * S,
//         or the largest id in K if rounding leaves none.
// Greedy mode is the argmax of the logits with the lowest id among ties.
//
// One 512-thread workgroup per row.  The k-th largest value is found by a
// radix select over order-preserving 32-bit keys, most significant byte
// first.  The running sum is a two-level scan: each thread owns a contiguous
// run of ids, the per-thread totals are scanned, then the owning thread walks
// its run.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace ngpt {

constexpr int kSampThreads = 512;

__device__ __forceinline__ float scaled(float logit, float T) {
  return (float)((double)logit / (double)T);
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
  double scan[kSampThreads];
  uint32_t prefix;
  uint32_t remaining;
  int found;
  int last_kept;
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
__device__ int row_argmax(const float* lg, int V, SampShared& sh) {
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
  return r == 0x7FFFFFFF ? 0 : r;
}

__device__ int row_sample(const float* lg, int V, float T, int top_k, double u,
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
      for (int i = tid; i < V; i += kSampThreads) {
        const uint32_t k = fkey(scaled(lg[i], T));
        if ((k & mask) == prefix) atomicAdd(&sh.hist[(k >> shift) & 0xFFu], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        uint32_t rem = sh.remaining, cum = 0;
        int d = 255;
        for (; d > 0; --d) {
          if (cum + sh.hist[d] >= rem) break;
          cum += sh.hist[d];
        }
        sh.remaining = rem - cum;
        sh.prefix = prefix | ((uint32_t)d << shift);
      }
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
  sh.scan[tid] = local;
  __syncthreads();
  if (tid == 0) {
    double acc = 0.0;
    for (int t = 0; t < kSampThreads; ++t) {
      const double v = sh.scan[t];
      sh.scan[t] = acc;   // exclusive prefix
      acc += v;
    }
    sh.dred[0] = acc;     // total S
    sh.found = 0x7FFFFFFF;
    sh.last_kept = -1;
  }
  __syncthreads();
  const double target = u * sh.dred[0];
  double c = sh.scan[tid];
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
    int32_t* __restrict__ status, const void* __restrict__ wte,
    const void* __restrict__ wpe, int C, int dtype, float* __restrict__ x) {
  __shared__ SampShared sh;
  const int b = blockIdx.x;
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
    if (p.greedy)
      id = row_argmax(lg, V, sh);
    else
      id = row_sample(lg, V, p.temperature, p.top_k, uniforms[b], sh);
  }
  if (threadIdx.x == 0) {
    if (next_ids) next_ids[b] = id;
    if (mode != SAMPLE_ONLY) {
      tok[b] = id;
      pos[b] = len;
      lens[b] = len + 1;
    }
  }
  if (mode != SAMPLE_ONLY) {
    float* xr = x + (size_t)b * C;
    if (dtype == NGPT_BF16)
      write_embedding((const bf16_t*)wte, (const bf16_t*)wpe, id, len, C, xr);
    else
      write_embedding((const float*)wte, (const float*)wpe, id, len, C, xr);
  }
}

void sampler_node_params(SamplerArgs& a, int B, hipKernelNodeParams* p) {
  void* vals[18] = {&a.mode, &a.logits, &a.ld, &a.V, &a.uniforms, &a.params,
                    &a.feed_ids, &a.next_ids, &a.tok, &a.pos, &a.lens,
                    &a.limit, &a.status, &a.wte, &a.wpe, &a.C, &a.dtype, &a.x};
  for (int i = 0; i < 18; ++i) a.ptrs[i] = vals[i];
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
                                       a.pos, a.lens, a.limit, a.status, a.wte,
                                       a.wpe, a.C, a.dtype, a.x);
}

}  // namespace ngpt
