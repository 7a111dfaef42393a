// Token + position embedding and LayerNorm kernels.
//
// Embedding: x = wte[id] + wpe[pos] with learned absolute positions that
// start at 0 in every sequence (model-building chapter "第 4 章 模型构建",
// section 4.5; SDK guide "模型架构解析": wte and wpe of the GPT class).
// LayerNorm: (x - mean) / sqrt(var + 1e-5) * w (+ b) over the C features,
// population variance, optional bias (serving page "原生 nanoGPT 模型服务首选",
// section 1).  Statistics are fp32, two-pass (mean, then the mean of the
// squared deviations).
#include "common.hpp"
#include "kernels.hpp"

namespace ngpt {

template <class T>
__global__ __launch_bounds__(256) void embed_prefill_kernel(
    const int32_t* __restrict__ ids, int Tmax, RowMap map,
    const T* __restrict__ wte, const T* __restrict__ wpe, int C, int V,
    float* __restrict__ x, int32_t* __restrict__ row_b,
    int32_t* __restrict__ row_pos, int32_t* __restrict__ last_rows,
    int32_t* __restrict__ last_slot, int32_t* __restrict__ hist, int Tb,
    int32_t* __restrict__ status) {
  const int r = blockIdx.x;
  // sequence owning packed row r: the last b with off[b] <= r
  int lo = 0, hi = map.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (map.off[mid] <= r) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int i = r - map.off[b];          // index among the sequence's new rows
  const int p = map.past[b] + i;         // its position
  int id = ids[Tmax > 0 ? (size_t)b * Tmax + i : (size_t)r];
  if (id < 0 || id >= V) {
    if (threadIdx.x == 0) atomicOr(status, 1);
    id = 0;
  }
  if (threadIdx.x == 0) {
    row_b[r] = map.slot[b];
    row_pos[r] = p;
    hist[(size_t)map.slot[b] * Tb + p] = id;
    if (r == map.off[b + 1] - 1) {
      last_rows[b] = r;
      last_slot[b] = map.slot[b];
    }
  }
  const T* te = wte + (size_t)id * C;
  const T* pe = wpe + (size_t)p * C;
  float* xr = x + (size_t)r * C;
  for (int c = threadIdx.x; c < C; c += blockDim.x)
    xr[c] = to_f32(te[c]) + to_f32(pe[c]);
}

template <class T>
__global__ __launch_bounds__(256) void embed_decode_kernel(
    const int32_t* __restrict__ tok, const int32_t* __restrict__ pos,
    const T* __restrict__ wte, const T* __restrict__ wpe, int C, int V,
    float* __restrict__ x, int32_t* __restrict__ status) {
  const int b = blockIdx.x;
  const int p = pos[b];
  float* xr = x + (size_t)b * C;
  if (p < 0) {  // inactive row: keep the residual finite, nothing is stored
    for (int c = threadIdx.x; c < C; c += blockDim.x) xr[c] = 0.f;
    return;
  }
  int id = tok[b];
  if (id < 0 || id >= V) {
    if (threadIdx.x == 0) atomicOr(status, 1);
    id = 0;
  }
  const T* te = wte + (size_t)id * C;
  const T* pe = wpe + (size_t)p * C;
  for (int c = threadIdx.x; c < C; c += blockDim.x)
    xr[c] = to_f32(te[c]) + to_f32(pe[c]);
}

// One wavefront per row; 4 rows per 256-thread block.  The row is held in
// registers (float4 per lane per 256 columns, up to 8 of them), so x is read
// once and every load is issued before the first reduction.
constexpr int kLnMaxVec = 8;  // C <= 2048

// Four consecutive elements at a multiple of 4 (C is a multiple of 32 and
// the parameter and output rows are 16-byte aligned), so the LayerNorm
// parameters are read and its output written with one access per lane.
__device__ __forceinline__ void load4(const bf16_t* p, float* f) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  f[0] = to_f32(static_cast<bf16_t>(u.x & 0xffffu));
  f[1] = to_f32(static_cast<bf16_t>(u.x >> 16));
  f[2] = to_f32(static_cast<bf16_t>(u.y & 0xffffu));
  f[3] = to_f32(static_cast<bf16_t>(u.y >> 16));
}
__device__ __forceinline__ void load4(const f16_t* p, float* f) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  f[0] = to_f32(__builtin_bit_cast(f16_t, static_cast<uint16_t>(u.x & 0xffffu)));
  f[1] = to_f32(__builtin_bit_cast(f16_t, static_cast<uint16_t>(u.x >> 16)));
  f[2] = to_f32(__builtin_bit_cast(f16_t, static_cast<uint16_t>(u.y & 0xffffu)));
  f[3] = to_f32(__builtin_bit_cast(f16_t, static_cast<uint16_t>(u.y >> 16)));
}
__device__ __forceinline__ void load4(const float* p, float* f) {
  const float4 t = *reinterpret_cast<const float4*>(p);
  f[0] = t.x; f[1] = t.y; f[2] = t.z; f[3] = t.w;
}
// The same four elements through a range-checked buffer load: offset kLnOut
// (past every buffer) and a buffer of 0 bytes read zeros, so the load can be
// issued on every path.
constexpr uint32_t kLnOut = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ln_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, p ? bytes : 0,
                                           0x00020000);
}
__device__ __forceinline__ void unpack4(uint2 u, const bf16_t*, float* f) {
  f[0] = to_f32(static_cast<bf16_t>(u.x & 0xffffu));
  f[1] = to_f32(static_cast<bf16_t>(u.x >> 16));
  f[2] = to_f32(static_cast<bf16_t>(u.y & 0xffffu));
  f[3] = to_f32(static_cast<bf16_t>(u.y >> 16));
}
__device__ __forceinline__ void unpack4(uint2 u, const f16_t*, float* f) {
  f[0] = to_f32(__builtin_bit_cast(f16_t, static_cast<uint16_t>(u.x & 0xffffu)));
  f[1] = to_f32(__builtin_bit_cast(f16_t, static_cast<uint16_t>(u.x >> 16)));
  f[2] = to_f32(__builtin_bit_cast(f16_t, static_cast<uint16_t>(u.y & 0xffffu)));
  f[3] = to_f32(__builtin_bit_cast(f16_t, static_cast<uint16_t>(u.y >> 16)));
}
template <class T>
__device__ __forceinline__ void load4_buf(__amdgpu_buffer_rsrc_t r, int c, bool ok, float* f) {
  const uint32_t off = ok ? (uint32_t)c * sizeof(T) : kLnOut;
  if constexpr (sizeof(T) == 2) {
    unpack4(__builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0)),
            static_cast<const T*>(nullptr), f);
  } else {
    const float4 t = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    f[0] = t.x; f[1] = t.y; f[2] = t.z; f[3] = t.w;
  }
}

__device__ __forceinline__ void store4(bf16_t* p, const float* f) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
}
__device__ __forceinline__ void store4(f16_t* p, const float* f) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_f16x2(f[0], f[1]), pack_f16x2(f[2], f[3]));
}
__device__ __forceinline__ void store4(float* p, const float* f) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
}

template <class T>
__global__ __launch_bounds__(256) void layernorm_kernel(
    const float* __restrict__ x, int ldx, const int32_t* __restrict__ rows,
    int M, const T* __restrict__ w, const T* __restrict__ bias,
    T* __restrict__ out, int ldo, int C) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= M) return;
  const int src = rows ? rows[i] : i;
  const float* xr = x + (size_t)src * ldx;
  // The row, the gain and the shift are all fetched before the first
  // reduction, through range-checked buffer loads (issued on every path;
  // guarded loads were each waited for in turn), so one memory latency is
  // exposed.
  const __amdgpu_buffer_rsrc_t rx = ln_rsrc(xr, C * 4);
  const __amdgpu_buffer_rsrc_t rw = ln_rsrc(w, C * (int)sizeof(T));
  const __amdgpu_buffer_rsrc_t rb = ln_rsrc(bias, C * (int)sizeof(T));
  float4 v[kLnMaxVec];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kLnMaxVec; ++j) {
    const int c = j * 256 + lane * 4;
    v[j] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
        rx, c < C ? (uint32_t)c * 4u : kLnOut, 0, 0));
  }
  float wv[kLnMaxVec][4], bv[kLnMaxVec][4];
#pragma unroll
  for (int j = 0; j < kLnMaxVec; ++j) {
    const int c = j * 256 + lane * 4;
    load4_buf<T>(rw, c, c < C, wv[j]);
    load4_buf<T>(rb, c, c < C, bv[j]);
  }
  // (keeps the scheduler from sinking the gain and shift loads below the
  // reductions, which would expose a second memory latency)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < kLnMaxVec; ++j) s += (v[j].x + v[j].y) + (v[j].z + v[j].w);
  const float mean = wave_sum_all(s) / (float)C;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < kLnMaxVec; ++j) {
    const int c = j * 256 + lane * 4;
    if (c < C) {
      const float a = v[j].x - mean, b = v[j].y - mean, d = v[j].z - mean, e = v[j].w - mean;
      q += (a * a + b * b) + (d * d + e * e);
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum_all(q) / (float)C + 1e-5f);
  T* o = out + (size_t)i * ldo;
#pragma unroll
  for (int j = 0; j < kLnMaxVec; ++j) {
    const int c = j * 256 + lane * 4;
    if (c < C) {
      const float xv[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
      float y[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        y[u] = (xv[u] - mean) * rstd * wv[j][u];
        if (bias) y[u] += bv[j][u];
      }
      store4(o + c, y);
    }
  }
}

void launch_embed_prefill(int dtype, const int32_t* ids, int Tmax,
                          const RowMap& map, int M, const void* wte,
                          const void* wpe, int C, int V, float* x,
                          int32_t* row_b, int32_t* row_pos, int32_t* last_rows,
                          int32_t* last_slot, int32_t* hist, int Tb,
                          int32_t* status, hipStream_t s) {
  if (M <= 0) return;
  if (dtype == NGPT_BF16)
    embed_prefill_kernel<bf16_t><<<M, 256, 0, s>>>(
        ids, Tmax, map, (const bf16_t*)wte, (const bf16_t*)wpe, C, V, x,
        row_b, row_pos, last_rows, last_slot, hist, Tb, status);
  else if (dtype == NGPT_F16)
    embed_prefill_kernel<f16_t><<<M, 256, 0, s>>>(
        ids, Tmax, map, (const f16_t*)wte, (const f16_t*)wpe, C, V, x,
        row_b, row_pos, last_rows, last_slot, hist, Tb, status);
  else
    embed_prefill_kernel<float><<<M, 256, 0, s>>>(
        ids, Tmax, map, (const float*)wte, (const float*)wpe, C, V, x, row_b,
        row_pos, last_rows, last_slot, hist, Tb, status);
}

void launch_embed_decode(int dtype, const int32_t* tok, const int32_t* pos,
                         int B, const void* wte, const void* wpe, int C, int V,
                         float* x, int32_t* status, hipStream_t s) {
  if (dtype == NGPT_BF16)
    embed_decode_kernel<bf16_t><<<B, 256, 0, s>>>(
        tok, pos, (const bf16_t*)wte, (const bf16_t*)wpe, C, V, x, status);
  else if (dtype == NGPT_F16)
    embed_decode_kernel<f16_t><<<B, 256, 0, s>>>(
        tok, pos, (const f16_t*)wte, (const f16_t*)wpe, C, V, x, status);
  else
    embed_decode_kernel<float><<<B, 256, 0, s>>>(
        tok, pos, (const float*)wte, (const float*)wpe, C, V, x, status);
}

void launch_layernorm(int dtype, const float* x, int ldx, const int32_t* rows,
                      int M, const void* w, const void* b, void* out, int ldo,
                      int C, hipStream_t s) {
  if (M <= 0) return;
  const int grid = (M + 3) / 4;
  if (dtype == NGPT_BF16)
    layernorm_kernel<bf16_t><<<grid, 256, 0, s>>>(
        x, ldx, rows, M, (const bf16_t*)w, (const bf16_t*)b, (bf16_t*)out, ldo,
        C);
  else if (dtype == NGPT_F16)
    layernorm_kernel<f16_t><<<grid, 256, 0, s>>>(
        x, ldx, rows, M, (const f16_t*)w, (const f16_t*)b, (f16_t*)out, ldo, C);
  else
    layernorm_kernel<float><<<grid, 256, 0, s>>>(
        x, ldx, rows, M, (const float*)w, (const float*)b, (float*)out, ldo, C);
}

}  // namespace ngpt
