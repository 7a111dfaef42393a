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
#include "ln_row.hpp"

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

// One wavefront per row; 4 rows per 256-thread block.
template <class T>
__global__ __launch_bounds__(256) void layernorm_kernel(
    const float* __restrict__ x, int ldx, const int32_t* __restrict__ rows,
    int M, const T* __restrict__ w, const T* __restrict__ bias,
    T* __restrict__ out, int ldo, int C) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= M) return;
  const int src = rows ? rows[i] : i;
  ln_row<T>(x + (size_t)src * ldx, C, w, bias, out + (size_t)i * ldo);
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
