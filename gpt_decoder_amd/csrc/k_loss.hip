// Cross-entropy of the evaluation forward.
//
// The forward with labels of the model-building chapter ("第 4 章 模型构建",
// section 4.6): logits at every position, the last position dropped and the
// labels shifted by one, so the logits of position t are scored against the
// id at t + 1; the loss is the mean of log(sum_j exp(l_j)) - l_target over
// the scored positions.  Rows are the packed prefill rows: row r is scored
// against ids[r + 1] unless it is its sequence's last row.
//
// Kernels:
//   cross_entropy_regs_kernel  one workgroup of 1024 per row for rows of up to
//                         1024 * PER logits: the row is read once, into
//                         registers (range-checked loads, all in flight), its
//                         maximum found, then the sum of exp(l - max) (fp32
//                         terms by the hardware exp2, per-thread fp32 sums
//                         combined in fp64 in a fixed order),
//                         loss = max + log(sum) - l_target
//   cross_entropy_kernel  the same for longer rows, reading the row twice
//   mean_loss_kernel      one workgroup: the losses summed in a fixed order
//                         (fp64), divided by the number of scored rows
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace ngpt {

constexpr int kCeThreads = 256;

__global__ __launch_bounds__(kCeThreads) void cross_entropy_kernel(
    const float* __restrict__ logits, int ld, int V, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ row_b, const int32_t* __restrict__ last_rows,
    float* __restrict__ losses) {
  __shared__ float fred[kCeThreads / 64];
  __shared__ double dred[kCeThreads / 64];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (r == last_rows[row_b[r]]) {   // the last position has no label
    if (tid == 0) losses[r] = 0.f;
    return;
  }
  const int tgt = ids[r + 1];
  const float* row = logits + (size_t)r * ld;
  float mx = -INFINITY;
  for (int i = tid; i < V; i += kCeThreads) mx = fmaxf(mx, row[i]);
  mx = wave_max(mx);
  if (lane == 0) fred[w] = mx;
  __syncthreads();
  mx = fred[0];
  for (int i = 1; i < kCeThreads / 64; ++i) mx = fmaxf(mx, fred[i]);
  float sum = 0.f;
  for (int i = tid; i < V; i += kCeThreads) sum += expf(row[i] - mx);
  double ds = sum;
  for (int o = 32; o > 0; o >>= 1) ds += __shfl_xor(ds, o, 64);
  if (lane == 0) dred[w] = ds;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int i = 0; i < kCeThreads / 64; ++i) t += dred[i];
    losses[r] = (float)((double)mx + log(t) - (double)row[tgt]);
  }
}

constexpr int kCeRegThreads = 1024;

template <int PER>
__global__ __launch_bounds__(kCeRegThreads) void cross_entropy_regs_kernel(
    const float* __restrict__ logits, int ld, int V, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ row_b, const int32_t* __restrict__ last_rows,
    float* __restrict__ losses) {
  constexpr int NW = kCeRegThreads / 64;
  __shared__ float fred[NW];
  __shared__ double dred[NW];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (r == last_rows[row_b[r]]) {   // the last position has no label
    if (tid == 0) losses[r] = 0.f;
    return;
  }
  const float* row = logits + (size_t)r * ld;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(row), (short)0, (int)((uint32_t)V * 4u), 0x00020000);
  constexpr uint32_t kOut = 0x80000000u;   // past the row: reads 0
  float v[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = tid + k * kCeRegThreads;
    v[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                         rs, i < V ? (uint32_t)i * 4u : kOut, 0, 0));
  }
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (tid + k * kCeRegThreads >= V) v[k] = -INFINITY;   // not a logit
    mx = fmaxf(mx, v[k]);
  }
  mx = wave_max(mx);
  if (lane == 0) fred[w] = mx;
  __syncthreads();
  mx = fred[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) mx = fmaxf(mx, fred[i]);
  // exp(l - max) = 2^((l - max) log2 e); entries that are not logits give 0
  constexpr float kLog2e = 1.44269504088896340736f;
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k) sum += exp2_fast((v[k] - mx) * kLog2e);
  double ds = sum;
  for (int o = 32; o > 0; o >>= 1) ds += __shfl_xor(ds, o, 64);
  if (lane == 0) dred[w] = ds;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int i = 0; i < NW; ++i) t += dred[i];
    losses[r] = (float)((double)mx + log(t) - (double)row[ids[r + 1]]);
  }
}

__global__ __launch_bounds__(kCeThreads) void mean_loss_kernel(
    const float* __restrict__ losses, int M, int nscored, float* __restrict__ mean) {
  __shared__ double part[kCeThreads];
  const int tid = threadIdx.x;
  // contiguous ranges per thread, then a fixed-order sum of the ranges
  const int per = (M + kCeThreads - 1) / kCeThreads;
  double s = 0.0;
  for (int i = tid * per; i < min(M, (tid + 1) * per); ++i) s += losses[i];
  part[tid] = s;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int i = 0; i < kCeThreads; ++i) t += part[i];
    mean[0] = nscored > 0 ? (float)(t / nscored) : 0.f;
  }
}

void launch_cross_entropy(const float* logits, int ld, int V, int M, int nscored,
                          const int32_t* ids, const int32_t* row_b,
                          const int32_t* last_rows, float* losses, float* mean,
                          hipStream_t s) {
  if (M <= 0) return;
  // (the row held in registers: the 1024-position evaluation pass at a
  // vocabulary of 50304 measured 1172 -> 1068 us against the two-pass
  // kernel, whose cross-entropy took 145 us)
  if (V <= 4 * kCeRegThreads)
    cross_entropy_regs_kernel<4><<<M, kCeRegThreads, 0, s>>>(logits, ld, V, ids, row_b, last_rows, losses);
  else if (V <= 16 * kCeRegThreads)
    cross_entropy_regs_kernel<16><<<M, kCeRegThreads, 0, s>>>(logits, ld, V, ids, row_b, last_rows, losses);
  else if (V <= 52 * kCeRegThreads)
    cross_entropy_regs_kernel<52><<<M, kCeRegThreads, 0, s>>>(logits, ld, V, ids, row_b, last_rows, losses);
  else
    cross_entropy_kernel<<<M, kCeThreads, 0, s>>>(logits, ld, V, ids, row_b, last_rows, losses);
  mean_loss_kernel<<<1, kCeThreads, 0, s>>>(losses, M, nscored, mean);
}

}  // namespace ngpt
