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
//   cross_entropy_kernel  one workgroup per row: the row maximum, then the sum
//                         of exp(l - max) (fp32 terms, per-thread fp32 sums,
//                         combined in fp64), loss = max + log(sum) - l_target
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
  cross_entropy_kernel<<<M, kCeThreads, 0, s>>>(logits, ld, V, ids, row_b, last_rows, losses);
  mean_loss_kernel<<<1, kCeThreads, 0, s>>>(losses, M, nscored, mean);
}

}  // namespace ngpt
