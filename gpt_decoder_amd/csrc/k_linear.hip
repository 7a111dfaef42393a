// Linear layers: acc = A W^T with nn.Linear weights W [N][K] (both operands
// K-contiguous), followed by a fused epilogue (bias, GELU, residual add,
// q/K/V split into the cache, fp32 logits).
//
// The layers are the model's c_attn, attention c_proj, MLP c_fc and MLP
// c_proj, plus the tied lm_head (SDK guide "极速上手nanoGPT", "模型架构解析";
// architecture analysis "nanoGPT 架构分析", section 4.1: 4x MLP with GELU,
// pre-LN residual adds, lm_head = wte evaluated on the last position only).
// The q/k/v split follows the serving page's KV-cache section: the c_attn
// output is split at n_embd into q, k, v; head j is the hs-wide slice j.
//
// Kernels:
//   gemm_mfma_kernel  bf16 MFMA (v_mfma_f32_16x16x32_bf16) tile GEMM for
//                     many rows (prefill, batched decode);
//   gemv_kernel       streaming matrix-vector kernel for a few rows (decode),
//                     bandwidth-bound: 16-byte weight loads, one wavefront per
//                     output column;
//   gemm_f32_kernel   fp32 tiled kernel (the fp32 model).
#include "common.hpp"
#include "kernels.hpp"

namespace ngpt {

template <class T, int EPI>
__device__ __forceinline__ void epi_apply(const EpiArgs& e, int r, int n,
                                          float acc) {
  if constexpr (EPI == EPI_LOGITS) {
    if (e.row_pos && e.row_pos[r] < 0) return;
    static_cast<float*>(e.out)[(size_t)r * e.ldo + n] = acc;
    return;
  } else {
    float v = acc;
    if (e.bias) v += to_f32(static_cast<const T*>(e.bias)[n]);
    if constexpr (EPI == EPI_STORE) {
      static_cast<T*>(e.out)[(size_t)r * e.ldo + n] = from_f32<T>(v);
    } else if constexpr (EPI == EPI_GELU) {
      static_cast<T*>(e.out)[(size_t)r * e.ldo + n] = from_f32<T>(gelu_erf(v));
    } else if constexpr (EPI == EPI_RESID) {
      static_cast<float*>(e.out)[(size_t)r * e.ldo + n] += v;
    } else if constexpr (EPI == EPI_QKV) {
      const int which = n / e.C;
      const int c = n - which * e.C;
      if (which == 0) {
        static_cast<T*>(e.out)[(size_t)r * e.ldo + c] = from_f32<T>(v);
        return;
      }
      const int p = e.row_pos[r];
      if (p < 0) return;
      const int b = e.row_b ? e.row_b[r] : r;
      const int h = c / e.hs;
      const int d = c - h * e.hs;
      T* cache = static_cast<T*>(which == 1 ? e.kc : e.vc);
      cache[(((size_t)b * e.H + h) * e.Tb + p) * e.hs + d] = from_f32<T>(v);
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA tile GEMM.  256 threads = 4 wavefronts in a 2x2 arrangement; each
// wavefront owns a (BM/2) x (BN/2) sub-tile built from 16x16 MFMA tiles.  K is
// consumed 64 at a time: the next K-slab is fetched into registers while the
// current one is multiplied out of LDS.
//
// MFMA operand layout used (v_mfma_f32_16x16x32_bf16): lane l supplies row
// (l % 16) of A and column (l % 16) of B, each as 8 consecutive K values
// starting at 8 * (l / 16); the 16x16 fp32 result holds row 4 * (l / 16) + i,
// column l % 16 in element i of lane l.  A and B are fed with the same K
// order, so the dot products do not depend on how the hardware numbers K.
// ---------------------------------------------------------------------------
template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(
    const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ W, int M,
    int N, int K, EpiArgs e) {
  constexpr int BK = 64;
  constexpr int LDS = BK + 8;  // padded row stride (elements)
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int ACH = BM * 8 / 256;  // 16-byte chunks per thread (A tile)
  constexpr int BCH = BN * 8 / 256;
  __shared__ __attribute__((aligned(16))) bf16_t sA[BM * LDS];
  __shared__ __attribute__((aligned(16))) bf16_t sB[BN * LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 ra[ACH], rb[BCH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int c = tid + i * 256;
      const int r = c >> 3, kc = (c & 7) * 8;
      const int row = m0 + r;
      ra[i] = row < M ? *reinterpret_cast<const uint4*>(A + (size_t)row * lda + k0 + kc)
                      : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int c = tid + i * 256;
      const int r = c >> 3, kc = (c & 7) * 8;
      const int row = n0 + r;
      rb[i] = row < N ? *reinterpret_cast<const uint4*>(W + (size_t)row * K + k0 + kc)
                      : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int c = tid + i * 256;
      *reinterpret_cast<uint4*>(sA + (c >> 3) * LDS + (c & 7) * 8) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int c = tid + i * 256;
      *reinterpret_cast<uint4*>(sB + (c >> 3) * LDS + (c & 7) * 8) = rb[i];
    }
  };

  gload(0);
  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
    sstore();
    __syncthreads();
    if (k0 + BK < K) gload(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WM + i * 16 + (lane & 15);
        af[i] = *reinterpret_cast<const bf16x8_t*>(sA + r * LDS + kk + (lane >> 4) * 8);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * WN + j * 16 + (lane & 15);
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(sB + r * LDS + kk + (lane >> 4) * 8);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j],
                                                              acc[i][j], 0, 0, 0);
    }
  }

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * WN + j * 16 + (lane & 15);
      if (col >= N) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m0 + wm * WM + i * 16 + (lane >> 4) * 4 + v;
        if (row < M) epi_apply<bf16_t, EPI>(e, row, col, acc[i][j][v]);
      }
    }
}

// ---------------------------------------------------------------------------
// Streaming GEMV for M <= MR rows: one wavefront per output column n reads the
// weight row W[n][:] once with 16-byte loads and multiplies it with every A
// row; a wavefront-wide reduction finishes each dot product.
// ---------------------------------------------------------------------------
template <class T, int EPI, int MR>
__global__ __launch_bounds__(256) void gemv_kernel(
    const T* __restrict__ A, int lda, const T* __restrict__ W, int M, int N,
    int K, EpiArgs e) {
  constexpr int VE = 16 / sizeof(T);
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.f;
  const T* wr = W + (size_t)n * K;
  for (int k = lane * VE; k < K; k += 64 * VE) {
    float wf[VE];
    if constexpr (sizeof(T) == 2) {
      bf16x8_to_f32(*reinterpret_cast<const uint4*>(wr + k), wf);
    } else {
      const float4 t = *reinterpret_cast<const float4*>(wr + k);
      wf[0] = t.x; wf[1] = t.y; wf[2] = t.z; wf[3] = t.w;
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (m < M) {
        float af[VE];
        if constexpr (sizeof(T) == 2) {
          bf16x8_to_f32(*reinterpret_cast<const uint4*>(A + (size_t)m * lda + k), af);
        } else {
          const float4 t = *reinterpret_cast<const float4*>(A + (size_t)m * lda + k);
          af[0] = t.x; af[1] = t.y; af[2] = t.z; af[3] = t.w;
        }
#pragma unroll
        for (int q = 0; q < VE; ++q) acc[m] = fmaf(af[q], wf[q], acc[m]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = wave_sum(acc[m]);
  if (lane == 0) {
#pragma unroll
    for (int m = 0; m < MR; ++m)
      if (m < M) epi_apply<T, EPI>(e, m, n, acc[m]);
  }
}

// ---------------------------------------------------------------------------
// fp32 tiled GEMM, 16x16 outputs per 256-thread block.
// ---------------------------------------------------------------------------
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float* __restrict__ A, int lda, const float* __restrict__ W, int M,
    int N, int K, EpiArgs e) {
  __shared__ float sA[16][17], sW[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int r = blockIdx.y * 16 + ty;
  const int n = blockIdx.x * 16 + tx;
  const int nw = blockIdx.x * 16 + ty;
  float acc = 0.f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const int k = k0 + tx;
    sA[ty][tx] = (r < M && k < K) ? A[(size_t)r * lda + k] : 0.f;
    sW[ty][tx] = (nw < N && k < K) ? W[(size_t)nw * K + k] : 0.f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) acc = fmaf(sA[ty][kk], sW[tx][kk], acc);
    __syncthreads();
  }
  if (r < M && n < N) epi_apply<float, EPI>(e, r, n, acc);
}

// ---------------------------------------------------------------------------
template <int EPI>
static void dispatch(int dtype, const void* A, int lda, const void* W, int M,
                     int N, int K, const EpiArgs& e, hipStream_t s) {
  if (dtype == NGPT_BF16) {
    const bf16_t* a = static_cast<const bf16_t*>(A);
    const bf16_t* w = static_cast<const bf16_t*>(W);
    if (M <= 8) {
      const dim3 grid((N + 3) / 4);
      if (M <= 1)      gemv_kernel<bf16_t, EPI, 1><<<grid, 256, 0, s>>>(a, lda, w, M, N, K, e);
      else if (M <= 2) gemv_kernel<bf16_t, EPI, 2><<<grid, 256, 0, s>>>(a, lda, w, M, N, K, e);
      else if (M <= 4) gemv_kernel<bf16_t, EPI, 4><<<grid, 256, 0, s>>>(a, lda, w, M, N, K, e);
      else             gemv_kernel<bf16_t, EPI, 8><<<grid, 256, 0, s>>>(a, lda, w, M, N, K, e);
    } else if (M <= 64) {
      const dim3 grid((N + 63) / 64, (M + 63) / 64);
      gemm_mfma_kernel<64, 64, EPI><<<grid, 256, 0, s>>>(a, lda, w, M, N, K, e);
    } else {
      const dim3 grid((N + 127) / 128, (M + 127) / 128);
      gemm_mfma_kernel<128, 128, EPI><<<grid, 256, 0, s>>>(a, lda, w, M, N, K, e);
    }
  } else {
    const float* a = static_cast<const float*>(A);
    const float* w = static_cast<const float*>(W);
    if (M <= 4) {
      const dim3 grid((N + 3) / 4);
      if (M <= 1) gemv_kernel<float, EPI, 1><<<grid, 256, 0, s>>>(a, lda, w, M, N, K, e);
      else        gemv_kernel<float, EPI, 4><<<grid, 256, 0, s>>>(a, lda, w, M, N, K, e);
    } else {
      const dim3 grid((N + 15) / 16, (M + 15) / 16);
      gemm_f32_kernel<EPI><<<grid, 256, 0, s>>>(a, lda, w, M, N, K, e);
    }
  }
}

void launch_linear(int dtype, int epi, const void* A, int lda, const void* W,
                   int M, int N, int K, const EpiArgs& e, hipStream_t s) {
  if (M <= 0 || N <= 0) return;
  switch (epi) {
    case EPI_STORE: dispatch<EPI_STORE>(dtype, A, lda, W, M, N, K, e, s); break;
    case EPI_GELU: dispatch<EPI_GELU>(dtype, A, lda, W, M, N, K, e, s); break;
    case EPI_RESID: dispatch<EPI_RESID>(dtype, A, lda, W, M, N, K, e, s); break;
    case EPI_QKV: dispatch<EPI_QKV>(dtype, A, lda, W, M, N, K, e, s); break;
    default: dispatch<EPI_LOGITS>(dtype, A, lda, W, M, N, K, e, s); break;
  }
}

}  // namespace ngpt
