// Skinny 16-bit MFMA GEMM for a few rows (5 <= M <= 64: the rows of a
// batched decode step, or a short prefill), where a tile GEMM has too few
// tiles to keep the chip busy and its K loop waits on workgroup barriers.
//
// The layers are those of k_linear.hip (c_attn, c_proj, c_fc, the MLP
// c_proj and the tied lm_head of the SDK guide's GPT class), with the same
// per-element epilogues.
//
// A workgroup owns a strip of 16 * NT output columns and a block of 16 * MT
// rows (blockIdx.y; rows past M read zeros); narrow layers (the n_embd-wide
// projections) split the rows over several workgroups so that enough CUs
// stream the weights.  K goes in pairs of MFMA steps (64 values); wavefront w of
// the NWV takes the NP consecutive pairs starting at pair w * NP (pairs past
// K read zeros).  Each 16-row operand fragment of a pair is fetched with two
// loads that cover 8 rows x 128 bytes each (whole cache lines; a load in the
// MFMA operand layout would touch 16 half lines), D pairs ahead in registers,
// then rearranged into the operand layout through the wavefront's own slice
// of LDS, so no workgroup barrier is needed in the loop.  The NWV partial
// sums meet in LDS and are added in wavefront order, then the epilogue runs
// per element.  MFMA operand layout (v_mfma_f32_16x16x32, A fragment first):
// for step s of the pair, lane l feeds row l % 16 of A and column l % 16 of W
// with the 8 K values of 16-byte chunk 4 s + l / 16 of the pair (the same K
// order for both operands); element i of the 16x16 result is row
// 4 * (l / 16) + i, column l % 16.
#include "common.hpp"
#include "epilogue.hpp"
#include "kernels.hpp"

namespace ngpt {

constexpr int kSkinnyMaxRows = 64;

// Epilogue inputs of one output element (row r, column n), fetched before the
// K loop so that their latency overlaps it: the bias, the residual being
// added to, the row's position and cache row or logits row.  The caller
// clamps r and n into range, so every load is issued on every path.
struct SkinnyEpi {
  float pb, pr;
  int pp;
  int64_t pbase;
};
template <class T, int EPI>
__device__ __forceinline__ SkinnyEpi skinny_epi_fetch(const EpiArgs& e, int r, int n) {
  SkinnyEpi p;
  p.pb = (EPI != EPI_LOGITS && e.bias) ? to_f32(static_cast<const T*>(e.bias)[n]) : 0.f;
  p.pr = EPI == EPI_RESID ? static_cast<const float*>(e.out)[(size_t)r * e.ldo + n] : 0.f;
  p.pp = e.row_pos ? e.row_pos[r] : 0;
  p.pbase = 0;
  if constexpr (EPI == EPI_QKV) {
    const int b = e.row_b ? e.row_b[r] : r;
    const int64_t base = kv_block_base(e.kv, b, max(p.pp, 0) / kPageTokens);
    p.pbase = (n >= e.C && p.pp >= 0) ? base : -1;
  } else if constexpr (EPI == EPI_LOGITS) {
    p.pbase = e.row_b ? e.row_b[r] : r;   // the sequence's logits row
  }
  return p;
}
// The epilogue of epi_apply (epilogue.hpp) for one element, acc1 = the dot
// product, with the prefetched inputs.
template <class T, int EPI>
__device__ __forceinline__ void skinny_epi_store(const EpiArgs& e, int r, int n, float acc1,
                                                 const SkinnyEpi& p) {
  if constexpr (EPI == EPI_LOGITS) {
    if (e.row_pos && p.pp < 0) return;
    static_cast<float*>(e.out)[(size_t)p.pbase * e.ldo + n] = acc1;
  } else {
    float v = acc1;
    if (e.bias) v += p.pb;
    if constexpr (EPI == EPI_GELU) {
      static_cast<T*>(e.out)[(size_t)r * e.ldo + n] = from_f32<T>(gelu_erf(v));
    } else if constexpr (EPI == EPI_RESID) {
      static_cast<float*>(e.out)[(size_t)r * e.ldo + n] = p.pr + v;
    } else {   // EPI_QKV
      const int which = n / e.C;
      const int cc = n - which * e.C;
      if (which == 0) {
        static_cast<T*>(e.out)[(size_t)r * e.ldo + cc] = from_f32<T>(v);
        return;
      }
      if (p.pp < 0) return;
      if (p.pbase < 0) {   // unmapped block of a paged cache
        if (e.status) atomicOr(e.status, 4);
        return;
      }
      const int h = cc / e.hs;
      const int d = cc - h * e.hs;
      T* cache = static_cast<T*>(which == 1 ? e.kc : e.vc);
      cache[(size_t)(p.pbase + (int64_t)h * kv_hstride(e.kv) + p.pp % kPageTokens) * e.hs + d] =
          from_f32<T>(v);
    }
  }
}

template <class T, int EPI, int MT, int NT, int NWV, int NP>
__global__ __launch_bounds__(64 * NWV) void gemm_skinny_kernel(
    const T* __restrict__ A, int lda, const T* __restrict__ W, int M, int N, int K,
    EpiArgs e) {
  typedef typename Half16<T>::vec8 vec8;
  constexpr int NF = MT + NT;           // operand fragments per pair
  constexpr int D = NP < 3 ? NP : 3;    // pairs in flight per wavefront
  constexpr uint32_t kOut = 0x80000000u;
  constexpr int BN = 16 * NT, BM = 16 * MT;
  constexpr int RS = 72;                // staging row stride (elements): 64 + 8
  constexpr int STAGE = NF * 16 * RS;   // one wavefront's staging (elements)
  constexpr int kStageBytes = NWV * STAGE * 2;
  constexpr int kRedBytes = NWV * BM * (BN + 1) * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStageBytes > kRedBytes ? kStageBytes
                                                                                     : kRedBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  bf16_t* stage = reinterpret_cast<bf16_t*>(smem) + wave * STAGE;
  const int n0 = blockIdx.x * BN;
  const int r0 = blockIdx.y * BM;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(A), (short)0, (int)((uint32_t)M * (uint32_t)lda * 2u), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(W), (short)0, (int)((uint32_t)N * (uint32_t)K * 2u), 0x00020000);
  // fetch lanes: row 8 u + lane / 8 of a fragment, 16-byte chunk lane % 8
  const int frow = lane >> 3, fch = lane & 7;
  uint32_t off[NF][2];   // byte offsets at K = 0 (kOut: rows past M / N)
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = 8 * u + frow;
      if (f < MT) {
        const int row = r0 + 16 * f + r;
        off[f][u] = row < M ? ((uint32_t)row * (uint32_t)lda + 8u * fch) * 2u : kOut;
      } else {
        const int n = n0 + 16 * (f - MT) + r;
        off[f][u] = n < N ? ((uint32_t)n * (uint32_t)K + 8u * fch) * 2u : kOut;
      }
    }
  const int npairs = K / 64;
  uint4 g[D][NF][2];
  auto load = [&](int st, int i) {
    const int pr = wave * NP + i;
    const bool in = i < NP && pr < npairs;
    const uint32_t kb = (uint32_t)(64 * pr) * 2u;   // this pair's K, bytes
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t o = (off[f][u] == kOut || !in) ? kOut : off[f][u] + kb;
        g[st][f][u] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(f < MT ? ra : rw, o, 0, 0));
      }
  };
  f32x4_t acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[m][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Epilogue inputs of this thread's output elements (idx = tid + q * 64 NWV,
  // row idx / BN, column idx % BN), fetched before the K loop so that their
  // latency overlaps it: the bias, the residual being added to, the row's
  // position and cache row or logits row.  Indices are clamped into range,
  // so every load is issued on every path.
  constexpr int NTHR = 64 * NWV;
  constexpr int EPT = (BM * BN + NTHR - 1) / NTHR;
  SkinnyEpi pre[EPT];
#pragma unroll
  for (int q = 0; q < EPT; ++q) {
    const int idx = tid + q * NTHR;
    pre[q] = skinny_epi_fetch<T, EPI>(e, min(r0 + idx / BN, M - 1), min(n0 + idx % BN, N - 1));
  }
  // (scheduling barriers keep the compiler from sinking the loads towards
  // their use, which would leave fewer pairs in flight)
#pragma unroll
  for (int i = 0; i < D; ++i) load(i, i);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int st = i % D;
    // rows 8 u + frow, chunk fch of every fragment into the staging slice
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        *reinterpret_cast<uint4*>(stage + (f * 16 + 8 * u + frow) * RS + 8 * fch) = g[st][f][u];
    if (i + D < NP) load(st, i + D);
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
      vec8 fr[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f)
        fr[f] = *reinterpret_cast<const vec8*>(stage + (f * 16 + (lane & 15)) * RS +
                                               8 * (4 * sp + (lane >> 4)));
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[m][j] = Half16<T>::mfma(fr[m], fr[MT + j], acc[m][j]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();   // every wavefront is done with its staging slice
  float (*red)[BM][BN + 1] = reinterpret_cast<float (*)[BM][BN + 1]>(smem);
  const int g4 = lane >> 4;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][16 * m + 4 * g4 + v][16 * j + (lane & 15)] = acc[m][j][v];
  __syncthreads();
  // the epilogue of epi_apply (epilogue.hpp) with the prefetched inputs
#pragma unroll
  for (int q = 0; q < EPT; ++q) {
    const int idx = tid + q * NTHR;
    const int rl = idx / BN, c = idx % BN;
    const int r = r0 + rl, n = n0 + c;
    if (idx >= BM * BN || r >= M || n >= N) continue;
    float acc1 = red[0][rl][c];
#pragma unroll
    for (int w = 1; w < NWV; ++w) acc1 += red[w][rl][c];
    skinny_epi_store<T, EPI>(e, r, n, acc1, pre[q]);
  }
}

// Wavefronts per workgroup and pairs per wavefront: 8 wavefronts above 12
// pairs (K > 768) or under 256 workgroups, else 4 (measured at 64 rows of
// GPT-2 small: c_attn 6.0 -> 5.2 us with 8, the lm_head 30.6 -> 24.1 us with
// 4); the pairs per wavefront are bucketed to 2, 4, 7 or 13 (7 and 13 for
// the MLP projection's K = 4 n_embd only).
template <class T, int EPI>
static bool skinny_t(const T* a, int lda, const T* w, int M, int N, int K, const EpiArgs& e,
                     hipStream_t s) {
  constexpr int NT = EPI == EPI_LOGITS ? 2 : 1;
  const int grid = (N + 16 * NT - 1) / (16 * NT);
  const int npairs = K / 64;
  const int nw = (npairs > 12 || grid < 256) ? 8 : 4;
  const int np = (npairs + nw - 1) / nw;
  // rows per workgroup: all of them (up to 64) when the column strips
  // alone fill the chip, else blocks of 32 or 16 rows, so that narrow
  // layers (n_embd outputs: 48 strips at GPT-2 small) are streamed by more
  // CUs; each workgroup then reads a smaller share of the activation rows
  int mt = M > 32 ? 4 : M > 16 ? 2 : 1;
  while (mt > 1 && grid * ((M + 16 * mt - 1) / (16 * mt)) < 256) mt /= 2;
  const dim3 g2(grid, (M + 16 * mt - 1) / (16 * mt));
#define NGPT_SKINNY(NWV, NP)                                                                   \
  do {                                                                                         \
    if (mt == 1)                                                                               \
      gemm_skinny_kernel<T, EPI, 1, NT, NWV, NP><<<g2, 64 * NWV, 0, s>>>(a, lda, w, M, N, K, e); \
    else if (mt == 2)                                                                          \
      gemm_skinny_kernel<T, EPI, 2, NT, NWV, NP><<<g2, 64 * NWV, 0, s>>>(a, lda, w, M, N, K, e); \
    else                                                                                       \
      gemm_skinny_kernel<T, EPI, 4, NT, NWV, NP><<<g2, 64 * NWV, 0, s>>>(a, lda, w, M, N, K, e); \
    return true;                                                                               \
  } while (0)
  if (nw == 4) {
    if (np <= 2) NGPT_SKINNY(4, 2);
    if (np <= 4) NGPT_SKINNY(4, 4);
  } else {
    if (np <= 2) NGPT_SKINNY(8, 2);
    if (np <= 4) NGPT_SKINNY(8, 4);
    if constexpr (EPI == EPI_RESID) {
      if (np <= 7) NGPT_SKINNY(8, 7);
      if (np <= 13) NGPT_SKINNY(8, 13);
    }
  }
#undef NGPT_SKINNY
  return false;
}

template <int EPI>
static bool skinny_epi(int dtype, const void* A, int lda, const void* W, int M, int N, int K,
                       const EpiArgs& e, hipStream_t s) {
  if (dtype == NGPT_BF16)
    return skinny_t<bf16_t, EPI>(static_cast<const bf16_t*>(A), lda,
                                 static_cast<const bf16_t*>(W), M, N, K, e, s);
  return skinny_t<f16_t, EPI>(static_cast<const f16_t*>(A), lda, static_cast<const f16_t*>(W),
                              M, N, K, e, s);
}

bool launch_skinny(int dtype, int epi, const void* A, int lda, const void* W, int M, int N,
                   int K, const EpiArgs& e, hipStream_t s) {
  if (dtype != NGPT_BF16 && dtype != NGPT_F16) return false;
  if (M < 1 || M > kSkinnyMaxRows || K % 64 != 0) return false;
  switch (epi) {
    case EPI_GELU: return skinny_epi<EPI_GELU>(dtype, A, lda, W, M, N, K, e, s);
    case EPI_RESID: return skinny_epi<EPI_RESID>(dtype, A, lda, W, M, N, K, e, s);
    case EPI_QKV: return skinny_epi<EPI_QKV>(dtype, A, lda, W, M, N, K, e, s);
    case EPI_LOGITS: return skinny_epi<EPI_LOGITS>(dtype, A, lda, W, M, N, K, e, s);
    default: return false;
  }
}


}  // namespace ngpt
