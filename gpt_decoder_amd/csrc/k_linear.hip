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
//                     many rows (prefill, eval);
//   gemv_kernel       streaming matrix-vector kernel for up to 4 rows (decode),
//                     bandwidth-bound: 16-byte weight loads issued ahead of the
//                     activations, optional fused LayerNorm prologue;
//   gemm_f32_kernel   fp32 tiled kernel (the fp32 model).
// (5 to 64 rows of a batched decode step go to the skinny kernel of
// k_skinny.hip.)
#include "common.hpp"
#include "epilogue.hpp"
#include "kernels.hpp"

namespace ngpt {

constexpr int kGemvMaxRows = 4;  // rows handled by the streaming kernels
constexpr int kGemvLnMaxK = 2048;  // widest row the fused LayerNorm holds (n_embd limit)

// A 16-bit element from its bit pattern.
template <class T> __device__ __forceinline__ float bits_to_f32(uint32_t u16);
template <> __device__ __forceinline__ float bits_to_f32<bf16_t>(uint32_t u16) {
  return to_f32(static_cast<bf16_t>(u16));
}
template <> __device__ __forceinline__ float bits_to_f32<f16_t>(uint32_t u16) {
  return to_f32(__builtin_bit_cast(f16_t, static_cast<uint16_t>(u16)));
}

// Bias of four consecutive output columns col .. col + 3 (the MFMA kernel's
// 16-bit epilogues), by value so that nothing goes to scratch; columns at or
// past N get none.
template <class T>
__device__ __forceinline__ uint2 pack4(float4 v) {
  return make_uint2(Half16<T>::pack2(v.x, v.y), Half16<T>::pack2(v.z, v.w));
}

// Wait until at most N vector-memory operations of this wavefront are
// outstanding (s_waitcnt with vmcnt = N; lgkm and export counts not waited).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
template <int P>
__device__ __forceinline__ void wait_vmcnt_stages(int n) {
  // n whole stages of P loads may stay in flight (n <= 3)
  switch (n) {
    case 3: wait_vmcnt<3 * P>(); break;
    case 2: wait_vmcnt<2 * P>(); break;
    case 1: wait_vmcnt<P>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

// One 16-byte direct-to-LDS buffer load per lane: lane i's bytes land at
// lds + 16 i (the LDS address must be the same in every lane).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
}

// K loop of the tile GEMM with its operands loaded straight into LDS
// (buffer_load ... lds), NS stages of one 64-wide K-slab each, NS - 1
// slabs in flight.  No registers stage the operands and no LDS store
// instructions are issued, so the ring can be deeper than the register
// path's two LDS buffers (four 28 KB stages for 128 x 96 tiles).
//
// Stage layout: A rows then W rows of the slab, 128 bytes (64 elements)
// each.  One load instruction fills 1 KB = 8 rows: lane i brings row i / 8
// and places it in 16-byte slot i % 8 of that row, which holds K-chunk
// (i % 8) ^ (row % 8); the XOR lets the 16 lanes of an MFMA fragment read
// (16 rows at one K-chunk) fall in different LDS banks.
//
// Each stage lives in its own __shared__ array, and every slab index is a
// compile-time constant (NK slabs, fully unrolled), so each wait is exact:
// before slab it is used, every wavefront waits until only the loads of
// the later slabs it has issued are outstanding, then all meet at a
// barrier (their loads of slab it are then complete); the slab it + NS - 1
// loads then go into the stage that slab it - 1 used, which every
// wavefront has finished reading by that barrier.
template <class T, int BM, int BN, int NS, int NK, bool kSwap, int TM, int TN, int NW = 4>
__device__ __forceinline__ void kloop_dma(__amdgpu_buffer_rsrc_t ra_rs, __amdgpu_buffer_rsrc_t rb_rs,
                                          int lda, int K, int M, int N, int m0, int n0,
                                          f32x4_t (&acc)[TM][TN]) {
  typedef typename Half16<T>::vec8 vec8;
  static_assert(NS >= 2 && NS <= 4 && NK >= 0, "stages / slabs (NK = 0: K / 64 at run time)");
  constexpr int WM = BM / (NW / 2), WN = BN / 2;   // NW wavefronts as (NW / 2) x 2
  constexpr int PA = BM / (8 * NW), PB = BN / (8 * NW);   // load instructions per wavefront per slab
  static_assert(PA * 8 * NW == BM && PB * 8 * NW == BN, "whole 8-row loads per wavefront");
  constexpr int P = PA + PB;
  constexpr int SB = (BM + BN) * 128;         // bytes per stage
  constexpr uint32_t kOut = 0x80000000u;      // offset past every buffer: reads 0
  __shared__ __attribute__((aligned(1024))) char st0[SB];
  __shared__ __attribute__((aligned(1024))) char st1[SB];
  __shared__ __attribute__((aligned(1024))) char st2[NS > 2 ? SB : 16];
  __shared__ __attribute__((aligned(1024))) char st3[NS > 3 ? SB : 16];
  auto stage = [&](int i) -> char* {
    const int q = i % NS;
    return q == 0 ? st0 : q == 1 ? st1 : q == 2 ? st2 : st3;
  };
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane >> 3;          // row within the 8 rows of a load
  const int lc = (lane & 7) ^ lr;    // the K-chunk this lane brings
  uint32_t aoff[PA], boff[PB];
#pragma unroll
  for (int j = 0; j < PA; ++j) {
    const int row = m0 + (wave * PA + j) * 8 + lr;
    aoff[j] = row < M ? ((uint32_t)row * (uint32_t)lda + (uint32_t)lc * 8u) * 2u : kOut;
  }
#pragma unroll
  for (int j = 0; j < PB; ++j) {
    const int row = n0 + (wave * PB + j) * 8 + lr;
    boff[j] = row < N ? ((uint32_t)row * (uint32_t)K + (uint32_t)lc * 8u) * 2u : kOut;
  }
  auto issue = [&](int it) {
    char* base = stage(it);
    const uint32_t kb = (uint32_t)it * 128u;   // byte offset of the slab within a row
#pragma unroll
    for (int j = 0; j < PA; ++j)
      dma16(ra_rs, base + (wave * PA + j) * 1024, aoff[j] == kOut ? kOut : aoff[j] + kb);
#pragma unroll
    for (int j = 0; j < PB; ++j)
      dma16(rb_rs, base + BM * 128 + (wave * PB + j) * 1024, boff[j] == kOut ? kOut : boff[j] + kb);
  };

  auto slab = [&](int it, int nk) {
    const int last = (it + NS - 2 < nk - 1) ? it + NS - 2 : nk - 1;
    wait_vmcnt_stages<P>(last - it);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (it + NS - 1 < nk) issue(it + NS - 1);
    const char* sa = stage(it);
    const char* sb = sa + BM * 128;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      vec8 af[TM], bfr[TN];
      const int c = kk * 4 + (lane >> 4);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WM + i * 16 + (lane & 15);
        af[i] = *reinterpret_cast<const vec8*>(sa + r * 128 + ((c ^ (r & 7)) << 4));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * WN + j * 16 + (lane & 15);
        bfr[j] = *reinterpret_cast<const vec8*>(sb + r * 128 + ((c ^ (r & 7)) << 4));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = kSwap ? Half16<T>::mfma(bfr[j], af[i], acc[i][j])
                            : Half16<T>::mfma(af[i], bfr[j], acc[i][j]);
    }
  };
  if constexpr (NK > 0) {
#pragma unroll
    for (int i = 0; i < NS - 1; ++i)
      if (i < NK) issue(i);
#pragma unroll
    for (int it = 0; it < NK; ++it) slab(it, NK);
  } else {
    // K known at run time: the loop goes in rounds of NS slabs, so that
    // each slab's stage is still a compile-time constant
    const int nk = K / 64;
#pragma unroll
    for (int i = 0; i < NS - 1; ++i)
      if (i < nk) issue(i);
    for (int it0 = 0; it0 < nk; it0 += NS) {
#pragma unroll
      for (int st = 0; st < NS; ++st)
        if (it0 + st < nk) slab(it0 + st, nk);
    }
  }
}

// ---------------------------------------------------------------------------
// 16-bit MFMA tile GEMM (bf16 or fp16 operands, fp32 accumulation; the
// v_mfma_f32_16x16x32 bf16 / f16 instruction of the operand type).  256
// threads = 4 wavefronts in a 2x2 arrangement; each
// wavefront owns a (BM/2) x (BN/2) sub-tile built from 16x16 MFMA tiles.  K is
// consumed 64 at a time through a two-stage LDS ring: the next K-slab is
// fetched into registers while the current one is multiplied, then written
// to the other LDS stage, so one barrier per K-slab suffices.
//
// Tile order is XCD-aware: workgroups are dealt round-robin to the 8 XCDs,
// so tile t goes to the workgroup that lands on XCD t / (tiles / 8); each XCD
// then walks its tiles with the row-block index fastest, and tiles sharing a
// weight panel run back to back on the same L2.
//
// MFMA operand layout used (v_mfma_f32_16x16x32_bf16): lane l supplies row
// (l % 16) of the first operand and column (l % 16) of the second, each as 8
// consecutive K values starting at 8 * (l / 16); the 16x16 fp32 result holds
// row 4 * (l / 16) + i, column l % 16 in element i of lane l.  For the bf16
// outputs (q/k/v and GELU) the weight fragment goes first: each
// 16x16 result is then a tile of (A W^T)^T, and lane l holds output row
// (l % 16) at four consecutive columns, written with one 8-byte store.  For
// the fp32 outputs (residual add, logits) the A fragment goes first, and 16
// lanes cover 16 consecutive columns of a row (measured faster for the
// read-modify-write of the residual).  Both operands are fed with the same K
// order, so the dot products do not depend on how the hardware numbers K.
// ---------------------------------------------------------------------------
template <class T, int BM, int BN, int EPI, int S, int NKC = 0, bool DMA = false, int NW = 4>
__global__ __launch_bounds__(64 * NW) void gemm_mfma_kernel(
    const T* __restrict__ A, int lda, const T* __restrict__ W, int M,
    int N, int K, EpiArgs e) {
  typedef typename Half16<T>::vec8 vec8;
  constexpr int BK = 64;
  constexpr int LDS = BK + 8;  // padded row stride (elements)
  static_assert(NW == 4 || (NW == 8 && DMA), "eight wavefronts only with the direct-to-LDS loop");
  constexpr int WM = BM / (NW / 2), WN = BN / 2;   // NW wavefronts as (NW / 2) x 2
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int ACH = BM * 8 / 256;  // 16-byte chunks per thread (A tile)
  constexpr int BCH = BN * 8 / 256;
  constexpr uint32_t kOut = 0x80000000u;  // offset past every buffer: reads 0
  // weight fragment first for the bf16-output epilogues (see the epilogue)
  constexpr bool kSwap = (EPI == EPI_QKV || EPI == EPI_GELU);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int mt = (M + BM - 1) / BM;
  const int ntile = gridDim.x;
  int t = blockIdx.x;
  if ((ntile & 7) == 0) t = (t & 7) * (ntile >> 3) + (t >> 3);
  const int m0 = (t % mt) * BM;
  const int n0 = (t / mt) * BN;

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Range-checked buffer loads: rows past M / N and K-slabs past K read
  // zeros, and every load is issued on every path, so the wait before a
  // stage is used covers exactly that stage.
  const __amdgpu_buffer_rsrc_t ra_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(A), (short)0, (int)((uint32_t)M * (uint32_t)lda * 2u), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(W), (short)0, (int)((uint32_t)N * (uint32_t)K * 2u), 0x00020000);
  auto ld16 = [](__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  };
  uint4 ra[DMA ? 1 : S][ACH], rb[DMA ? 1 : S][BCH];
  auto gload = [&](int st, int k0) {
    const bool kin = k0 < K;
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int c = tid + i * 256;
      const int row = m0 + (c >> 3), kc = (c & 7) * 8;
      ra[st][i] = ld16(ra_rs, (kin && row < M)
                                  ? ((uint32_t)row * (uint32_t)lda + (uint32_t)(k0 + kc)) * 2u
                                  : kOut);
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int c = tid + i * 256;
      const int row = n0 + (c >> 3), kc = (c & 7) * 8;
      rb[st][i] = ld16(rb_rs, (kin && row < N)
                                  ? ((uint32_t)row * (uint32_t)K + (uint32_t)(k0 + kc)) * 2u
                                  : kOut);
    }
  };

  // Register path: S K-slabs in flight in registers; slab it goes
  // registers -> LDS buffer it % 2 -> MFMA.  The trip count is rounded up
  // to a multiple of S (the extra slabs are zeros).
  const int nk = NKC > 0 ? NKC : K / BK;
  const int nkp = ((nk + S - 1) / S) * S;
  constexpr int kUnroll = NKC > 0 ? 64 : 1;   // whole loop when K is known
  if constexpr (!DMA) {
#pragma unroll
    for (int st = 0; st < S; ++st) gload(st, st * BK);
  }

  // Epilogue inputs that do not depend on the product are fetched before
  // the K loop (after its first slabs' loads are issued), which hides their
  // latency: the rows' cache positions (QKV), the bias of the 16-bit
  // epilogues and, for small tiles, the residual values being added to
  // (RESID).  Every fetch is a range-checked buffer load issued on every
  // path: loads behind per-lane branches were each waited for in turn,
  // before the K loop's first loads were even issued.
  // (kSwap: lane l holds output row (l % 16) of each row fragment at the
  // four consecutive columns 4 * (l / 16) + i of each column fragment;
  // otherwise column (l % 16) at rows 4 * (l / 16) + i)
  auto out_row = [&](int i) { return m0 + wm * WM + i * 16 + (lane & 15); };
  auto out_col = [&](int j) { return n0 + wn * WN + j * 16 + (lane >> 4) * 4; };
  auto rsrc = [](const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0,
                                             p ? (int)bytes : 0, 0x00020000);
  };
  // QKV: each output row's position and sequence (the cache rows are
  // formed after the K loop, where a paged cache's table read costs no
  // wait in front of the loop)
  constexpr bool kQkv = EPI == EPI_QKV;
  int pv[kQkv ? TM : 1], sv[kQkv ? TM : 1];
  constexpr bool kPreRes = (EPI == EPI_RESID) && TM * TN * 4 <= 16;
  float res[kPreRes ? TM : 1][kPreRes ? TN : 1][4];
  constexpr bool kPreBias = (EPI == EPI_QKV || EPI == EPI_GELU);
  float bias4[kPreBias ? TN : 1][4];
  if constexpr (kQkv) {
    const __amdgpu_buffer_rsrc_t rp = rsrc(e.row_pos, (uint32_t)M * 4u);
    const __amdgpu_buffer_rsrc_t rbq = rsrc(e.row_b, (uint32_t)M * 4u);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const uint32_t off = (uint32_t)min(out_row(i), M - 1) * 4u;
      pv[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(rp, off, 0, 0);
      sv[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(rbq, off, 0, 0);
    }
  }
  if constexpr (kPreBias) {
    const __amdgpu_buffer_rsrc_t rb16 = rsrc(e.bias, (uint32_t)N * 2u);
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int col = out_col(j) + v;
        const uint32_t u = __builtin_amdgcn_raw_buffer_load_b16(
            rb16, col < N ? (uint32_t)col * 2u : kOut, 0, 0);
        bias4[j][v] = bits_to_f32<T>(u & 0xffffu);
      }
  }
  float biasr[kPreRes ? TN : 1];   // RESID: the bias of this lane's column
  if constexpr (kPreRes) {
    const __amdgpu_buffer_rsrc_t rb16 = rsrc(e.bias, (uint32_t)N * 2u);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * WN + j * 16 + (lane & 15);
      biasr[j] = bits_to_f32<T>(__builtin_amdgcn_raw_buffer_load_b16(
                     rb16, col < N ? (uint32_t)col * 2u : kOut, 0, 0) & 0xffffu);
    }
    const float* o = static_cast<const float*>(e.out);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = min(m0 + wm * WM + i * 16 + (lane >> 4) * 4 + v, M - 1);
          const int col = min(n0 + wn * WN + j * 16 + (lane & 15), N - 1);
          res[i][j][v] = o[(size_t)row * e.ldo + col];
        }
  }

  if constexpr (DMA) {
    kloop_dma<T, BM, BN, S, NKC, kSwap, TM, TN, NW>(ra_rs, rb_rs, lda, K, M, N, m0, n0, acc);
  } else {
    __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * LDS];
    __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * LDS];
    auto sstore = [&](int st, int buf) {
#pragma unroll
      for (int i = 0; i < ACH; ++i) {
        const int c = tid + i * 256;
        *reinterpret_cast<uint4*>(sA[buf] + (c >> 3) * LDS + (c & 7) * 8) = ra[st][i];
      }
#pragma unroll
      for (int i = 0; i < BCH; ++i) {
        const int c = tid + i * 256;
        *reinterpret_cast<uint4*>(sB[buf] + (c >> 3) * LDS + (c & 7) * 8) = rb[st][i];
      }
    };
#pragma unroll kUnroll
    for (int it0 = 0; it0 < nkp; it0 += S) {
#pragma unroll
      for (int st = 0; st < S; ++st) {
        const int it = it0 + st;
        const int buf = st & 1;   // S is even, so it % 2 == st % 2
        sstore(st, buf);
        __syncthreads();
        gload(st, (it + S) * BK);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
          vec8 af[TM], bfr[TN];
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            const int r = wm * WM + i * 16 + (lane & 15);
            af[i] = *reinterpret_cast<const vec8*>(sA[buf] + r * LDS + kk + (lane >> 4) * 8);
          }
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int r = wn * WN + j * 16 + (lane & 15);
            bfr[j] = *reinterpret_cast<const vec8*>(sB[buf] + r * LDS + kk + (lane >> 4) * 8);
          }
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i][j] = kSwap ? Half16<T>::mfma(bfr[j], af[i], acc[i][j])
                                : Half16<T>::mfma(af[i], bfr[j], acc[i][j]);
        }
      }
    }
  }

  if constexpr (EPI == EPI_QKV) {
    // cache row (of hs elements, head 0) of each output row's position, -1
    // for inactive rows and unmapped blocks (the latter flagged); the block
    // table of a paged cache is read here, the entries of inactive rows not
    // at all (offset past the end)
    int64_t rrow[TM];
    const __amdgpu_buffer_rsrc_t rt = rsrc(e.kv.table, 0x7FFFFFF0u);
    int pg[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int sq = e.row_b ? sv[i] : min(out_row(i), M - 1);
      sv[i] = sq;
      const uint32_t off = pv[i] >= 0 ? (uint32_t)(sq * e.kv.nblk + pv[i] / kPageTokens) * 4u
                                       : kOut;
      pg[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(rt, off, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int p = pv[i];
      int64_t base = -1;
      if (p >= 0) {
        if (!e.kv.table)
          base = (int64_t)sv[i] * e.kv.H * e.kv.Tb + (int64_t)(p / kPageTokens) * kPageTokens;
        else if ((uint32_t)pg[i] < (uint32_t)e.kv.npages)
          base = (int64_t)pg[i] * e.kv.H * kPageTokens;
      }
      if (p >= 0 && base < 0 && e.status) atomicOr(e.status, 4);
      rrow[i] = base < 0 ? -1 : base + p % kPageTokens;
    }
    // columns -> q / k / v, head, dim once per column fragment (the four
    // columns of a lane lie in one head: 4 | hs, and 4 | ldo = n_embd)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = out_col(j);
      if (col >= N) continue;
      const int which = col / e.C;
      const int c = col - which * e.C;
      const int hh = c / e.hs, d = c - hh * e.hs;
      const int64_t hoff = (int64_t)hh * kv_hstride(e.kv);
      T* cache = static_cast<T*>(which == 1 ? e.kc : e.vc);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = out_row(i);
        if (row >= M) continue;
        float4 v = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        if (e.bias) v = make_float4(v.x + bias4[j][0], v.y + bias4[j][1], v.z + bias4[j][2],
                                    v.w + bias4[j][3]);
        const uint2 packed = pack4<T>(v);
        if (which == 0) {
          *reinterpret_cast<uint2*>(static_cast<T*>(e.out) + (size_t)row * e.ldo + c) = packed;
        } else if (rrow[i] >= 0) {
          *reinterpret_cast<uint2*>(cache + (size_t)(rrow[i] + hoff) * e.hs + d) = packed;
        }
      }
    }
  } else if constexpr (kSwap) {  // EPI_GELU: 16-bit rows
    const bool vec = (e.ldo & 3) == 0;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = out_row(i), col = out_col(j);
        if (row >= M || col >= N) continue;
        float4 v = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        if (e.bias) v = make_float4(v.x + bias4[j][0], v.y + bias4[j][1], v.z + bias4[j][2],
                                    v.w + bias4[j][3]);
        v = make_float4(gelu_erf(v.x), gelu_erf(v.y), gelu_erf(v.z), gelu_erf(v.w));
        T* o = static_cast<T*>(e.out) + (size_t)row * e.ldo + col;
        if (vec && col + 3 < N) {
          *reinterpret_cast<uint2*>(o) = pack4<T>(v);
        } else {
          o[0] = from_f32<T>(v.x);
          if (col + 1 < N) o[1] = from_f32<T>(v.y);
          if (col + 2 < N) o[2] = from_f32<T>(v.z);
          if (col + 3 < N) o[3] = from_f32<T>(v.w);
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = n0 + wn * WN + j * 16 + (lane & 15);
        if (col >= N) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = m0 + wm * WM + i * 16 + (lane >> 4) * 4 + v;
          if (row >= M) continue;
          if constexpr (kPreRes) {
            float val = acc[i][j][v];
            if (e.bias) val += biasr[j];
            static_cast<float*>(e.out)[(size_t)row * e.ldo + col] = res[i][j][v] + val;
          } else {
            epi_apply<T, EPI>(e, row, col, acc[i][j][v]);
          }
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Streaming GEMV for M <= MR (1, 2 or 4) rows, one wavefront per workgroup.
// A wavefront owns CPW consecutive output columns; lane l multiplies the
// K-elements l*VE .. l*VE+VE-1 of each 64*VE-wide chunk.  Every chunk's
// weight loads (16 bytes per lane per column) are issued before the
// activations are touched, so the weight stream is in flight while the
// activation rows (and their LayerNorm statistics) arrive.
//
// With LN, the A rows are LN(x) computed here from the fp32 residual x:
// each lane normalises exactly the elements it multiplies, and rounds them to
// the model dtype as the bf16 data path stores its LayerNorm output.
// ---------------------------------------------------------------------------

// Sum R = 2^LG values across the wavefront.  Returns the sum of value index
// (lane >> (6 - LG)) in lanes whose low (6 - LG) bits are zero.
template <int LG>
__device__ __forceinline__ float wave_reduce_multi(float* v) {
  constexpr int R = 1 << LG;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int st = 0; st < LG; ++st) {
    const int o = 32 >> st;
    const int cnt = R >> st;
    const bool hi = (lane & o) != 0;
#pragma unroll
    for (int i = 0; i < cnt / 2; ++i) {
      const float send = hi ? v[i] : v[i + cnt / 2];
      const float keep = hi ? v[i + cnt / 2] : v[i];
      v[i] = keep + __shfl_xor(send, o, 64);
    }
  }
  float r = v[0];
#pragma unroll
  for (int o = 32 >> LG; o > 0; o >>= 1) r += __shfl_xor(r, o, 64);
  return r;
}

__device__ __forceinline__ void load_vec(const bf16_t* p, float* f) {
  bf16x8_to_f32(*reinterpret_cast<const uint4*>(p), f);
}
__device__ __forceinline__ void load_vec(const f16_t* p, float* f) {
  f16x8_to_f32(*reinterpret_cast<const uint4*>(p), f);
}
__device__ __forceinline__ void load_vec(const float* p, float* f) {
  const float4 t = *reinterpret_cast<const float4*>(p);
  f[0] = t.x; f[1] = t.y; f[2] = t.z; f[3] = t.w;
}
template <class T>
__device__ __forceinline__ float round_to(float v) {
  return to_f32(from_f32<T>(v));
}

template <class T, int EPI, int MR, int CPW, int NCH, bool LN>
__global__ __launch_bounds__(64) void gemv_kernel(
    const T* __restrict__ A, int lda, LnArgs ln, const T* __restrict__ W,
    int M, int N, int K, EpiArgs e) {
  constexpr int VE = 16 / sizeof(T);
  constexpr int SPAN = 64 * VE;
  constexpr int LG = (MR * CPW == 1) ? 0 : (MR * CPW == 2) ? 1
                   : (MR * CPW == 4) ? 2 : (MR * CPW == 8) ? 3 : 4;
  static_assert((1 << LG) == MR * CPW, "MR*CPW must be a power of two <= 16");
  const int lane = threadIdx.x;
  const int n0 = blockIdx.x * CPW;

  // 1. every load of this lane, issued before any of them is used, through
  // range-checked buffer loads: a lane past K (the last chunk of a K that is
  // not a multiple of the span) or a row past M reads zeros, and no load
  // sits behind a per-lane branch (each such load was waited for before the
  // next was issued)
  constexpr uint32_t kOut = 0x80000000u;   // offset past every buffer: reads 0
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(W), (short)0, (int)((uint32_t)N * (uint32_t)K * (uint32_t)sizeof(T)),
      0x00020000);
  uint4 wv[NCH][CPW];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int k = j * SPAN + lane * VE;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int n = min(n0 + c, N - 1);
      wv[j][c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
          rw, k < K ? ((uint32_t)n * (uint32_t)K + (uint32_t)k) * (uint32_t)sizeof(T) : kOut,
          0, 0));
    }
  }
  // A rows: LN keeps the raw fp32 x values (normalised below); otherwise the
  // packed 16-byte vectors are kept and widened at use
  float av[LN ? MR : 1][LN ? NCH : 1][VE];
  uint4 araw[LN ? 1 : MR][LN ? 1 : NCH];
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      LN ? const_cast<float*>(ln.x) : static_cast<void*>(const_cast<T*>(A)), (short)0,
      LN ? (int)((uint32_t)M * (uint32_t)ln.ldx * 4u)
         : (int)((uint32_t)M * (uint32_t)lda * (uint32_t)sizeof(T)),
      0x00020000);
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int k = j * SPAN + lane * VE;
      const bool ok = m < M && k < K;
      if constexpr (LN) {
        const uint32_t xo = ok ? ((uint32_t)m * (uint32_t)ln.ldx + (uint32_t)k) * 4u : kOut;
#pragma unroll
        for (int q = 0; q < VE; q += 4) {
          const float4 t4 = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
              ra, xo == kOut ? kOut : xo + (uint32_t)q * 4u, 0, 0));
          av[m][j][q] = t4.x; av[m][j][q + 1] = t4.y;
          av[m][j][q + 2] = t4.z; av[m][j][q + 3] = t4.w;
        }
      } else {
        araw[m][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
            ra, ok ? ((uint32_t)m * (uint32_t)lda + (uint32_t)k) * (uint32_t)sizeof(T) : kOut,
            0, 0));
      }
    }

  // 2. LayerNorm of the A rows (two-pass statistics over the K features)
  if constexpr (LN) {
    float g[NCH][VE], bb[NCH][VE];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int k = j * SPAN + lane * VE;
      if (k < K) {
        load_vec(static_cast<const T*>(ln.w) + k, g[j]);
        if (ln.b) load_vec(static_cast<const T*>(ln.b) + k, bb[j]);
        else {
#pragma unroll
          for (int q = 0; q < VE; ++q) bb[j][q] = 0.f;
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float sm = 0.f;
#pragma unroll
      for (int j = 0; j < NCH; ++j)
#pragma unroll
        for (int q = 0; q < VE; ++q) sm += av[m][j][q];
      const float mu = wave_sum(sm) / (float)K;
      float sq = 0.f;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int k = j * SPAN + lane * VE;
        if (k < K) {
#pragma unroll
          for (int q = 0; q < VE; ++q) {
            const float d = av[m][j][q] - mu;
            sq += d * d;
          }
        }
      }
      const float rs = 1.0f / sqrtf(wave_sum(sq) / (float)K + 1e-5f);
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int k = j * SPAN + lane * VE;
#pragma unroll
        for (int q = 0; q < VE; ++q)
          av[m][j][q] = (k < K) ? round_to<T>((av[m][j][q] - mu) * rs * g[j][q] + bb[j][q]) : 0.f;
      }
    }
  }

  // 3. dot products
  float acc[MR * CPW];
#pragma unroll
  for (int i = 0; i < MR * CPW; ++i) acc[i] = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      float wf[VE];
      if constexpr (sizeof(T) == 2) {
        Half16<T>::unpack8(wv[j][c], wf);
      } else {
        wf[0] = __uint_as_float(wv[j][c].x);
        wf[1] = __uint_as_float(wv[j][c].y);
        wf[2] = __uint_as_float(wv[j][c].z);
        wf[3] = __uint_as_float(wv[j][c].w);
      }
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        float af[VE];
        if constexpr (LN) {
#pragma unroll
          for (int q = 0; q < VE; ++q) af[q] = av[m][j][q];
        } else if constexpr (sizeof(T) == 2) {
          Half16<T>::unpack8(araw[m][j], af);
        } else {
          af[0] = __uint_as_float(araw[m][j].x);
          af[1] = __uint_as_float(araw[m][j].y);
          af[2] = __uint_as_float(araw[m][j].z);
          af[3] = __uint_as_float(araw[m][j].w);
        }
#pragma unroll
        for (int q = 0; q < VE; ++q)
          acc[m * CPW + c] = fmaf(af[q], wf[q], acc[m * CPW + c]);
      }
    }
  }

  const float r = wave_reduce_multi<LG>(acc);
  constexpr int LOW = (1 << (6 - LG)) - 1;
  if ((lane & LOW) == 0) {
    const int idx = lane >> (6 - LG);
    const int m = idx / CPW, c = idx % CPW;
    const int n = n0 + c;
    if (m < M && n < N) epi_apply<T, EPI>(e, m, n, r);
  }
}

// ---------------------------------------------------------------------------
// Decode output projection with the attention chunk merge folded in:
//   y[m] = merge over key chunks of the split-K attention records,
//   x[m] += y[m] W_proj^T + b.
// 256 threads; each wavefront owns 4 output columns.  Weight loads are issued
// first; the merge of every (row, head, dim) item then fills an LDS copy of
// y (rounded to the model dtype, as the attention output is stored), records
// merged in chunk order with eight records' loads in flight at a time.
// ---------------------------------------------------------------------------
constexpr int kProjCols = 16;       // output columns per workgroup
constexpr int kProjMaxK = 2048;     // n_embd bound

template <class T, int HS, int MR, int NCH>
__global__ __launch_bounds__(256) void attn_proj_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ pos, int H,
    int nchunk, int chunk_keys, const T* __restrict__ W, int M, int N, int K,
    EpiArgs e) {
  constexpr int VE = 16 / sizeof(T);
  constexpr int SPAN = 64 * VE;
  constexpr int CPW = 4;
  constexpr int PS = HS + 2;
  constexpr int LG = (MR * CPW == 4) ? 2 : (MR * CPW == 8) ? 3 : 4;
  __shared__ __attribute__((aligned(16))) float sy[MR][kProjMaxK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * kProjCols + wave * CPW;

  // weight loads first, range-checked on every path (lanes past K read 0)
  constexpr uint32_t kOut = 0x80000000u;
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(W), (short)0, (int)((uint32_t)N * (uint32_t)K * (uint32_t)sizeof(T)),
      0x00020000);
  uint4 wv[NCH][CPW];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int k = j * SPAN + lane * VE;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int n = min(n0 + c, N - 1);
      wv[j][c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
          rw, k < K ? ((uint32_t)n * (uint32_t)K + (uint32_t)k) * (uint32_t)sizeof(T) : kOut,
          0, 0));
    }
  }

  for (int it = tid; it < M * K; it += 256) {
    const int m = it / K, f = it - m * K;
    const int h = f / HS, d = f - h * HS;
    const int p = pos[m];
    float yv = 0.f;
    if (p >= 0) {
      const int nact = p / chunk_keys + 1;
      const float* base = part + ((size_t)m * H + h) * nchunk * PS;
      float mm = -INFINITY, ll = 0.f, oo = 0.f;
      for (int c0 = 0; c0 < nact; c0 += 8) {
        float rm[8], rl[8], ro[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float* r = base + (size_t)(c0 + u) * PS;
          const bool ok = c0 + u < nact;
          rm[u] = ok ? r[0] : -INFINITY;
          rl[u] = ok ? r[1] : 0.f;
          ro[u] = ok ? r[2 + d] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) merge_state(mm, ll, &oo, rm[u], rl[u], &ro[u], 1);
      }
      yv = round_to<T>(oo / ll);
    }
    sy[m][f] = yv;
  }
  __syncthreads();

  float acc[MR * CPW];
#pragma unroll
  for (int i = 0; i < MR * CPW; ++i) acc[i] = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int k = j * SPAN + lane * VE;
    if (k >= K) break;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      float wf[VE];
      if constexpr (sizeof(T) == 2) {
        Half16<T>::unpack8(wv[j][c], wf);
      } else {
        wf[0] = __uint_as_float(wv[j][c].x);
        wf[1] = __uint_as_float(wv[j][c].y);
        wf[2] = __uint_as_float(wv[j][c].z);
        wf[3] = __uint_as_float(wv[j][c].w);
      }
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int q = 0; q < VE; ++q)
          acc[m * CPW + c] = fmaf(sy[m][k + q], wf[q], acc[m * CPW + c]);
    }
  }
  const float r = wave_reduce_multi<LG>(acc);
  constexpr int LOW = (1 << (6 - LG)) - 1;
  if ((lane & LOW) == 0) {
    const int idx = lane >> (6 - LG);
    const int m = idx / CPW, c = idx % CPW;
    const int n = n0 + c;
    if (m < M && n < N) epi_apply<T, EPI_RESID>(e, m, n, r);
  }
}

template <class T, int HS, int MR>
static void launch_attn_proj_t(const float* part, const int32_t* pos, int H,
                               int nchunk, int chunk_keys, const T* W, int M,
                               int N, int K, const EpiArgs& e, hipStream_t s) {
  constexpr int SPAN = 64 * (16 / sizeof(T));
  const int grid = (N + kProjCols - 1) / kProjCols;
  if (K <= 2 * SPAN)
    attn_proj_kernel<T, HS, MR, 2><<<grid, 256, 0, s>>>(part, pos, H, nchunk, chunk_keys, W, M, N, K, e);
  else if (K <= 4 * SPAN)
    attn_proj_kernel<T, HS, MR, 4><<<grid, 256, 0, s>>>(part, pos, H, nchunk, chunk_keys, W, M, N, K, e);
  else
    attn_proj_kernel<T, HS, MR, 8><<<grid, 256, 0, s>>>(part, pos, H, nchunk, chunk_keys, W, M, N, K, e);
}

template <class T, int HS>
static void launch_attn_proj_h(const float* part, const int32_t* pos, int H,
                               int nchunk, int chunk_keys, const T* W, int M,
                               int N, int K, const EpiArgs& e, hipStream_t s) {
  if (M <= 1) launch_attn_proj_t<T, HS, 1>(part, pos, H, nchunk, chunk_keys, W, M, N, K, e, s);
  else if (M <= 2) launch_attn_proj_t<T, HS, 2>(part, pos, H, nchunk, chunk_keys, W, M, N, K, e, s);
  else launch_attn_proj_t<T, HS, 4>(part, pos, H, nchunk, chunk_keys, W, M, N, K, e, s);
}

void launch_attn_proj(int dtype, const float* part, const int32_t* pos, int H,
                      int hs, int nchunk, int chunk_keys, const void* W, int M,
                      int C, const EpiArgs& e, hipStream_t s) {
  if (dtype == NGPT_BF16) {
    const bf16_t* w = static_cast<const bf16_t*>(W);
    if (hs == 64) launch_attn_proj_h<bf16_t, 64>(part, pos, H, nchunk, chunk_keys, w, M, C, C, e, s);
    else launch_attn_proj_h<bf16_t, 32>(part, pos, H, nchunk, chunk_keys, w, M, C, C, e, s);
  } else if (dtype == NGPT_F16) {
    const f16_t* w = static_cast<const f16_t*>(W);
    if (hs == 64) launch_attn_proj_h<f16_t, 64>(part, pos, H, nchunk, chunk_keys, w, M, C, C, e, s);
    else launch_attn_proj_h<f16_t, 32>(part, pos, H, nchunk, chunk_keys, w, M, C, C, e, s);
  } else {
    const float* w = static_cast<const float*>(W);
    if (hs == 64) launch_attn_proj_h<float, 64>(part, pos, H, nchunk, chunk_keys, w, M, C, C, e, s);
    else launch_attn_proj_h<float, 32>(part, pos, H, nchunk, chunk_keys, w, M, C, C, e, s);
  }
}

bool decode_fused_proj(int M) { return M <= kGemvMaxRows; }

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
template <class T, int EPI, int MR, int CPW, bool LN>
static void launch_gemv_c(const T* A, int lda, const LnArgs& ln, const T* W,
                          int M, int N, int K, const EpiArgs& e, hipStream_t s) {
  constexpr int SPAN = 64 * (16 / sizeof(T));
  const int nch = (K + SPAN - 1) / SPAN;
  const int grid = (N + CPW - 1) / CPW;
  // with a fused LayerNorm (K = n_embd <= kGemvLnMaxK) only the chunk counts
  // that K can need are built: the larger ones would not fit in registers
  constexpr int kMaxNch = LN ? kGemvLnMaxK / SPAN : 16;
  if (nch <= 2) {
    gemv_kernel<T, EPI, MR, CPW, 2, LN><<<grid, 64, 0, s>>>(A, lda, ln, W, M, N, K, e);
  } else if (nch <= 4) {
    gemv_kernel<T, EPI, MR, CPW, 4, LN><<<grid, 64, 0, s>>>(A, lda, ln, W, M, N, K, e);
  } else if constexpr (kMaxNch >= 8) {
    if (nch <= 8)
      gemv_kernel<T, EPI, MR, CPW, 8, LN><<<grid, 64, 0, s>>>(A, lda, ln, W, M, N, K, e);
    else if constexpr (kMaxNch >= 16)
      gemv_kernel<T, EPI, MR, CPW, 16, LN><<<grid, 64, 0, s>>>(A, lda, ln, W, M, N, K, e);
  }
}

template <class T, int EPI, int MR, bool LN>
static void launch_gemv(const T* A, int lda, const LnArgs& ln, const T* W,
                        int M, int N, int K, const EpiArgs& e, hipStream_t s) {
  // enough wavefronts to cover every CU several times over; more columns per
  // wavefront only where the weight rows are short
  constexpr int SPAN = 64 * (16 / sizeof(T));
  const int nch = (K + SPAN - 1) / SPAN;
  if (N >= 16384 && MR == 1 && nch <= 4)
    launch_gemv_c<T, EPI, MR, 4, LN>(A, lda, ln, W, M, N, K, e, s);
  else if (N >= 2048 && MR <= 2 && nch <= 4)
    launch_gemv_c<T, EPI, MR, 2, LN>(A, lda, ln, W, M, N, K, e, s);
  else
    launch_gemv_c<T, EPI, MR, 1, LN>(A, lda, ln, W, M, N, K, e, s);
}

template <class T, int EPI, bool LN>
static void gemv_rows(const T* A, int lda, const LnArgs& ln, const T* W, int M,
                      int N, int K, const EpiArgs& e, hipStream_t s) {
  if (M <= 1) launch_gemv<T, EPI, 1, LN>(A, lda, ln, W, M, N, K, e, s);
  else if (M <= 2) launch_gemv<T, EPI, 2, LN>(A, lda, ln, W, M, N, K, e, s);
  else launch_gemv<T, EPI, 4, LN>(A, lda, ln, W, M, N, K, e, s);
}


// 16-bit MFMA tile GEMM: tile shape and K-slab staging chosen per shape.
template <class T, int EPI>
static void dispatch_mfma(const T* a, int lda, const T* w, int M, int N, int K,
                          const EpiArgs& e, hipStream_t s) {
  // Tile size: a workgroup's time is set by the operand bytes it streams,
  // (BM + BN) * K, and the grid runs in rounds of one workgroup per CU;
  // pick the smaller rounds * (BM + BN), 128x64 on a tie.
  auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  auto cost = [&](int bm, int bn) {
    constexpr int kCUs = 256;
    return ((tiles(bm, bn) + kCUs - 1) / kCUs) * (bm + bn);
  };
  // K-slab counts of the GPT-2-small widths (768 and 4 * 768) are
  // compile-time constants, so the K loop is fully unrolled: at every trip
  // of a rolled loop the compiler waits for all loads in flight.
  const bool big = M > 64 && cost(128, 64) <= cost(64, 64);
  // 128x96 tiles for c_attn, c_fc and an all-position lm_head when they
  // cost less (at 1024 rows of GPT-2 small: 192 and 256 tiles, one round;
  // measured 2-2.5 us faster per launch than 128x64)
  constexpr bool kWideEpi = EPI == EPI_QKV || EPI == EPI_GELU || EPI == EPI_LOGITS;
  const bool wide = kWideEpi && M > 64 && cost(128, 96) < cost(big ? 128 : 64, 64);
  const int g = wide ? tiles(128, 96) : big ? tiles(128, 64) : tiles(64, 64);
  constexpr int kCUs = 256;
  // Grids of several rounds (batched prefills, the XL shape, the
  // all-position lm_head): eight-wavefront tiles with the direct-to-LDS K
  // loop (kloop_dma), two stages, two wavefronts per SIMD: 192x128 for the
  // 16-bit epilogues at 4096 rows or more, else 128x128.  Against the
  // four-wavefront 128x96 tiles at 16384 rows of the XL shape: c_attn
  // 452 -> 354 us, c_fc 600 -> 477 us, c_proj 201 -> 151 us, MLP c_proj
  // 674 -> 525 us; batch-64 prompts (17408 rows): c_fc 171 -> 133 us, MLP
  // c_proj 205 -> 121 us; bit-identical.  Whole passes: XL batch-32 prefill
  // 98.8 -> 87.3 ms, batch-64 prefill 8.98 -> 7.72 ms, the 1024-position
  // evaluation forward (its lm_head) 1215 -> 1168 us.
  if (M > 64 && tiles(128, 128) > kCUs) {
    if constexpr (kWideEpi) {
      if (M >= 4096) {
        gemm_mfma_kernel<T, 192, 128, EPI, 2, 0, true, 8><<<tiles(192, 128), 512, 0, s>>>(
            a, lda, w, M, N, K, e);
        return;
      }
    }
    if constexpr (kWideEpi || EPI == EPI_RESID) {
      gemm_mfma_kernel<T, 128, 128, EPI, 2, 0, true, 8><<<tiles(128, 128), 512, 0, s>>>(
          a, lda, w, M, N, K, e);
      return;
    }
  }
  // One round of 128x96 tiles (c_attn / c_fc at 1024 rows): the same loop
  // with four wavefronts and three stages (13.1 -> 9.8 and 13.6 -> 10.5 us
  // against the register-staged loop).
  if constexpr (kWideEpi) {
    if (wide) {
      if (K == 768) gemm_mfma_kernel<T, 128, 96, EPI, 3, 12, true><<<g, 256, 0, s>>>(a, lda, w, M, N, K, e);
      else gemm_mfma_kernel<T, 128, 96, EPI, 3, 0, true><<<g, 256, 0, s>>>(a, lda, w, M, N, K, e);
      return;
    }
  }
  // (only the pairs a block issues: c_attn, c_fc, c_proj at K = 768, the
  // MLP projection at K = 3072)
  constexpr bool k768 = EPI == EPI_QKV || EPI == EPI_GELU || EPI == EPI_RESID;
  constexpr bool k3072 = EPI == EPI_RESID;
  bool done = false;
  if constexpr (k768) {
    if (K == 768) {
      if (big) gemm_mfma_kernel<T, 128, 64, EPI, 4, 12><<<g, 256, 0, s>>>(a, lda, w, M, N, K, e);
      else gemm_mfma_kernel<T, 64, 64, EPI, 4, 12><<<g, 256, 0, s>>>(a, lda, w, M, N, K, e);
      done = true;
    }
  }
  if constexpr (k3072) {
    if (K == 3072) {
      if (big) gemm_mfma_kernel<T, 128, 64, EPI, 4, 48><<<g, 256, 0, s>>>(a, lda, w, M, N, K, e);
      else gemm_mfma_kernel<T, 64, 64, EPI, 4, 48><<<g, 256, 0, s>>>(a, lda, w, M, N, K, e);
      done = true;
    }
  }
  if (!done) {
    if (big) gemm_mfma_kernel<T, 128, 64, EPI, 4><<<g, 256, 0, s>>>(a, lda, w, M, N, K, e);
    else gemm_mfma_kernel<T, 64, 64, EPI, 8><<<g, 256, 0, s>>>(a, lda, w, M, N, K, e);
  }
}

template <class T, int EPI>
static void dispatch_gemv(const void* A, int lda, const LnArgs* ln, const void* W,
                          int M, int N, int K, const EpiArgs& e, hipStream_t s) {
  const LnArgs none{};
  const T* a = static_cast<const T*>(A);
  const T* w = static_cast<const T*>(W);
  if (ln) gemv_rows<T, EPI, true>(a, lda, *ln, w, M, N, K, e, s);
  else gemv_rows<T, EPI, false>(a, lda, none, w, M, N, K, e, s);
}

template <int EPI>
static void dispatch(int dtype, const void* A, int lda, const LnArgs* ln,
                     const void* W, int M, int N, int K, const EpiArgs& e,
                     hipStream_t s) {
  // streaming path: up to 16 chunks of 64 16-byte vectors per row (K <= 8192
  // 16-bit / 4096 fp32), with a fused LayerNorm only up to kGemvLnMaxK
  const bool half = dtype == NGPT_BF16 || dtype == NGPT_F16;
  const int gemv_max_k = 16 * 64 * (half ? 8 : 4);
  if (M <= kGemvMaxRows && K <= gemv_max_k && (!ln || K <= kGemvLnMaxK)) {
    if (dtype == NGPT_BF16) dispatch_gemv<bf16_t, EPI>(A, lda, ln, W, M, N, K, e, s);
    else if (dtype == NGPT_F16) dispatch_gemv<f16_t, EPI>(A, lda, ln, W, M, N, K, e, s);
    else dispatch_gemv<float, EPI>(A, lda, ln, W, M, N, K, e, s);
    return;
  }
  if (ln) {  // tiled paths read a materialised LayerNorm output
    launch_layernorm(dtype, ln->x, ln->ldx, nullptr, M, ln->w, ln->b, ln->h, K, K, s);
    A = ln->h;
    lda = K;
  }
  if (dtype == NGPT_BF16) {
    const bf16_t* a = static_cast<const bf16_t*>(A);
    const bf16_t* w = static_cast<const bf16_t*>(W);
    if (!launch_skinny(NGPT_BF16, EPI, a, lda, w, M, N, K, e, s))
      dispatch_mfma<bf16_t, EPI>(a, lda, w, M, N, K, e, s);
  } else if (dtype == NGPT_F16) {
    const f16_t* a = static_cast<const f16_t*>(A);
    const f16_t* w = static_cast<const f16_t*>(W);
    if (!launch_skinny(NGPT_F16, EPI, a, lda, w, M, N, K, e, s))
      dispatch_mfma<f16_t, EPI>(a, lda, w, M, N, K, e, s);
  } else {
    const dim3 grid((N + 15) / 16, (M + 15) / 16);
    gemm_f32_kernel<EPI><<<grid, 256, 0, s>>>(static_cast<const float*>(A), lda,
        static_cast<const float*>(W), M, N, K, e);
  }
}

void launch_linear(int dtype, int epi, const void* A, int lda,
                   const LnArgs* ln, const void* W, int M, int N, int K,
                   const EpiArgs& e, hipStream_t s) {
  if (M <= 0 || N <= 0) return;
  switch (epi) {
    case EPI_GELU: dispatch<EPI_GELU>(dtype, A, lda, ln, W, M, N, K, e, s); break;
    case EPI_RESID: dispatch<EPI_RESID>(dtype, A, lda, ln, W, M, N, K, e, s); break;
    case EPI_QKV: dispatch<EPI_QKV>(dtype, A, lda, ln, W, M, N, K, e, s); break;
    case EPI_LOGITS: dispatch<EPI_LOGITS>(dtype, A, lda, ln, W, M, N, K, e, s); break;
    default: break;   // (no other epilogue exists)
  }
}

}  // namespace ngpt
