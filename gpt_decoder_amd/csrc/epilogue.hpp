// Per-element epilogue of the linear layers (shared by the tile, streaming
// and skinny kernels): what happens to acc = (A W^T)[r][n].
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace ngpt {

template <class T, int EPI>
__device__ __forceinline__ void epi_apply(const EpiArgs& e, int r, int n,
                                          float acc) {
  if constexpr (EPI == EPI_LOGITS) {
    if (e.row_pos && e.row_pos[r] < 0) return;
    const int orow = e.row_b ? e.row_b[r] : r;   // the sequence's logits row
    static_cast<float*>(e.out)[(size_t)orow * e.ldo + n] = acc;
    return;
  } else {
    float v = acc;
    if (e.bias) v += to_f32(static_cast<const T*>(e.bias)[n]);
    if constexpr (EPI == EPI_GELU) {
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
      const int64_t base = kv_block_base(e.kv, b, p / kPageTokens);
      if (base < 0) {   // unmapped block of a paged cache
        if (e.status) atomicOr(e.status, 4);
        return;
      }
      const int h = c / e.hs;
      const int d = c - h * e.hs;
      T* cache = static_cast<T*>(which == 1 ? e.kc : e.vc);
      cache[(size_t)(base + (int64_t)h * kv_hstride(e.kv) + p % kPageTokens) * e.hs + d] =
          from_f32<T>(v);
    }
  }
}

}  // namespace ngpt
