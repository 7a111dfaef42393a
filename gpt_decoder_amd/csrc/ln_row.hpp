// LayerNorm of one fp32 row by one wavefront: (x - mean) / sqrt(var + 1e-5)
// * w (+ b) over the C features, population variance, fp32 two-pass
// statistics (serving page "原生 nanoGPT 模型服务首选", section 1).
#pragma once
#include "common.hpp"

namespace ngpt {

// The row is held in registers (float4 per lane per 256 columns, up to 8 of
// them), so x is read once and every load is issued before the first
// reduction.
constexpr int kLnMaxVec = 8;  // C <= 2048

// Four consecutive elements at a multiple of 4 (C is a multiple of 32 and
// the parameter and output rows are 16-byte aligned), so the LayerNorm
// parameters are read and its output written with one access per lane,
// through range-checked buffer loads: offset kLnOut (past every buffer) and
// a buffer of 0 bytes read zeros, so the load can be issued on every path.
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

// out[0..C) = LayerNorm(xr[0..C)) for one row, by the calling wavefront
// (lane l holds columns 256 j + 4 l .. + 3).  The row, the gain and the
// shift are all fetched before the first reduction, through range-checked
// buffer loads (issued on every path; guarded loads were each waited for in
// turn), so one memory latency is exposed.
template <class T>
__device__ __forceinline__ void ln_row(const float* __restrict__ xr, int C,
                                       const T* __restrict__ w, const T* __restrict__ bias,
                                       T* __restrict__ o) {
  const int lane = threadIdx.x & 63;
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


}  // namespace ngpt
