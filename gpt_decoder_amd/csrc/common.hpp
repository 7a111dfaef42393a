// Device-side helpers shared by the gfx950 kernels of libngpt.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ngpt {

typedef uint16_t bf16_t;  // bfloat16 storage: the top 16 bits of an fp32
typedef _Float16 f16_t;   // IEEE binary16 storage (the fp16 model)
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// fp32 -> bf16, round to nearest, ties to even: gfx950's v_cvt_pk_bf16_f32
// (checked bit-identical to integer round-to-nearest-even on every finite
// fp32 input, denormals included).
typedef __bf16 bf16x2_hw_t __attribute__((ext_vector_type(2)));
typedef float f32x2_hw_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

template <class T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  return f32_to_bf16(x);
}
// fp32 -> fp16, round to nearest even (v_cvt_f16_f32 in the default mode)
__device__ __forceinline__ float to_f32(f16_t x) { return static_cast<float>(x); }
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float x) {
  return static_cast<f16_t>(x);
}

// Unpack 8 bf16 held in a uint4 (little-endian pairs) to fp32.
__device__ __forceinline__ void bf16x8_to_f32(const uint4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// two values to bf16 (a in the low half), one instruction
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_hw_t{a, b}, bf16x2_hw_t));
}

// Unpack 8 fp16 held in a uint4 (little-endian pairs) to fp32.
__device__ __forceinline__ void f16x8_to_f32(const uint4 v, float* f) {
  const f16x8_t h = __builtin_bit_cast(f16x8_t, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = static_cast<float>(h[i]);
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<f16_t>(a));
  const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<f16_t>(b));
  return lo | (hi << 16);
}

// The same operations chosen by storage type T (bf16_t or f16_t): 8 values
// of a 16-byte vector to fp32, two values packed into 32 bits, the MFMA
// operand vector type and its 16x16x32 MFMA.
template <class T> struct Half16;
template <> struct Half16<bf16_t> {
  typedef bf16x8_t vec8;
  static __device__ __forceinline__ void unpack8(const uint4 v, float* f) { bf16x8_to_f32(v, f); }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_bf16x2(a, b); }
  static __device__ __forceinline__ f32x4_t mfma(vec8 a, vec8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Half16<f16_t> {
  typedef f16x8_t vec8;
  static __device__ __forceinline__ void unpack8(const uint4 v, float* f) { f16x8_to_f32(v, f); }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_f16x2(a, b); }
  static __device__ __forceinline__ f32x4_t mfma(vec8 a, vec8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// 2^x with the hardware v_exp_f32: the same value as exp2f wherever that is
// a normal float, 2^-inf = 0; results below 2^-126 (softmax weights too
// small to change any sum) come out as 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// GELU, exact erf form: z/2 (1 + erf(z / sqrt 2)) = z/2 erfc(-z / sqrt 2).
// erfc(u) for u >= 0 is the rational-exponential formula of Abramowitz &
// Stegun 7.1.26 (after Hastings): t = 1 / (1 + p u),
// erfc(u) ~ t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-u^2), absolute
// error at most 1.5e-7; for u < 0, erfc(u) = 2 - erfc(-u).  Branch-free, a
// dozen instructions: the library erff spent about 30 instructions and two
// data-dependent branches per element, which made the GELU epilogue of the
// MLP up-projection cost as much as its matrix product.  Against the exact
// function in fp64 the result is within 4.3e-7 absolute (the library form:
// 4.5e-7).
__device__ __forceinline__ float gelu_erf(float z) {
  const float u = -z * 0.70710678118654752440f;
  const float au = fabsf(u);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, au, 1.0f));
  float p = fmaf(1.061405429f, t, -1.453152027f);
  p = fmaf(p, t, 1.421413741f);
  p = fmaf(p, t, -0.284496736f);
  p = fmaf(p, t, 0.254829592f);
  const float q = p * t * __builtin_amdgcn_exp2f(-(au * au) * 1.44269504088896340736f);
  return 0.5f * z * (u >= 0.f ? q : 2.0f - q);
}

// Merge two partial softmax states (running max m in the log2 domain, sum l,
// weighted value sums o[n]) into the first.
__device__ __forceinline__ void merge_state(float& m, float& l, float* o,
                                            float m2, float l2,
                                            const float* o2, int n) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  const float a = (m == -INFINITY) ? 0.f : exp2_fast(m - mn);
  const float c = (m2 == -INFINITY) ? 0.f : exp2_fast(m2 - mn);
  l = l * a + l2 * c;
  for (int j = 0; j < n; ++j) o[j] = o[j] * a + o2[j] * c;
  m = mn;
}

// Cross-lane moves (gfx950).
// DPP within a row of 16 lanes, the gfx950 permlane swaps across rows.  Each
// returns the value of the partner lane named in the comment.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float lane_xor1(float v) { return dpp_mov<0xB1>(v); }  // quad_perm 1,0,3,2
__device__ __forceinline__ float lane_xor2(float v) { return dpp_mov<0x4E>(v); }  // quad_perm 2,3,0,1
__device__ __forceinline__ float lane_mirror8(float v) { return dpp_mov<0x141>(v); }  // 7 - i in 8
__device__ __forceinline__ float lane_xor8(float v) { return dpp_mov<0x128>(v); }  // row_ror:8
__device__ __forceinline__ float lane_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(((threadIdx.x >> 4) & 1) ? r[0] : r[1]);
}
__device__ __forceinline__ float lane_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
// [a_lo + a_hi | b_lo + b_hi]: lanes 0..31 sum a over the two halves, lanes
// 32..63 sum b.
__device__ __forceinline__ float halves_sum2(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Row r of the result sums rows (r & ~1), (r | 1) of a (r even) or of b
// (r odd): [a0+a1, b0+b1, a2+a3, b2+b3].
__device__ __forceinline__ float rows_sum2(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// sum over each row of 16 lanes, in every lane of the row (bit-identical:
// each step adds a symmetric partner)
__device__ __forceinline__ float row_sum16(float v) {
  v += lane_xor1(v);
  v += lane_xor2(v);
  v += lane_mirror8(v);
  v += lane_xor8(v);
  return v;
}
__device__ __forceinline__ float wave_sum_all(float v) {
  v = row_sum16(v);
  v += lane_xor16(v);
  v += lane_xor32(v);
  return v;
}

}  // namespace ngpt
