// device_common.h — constants and small device helpers shared by the LOCKS
// kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace locks {

constexpr int kDim = 128;        // head dimension
constexpr int kPage = 16;        // tokens per page
constexpr int kRank = 8;         // summary rank
constexpr int kStride = 784;     // bytes per summary record
constexpr int kVOff = 0;         // V codes, k-major nibbles
constexpr int kMuOff = 512;      // centroid codes, int8[128]
constexpr int kCOff = 640;       // coefficient codes, int8[16][8]
constexpr int kSOff = 768;       // fp16 scales {s_mu, s_V, s_C, 0}
constexpr int kMaxGroup = 16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kInvSqrtD = 0.08838834764831845f;  // 1/sqrt(128)

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float f16bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xffffu));
}

// Number of full pages of sequence b, clamped to [0, max_pages].
__device__ __forceinline__ int full_pages(const int32_t* seq_lens, int b, int max_pages) {
  int n = seq_lens[b] / kPage;
  n = n < 0 ? 0 : n;
  return n > max_pages ? max_pages : n;
}

// Orders LDS traffic of one wave around a point where lanes exchange data
// through LDS (a wave's LDS operations complete in issue order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Raw hardware 2^x and log2(x) (v_exp_f32 / v_log_f32): results that would be
// fp32 denormals flush to zero, which only drops terms below 2^-126 of a sum.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Butterfly partners across 32-lane halves and across 16-lane rows (gfx950
// v_permlane32_swap / v_permlane16_swap): returns op(x, x of lane ^ 32 / ^ 16).
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Merge of two (max, sum-of-exp2) pairs in base-2 log units; m = -inf means empty.
__device__ __forceinline__ void lse2_merge(float& m, float& s, float m2, float s2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) { m = m2; s = s2; return; }
  if (m2 > m) { s = s * exp2f(m - m2) + s2; m = m2; }
  else s += s2 * exp2f(m2 - m);
}

}  // namespace locks
