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

// Pages of sequence b that have a summary: its full pages, clamped to [0,
// max_pages], less the last one when `fill` (nullable) marks it as having
// filled in this step (fill[b] != 0 and seq_lens[b] a multiple of 16): that
// page's summary is being built concurrently, so it is attended like a tail
// instead of scored.
__device__ __forceinline__ int full_pages(const int32_t* seq_lens, const int32_t* fill, int b,
                                          int max_pages) {
  const int len = seq_lens[b];
  int n = len / kPage;
  n = n < 0 ? 0 : n;
  n = n > max_pages ? max_pages : n;
  if (fill && n > 0 && len == n * kPage && fill[b] != 0) --n;
  return n;
}

// Tokens of sequence b after its scored pages: they sit in logical page
// full_pages(), which has no summary yet (a page's summary is built when its
// 16th token lands): the partly filled last page, or all 16 tokens of a page
// that filled in this step; 0 when the scored pages already reach max_pages.
__device__ __forceinline__ int tail_tokens(const int32_t* seq_lens, const int32_t* fill, int b,
                                           int max_pages) {
  const int len = seq_lens[b];
  const int n = full_pages(seq_lens, fill, b, max_pages);
  return (len <= 0 || n >= max_pages) ? 0 : len - n * kPage;
}

// Orders LDS traffic of one wave around a point where lanes exchange data
// through LDS (a wave's LDS operations complete in issue order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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

// ---- wave-level data movement without LDS round trips (gfx950 DPP and
// permlane swaps; every helper expects all 64 lanes active).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within each 8-lane half row
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within each 16-lane row
constexpr int kDppShr1 = 0x111;       // row_shr:n, lanes n..15 of a row read lane i-n
constexpr int kDppShr2 = 0x112;
constexpr int kDppShr4 = 0x114;
constexpr int kDppShr8 = 0x118;

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kCtrl, 0xF, 0xF, false);
}
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float x) {
  return __uint_as_float(dpp_mov<kCtrl>(__float_as_uint(x)));
}
// row_shr with zero fill for lanes whose source lies outside the row
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_shr(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kCtrl, 0xF, 0xF, true);
}

// op over the 16 lanes of each row: a butterfly whose pairings are lane^1,
// lane^2, then the 8-lane halves and the 16-lane row mirrored onto each other.
// op must be commutative (every lane then gets bit-identical results).
template <typename T, typename Op>
__device__ __forceinline__ T row16_reduce(T x, Op op) {
  x = op(x, dpp_mov<kDppXor1>(x));
  x = op(x, dpp_mov<kDppXor2>(x));
  x = op(x, dpp_mov<kDppHalfMirror>(x));
  x = op(x, dpp_mov<kDppMirror>(x));
  return x;
}
// op over lanes l and l^16 / l^32 (both operands in the same order in both lanes)
template <typename Op>
__device__ __forceinline__ uint32_t xor16_op(uint32_t x, Op op) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return op((uint32_t)r[0], (uint32_t)r[1]);
}
template <typename Op>
__device__ __forceinline__ uint32_t xor32_op(uint32_t x, Op op) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op((uint32_t)r[0], (uint32_t)r[1]);
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  auto add = [](uint32_t a, uint32_t b) { return a + b; };
  x = row16_reduce(x, add);
  x = xor16_op(x, add);
  return xor32_op(x, add);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  auto mn = [](uint32_t a, uint32_t b) { return a < b ? a : b; };
  x = row16_reduce(x, mn);
  x = xor16_op(x, mn);
  return xor32_op(x, mn);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  x = row16_reduce(x, mx);
  x = xor16_op(x, mx);
  return xor32_op(x, mx);
}
__device__ __forceinline__ float wave_max(float x) {
  auto mx = [](float a, float b) { return fmaxf(a, b); };
  x = row16_reduce(x, mx);
  x = xor16_max(x);
  return xor32_max(x);
}
__device__ __forceinline__ float wave_sum(float x) {
  auto add = [](float a, float b) { return a + b; };
  x = row16_reduce(x, add);
  x = xor16_sum(x);
  return xor32_sum(x);
}

// Inclusive prefix sum over the 64 lanes (lane order).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_shr<kDppShr1>(x);
  x += dpp_shr<kDppShr2>(x);
  x += dpp_shr<kDppShr4>(x);
  x += dpp_shr<kDppShr8>(x);
  const uint32_t t0 = __builtin_amdgcn_readlane(x, 15), t1 = __builtin_amdgcn_readlane(x, 31),
                 t2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? t0 : 0u) + (row >= 2 ? t1 : 0u) + (row >= 3 ? t2 : 0u);
}

// Merge of two (max, sum-of-exp2) pairs in base-2 log units; m = -inf means empty.
__device__ __forceinline__ void lse2_merge(float& m, float& s, float m2, float s2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) { m = m2; s = s2; return; }
  if (m2 > m) { s = s * exp2f(m - m2) + s2; m = m2; }
  else s += s2 * exp2f(m2 - m);
}

}  // namespace locks
