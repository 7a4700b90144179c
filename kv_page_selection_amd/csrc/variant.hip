// variant.hip — page scores from the variant summary formats (gfx950): the
// precision / rank ablation (blog post, "Caveats": Theorem 1 covers
// unquantised summaries; int4 loses a few recall points; int2 collapses).
//
// The same page score as the shipped path (blog post, "How LOCKS works",
// page-score equation), s_hat = log sum_i exp((q.mu + (V^T q).c_i) / sqrt(128)),
// at rank R with V held in VB bits (2, 4: signed codes; 16: fp16) and mu, C
// as int8 codes (fp16 values when VB = 16); the record layout is the one
// build.hip's variant kernel writes (V [d][k] bit-packed, mu, C [16][R], fp16
// scales). Outputs have the layout of the shipped scorer (page scores,
// per-range (max, sum) partials, tile maxima for sequences bounded by tiles),
// so the selection and attention passes run on them unchanged.
//
// This is a measurement path, not a tuned one: one wave per 64-page range of
// one KV head, lane = page; each lane decodes its own record (L1-cached
// 16-byte loads) once per group of up to 4 query heads, accumulating q.mu and
// V^T q in fp32, then the 16 token logits and their log-sum-exp in base 2.
#include "device_common.h"
#include "internal.h"

namespace locks {

namespace {

struct VarArgs {
  const float* q;
  const uint8_t* summ;
  const int32_t* page_table;
  const int32_t* seq_lens;
  float* scores;
  float* partials;
  float* tile_max;
  int Hq, Hkv, N, num_blocks, n_ranges, tile_pages;
};

template <int R, int VB>
struct Fmt {
  static constexpr int MB = VB == 16 ? 16 : 8;
  static constexpr int kV = kDim * R * VB / 8;
  static constexpr int kMu = kV;
  static constexpr int kC = kMu + kDim * MB / 8;
  static constexpr int kS = kC + kPage * R * MB / 8;
  static constexpr int kBytes = (kS + 8 + 15) / 16 * 16;
  static constexpr int kDB = 512 / (R * VB);  // V rows per 512-bit step
};

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// field j of width BITS (< 32 or 16 = fp16) from a little-endian word array
template <int BITS>
__device__ __forceinline__ float field(const uint32_t* w, int j, float scale) {
  const uint32_t x = (w[(j * BITS) / 32] >> ((j * BITS) % 32)) & ((1u << BITS) - 1u);
  if constexpr (BITS == 16) return half_bits_to_float(x);
  const int c = (int)(x << (32 - BITS)) >> (32 - BITS);  // sign-extend
  return scale * (float)c;
}

template <int NW>
__device__ __forceinline__ void load_words(const uint8_t* p, uint32_t (&w)[NW]) {
  if constexpr (NW % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const uint4 x = reinterpret_cast<const uint4*>(p)[i];
      w[4 * i] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z; w[4 * i + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = reinterpret_cast<const uint32_t*>(p)[i];
  }
}

template <int R, int VB, int G>
__global__ __launch_bounds__(64) void score_variant_kernel(VarArgs a) {
  using F = Fmt<R, VB>;
  constexpr int MB = F::MB, DB = F::kDB;
  constexpr int HG = G < 4 ? G : 4;            // heads per decode pass
  constexpr int kMuW = (DB * MB / 8 + 3) / 4;  // mu words per step
  const int range = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int N = a.N;
  const int n_b = full_pages(a.seq_lens, nullptr, b, N);
  if (range * 64 >= n_b) return;  // nothing of the sequence here (partials not read)
  __shared__ float qs[G][kDim];
  {
    const float qscale = kLog2e * kInvSqrtD;  // base-2 logits
    const float* qg = a.q + ((size_t)b * a.Hq + (size_t)kvh * G) * kDim;
    for (int i = lane; i < G * kDim; i += 64) qs[i / kDim][i % kDim] = qg[i] * qscale;
  }
  wave_lds_sync();

  const int p = range * 64 + lane;
  int blk = (p < n_b) ? a.page_table[(size_t)b * N + p] : -1;
  const bool present = blk >= 0 && blk < a.num_blocks;
  const uint8_t* rec = a.summ + ((size_t)(present ? blk : 0) * a.Hkv + kvh) * F::kBytes;
  const uint32_t sw0 = reinterpret_cast<const uint32_t*>(rec + F::kS)[0];
  const uint32_t sw1 = reinterpret_cast<const uint32_t*>(rec + F::kS)[1];
  const float s_mu = half_bits_to_float(sw0 & 0xffffu), s_v = half_bits_to_float(sw0 >> 16),
              s_c = half_bits_to_float(sw1 & 0xffffu);

  float out[G];
#pragma unroll
  for (int hg = 0; hg < G / HG; ++hg) {
    float am[HG], pv[HG][R];
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      am[h] = 0.f;
#pragma unroll
      for (int k = 0; k < R; ++k) pv[h][k] = 0.f;
    }
#pragma unroll 1
    for (int d0 = 0; d0 < kDim; d0 += DB) {
      uint32_t vw[16], mw[kMuW];
      load_words<16>(rec + (size_t)d0 * R * VB / 8, vw);
      load_words<kMuW>(rec + F::kMu + d0 * MB / 8, mw);
#pragma unroll
      for (int dl = 0; dl < DB; ++dl) {
        const float mu = field<MB>(mw, dl, s_mu);
        float vk[R];
#pragma unroll
        for (int k = 0; k < R; ++k) vk[k] = field<VB>(vw, dl * R + k, s_v);
#pragma unroll
        for (int h = 0; h < HG; ++h) {
          const float qd = qs[hg * HG + h][d0 + dl];
          am[h] = fmaf(mu, qd, am[h]);
#pragma unroll
          for (int k = 0; k < R; ++k) pv[h][k] = fmaf(vk[k], qd, pv[h][k]);
        }
      }
    }
    // the 16 token logits and their log-sum-exp (online, base 2)
    float m[HG], s[HG];
#pragma unroll
    for (int h = 0; h < HG; ++h) { m[h] = -INFINITY; s[h] = 0.f; }
#pragma unroll 4
    for (int i = 0; i < kPage; ++i) {
      uint32_t cw[R * MB / 32];
      load_words<R * MB / 32>(rec + F::kC + i * R * MB / 8, cw);
      float ck[R];
#pragma unroll
      for (int k = 0; k < R; ++k) ck[k] = field<MB>(cw, k, s_c);
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        float t = am[h];
#pragma unroll
        for (int k = 0; k < R; ++k) t = fmaf(ck[k], pv[h][k], t);
        const float mn = fmaxf(m[h], t);
        s[h] = s[h] * fast_exp2(m[h] - mn) + fast_exp2(t - mn);
        m[h] = mn;
      }
    }
#pragma unroll
    for (int h = 0; h < HG; ++h) out[hg * HG + h] = present ? m[h] + fast_log2(s[h]) : -INFINITY;
  }

  // ---- scores (natural log), partials, tile maxima
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (p < n_b)
      a.scores[((size_t)b * a.Hq + (size_t)kvh * G + h) * N + p] = out[h] * kLn2;
    float mx = wave_max(out[h]);
    const float ms = mx == -INFINITY ? 0.f : mx;
    const float sm = wave_sum(fast_exp2(out[h] - ms));
    if (lane == 0) {
      float* dst = a.partials + (((size_t)b * a.Hq + (size_t)kvh * G + h) * a.n_ranges + range) * 2;
      dst[0] = sm > 0.f ? mx : -INFINITY;
      dst[1] = sm;
    }
    if (n_b < a.tile_pages) {
      const float tm = row16_reduce(out[h], [](float x, float y) { return fmaxf(x, y); });
      if ((lane & 15) == 0)
        a.tile_max[((size_t)b * a.Hq + (size_t)kvh * G + h) * ((size_t)a.n_ranges * 4) +
                   (size_t)range * 4 + (lane >> 4)] = tm;
    }
  }
}

template <int R, int VB, int G>
hipError_t launch_rvg(const locks_dims& d, const WsLayout& L, const DevPtrs& P, const float* q,
                      const uint8_t* summ, const int32_t* pt, const int32_t* sl, hipStream_t s) {
  VarArgs a;
  a.q = q;
  a.summ = summ;
  a.page_table = pt;
  a.seq_lens = sl;
  a.scores = P.scores;
  a.partials = P.score_part;
  a.tile_max = P.tile_max;
  a.Hq = d.n_q_heads;
  a.Hkv = d.n_kv_heads;
  a.N = d.max_pages_per_seq;
  a.num_blocks = d.num_blocks;
  a.n_ranges = L.n_score_wg;
  a.tile_pages = kTileBoundPages * L.k;
  hipLaunchKernelGGL((score_variant_kernel<R, VB, G>), dim3(L.n_score_wg, d.n_kv_heads, d.batch),
                     dim3(64), 0, s, a);
  return hipGetLastError();
}

template <int R, int VB>
hipError_t launch_rv(const locks_dims& d, const WsLayout& L, const DevPtrs& P, const float* q,
                     const uint8_t* summ, const int32_t* pt, const int32_t* sl, hipStream_t s) {
  switch (d.n_q_heads / d.n_kv_heads) {
    case 1: return launch_rvg<R, VB, 1>(d, L, P, q, summ, pt, sl, s);
    case 2: return launch_rvg<R, VB, 2>(d, L, P, q, summ, pt, sl, s);
    case 4: return launch_rvg<R, VB, 4>(d, L, P, q, summ, pt, sl, s);
    case 8: return launch_rvg<R, VB, 8>(d, L, P, q, summ, pt, sl, s);
    case 16: return launch_rvg<R, VB, 16>(d, L, P, q, summ, pt, sl, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_score_variant(const locks_dims& d, const WsLayout& L, const DevPtrs& P,
                                const float* q, const uint8_t* summ, const int32_t* pt,
                                const int32_t* sl, int rank, int v_bits, hipStream_t s) {
#define LOCKS_VARIANT_SCORE(R, VB) \
  if (rank == R && v_bits == VB) return launch_rv<R, VB>(d, L, P, q, summ, pt, sl, s);
  LOCKS_VARIANT_SCORE(4, 2) LOCKS_VARIANT_SCORE(4, 4) LOCKS_VARIANT_SCORE(4, 16)
  LOCKS_VARIANT_SCORE(8, 2) LOCKS_VARIANT_SCORE(8, 4) LOCKS_VARIANT_SCORE(8, 16)
  LOCKS_VARIANT_SCORE(16, 2) LOCKS_VARIANT_SCORE(16, 4) LOCKS_VARIANT_SCORE(16, 16)
#undef LOCKS_VARIANT_SCORE
  return hipErrorInvalidValue;
}

}  // namespace locks
