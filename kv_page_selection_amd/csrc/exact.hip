// exact.hip — exact-mass page scores (gfx950): the reference selector.
//
// For every (sequence b, KV head, full page j) and each of the G query heads
// of the group: the exact log-sum-exp of q.k/sqrt(128) over the page's 16 real
// keys. Selecting by these masses is the exact mass selector that Theorem 1
// measures LOCKS's summary scores against (blog post, "How LOCKS works",
// Theorem 1; technical summary, section 3). It reads every key (4 KiB per
// page-head instead of a 784-byte summary), so it is a quality reference, not
// a decode path. Its outputs have the layout the summary scorer writes (page
// scores, per-range (max, sum) partials, tile maxima when the selection bounds
// by tiles), so the selection and attention passes run on it unchanged.
//
// Mapping: a workgroup is one 64-page range of one KV head; wave w takes its
// 16 pages one at a time, the next page's key tile in flight. Per page,
// S = K Q^T (16 tokens x 16 head columns, G used) is 32 chained
// v_mfma_f32_16x16x4_f32: lane (token l%16, group l/16) supplies key
// dimensions 32(l/16) + s at step s and the query lane (head l%16) the same
// dimensions, so the 4 k-slots of a step cover 4 disjoint d ranges and the 32
// steps all 128 dims, with fp32 products of the bf16 keys and fp32 queries.
#include "device_common.h"
#include "internal.h"

namespace locks {

namespace {

struct ExactArgs {
  const float* q;
  const uint16_t* kc;
  const int32_t* page_table;
  const int32_t* seq_lens;
  float* scores;
  float* partials;
  float* tile_max;
  int Hq, Hkv, N, num_blocks, n_ranges, tile_pages;  // tile maxima for n_b < tile_pages
};

template <int G>
__global__ __launch_bounds__(256) void exact_score_kernel(ExactArgs a) {
  static_assert(G >= 1 && G <= 16, "query heads per KV head");
  const int range = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, lj = lane >> 4;
  const int N = a.N;
  const int n_b = full_pages(a.seq_lens, nullptr, b, N);
  const int p0 = range * 64 + wave * 16;  // this wave's first page
  __shared__ float out[64][G];            // base-2 page scores, [page][head]; -inf: absent

  // physical block of page p0 + t in lane t (-1: absent)
  int myblk = -1;
  if (lane < 16 && p0 + lane < n_b) {
    const int blk = a.page_table[(size_t)b * N + p0 + lane];
    myblk = (blk >= 0 && blk < a.num_blocks) ? blk : -1;
  }

  // query operand: head li's dims 32 lj + s, in base-2 logit units (0 past G)
  float qv[32];
  {
    const float qscale = kLog2e * kInvSqrtD;
    const float* qrow = a.q + ((size_t)b * a.Hq + (size_t)kvh * G + (li < G ? li : 0)) * kDim + 32 * lj;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float4 x = *reinterpret_cast<const float4*>(qrow + 4 * c);
      qv[4 * c] = li < G ? x.x * qscale : 0.f;
      qv[4 * c + 1] = li < G ? x.y * qscale : 0.f;
      qv[4 * c + 2] = li < G ? x.z * qscale : 0.f;
      qv[4 * c + 3] = li < G ? x.w * qscale : 0.f;
    }
  }

  // key row li, dims [32 lj, 32 lj + 32) of page p0 + t
  auto load_tile = [&](int blk, uint4 (&kr)[4]) {
    if (blk >= 0) {
      const uint4* src = reinterpret_cast<const uint4*>(
          a.kc + ((size_t)blk * a.Hkv + kvh) * (kPage * kDim) + li * kDim + 32 * lj);
#pragma unroll
      for (int u = 0; u < 4; ++u) kr[u] = src[u];
    }
  };
  uint4 cur[4], nxt[4];
  int blk = __shfl(myblk, 0);
  load_tile(blk, cur);
  for (int t = 0; t < 16; ++t) {
    const int blk_n = (t + 1 < 16) ? __shfl(myblk, t + 1) : -1;
    load_tile(blk_n, nxt);
    float sh = -INFINITY;
    if (blk >= 0) {  // wave-uniform
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t w[4] = {cur[u].x, cur[u].y, cur[u].z, cur[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bf16lo(w[e]), qv[8 * u + 2 * e], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bf16hi(w[e]), qv[8 * u + 2 * e + 1], acc, 0, 0, 0);
        }
      }
      // lane holds tokens 4 lj + r of head li: log-sum-exp over the 16 tokens
      float mx = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
      mx = xor32_max(xor16_max(mx));
      float s = (fast_exp2(acc[0] - mx) + fast_exp2(acc[1] - mx)) +
                (fast_exp2(acc[2] - mx) + fast_exp2(acc[3] - mx));
      s = xor32_sum(xor16_sum(s));
      sh = mx + fast_log2(s);
    }
    if (lj == 0 && li < G) out[wave * 16 + t][li] = sh;
    blk = blk_n;
#pragma unroll
    for (int u = 0; u < 4; ++u) cur[u] = nxt[u];
  }
  __syncthreads();

  // ---- page scores (natural log), one row per head
  const int pbase = range * 64;
  for (int i = threadIdx.x; i < 64 * G; i += 256) {
    const int h = i / 64, pg = i % 64;
    if (pbase + pg < n_b)
      __builtin_nontemporal_store(out[pg][h] * kLn2, &a.scores[((size_t)b * a.Hq + (size_t)kvh * G + h) * N + pbase + pg]);
  }
  if (wave == 0) {
    // ---- per-head (max, sum of exp2) over the range: lane takes head
    // lane % G and pages i * 64/G + lane / G, then lanes of one head merge
    constexpr int LPH = 64 / G;
    float m = -INFINITY, v[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      v[i] = out[i * LPH + lane / G][lane % G];
      m = fmaxf(m, v[i]);
    }
    float ssum = 0.f;
    {
      const float ms = m == -INFINITY ? 0.f : m;
#pragma unroll
      for (int i = 0; i < G; ++i) ssum += fast_exp2(v[i] - ms);
    }
#pragma unroll
    for (int off = G; off < 64; off <<= 1) {
      const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(ssum, off);
      const float mn = fmaxf(m, m2);
      const float ms = mn == -INFINITY ? 0.f : mn;
      ssum = ssum * fast_exp2(m - ms) + s2 * fast_exp2(m2 - ms);
      m = mn;
    }
    if (lane < G) {
      float* dst = a.partials + (((size_t)b * a.Hq + (size_t)kvh * G + lane) * a.n_ranges + range) * 2;
      dst[0] = (ssum > 0.f) ? m : -INFINITY;
      dst[1] = ssum;
    }
    // ---- per head and 16-page tile: the max (for a sequence bounded by tiles)
    if (n_b < a.tile_pages && lane < 4 * G) {
      const int tt = lane / G, hh = lane % G;
      float tm = -INFINITY;
#pragma unroll
      for (int p = 0; p < 16; ++p) tm = fmaxf(tm, out[tt * 16 + p][hh]);
      a.tile_max[((size_t)b * a.Hq + (size_t)kvh * G + hh) * ((size_t)a.n_ranges * 4) +
                 (size_t)range * 4 + tt] = tm;
    }
  }
}

template <int G>
hipError_t launch_g(const locks_dims& d, const WsLayout& L, const DevPtrs& P, const float* q,
                    const uint16_t* kc, const int32_t* pt, const int32_t* sl, hipStream_t s) {
  ExactArgs a;
  a.q = q;
  a.kc = kc;
  a.page_table = pt;
  a.seq_lens = sl;
  a.scores = P.scores;
  a.partials = P.score_part;
  a.tile_max = P.tile_max;
  a.tile_pages = kTileBoundPages * L.k;
  a.Hq = d.n_q_heads;
  a.Hkv = d.n_kv_heads;
  a.N = d.max_pages_per_seq;
  a.num_blocks = d.num_blocks;
  a.n_ranges = L.n_score_wg;
  hipLaunchKernelGGL(exact_score_kernel<G>, dim3(L.n_score_wg, d.n_kv_heads, d.batch), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_exact_score(const locks_dims& d, const WsLayout& L, const DevPtrs& P,
                              const float* q, const uint16_t* kc, const int32_t* pt,
                              const int32_t* sl, hipStream_t s) {
  switch (d.n_q_heads / d.n_kv_heads) {
    case 1: return launch_g<1>(d, L, P, q, kc, pt, sl, s);
    case 2: return launch_g<2>(d, L, P, q, kc, pt, sl, s);
    case 4: return launch_g<4>(d, L, P, q, kc, pt, sl, s);
    case 8: return launch_g<8>(d, L, P, q, kc, pt, sl, s);
    case 16: return launch_g<16>(d, L, P, q, kc, pt, sl, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace locks
