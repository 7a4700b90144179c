// select.hip — group-shared page selection (gfx950).
//
// Group combine (technical summary, section 2 mechanism 3): each head g of a
// GQA group has total mass L_g = log sum_j exp(s_hat[g][j]) over the
// sequence's pages; a page's key is the log of the group-mean normalised mass
// share, key_j = log((1/G) sum_g exp(s_hat[g][j] - L_g)).
// Top-k (blog post, "Code": keep budget/16 pages with the largest score, ids
// ascending): the k largest keys, ties to the lower page id.
//
// Two launches, no float atomics:
//  1. chunk pass, grid (chunk, KV head, sequence), 1024 threads:
//     a. bound: every workgroup folds the scoring pass's per-range (max, sum)
//        partials (a few tens of KB, L2-resident) into L_g, and from the
//        maxima of s_hat over bound units (the 64-page ranges, or 16-page
//        tiles when a sequence has fewer than 2k ranges) a lower bound T on
//        the k-th largest key: every unit holds a page whose key is at least
//        max_g(unit max of s_hat_g - L_g) - log2 G, so the k-th largest of
//        these per-unit bounds (over distinct units) cannot exceed the k-th
//        largest key. One 2048-bucket histogram that keeps each bucket's
//        smallest member gives that k-th largest bound; it spans 128 (base-2
//        log) below the largest bound, which the fold already knows (the max
//        over heads of max s_hat_g - L_g), so no reduction finds its range.
//        Units are pooled into super-ranges when the (head, unit) maxima
//        exceed what LDS holds (the maximum over a super-range still bounds
//        one of its pages).
//        Computing this in every workgroup costs less than a launch of its
//        own.
//     b. the keys of the workgroup's <= 4096 pages as 64-bit sort keys
//        (order-preserving key bits << 32 | ~page id, so one integer
//        comparison applies "larger key, then lower id"); those with key >= T
//        are written, with their physical blocks, in page order (typically a
//        few hundred per (sequence, KV head) in all).
//  2. merge: one workgroup per (sequence, KV head) ranks the chunk lists in
//     page order and writes the kept ids, sorted without a sort because the
//     lists are in page order, with their physical blocks for the attention
//     pass. Up to 1024 candidates (the usual case) the waves rank them in
//     registers, two candidates per lane; up to 4,608 the workgroup ranks an LDS copy;
//     beyond that a radix select runs over the lists where they lie. (For
//     small budgets the decode step skips this launch: each sparse attention
//     workgroup ranks its own (sequence, KV head)'s lists the same way.)
// Ranking = exact selection by bucket refinement on the key bits: a histogram
// over the live [lo, hi] key range (2048 buckets; 512 on the register
// path) picks the bucket holding the k-th key; everything above it
// is in, below it out; repeat inside that bucket (range shrinks ~2^11, or
// ~2^9, per pass) until the count fits or all live keys are equal, where the
// lowest ids win.
#include "device_common.h"
#include "internal.h"
#include "rank_device.h"

namespace locks {

namespace {

constexpr int kThreads = 1024;
constexpr int kNW = kThreads / 64;
constexpr int kHistBuckets = 2 * kThreads;                // 2 buckets per thread
constexpr int kChunkEpt = kSelectChunk / kThreads;        // <= 4 pages per thread
// log2 range of the bound histogram below the largest unit bound; bounds
// further down share its lowest bucket (a looser but still valid threshold)
constexpr float kBoundSpan = 128.0f;

struct SelectArgs {
  const float* scores;
  const float* score_part;
  const float* tile_max;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* fill;  // nullable: pages that filled in this step (attended as the tail)
  unsigned long long* cand;
  int32_t* cand_blk;
  int32_t* cand_count;
  int32_t* selected;
  int32_t* sel_blk;
  int Hq, Hkv, N, k, n_ranges, n_tiles, sup_r, sup_t, chunk, n_chunks;
};

struct BoundLds {
  uint32_t msup[kBoundSlots];  // order bits of each (head, super-range) max; 0 = none
  uint32_t hmin[kHistBuckets];
};
struct ChunkShared {
  BoundLds bound;
  uint32_t hcnt[kHistBuckets];
  uint32_t scn[2][kNW];
  float redf[kNW][2];
  float reds[kNW];  // each wave's sum rescaled to its head's max
  uint32_t wsum[kNW];
  int scan[kNW];
  float tlb;
};

__device__ __forceinline__ uint32_t key_order_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // monotone in f
}

__device__ __forceinline__ float key_from_order_bits(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// Branch-free merge of base-2 (max, sum) pairs; an empty pair is (-1e30, 0).
__device__ __forceinline__ void lse2_acc(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  s = s * fast_exp2(m - mn) + s2 * fast_exp2(m2 - mn);
  m = mn;
}

// (max, sum) pairs merged over the 64 lanes; every lane gets the same result.
// Max first, then one rescale per lane and a plain sum: one exp2 per lane
// instead of two per butterfly step (an empty pair is (-1e30, 0)).
__device__ __forceinline__ void wave_lse2(float& m, float& s) {
  const float M = wave_max(m);
  s = wave_sum(s * fast_exp2(m - M));
  m = M;
}

// Bucket of order bits u among kHistBuckets linear buckets over [lo, hi]
// (monotone in u; lo -> 0, hi -> the top buckets).
__device__ __forceinline__ int hbucket(uint32_t u, uint32_t lo, float scale) {
  return min(kHistBuckets - 1, (int)((float)(u - lo) * scale));
}

// Suffix scan of a 2048-bucket histogram held as 2 buckets per thread
// (thread t: buckets 2t, 2t+1). Returns, for this thread, the count in
// buckets above 2t+1; one barrier.
__device__ __forceinline__ uint32_t hist_above(uint32_t mine, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t pre = wave_incl_scan(mine);  // lanes 0..this one
  const uint32_t wtot = __builtin_amdgcn_readlane(pre, 63);
  if (lane == 0) wsum[wave] = wtot;
  __syncthreads();
  uint32_t above = wtot - pre;  // lanes above this one in the wave
#pragma unroll
  for (int w = 0; w < kNW; ++w)
    if (w > wave) above += wsum[w];
  return above;
}

// Exclusive prefix sums over the 1024 threads (thread order) of two u32
// values at once; on return a, b hold this thread's exclusive prefixes and
// *ta, *tb the block totals. One barrier.
__device__ void big_exclusive_scan2(uint32_t& a, uint32_t& b, uint32_t* ta, uint32_t* tb,
                                    ChunkShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t ia = wave_incl_scan(a), ib = wave_incl_scan(b);
  if (lane == 63) { sh.scn[0][wave] = ia; sh.scn[1][wave] = ib; }
  __syncthreads();
  uint32_t pa = 0, pb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int w = 0; w < kNW; ++w) {
    const uint32_t ca = sh.scn[0][w], cb = sh.scn[1][w];
    if (w < wave) { pa += ca; pb += cb; }
    sa += ca;
    sb += cb;
  }
  a = pa + ia - a;
  b = pb + ib - b;
  *ta = sa;
  *tb = sb;
}

// EPT = pages per thread (1, 2 or 4 slabs of 1024), fixed by the chunk size
template <int G, int EPT>
__global__ __launch_bounds__(kThreads) void select_chunk_kernel(SelectArgs a) {
  static_assert(EPT >= 1 && EPT <= kChunkEpt, "pages per thread");
  constexpr int P = kThreads / G;  // threads per head in the bound pass
  constexpr int WPG = P / 64;      // waves per head
  constexpr int kLbPt = kBoundSlots / G / kThreads;  // super-ranges per thread at most
  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = a.N, nt = a.n_tiles;
  const int n_b = full_pages(a.seq_lens, a.fill, b, N);
  // bound units of this sequence: 16-page tiles when it has fewer than 2k
  // ranges (a bound over so few units prunes little; the scoring pass wrote
  // tile maxima exactly for such sequences), else 64-page ranges; only the
  // ranges and tiles that hold its pages are read
  const bool tiles = n_b < kTileBoundPages * a.k;
  const int nr = (n_b + kScorePagesPerWave - 1) / kScorePagesPerWave;
  const int nu = tiles ? (n_b + 15) / 16 : nr;
  const int S = tiles ? a.sup_t : a.sup_r;
  const int nR = (nu + S - 1) / S;  // super-ranges (G * nR fits the LDS slots)
  const size_t head = (size_t)b * a.Hkv + kvh;
  __shared__ ChunkShared sh;
  if (chunk * a.chunk >= n_b) {  // workgroup-uniform: no page of the sequence here
    if (tid == 0) a.cand_count[head * a.n_chunks + chunk] = 0;
    return;
  }

  // ---- this chunk's scores and page-table entries, in flight during the bound pass
  const int p0 = chunk * a.chunk + tid;  // page of slab i: p0 + 1024 i (coalesced loads)
  float sc[G][EPT];
  int blk[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const bool in = p0 + i * kThreads < n_b;
    const int p = in ? p0 + i * kThreads : 0;
    blk[i] = a.page_table[(size_t)b * N + p];
#pragma unroll
    for (int g = 0; g < G; ++g) sc[g][i] = a.scores[((size_t)b * a.Hq + (size_t)kvh * G + g) * N + p];
  }

  // ================================================================ 1. bound
  const int g = tid / P, j = tid % P;
  sh.hcnt[2 * tid] = 0u;
  sh.hcnt[2 * tid + 1] = 0u;
  sh.bound.hmin[2 * tid] = 0xffffffffu;
  sh.bound.hmin[2 * tid + 1] = 0xffffffffu;
  if (S > 1) {  // super-ranges are filled by atomics
    for (int i = tid; i < G * nR; i += kThreads) sh.bound.msup[i] = 0u;
    __syncthreads();
  }
  const float2* part =
      reinterpret_cast<const float2*>(a.score_part) + ((size_t)b * a.Hq + (size_t)kvh * G + g) * a.n_ranges;
  float lm = -1e30f, ls = 0.f;
  // partials per thread in flight at once: 16 for 16-head groups at one page
  // per thread (P = 64 threads per head: one round trip for 1024 ranges),
  // else 8 (P >= 128: one batch covers 1024 ranges already)
  constexpr int PB = (G == 16 && EPT == 1) ? 16 : 8;
  for (int r0 = 0; r0 < nr; r0 += PB * P) {
    float2 v[PB];
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int r = r0 + j + i * P;
      v[i] = (r < nr) ? part[r] : make_float2(-INFINITY, 0.f);
    }
    if (r0 + PB * P <= nr) {  // workgroup-uniform: a full batch, max first, one exp2 per partial
      float bm = -1e30f, bs = 0.f;
#pragma unroll
      for (int i = 0; i < PB; ++i) bm = fmaxf(bm, v[i].y > 0.f ? v[i].x : -1e30f);
#pragma unroll
      for (int i = 0; i < PB; ++i) bs += v[i].y * fast_exp2(v[i].x - bm);  // empty: (-inf, 0) adds 0
      lse2_acc(lm, ls, bm, bs);
    } else {
#pragma unroll
      for (int i = 0; i < PB; ++i)
        if (v[i].y > 0.f) lse2_acc(lm, ls, v[i].x, v[i].y);
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int r = r0 + j + i * P;
      const bool ne = v[i].y > 0.f;  // range holds a present page
      if (tiles) continue;
      if (S == 1) {
        if (r < nr) sh.bound.msup[g * nR + r] = ne ? key_order_bits(v[i].x) : 0u;
      } else if (ne) {
        atomicMax(&sh.bound.msup[g * nR + r / S], key_order_bits(v[i].x));
      }
    }
  }
  // tile units: the 16-page tiles' maxima (-inf: no present page)
  if (tiles) {
    const float* tmx = a.tile_max + ((size_t)b * a.Hq + (size_t)kvh * G + g) * nt;
    for (int u0 = 0; u0 < nu; u0 += 8 * P) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int u = u0 + j + i * P;
        v[i] = (u < nu) ? tmx[u] : -INFINITY;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int u = u0 + j + i * P;
        const bool ne = v[i] > -INFINITY;
        if (S == 1) {
          if (u < nu) sh.bound.msup[g * nR + u] = ne ? key_order_bits(v[i]) : 0u;
        } else if (ne) {
          atomicMax(&sh.bound.msup[g * nR + u / S], key_order_bits(v[i]));
        }
      }
    }
  }
  wave_lse2(lm, ls);
  if (lane == 0) {
    if constexpr (WPG > 1) {
      sh.redf[wave][0] = lm;
      sh.redf[wave][1] = ls;
    } else {  // one wave per head: its L and max - L, so readers need no log2
      const float Lw = (ls > 0.f) ? lm + fast_log2(ls) : -INFINITY;
      sh.redf[wave][0] = Lw;
      sh.redf[wave][1] = (ls > 0.f) ? lm - Lw : -INFINITY;
    }
  }
  if (tid == 0) sh.tlb = -INFINITY;  // kept when fewer than k units have pages: no pruning
  __syncthreads();
  // L_g: with several waves per head, each wave first rescales its sum to the
  // head's max (one exp2, a second barrier), so every thread then only adds
  float L[G];  // base 2
  float top = -INFINITY;  // the largest unit bound plus log2 G: max over heads of (max s_hat_g - L_g)
  if constexpr (WPG > 1) {
    float Mg = sh.redf[g * WPG][0];
#pragma unroll
    for (int w = 1; w < WPG; ++w) Mg = fmaxf(Mg, sh.redf[g * WPG + w][0]);
    if (lane == 0) sh.reds[wave] = ls * fast_exp2(lm - Mg);
    __syncthreads();
  }
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    if constexpr (WPG > 1) {
      float m = sh.redf[gg * WPG][0], sv = 0.f;
#pragma unroll
      for (int w = 1; w < WPG; ++w) m = fmaxf(m, sh.redf[gg * WPG + w][0]);
#pragma unroll
      for (int w = 0; w < WPG; ++w) sv += sh.reds[gg * WPG + w];
      L[gg] = (sv > 0.f) ? m + fast_log2(sv) : -INFINITY;
      if (sv > 0.f) top = fmaxf(top, m - L[gg]);
    } else {
      L[gg] = sh.redf[gg][0];
      top = fmaxf(top, sh.redf[gg][1]);
    }
    // the same in every lane: held in a scalar register
    L[gg] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(L[gg])));
  }
  top = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(top)));
  const float log2G = (float)__builtin_ctz(G);
  // bucket range of the bounds: [top - kBoundSpan, top] in order bits, known
  // without a reduction (lower bounds share the lowest bucket)
  const float topb = top - log2G;
  const uint32_t hi = key_order_bits(topb), lo = key_order_bits(topb - kBoundSpan);
  const float scale = (float)kHistBuckets / ((float)(hi - lo) + 1.0f);
  uint32_t lb[kLbPt];
#pragma unroll
  for (int i = 0; i < kLbPt; ++i) {
    lb[i] = 0u;
    const int R = tid + i * kThreads;
    if (R < nR) {
      uint32_t mu[G];  // all G maxima read before any is used
#pragma unroll
      for (int gg = 0; gg < G; ++gg) mu[gg] = sh.bound.msup[gg * nR + R];
      float v = -INFINITY;
#pragma unroll
      for (int gg = 0; gg < G; ++gg)
        if (mu[gg]) v = fmaxf(v, key_from_order_bits(mu[gg]) - L[gg]);
      if (v > -INFINITY) lb[i] = key_order_bits(v - log2G);
    }
  }
  float tlb = -INFINITY;  // fewer than k units (some may hold no page): no pruning
  if (nR >= a.k) {        // workgroup-uniform
    // the minimum of the bucket holding the k-th largest bound is at most it
#pragma unroll
    for (int i = 0; i < kLbPt; ++i)
      if (lb[i]) {
        const int bk = hbucket(max(lb[i], lo), lo, scale);
        atomicAdd(&sh.hcnt[bk], 1u);
        atomicMin(&sh.bound.hmin[bk], lb[i]);
      }
    __syncthreads();
    const uint32_t c0 = sh.hcnt[2 * tid], c1 = sh.hcnt[2 * tid + 1];
    const uint32_t above = hist_above(c0 + c1, sh.wsum);
    const uint32_t k = (uint32_t)a.k;
    uint32_t t = 0u;
    if (above < k && k <= above + c1) t = sh.bound.hmin[2 * tid + 1];
    else if (above + c1 < k && k <= above + c1 + c0) t = sh.bound.hmin[2 * tid];
    // margin for fp32 rounding between these bounds and the keys formed below
    if (t) sh.tlb = key_from_order_bits(t) - 1e-3f;
    __syncthreads();
    tlb = sh.tlb;  // -inf if fewer than k units held a page
  }

  // ================================================================ 2. chunk
  unsigned long long x[kChunkEpt];  // slots past EPT stay 0 (no candidate)
#pragma unroll
  for (int i = 0; i < kChunkEpt; ++i) x[i] = 0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    // log2 of sum_g exp2(s_hat_g - L_g): the max over the group first, then
    // one exp2 per head
    float v[G], km = -1e30f, ks = 0.f;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      v[gg] = fmaf(sc[gg][i], kLog2e, -L[gg]);
      km = fmaxf(km, v[gg]);
    }
#pragma unroll
    for (int gg = 0; gg < G; ++gg) ks += fast_exp2(v[gg] - km);
    const bool in = p0 + i * kThreads < n_b;
    // log2 of the summed shares minus log2 G; absent pages score -inf
    const float key2 = (in && ks > 0.f && km > -1e29f) ? km + fast_log2(ks) - log2G : -INFINITY;
    if (key2 > -INFINITY && key2 >= tlb) {
      const uint32_t jj = (uint32_t)(p0 + i * kThreads);
      x[i] = ((unsigned long long)key_order_bits(key2) << 32) | (unsigned long long)(0xffffffffu - jj);
    }
  }
  {
    // page order = (slab, thread) order: two packed scans give every
    // survivor its rank (slab counts fit 16 bits)
    const uint32_t f01 = (x[0] != 0 ? 1u : 0u) | (x[1] != 0 ? 0x10000u : 0u);
    const uint32_t f23 = (x[2] != 0 ? 1u : 0u) | (x[3] != 0 ? 0x10000u : 0u);
    uint32_t t01, t23;
    uint32_t e01 = f01, e23 = f23;
    big_exclusive_scan2(e01, e23, &t01, &t23, sh);
    const uint32_t T0 = t01 & 0xffffu, T1 = t01 >> 16, T2 = t23 & 0xffffu, T3 = t23 >> 16;
    const uint32_t off[4] = {e01 & 0xffffu, T0 + (e01 >> 16), T0 + T1 + (e23 & 0xffffu),
                             T0 + T1 + T2 + (e23 >> 16)};
    const size_t base = (head * a.n_chunks + chunk) * a.chunk;
#pragma unroll
    for (int i = 0; i < EPT; ++i)
      if (x[i] != 0) {
        a.cand[base + off[i]] = x[i];
        a.cand_blk[base + off[i]] = blk[i];
      }
    if (tid == 0) a.cand_count[head * a.n_chunks + chunk] = (int)(T0 + T1 + T2 + T3);
  }

}

// ============================================================ merge
//
// One workgroup of kMergeThreads per (sequence, KV head). Up to kFastCap
// candidates (the usual case) its waves rank them in registers. Up to kRoundCap the whole workgroup copies the chunk
// lists, in page order, into one LDS list and ranks it by bucket refinement
// over the live key range with a 2048-bucket LDS histogram (4 buckets per
// thread): elements above the bucket of the need-th key in, below it out,
// until the count fits or the live keys are all equal (then the earliest,
// i.e. lowest page ids, win). Larger sets: rank_global, a radix select over
// the lists where they lie.

constexpr int kMergeThreads = 512;               // 8 waves: up to 256 VGPRs, no spills
constexpr int kRoundCap = kSelectMaxK + 512;     // candidates the LDS list holds
constexpr int kMergeBpt = kRankBuckets / kMergeThreads;           // histogram buckets per thread
constexpr int kMergeEpt = (kRoundCap + kMergeThreads - 1) / kMergeThreads;  // list entries per thread

struct MergeLds {
  unsigned long long x[kRoundCap];  // sort keys; 0 = rejected
  int blk[kRoundCap];
  uint8_t state[kRoundCap];         // 0 live, 1 selected, 2 rejected
  RankLds<kMergeThreads> r;         // histogram, list offsets, reduction slots
};

// Ranks x[0..n) (state all live on entry) and marks the `need` largest
// selected; every thread of the workgroup takes part.
__device__ void merge_topk(MergeLds& W, int n, int need) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int iter = 0; iter < 8 && need > 0; ++iter) {
    uint32_t cnt = 0, lo = 0xffffffffu, hi = 0u;
    for (int e = tid; e < n; e += kMergeThreads)
      if (W.state[e] == 0) {
        const uint32_t v = (uint32_t)(W.x[e] >> 32);
        ++cnt;
        lo = min(lo, v);
        hi = max(hi, v);
      }
    cnt = wave_sum_u32(cnt);
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    if (lane == 0) { W.r.red3[0][wave] = cnt; W.r.red3[1][wave] = lo; W.r.red3[2][wave] = hi; }
    __syncthreads();
    cnt = 0;
    lo = 0xffffffffu;
    hi = 0u;
#pragma unroll
    for (int w = 0; w < kMergeThreads / 64; ++w) {
      cnt += W.r.red3[0][w];
      lo = min(lo, W.r.red3[1][w]);
      hi = max(hi, W.r.red3[2][w]);
    }
    if ((int)cnt <= need) {  // every live element is in
      for (int e = tid; e < n; e += kMergeThreads)
        if (W.state[e] == 0) W.state[e] = 1;
      __syncthreads();
      return;
    }
    if (lo == hi) break;
    const float scale = (float)kRankBuckets / ((float)(hi - lo) + 1.0f);
#pragma unroll
    for (int q = 0; q < kMergeBpt; ++q) W.r.hist[kMergeBpt * tid + q] = 0u;
    __syncthreads();
    for (int e = tid; e < n; e += kMergeThreads)
      if (W.state[e] == 0) atomicAdd(&W.r.hist[hbucket((uint32_t)(W.x[e] >> 32), lo, scale)], 1u);
    __syncthreads();
    // thread t owns buckets [4t, 4t+4): counts above them, then the bucket
    // holding the need-th key from the top
    uint32_t hb[kMergeBpt], mine = 0;
#pragma unroll
    for (int q = 0; q < kMergeBpt; ++q) {
      hb[q] = W.r.hist[kMergeBpt * tid + q];
      mine += hb[q];
    }
    uint32_t tot;
    const uint32_t pre = rank_excl_scan<kMergeThreads>(mine, W.r.scn, &tot);
    uint32_t acc = tot - pre - mine;
#pragma unroll
    for (int q = kMergeBpt - 1; q >= 0; --q) {
      if (acc < (uint32_t)need && (uint32_t)need <= acc + hb[q]) {
        W.r.bstar = kMergeBpt * tid + q;  // exactly one thread finds it
        W.r.babove = acc;
      }
      acc += hb[q];
    }
    __syncthreads();
    const int bstar = W.r.bstar;
    const uint32_t above = W.r.babove;
    for (int e = tid; e < n; e += kMergeThreads)
      if (W.state[e] == 0) {
        const int bk = hbucket((uint32_t)(W.x[e] >> 32), lo, scale);
        if (bk > bstar) W.state[e] = 1;
        else if (bk < bstar) W.state[e] = 2;
      }
    need -= (int)above;
    __syncthreads();
  }
  if (need > 0) {
    // live keys all equal (or, unreachably, out of passes): earliest live
    // win; thread t owns entries [t E, t E + E)
    const int E = (n + kMergeThreads - 1) / kMergeThreads;
    uint32_t nl = 0;
    for (int i = 0; i < E; ++i) {
      const int e = tid * E + i;
      if (e < n && W.state[e] == 0) ++nl;
    }
    uint32_t tot;
    uint32_t before = rank_excl_scan<kMergeThreads>(nl, W.r.scn, &tot);
    for (int i = 0; i < E; ++i) {
      const int e = tid * E + i;
      if (e < n && W.state[e] == 0) {
        if ((int)before < need) W.state[e] = 1;
        ++before;
      }
    }
    __syncthreads();
  }
}

// The exact top-k of one (sequence, KV head)'s candidate lists (at most
// kRoundCap of them: larger sets take rank_global), run by the whole
// workgroup in one pass: the lists are copied into the LDS list in page order
// and ranked there; leaves the kept sort keys and blocks, in page order, in
// W.x / W.blk and returns their count.
__device__ int merge_lists(MergeLds& W, const CandLists& L, int k) {
  const int tid = threadIdx.x;
  rank_list_offsets<kMergeThreads>(W.r, L);
  const int n = W.r.off[L.nc];  // <= kRoundCap (the caller's condition)
  unsigned long long xv[kMergeEpt];
  int bv[kMergeEpt];
#pragma unroll
  for (int i = 0; i < kMergeEpt; ++i) {
    const int e = tid + kMergeThreads * i;
    int sidx = 0;
    if (e < n) {
      int c = 0;
      for (int lo = 0, hi = L.nc - 1; lo <= hi;) {
        const int mid = (lo + hi) >> 1;
        if (W.r.off[mid] <= e) { c = mid; lo = mid + 1; } else hi = mid - 1;
      }
      sidx = c * L.chunk + (e - W.r.off[c]);
    }
    xv[i] = L.x[sidx];
    bv[i] = L.blk[sidx];
  }
#pragma unroll
  for (int i = 0; i < kMergeEpt; ++i) {
    const int e = tid + kMergeThreads * i;
    if (e < n) {
      W.x[e] = xv[i];
      W.blk[e] = bv[i];
    }
  }
  for (int e = tid; e < n; e += kMergeThreads) W.state[e] = 0;
  __syncthreads();
  merge_topk(W, n, k);
  // keep the selected, in order: thread t owns entries [t E, t E + E), all
  // read before the scan's barrier, written after it
  const int E = (n + kMergeThreads - 1) / kMergeThreads;
  unsigned long long xs[kMergeEpt];
  int bs[kMergeEpt];
  uint32_t sel = 0, ns = 0;
#pragma unroll
  for (int i = 0; i < kMergeEpt; ++i) {
    const int e = tid * E + i;
    xs[i] = 0;
    bs[i] = 0;
    if (i < E && e < n && W.state[e] == 1) {
      xs[i] = W.x[e];
      bs[i] = W.blk[e];
      sel |= 1u << i;
      ++ns;
    }
  }
  uint32_t kept;
  uint32_t dst = rank_excl_scan<kMergeThreads>(ns, W.r.scn, &kept);
#pragma unroll
  for (int i = 0; i < kMergeEpt; ++i)
    if ((sel >> i) & 1u) {
      W.x[dst] = xs[i];
      W.blk[dst] = bs[i];
      ++dst;
    }
  __syncthreads();
  return (int)kept;
}

// One workgroup per (sequence, KV head); writes the kept ids and their
// blocks in page order, -1 past them.
__global__ __launch_bounds__(kMergeThreads) void select_merge_kernel(SelectArgs a) {
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  __shared__ MergeLds W;
  const size_t head = (size_t)b * a.Hkv + kvh;
  const int nc = a.n_chunks;
  const CandLists L{a.cand + head * nc * a.chunk, a.cand_blk + head * nc * a.chunk,
                    a.cand_count + head * nc, nc, a.chunk};
  int32_t* out = a.selected + head * a.k;
  int32_t* outb = a.sel_blk + head * a.k;
  auto emit = [out, outb](int pos, int id, int blk) {
    out[pos] = id;
    outb[pos] = blk;
  };

  // the counts and the speculative slots, in one round trip
  const int lgS = fast_lg_slots(nc);
  int cc[16];
  fast_count_load(L, cc);
  constexpr int KPL = kFastCap / kMergeThreads;
  unsigned long long x[KPL];
  int bl[KPL], cof[KPL];
  fast_slots_load<kMergeThreads>(L, lgS, x, bl, cof);
  int total;
  const bool over = fast_count_check(L, lgS, cc, &total);  // the same in every wave
  if (over && total > kFastCap) {
    if (total > kRoundCap) {
      rank_global<kMergeThreads>(W.r, L, a.k, emit);
      return;
    }
    const int nk = merge_lists(W, L, a.k);
    for (int i = tid; i < a.k; i += kMergeThreads) {
      out[i] = (i < nk) ? (int32_t)(0xffffffffu - (uint32_t)(W.x[i] & 0xffffffffu)) : -1;
      outb[i] = (i < nk) ? W.blk[i] : -1;
    }
    return;
  }
  const uint32_t live = over ? fast_gather_exact<kMergeThreads>(L, W.r.off, total, x, bl)
                             : fast_slots_live<kMergeThreads>(L, lgS, cof);
  fast_emit<kMergeThreads>(x, bl, fast_rank<kMergeThreads>(x, live, a.k, !over, W.r), a.k, !over, 0, a.k, W.r,
                           emit);
}

}  // namespace

hipError_t launch_select(const locks_dims& d, const WsLayout& L, const DevPtrs& P,
                         const int32_t* pt, const int32_t* sl, const int32_t* fill,
                         int32_t* selected, bool merge, hipStream_t s) {
  SelectArgs a;
  a.scores = P.scores;
  a.score_part = P.score_part;
  a.tile_max = P.tile_max;
  a.page_table = pt;
  a.seq_lens = sl;
  a.fill = fill;
  a.cand = P.cand;
  a.cand_blk = P.cand_blk;
  a.cand_count = P.cand_count;
  a.selected = selected;
  a.sel_blk = P.sel_blk;
  a.Hq = d.n_q_heads;
  a.Hkv = d.n_kv_heads;
  a.N = d.max_pages_per_seq;
  a.k = L.k;
  a.n_ranges = L.n_score_wg;
  a.n_tiles = 4 * L.n_score_wg;
  a.sup_r = L.sup_r;
  a.sup_t = L.sup_t;
  a.chunk = L.sel_chunk;
  a.n_chunks = L.n_sel_chunks;
  const dim3 grid(L.n_sel_chunks, d.n_kv_heads, d.batch);
  const int ept = L.sel_chunk / kThreads;  // 1, 2 or 4
#define LOCKS_CHUNK(GG)                                                                               \
  case GG:                                                                                            \
    if (ept == 1) hipLaunchKernelGGL((select_chunk_kernel<GG, 1>), grid, dim3(kThreads), 0, s, a);   \
    else if (ept == 2) hipLaunchKernelGGL((select_chunk_kernel<GG, 2>), grid, dim3(kThreads), 0, s, a); \
    else if (ept == 4) hipLaunchKernelGGL((select_chunk_kernel<GG, 4>), grid, dim3(kThreads), 0, s, a); \
    else return hipErrorInvalidValue;                                                                 \
    break;
  switch (d.n_q_heads / d.n_kv_heads) {
    LOCKS_CHUNK(1) LOCKS_CHUNK(2) LOCKS_CHUNK(4) LOCKS_CHUNK(8) LOCKS_CHUNK(16)
    default: return hipErrorInvalidValue;
  }
#undef LOCKS_CHUNK
  if (merge)
    hipLaunchKernelGGL(select_merge_kernel, dim3(d.n_kv_heads, d.batch), dim3(kMergeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace locks
