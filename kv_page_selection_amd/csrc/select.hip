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
//        smallest member gives that k-th largest bound. Units are pooled into
//        super-ranges when the (head, unit) maxima exceed what LDS holds (the
//        maximum over a super-range still bounds one of its pages).
//        Computing this in every workgroup costs less than a launch of its
//        own.
//     b. the keys of the workgroup's <= 4096 pages as 64-bit sort keys
//        (order-preserving key bits << 32 | ~page id, so one integer
//        comparison applies "larger key, then lower id"); those with key >= T
//        are written, with their physical blocks, in page order (typically a
//        few hundred per (sequence, KV head) in all).
//  2. merge: one wave per (sequence, KV head) ranks the chunk lists in page
//     order, in rounds of up to 512 new candidates appended to the running
//     top-k; kept candidates always precede the new ones in page order, so the
//     result comes out sorted without a sort. It also writes the physical
//     blocks of the kept pages for the attention pass. One wave needs no
//     barriers; workgroup-wide ranking at this size is bound by barrier and
//     LDS round trips, not work.
// Ranking = exact selection by bucket refinement on the key bits: a 2048-bucket
// histogram over the live [lo, hi] key range picks the bucket holding the
// k-th key; everything above it is in, below it out; repeat inside that
// bucket (range shrinks ~2^11 per pass) until the count fits or all live keys
// are equal, where the lowest ids win.
#include "device_common.h"
#include "internal.h"

namespace locks {

namespace {

constexpr int kThreads = 1024;
constexpr int kNW = kThreads / 64;
constexpr int kHistBuckets = 2 * kThreads;                // 2 buckets per thread
constexpr int kChunkEpt = kSelectChunk / kThreads;        // <= 4 pages per thread

struct SelectArgs {
  const float* scores;
  const float* score_part;
  const float* tile_max;
  const int32_t* page_table;
  const int32_t* seq_lens;
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
  uint32_t red3[3][kNW];
  uint32_t scn[2][kNW];
  float redf[kNW][2];
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
__device__ __forceinline__ void wave_lse2(float& m, float& s) {
  lse2_acc(m, s, dpp_mov<kDppXor1>(m), dpp_mov<kDppXor1>(s));
  lse2_acc(m, s, dpp_mov<kDppXor2>(m), dpp_mov<kDppXor2>(s));
  lse2_acc(m, s, dpp_mov<kDppHalfMirror>(m), dpp_mov<kDppHalfMirror>(s));
  lse2_acc(m, s, dpp_mov<kDppMirror>(m), dpp_mov<kDppMirror>(s));
  {
    const auto rm = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    const auto rs = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    m = __uint_as_float(rm[0]);
    s = __uint_as_float(rs[0]);
    lse2_acc(m, s, __uint_as_float(rm[1]), __uint_as_float(rs[1]));
  }
  {
    const auto rm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    const auto rs = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    m = __uint_as_float(rm[0]);
    s = __uint_as_float(rs[0]);
    lse2_acc(m, s, __uint_as_float(rm[1]), __uint_as_float(rs[1]));
  }
}

// Block-wide (count, min, max) of u32 triples for 1024 threads, one barrier
// (red must not be reused before another barrier has passed).
__device__ __forceinline__ void big_reduce3(uint32_t& c, uint32_t& mn, uint32_t& mx,
                                            uint32_t (&red)[3][kNW]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  c = wave_sum_u32(c);
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  if (lane == 0) {
    red[0][wave] = c;
    red[1][wave] = mn;
    red[2][wave] = mx;
  }
  __syncthreads();
  c = 0;
  mn = 0xffffffffu;
  mx = 0u;
#pragma unroll
  for (int w = 0; w < kNW; ++w) {
    c += red[0][w];
    mn = min(mn, red[1][w]);
    mx = max(mx, red[2][w]);
  }
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
  const int n_b = full_pages(a.seq_lens, b, N);
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
  for (int r0 = 0; r0 < nr; r0 += 8 * P) {
    float2 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = r0 + j + i * P;
      v[i] = (r < nr) ? part[r] : make_float2(-INFINITY, 0.f);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = r0 + j + i * P;
      const bool ne = v[i].y > 0.f;  // range holds a present page
      if (ne) lse2_acc(lm, ls, v[i].x, v[i].y);
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
  if (lane == 0) { sh.redf[wave][0] = lm; sh.redf[wave][1] = ls; }
  __syncthreads();
  float L[G];  // base 2; every thread folds every head's wave partials itself
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    float m = sh.redf[gg * WPG][0], sv = sh.redf[gg * WPG][1];
#pragma unroll
    for (int w = 1; w < WPG; ++w) lse2_acc(m, sv, sh.redf[gg * WPG + w][0], sh.redf[gg * WPG + w][1]);
    L[gg] = (sv > 0.f) ? m + fast_log2(sv) : -INFINITY;
  }
  const float log2G = (float)__builtin_ctz(G);
  uint32_t lb[kLbPt];
  uint32_t cnt = 0, lo = 0xffffffffu, hi = 0u;
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
      if (v > -INFINITY) {
        lb[i] = key_order_bits(v - log2G);
        ++cnt;
        lo = min(lo, lb[i]);
        hi = max(hi, lb[i]);
      }
    }
  }
  big_reduce3(cnt, lo, hi, sh.red3);
  float tlb;
  if ((int)cnt < a.k) {
    tlb = -INFINITY;  // fewer bound units than k: no pruning
  } else if (lo == hi) {
    tlb = key_from_order_bits(lo) - 1e-3f;
  } else {
    // the minimum of the bucket holding the k-th largest bound is at most it
    const float scale = (float)kHistBuckets / ((float)(hi - lo) + 1.0f);
#pragma unroll
    for (int i = 0; i < kLbPt; ++i)
      if (lb[i]) {
        const int bk = hbucket(lb[i], lo, scale);
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
    tlb = sh.tlb;
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

// ============================================================ merge (one wave)
//
// One wave per (sequence, KV head) ranks the chunk lists, in page order, in
// rounds of up to kRoundNew new candidates appended to the running top-k in
// LDS; a wave needs no barriers, only the in-order completion of its own LDS
// operations. Ranking: bucket refinement over the live key range with a
// 2048-bucket LDS histogram (32 buckets per lane), elements above the bucket
// of the need-th key in, below it out, until the count fits or the live keys
// are all equal (then the earliest, i.e. lowest page ids, win).

constexpr int kRoundNew = 512;                   // new candidates per round
constexpr int kRoundCap = kSelectMaxK + kRoundNew;

struct WaveMergeLds {
  unsigned long long x[kRoundCap];  // sort keys; 0 = rejected
  int blk[kRoundCap];
  uint8_t state[kRoundCap];         // 0 live, 1 selected, 2 rejected
  uint32_t hist[kHistBuckets];
  int off[1025];
};

// LDS slot of histogram bucket bk when lane l owns buckets [32l, 32l+32):
// lane-major interleave, so the 64 lanes reading their q-th bucket hit 64
// different banks.
__device__ __forceinline__ int hslot(int bk) { return ((bk & 31) << 6) | (bk >> 5); }

__device__ __forceinline__ uint32_t wave_ballot_count(bool p) {
  return (uint32_t)__popcll(__ballot(p));
}

// Ranks x[0..n) (state all live on entry) and marks the `need` largest selected.
__device__ void wave_topk(WaveMergeLds& W, int n, int need) {
  const int lane = threadIdx.x & 63;
  for (int iter = 0; iter < 8 && need > 0; ++iter) {
    uint32_t cnt = 0, lo = 0xffffffffu, hi = 0u;
    for (int e = lane; e < n; e += 64)
      if (W.state[e] == 0) {
        const uint32_t v = (uint32_t)(W.x[e] >> 32);
        ++cnt;
        lo = min(lo, v);
        hi = max(hi, v);
      }
    cnt = wave_sum_u32(cnt);
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    if ((int)cnt <= need) {  // every live element is in
      for (int e = lane; e < n; e += 64)
        if (W.state[e] == 0) W.state[e] = 1;
      wave_lds_sync();
      return;
    }
    if (lo == hi) break;
    const float scale = (float)kHistBuckets / ((float)(hi - lo) + 1.0f);
    for (int i = lane; i < kHistBuckets; i += 64) W.hist[i] = 0u;  // layout-independent
    wave_lds_sync();
    for (int e = lane; e < n; e += 64)
      if (W.state[e] == 0) atomicAdd(&W.hist[hslot(hbucket((uint32_t)(W.x[e] >> 32), lo, scale))], 1u);
    wave_lds_sync();
    // lane l owns buckets [32l, 32l+32); suffix counts from the top bucket down
    uint32_t hb[32];
    uint32_t mine = 0;
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      hb[q] = W.hist[(q << 6) | lane];
      mine += hb[q];
    }
    const uint32_t pre = wave_incl_scan(mine);
    const uint32_t total = __builtin_amdgcn_readlane(pre, 63);
    uint32_t acc = total - pre;  // elements in buckets above this lane's
    int bstar = -1;
    uint32_t above = 0;
#pragma unroll
    for (int q = 31; q >= 0; --q) {
      if (acc < (uint32_t)need && (uint32_t)need <= acc + hb[q]) { bstar = 32 * lane + q; above = acc; }
      acc += hb[q];
    }
    // exactly one lane found the bucket: broadcast it
    const uint64_t owner = __ballot(bstar >= 0);
    if (owner == 0) break;  // unreachable: some bucket holds the need-th key
    const int src = __builtin_ctzll(owner);
    bstar = __builtin_amdgcn_readlane(bstar, src);
    above = __builtin_amdgcn_readlane(above, src);
    for (int e = lane; e < n; e += 64)
      if (W.state[e] == 0) {
        const int bk = hbucket((uint32_t)(W.x[e] >> 32), lo, scale);
        if (bk > bstar) W.state[e] = 1;
        else if (bk < bstar) W.state[e] = 2;
      }
    wave_lds_sync();
    need -= (int)above;
  }
  // live keys all equal (or, unreachably, out of passes): earliest live win
  int base = 0;
  for (int e0 = 0; e0 < n && need > 0; e0 += 64) {
    const int e = e0 + lane;
    const bool live = e < n && W.state[e] == 0;
    const uint32_t before = wave_incl_scan(live ? 1u : 0u) - (live ? 1u : 0u);
    if (live && (int)(base + before) < need) W.state[e] = 1;
    base += (int)wave_ballot_count(live);
  }
  wave_lds_sync();
}

// The exact top-k of one (sequence, KV head)'s candidate lists, run by one
// wave; leaves the kept sort keys and blocks, in page order, in W.x / W.blk
// and returns their count.
__device__ int wave_merge(WaveMergeLds& W, const unsigned long long* src, const int32_t* src_blk,
                          const int32_t* counts, int n_chunks, int chunk, int k) {
  const int lane = threadIdx.x & 63;
  // chunk offsets: lane l sums chunks [l*cpl, (l+1)*cpl)
  const int cpl = (n_chunks + 63) / 64;
  int c_loc[16];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = lane * cpl + i;
    c_loc[i] = (i < cpl && c < n_chunks) ? counts[c] : 0;
    mine += c_loc[i];
  }
  const int pre = (int)wave_incl_scan((uint32_t)mine);
  const int total = __builtin_amdgcn_readlane(pre, 63);
  {
    int o = pre - mine;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = lane * cpl + i;
      if (i < cpl && c < n_chunks) W.off[c] = o;
      o += c_loc[i];
    }
    if (lane == 0) W.off[n_chunks] = total;
  }
  wave_lds_sync();
  int nkept = 0, consumed = 0;
  do {
    const int take = min(total - consumed, kRoundNew);
    // gather the next `take` candidates (8 per lane, all loads in flight together)
    int slot[kRoundNew / 64];
#pragma unroll
    for (int i = 0; i < kRoundNew / 64; ++i) {
      const int e = lane + 64 * i;
      slot[i] = -1;
      if (e < take) {
        const int gidx = consumed + e;
        int c = 0;
        for (int lo = 0, hi = n_chunks - 1; lo <= hi;) {
          const int mid = (lo + hi) >> 1;
          if (W.off[mid] <= gidx) { c = mid; lo = mid + 1; } else hi = mid - 1;
        }
        slot[i] = c * chunk + (gidx - W.off[c]);
      }
    }
    unsigned long long xv[kRoundNew / 64];
    int bv[kRoundNew / 64];
#pragma unroll
    for (int i = 0; i < kRoundNew / 64; ++i) {
      const int sidx = slot[i] >= 0 ? slot[i] : 0;
      xv[i] = src[sidx];
      bv[i] = src_blk[sidx];
    }
#pragma unroll
    for (int i = 0; i < kRoundNew / 64; ++i) {
      const int e = lane + 64 * i;
      if (e < take) {
        W.x[nkept + e] = xv[i];
        W.blk[nkept + e] = bv[i];
      }
    }
    const int n = nkept + take;
    for (int e = lane; e < n; e += 64) W.state[e] = 0;
    wave_lds_sync();
    wave_topk(W, n, k);
    // keep the selected, in order (destinations never pass their sources)
    int base = 0;
    for (int e0 = 0; e0 < n; e0 += 64) {
      const int e = e0 + lane;
      const bool s = e < n && W.state[e] == 1;
      unsigned long long xe = 0;
      int be = 0;
      if (s) { xe = W.x[e]; be = W.blk[e]; }
      const uint32_t before = wave_incl_scan(s ? 1u : 0u) - (s ? 1u : 0u);
      wave_lds_sync();
      if (s) {
        W.x[base + before] = xe;
        W.blk[base + before] = be;
      }
      base += (int)wave_ballot_count(s);
      wave_lds_sync();
    }
    nkept = base;
    consumed += take;
  } while (consumed < total);
  return nkept;
}

constexpr int kFastPerLane = 16;
constexpr int kFastCap = 64 * kFastPerLane;  // candidates ranked in registers

// One wave per (sequence, KV head). Fast path (every chunk list fits the
// speculative slots, at most 1024 candidates): the counts and the first S
// slots of every chunk list arrive in one round trip, and the candidates are
// ranked in registers, 16 contiguous ones per lane, so lane order is page
// order. Otherwise the LDS rounds of wave_merge.
__global__ __launch_bounds__(64) void select_merge_kernel(SelectArgs a) {
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  __shared__ WaveMergeLds W;
  const size_t head = (size_t)b * a.Hkv + kvh;
  const int nc = a.n_chunks;
  const int32_t* counts = a.cand_count + head * nc;
  const unsigned long long* src = a.cand + head * nc * a.chunk;
  const int32_t* src_blk = a.cand_blk + head * nc * a.chunk;
  int32_t* out = a.selected + head * a.k;
  int32_t* outb = a.sel_blk + head * a.k;

  // slots per chunk loaded speculatively: a power of two with nc * S <= 1024
  const int lgS = 31 - __builtin_clz(max(1, kFastCap / nc));
  const int S = 1 << lgS;
  int ccnt[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = lane + 64 * i;
    ccnt[i] = (c < nc) ? counts[c] : 0;
  }
  unsigned long long x[kFastPerLane];
  int bl[kFastPerLane], cof[kFastPerLane];
#pragma unroll
  for (int i = 0; i < kFastPerLane; ++i) {
    const int e = lane * kFastPerLane + i;
    const int c = e >> lgS, sl = e & (S - 1);
    const int idx = (c < nc) ? c * a.chunk + sl : 0;
    x[i] = src[idx];
    bl[i] = src_blk[idx];
    cof[i] = (c < nc) ? counts[c] : 0;
  }
  int total = 0;
  bool over = false;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    total += ccnt[i];
    over |= ccnt[i] > S;
  }
  total = (int)wave_sum_u32((uint32_t)total);
  if (__ballot(over) != 0) {
    const int nk = wave_merge(W, src, src_blk, counts, nc, a.chunk, a.k);
    for (int i = lane; i < a.k; i += 64) {
      out[i] = (i < nk) ? (int32_t)(0xffffffffu - (uint32_t)(W.x[i] & 0xffffffffu)) : -1;
      outb[i] = (i < nk) ? W.blk[i] : -1;
    }
    return;
  }
  (void)total;

  uint32_t live = 0, sel = 0;
#pragma unroll
  for (int i = 0; i < kFastPerLane; ++i) {
    const int e = lane * kFastPerLane + i;
    if ((e >> lgS) < nc && (e & (S - 1)) < cof[i]) live |= 1u << i;
  }
  int need = a.k;
  for (int iter = 0; iter < 8; ++iter) {
    uint32_t cnt = __popc(live), lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int i = 0; i < kFastPerLane; ++i)
      if ((live >> i) & 1u) {
        const uint32_t v = (uint32_t)(x[i] >> 32);
        lo = min(lo, v);
        hi = max(hi, v);
      }
    cnt = wave_sum_u32(cnt);
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    if ((int)cnt <= need) { sel |= live; live = 0; break; }
    if (lo == hi) break;
    const float scale = (float)kHistBuckets / ((float)(hi - lo) + 1.0f);
#pragma unroll
    for (int q = 0; q < 32; ++q) W.hist[(q << 6) | lane] = 0u;
    wave_lds_sync();
    int bk[kFastPerLane];
#pragma unroll
    for (int i = 0; i < kFastPerLane; ++i) {
      bk[i] = -1;
      if ((live >> i) & 1u) {
        bk[i] = hbucket((uint32_t)(x[i] >> 32), lo, scale);
        atomicAdd(&W.hist[hslot(bk[i])], 1u);
      }
    }
    wave_lds_sync();
    uint32_t hb[32];
    uint32_t mine = 0;
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      hb[q] = W.hist[(q << 6) | lane];
      mine += hb[q];
    }
    const uint32_t pre = wave_incl_scan(mine);
    const uint32_t tot = __builtin_amdgcn_readlane(pre, 63);
    uint32_t acc = tot - pre;
    int bstar = -1;
    uint32_t above = 0;
#pragma unroll
    for (int q = 31; q >= 0; --q) {
      if (acc < (uint32_t)need && (uint32_t)need <= acc + hb[q]) { bstar = 32 * lane + q; above = acc; }
      acc += hb[q];
    }
    const uint64_t owner = __ballot(bstar >= 0);
    if (owner == 0) break;  // unreachable: some bucket holds the need-th key
    const int srcl = __builtin_ctzll(owner);
    bstar = __builtin_amdgcn_readlane(bstar, srcl);
    above = __builtin_amdgcn_readlane(above, srcl);
#pragma unroll
    for (int i = 0; i < kFastPerLane; ++i)
      if ((live >> i) & 1u) {
        if (bk[i] > bstar) sel |= 1u << i;
        if (bk[i] != bstar) live &= ~(1u << i);
      }
    need -= (int)above;
    wave_lds_sync();
  }
  if (__ballot(live != 0) != 0) {
    // live keys all equal: the earliest (lowest page ids) win
    const uint32_t nl = __popc(live);
    int before = (int)(wave_incl_scan(nl) - nl);
#pragma unroll
    for (int i = 0; i < kFastPerLane; ++i)
      if ((live >> i) & 1u) {
        if (before < need) sel |= 1u << i;
        ++before;
      }
  }
  // ---- write the kept pages in page order, then the -1 tail
  const uint32_t ns = __popc(sel);
  const uint32_t pre = wave_incl_scan(ns);
  const int nk = (int)__builtin_amdgcn_readlane(pre, 63);
  int o = (int)(pre - ns);
#pragma unroll
  for (int i = 0; i < kFastPerLane; ++i)
    if ((sel >> i) & 1u) {
      out[o] = (int32_t)(0xffffffffu - (uint32_t)(x[i] & 0xffffffffu));
      outb[o] = bl[i];
      ++o;
    }
  for (int i = nk + lane; i < a.k; i += 64) {
    out[i] = -1;
    outb[i] = -1;
  }
}

}  // namespace

hipError_t launch_select(const locks_dims& d, const WsLayout& L, const DevPtrs& P,
                         const int32_t* pt, const int32_t* sl, int32_t* selected, hipStream_t s) {
  SelectArgs a;
  a.scores = P.scores;
  a.score_part = P.score_part;
  a.tile_max = P.tile_max;
  a.page_table = pt;
  a.seq_lens = sl;
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
  hipLaunchKernelGGL(select_merge_kernel, dim3(d.n_kv_heads, d.batch), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace locks
