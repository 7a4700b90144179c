// select.hip — group-shared page selection (gfx950).
//
// Group combine (technical summary, section 2 mechanism 3): each head g of a
// GQA group has total mass L_g = log sum_j exp(s_hat[g][j]) over the
// sequence's pages; a page's key is the log of the group-mean normalised mass
// share, key_j = log((1/G) sum_g exp(s_hat[g][j] - L_g)).
// Top-k (blog post, "Code": keep budget/16 pages with the largest score, ids
// ascending): the k largest keys, ties to the lower page id.
//
// Three launches, no float atomics, every load of a phase issued before the
// first one is consumed:
//  1. bound: one 1024-thread workgroup per (sequence, KV head) folds the
//     scoring pass's per-range (max, sum) partials into L_g, and from the
//     per-range maxima a lower bound T on the k-th largest key: every 64-page
//     range holds a page whose key is at least max_g(range max of
//     s_hat_g - L_g) - log2 G, so the k-th largest of these per-range bounds
//     (taken over distinct ranges) cannot exceed the k-th largest key. Ranges
//     are pooled into super-ranges when there are too many to hold in LDS
//     (the maximum over a super-range is still a bound of one of its pages).
//  2. chunk: grid (chunk, KV head, sequence); every workgroup forms the keys of
//     <= 1024 pages as 64-bit sort keys (order-preserving key bits << 32 |
//     ~page id, so one integer comparison applies "larger key, then lower id")
//     and writes those with key >= T, with their physical blocks, in page
//     order (typically a few hundred per (sequence, KV head) in total).
//  3. merge: one 1024-thread workgroup per (sequence, KV head) streams over
//     the chunk lists in page order, up to 8192 candidates per round,
//     carrying the running top-k; kept candidates always precede the new ones
//     in page order, so the result comes out sorted without a sort.
// (Separate launches instead of last-workgroup hand-offs: on this chip a
// device-scope release from every workgroup costs an L2 write-back each.)
// Ranking = exact selection by bucket refinement on the key bits: a 2048-bucket
// histogram over the live [lo, hi] key range picks the bucket holding the
// k-th key; everything above it is in, below it out; repeat inside that
// bucket (range shrinks ~2^11 per pass) until the count fits or all live keys
// are equal, where the lowest ids win. The bound pass uses one such histogram,
// keeping each bucket's smallest member, to get its k-th largest range bound.
#include "device_common.h"
#include "internal.h"

namespace locks {

namespace {

constexpr int kChunkThreads = 256;
constexpr int kBigThreads = 1024;                          // bound and merge kernels
constexpr int kMergeEpt = kSelectMaxElems / kBigThreads;   // 8 candidates per thread per round
constexpr int kHistBuckets = 2 * kBigThreads;             // 2048 histogram buckets, 2 per thread

struct SelectArgs {
  const float* scores;
  const float* score_part;
  const int32_t* page_table;
  const int32_t* seq_lens;
  float* Lg;
  float* tlb;
  unsigned long long* cand;
  int32_t* cand_blk;
  int32_t* cand_count;
  int32_t* selected;
  int32_t* sel_blk;
  int Hq, Hkv, N, num_blocks, k, n_ranges, sup, n_sup, chunk, n_chunks;
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

// Exclusive prefix over the 256 threads of a chunk workgroup (thread order =
// element order); returns this thread's offset and the total in *total.
__device__ int chunk_exclusive_scan(int v, int* total, int* scan_s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) scan_s[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int c = scan_s[w];
    if (w < wave) before += c;
    tot += c;
  }
  *total = tot;
  return before + incl - v;
}

// ---------------------------------------------------------------- 1. bound

// Block-wide (count, min, max) of u32 triples for 1024 threads, one barrier
// (red must not be reused before another barrier has passed).
__device__ __forceinline__ void big_reduce3(uint32_t& c, uint32_t& mn, uint32_t& mx,
                                            uint32_t (&red)[3][16]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    c += __shfl_xor(c, o);
    mn = min(mn, (uint32_t)__shfl_xor(mn, o));
    mx = max(mx, (uint32_t)__shfl_xor(mx, o));
  }
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
  for (int w = 0; w < 16; ++w) {
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
  uint32_t incl = mine;  // this lane and the lanes above it in the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_down(incl, o);
    if (lane + o < 64) incl += y;
  }
  if (lane == 0) wsum[wave] = incl;
  __syncthreads();
  uint32_t above = incl - mine;
#pragma unroll
  for (int w = 0; w < 16; ++w)
    if (w > wave) above += wsum[w];
  return above;
}

template <int G>
__global__ __launch_bounds__(kBigThreads) void select_bound_kernel(SelectArgs a) {
  constexpr int P = kBigThreads / G;  // threads per head
  constexpr int WPG = P / 64;         // waves per head
  constexpr int kLbPt = kBoundSlots / G / kBigThreads;  // super-ranges per thread at most
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nr = a.n_ranges, S = a.sup, nR = a.n_sup;
  const int g = tid / P, j = tid % P;
  __shared__ uint32_t msup_s[kBoundSlots];  // order bits of each (head, super-range) max; 0 = none
  __shared__ uint32_t hcnt_s[kHistBuckets], hmin_s[kHistBuckets];
  __shared__ float red_s[16][2];
  __shared__ uint32_t red3_s[3][16];
  __shared__ uint32_t wsum_s[16];

  hcnt_s[2 * tid] = 0u;
  hcnt_s[2 * tid + 1] = 0u;
  hmin_s[2 * tid] = 0xffffffffu;
  hmin_s[2 * tid + 1] = 0xffffffffu;
  if (S > 1) {  // super-ranges are filled by atomics
    for (int i = tid; i < G * nR; i += kBigThreads) msup_s[i] = 0u;
    __syncthreads();
  }

  // ---- L_g (base 2) and the super-range maxima, 8 independent loads per pass
  const float2* part =
      reinterpret_cast<const float2*>(a.score_part) + ((size_t)b * a.Hq + (size_t)kvh * G + g) * nr;
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
      if (S == 1) {
        if (r < nr) msup_s[g * nR + r] = ne ? key_order_bits(v[i].x) : 0u;
      } else if (ne) {
        atomicMax(&msup_s[g * nR + r / S], key_order_bits(v[i].x));
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) lse2_acc(lm, ls, __shfl_xor(lm, o), __shfl_xor(ls, o));
  if (lane == 0) { red_s[wave][0] = lm; red_s[wave][1] = ls; }
  __syncthreads();
  float L[G];  // every thread folds every head's wave partials itself
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    float m = red_s[gg * WPG][0], sv = red_s[gg * WPG][1];
#pragma unroll
    for (int w = 1; w < WPG; ++w) lse2_acc(m, sv, red_s[gg * WPG + w][0], red_s[gg * WPG + w][1]);
    L[gg] = (sv > 0.f) ? m + fast_log2(sv) : -INFINITY;
    if (tid == gg) a.Lg[(size_t)b * a.Hq + (size_t)kvh * G + gg] = L[gg];
  }

  // ---- per-super-range bounds max_g(max s_hat_g - L_g) - log2 G
  const float log2G = (float)__builtin_ctz(G);
  uint32_t lb[kLbPt];
  uint32_t cnt = 0, lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int i = 0; i < kLbPt; ++i) {
    lb[i] = 0u;
    const int R = tid + i * kBigThreads;
    if (R < nR) {
      float v = -INFINITY;
#pragma unroll
      for (int gg = 0; gg < G; ++gg) {
        const uint32_t u = msup_s[gg * nR + R];
        if (u) v = fmaxf(v, key_from_order_bits(u) - L[gg]);
      }
      if (v > -INFINITY) {
        lb[i] = key_order_bits(v - log2G);
        ++cnt;
        lo = min(lo, lb[i]);
        hi = max(hi, lb[i]);
      }
    }
  }
  big_reduce3(cnt, lo, hi, red3_s);
  if ((int)cnt < a.k) {  // fewer ranges than k: no pruning
    if (tid == 0) a.tlb[(size_t)b * a.Hkv + kvh] = -INFINITY;
    return;
  }
  if (lo == hi) {
    if (tid == 0) a.tlb[(size_t)b * a.Hkv + kvh] = key_from_order_bits(lo) - 1e-3f;
    return;
  }
  // ---- k-th largest bound: one histogram pass keeping each bucket's minimum;
  // the minimum of the bucket holding the k-th is at most the k-th largest
  const float scale = (float)kHistBuckets / ((float)(hi - lo) + 1.0f);
#pragma unroll
  for (int i = 0; i < kLbPt; ++i)
    if (lb[i]) {
      const int bk = hbucket(lb[i], lo, scale);
      atomicAdd(&hcnt_s[bk], 1u);
      atomicMin(&hmin_s[bk], lb[i]);
    }
  __syncthreads();
  const uint32_t c0 = hcnt_s[2 * tid], c1 = hcnt_s[2 * tid + 1];
  const uint32_t above = hist_above(c0 + c1, wsum_s);
  const uint32_t k = (uint32_t)a.k;
  uint32_t t = 0u;
  if (above < k && k <= above + c1) t = hmin_s[2 * tid + 1];
  else if (above + c1 < k && k <= above + c1 + c0) t = hmin_s[2 * tid];
  // margin for fp32 rounding between these bounds and the keys formed later
  if (t) a.tlb[(size_t)b * a.Hkv + kvh] = key_from_order_bits(t) - 1e-3f;
}

// ---------------------------------------------------------------- 2. chunk

template <int G>
__global__ __launch_bounds__(kChunkThreads) void select_chunk_kernel(SelectArgs a) {
  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int N = a.N;
  const int n_b = full_pages(a.seq_lens, b, N);
  __shared__ int scan_s[4];
  constexpr int kEpt = kSelectChunk / kChunkThreads;  // <= 4 pages per thread
  const int ept = a.chunk / kChunkThreads;
  const int p0 = chunk * a.chunk + tid * ept;

  // ---- every load first: bound, L_g, scores, page-table entries
  const float tlb = a.tlb[(size_t)b * a.Hkv + kvh];
  float Lg[G];
#pragma unroll
  for (int g = 0; g < G; ++g) Lg[g] = a.Lg[(size_t)b * a.Hq + (size_t)kvh * G + g];
  float sc[G][kEpt];
  int blk[kEpt];
#pragma unroll
  for (int i = 0; i < kEpt; ++i) {
    const bool in = i < ept && p0 + i < n_b;
    const int p = in ? p0 + i : 0;
    blk[i] = a.page_table[(size_t)b * N + p];
#pragma unroll
    for (int g = 0; g < G; ++g) sc[g][i] = a.scores[((size_t)b * a.Hq + (size_t)kvh * G + g) * N + p];
  }

  // ---- keys: log2 of the summed shares minus log2 G; absent pages score -inf
  const float log2G = log2f((float)G);
  unsigned long long x[kEpt];
  int nlive = 0;
#pragma unroll
  for (int i = 0; i < kEpt; ++i) {
    float km = -1e30f, ks = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) lse2_acc(km, ks, sc[g][i] * kLog2e - Lg[g], 1.0f);
    const bool in = i < ept && p0 + i < n_b;
    const float key2 = (in && ks > 0.f && km > -1e29f) ? km + fast_log2(ks) - log2G : -INFINITY;
    x[i] = 0;
    if (key2 > -INFINITY && key2 >= tlb) {
      const uint32_t jj = (uint32_t)(p0 + i);
      x[i] = ((unsigned long long)key_order_bits(key2) << 32) | (unsigned long long)(0xffffffffu - jj);
      ++nlive;
    }
  }
  int tot;
  int off = chunk_exclusive_scan(nlive, &tot, scan_s);
  const size_t base = ((size_t)(b * a.Hkv + kvh) * a.n_chunks + chunk) * a.chunk;
#pragma unroll
  for (int i = 0; i < kEpt; ++i)
    if (x[i] != 0) {
      a.cand[base + off] = x[i];
      a.cand_blk[base + off] = blk[i];
      ++off;
    }
  if (tid == 0) a.cand_count[(size_t)(b * a.Hkv + kvh) * a.n_chunks + chunk] = tot;
}

// ---------------------------------------------------------------- 3. merge

struct MergeShared {
  uint32_t hcnt[kHistBuckets];
  uint32_t red3[2][3][16];
  uint32_t wsum[16];
  int scan[16];
  uint32_t bstar, above;
};

// Exclusive prefix over the 1024 threads (thread order = element order);
// returns this thread's offset and the total in *total. Two barriers.
__device__ int big_exclusive_scan(int v, int* total, MergeShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) sh.scan[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const int c = sh.scan[w];
    if (w < wave) before += c;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return before + incl - v;
}

// Marks (in `sel`) the `need` largest live elements (`live` bits) of
// x[0..kMergeEpt) across the 1024 threads; element order is thread-major, so
// among equal keys the earliest (lowest page id) win. Each pass: a
// 2048-bucket histogram over the live key range picks the bucket holding the
// need-th key; elements above it are in, below it out; the range shrinks by
// ~2^11 per pass, so 32-bit keys resolve in at most 3 passes plus a check.
__device__ void merge_topk(const unsigned long long* x, uint32_t live, uint32_t& sel, int need,
                           MergeShared& sh) {
  const int tid = threadIdx.x;
  int parity = 0;
  for (int iter = 0; iter < 8; ++iter) {
    // clear this thread's buckets; their last readers passed a barrier since
    sh.hcnt[2 * tid] = 0u;
    sh.hcnt[2 * tid + 1] = 0u;
    uint32_t cnt = __popc(live), lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int i = 0; i < kMergeEpt; ++i)
      if ((live >> i) & 1u) {
        const uint32_t v = (uint32_t)(x[i] >> 32);
        lo = min(lo, v);
        hi = max(hi, v);
      }
    big_reduce3(cnt, lo, hi, sh.red3[parity]);
    parity ^= 1;
    if ((int)cnt <= need) { sel |= live; return; }
    if (need <= 0) return;
    if (lo == hi) break;
    const float scale = (float)kHistBuckets / ((float)(hi - lo) + 1.0f);
    int bk[kMergeEpt];
#pragma unroll
    for (int i = 0; i < kMergeEpt; ++i) {
      bk[i] = -1;
      if ((live >> i) & 1u) {
        bk[i] = hbucket((uint32_t)(x[i] >> 32), lo, scale);
        atomicAdd(&sh.hcnt[bk[i]], 1u);
      }
    }
    __syncthreads();
    const uint32_t c0 = sh.hcnt[2 * tid], c1 = sh.hcnt[2 * tid + 1];
    const uint32_t above = hist_above(c0 + c1, sh.wsum);
    const uint32_t nd = (uint32_t)need;
    if (above < nd && nd <= above + c1) { sh.bstar = 2 * tid + 1; sh.above = above; }
    else if (above + c1 < nd && nd <= above + c1 + c0) { sh.bstar = 2 * tid; sh.above = above + c1; }
    __syncthreads();
    const int bstar = (int)sh.bstar;
    need -= (int)sh.above;
#pragma unroll
    for (int i = 0; i < kMergeEpt; ++i) {
      if (bk[i] > bstar) sel |= 1u << i;
      if (bk[i] != bstar) live &= ~(1u << i);
    }
  }
  // all live keys equal: the earliest live elements win
  int tot;
  int off = big_exclusive_scan(__popc(live), &tot, sh);
#pragma unroll
  for (int i = 0; i < kMergeEpt; ++i)
    if ((live >> i) & 1u) {
      if (off < need) sel |= 1u << i;
      ++off;
    }
}

__global__ __launch_bounds__(kBigThreads) void select_merge_kernel(SelectArgs a) {
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  __shared__ MergeShared sh;
  __shared__ int off_s[1025];
  __shared__ unsigned long long kept_s[kSelectMaxK];
  __shared__ int kept_blk_s[kSelectMaxK];
  __shared__ int nkept_s;
  const size_t head = (size_t)b * a.Hkv + kvh;
  // offsets of the chunk lists in their concatenation (n_chunks <= 1024)
  int tot_all = 0;
  {
    const int c = (tid < a.n_chunks) ? a.cand_count[head * a.n_chunks + tid] : 0;
    const int off = big_exclusive_scan(c, &tot_all, sh);
    if (tid < a.n_chunks) off_s[tid] = off;
    if (tid == 0) { off_s[a.n_chunks] = tot_all; nkept_s = 0; }
  }
  __syncthreads();
  const unsigned long long* src = a.cand + head * a.n_chunks * a.chunk;
  const int32_t* src_blk = a.cand_blk + head * a.n_chunks * a.chunk;
  // rounds: [kept (earlier pages) | next candidates in page order], <= 8192 per round
  int consumed = 0;
  do {
    const int nkept = nkept_s;
    const int take = min(tot_all - consumed, kSelectMaxElems - nkept);
    const int n = nkept + take;
    const int ept = (n + kBigThreads - 1) / kBigThreads;  // <= 8
    const int e0 = tid * ept;
    // source slot of every element: kept list, or (chunk, rank in chunk)
    int c = 0;
    {
      const int g0 = consumed + max(0, e0 - nkept);
      for (int lo = 0, hi = a.n_chunks - 1; lo <= hi;) {
        const int mid = (lo + hi) >> 1;
        if (off_s[mid] <= g0) { c = mid; lo = mid + 1; } else hi = mid - 1;
      }
    }
    int slot[kMergeEpt];  // >= 0: global slot; < 0: -1 - kept index
    uint32_t live = 0;
#pragma unroll
    for (int i = 0; i < kMergeEpt; ++i) {
      const int e = e0 + i;
      slot[i] = 0;
      if (i < ept && e < n) {
        if (e < nkept) {
          slot[i] = -1 - e;
        } else {
          const int gidx = consumed + (e - nkept);
          while (c + 1 < a.n_chunks && off_s[c + 1] <= gidx) ++c;
          slot[i] = c * a.chunk + (gidx - off_s[c]);
        }
        live |= 1u << i;
      }
    }
    unsigned long long x[kMergeEpt];
    int bl[kMergeEpt];
#pragma unroll
    for (int i = 0; i < kMergeEpt; ++i) {
      const int sidx = slot[i] >= 0 ? slot[i] : 0;
      x[i] = src[sidx];
      bl[i] = src_blk[sidx];
    }
#pragma unroll
    for (int i = 0; i < kMergeEpt; ++i) {
      if (slot[i] < 0) {
        x[i] = kept_s[-1 - slot[i]];
        bl[i] = kept_blk_s[-1 - slot[i]];
      }
      if (!((live >> i) & 1u)) x[i] = 0;
    }
    __syncthreads();  // every thread has read kept_s
    uint32_t sel = 0;
    merge_topk(x, live, sel, a.k, sh);
    int tot;
    int off = big_exclusive_scan(__popc(sel), &tot, sh);
#pragma unroll
    for (int i = 0; i < kMergeEpt; ++i)
      if ((sel >> i) & 1u) {
        kept_s[off] = x[i];
        kept_blk_s[off] = bl[i];
        ++off;
      }
    if (tid == 0) nkept_s = tot;
    consumed += take;
    __syncthreads();
  } while (consumed < tot_all);
  const int nk = nkept_s;
  int32_t* out = a.selected + head * a.k;
  int32_t* outb = a.sel_blk + head * a.k;
  for (int i = tid; i < a.k; i += kBigThreads) {
    out[i] = (i < nk) ? (int32_t)(0xffffffffu - (uint32_t)(kept_s[i] & 0xffffffffu)) : -1;
    outb[i] = (i < nk) ? kept_blk_s[i] : -1;
  }
}

// bound and chunk launches of group size G
template <int G>
void launch_first(const locks_dims& d, const WsLayout& L, const SelectArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(select_bound_kernel<G>, dim3(d.n_kv_heads, d.batch), dim3(kBigThreads), 0, s, a);
  hipLaunchKernelGGL(select_chunk_kernel<G>, dim3(L.n_sel_chunks, d.n_kv_heads, d.batch),
                     dim3(kChunkThreads), 0, s, a);
}

}  // namespace

hipError_t launch_select(const locks_dims& d, const WsLayout& L, const DevPtrs& P,
                         const int32_t* pt, const int32_t* sl, int32_t* selected, hipStream_t s) {
  SelectArgs a;
  a.scores = P.scores;
  a.score_part = P.score_part;
  a.page_table = pt;
  a.seq_lens = sl;
  a.Lg = P.Lg;
  a.tlb = P.tlb;
  a.cand = P.cand;
  a.cand_blk = P.cand_blk;
  a.cand_count = P.cand_count;
  a.selected = selected;
  a.sel_blk = P.sel_blk;
  a.Hq = d.n_q_heads;
  a.Hkv = d.n_kv_heads;
  a.N = d.max_pages_per_seq;
  a.num_blocks = d.num_blocks;
  a.k = L.k;
  a.n_ranges = L.n_score_wg;
  a.sup = L.bound_sup;
  a.n_sup = L.bound_n_sup;
  a.chunk = L.sel_chunk;
  a.n_chunks = L.n_sel_chunks;
  switch (d.n_q_heads / d.n_kv_heads) {
    case 1: launch_first<1>(d, L, a, s); break;
    case 2: launch_first<2>(d, L, a, s); break;
    case 4: launch_first<4>(d, L, a, s); break;
    case 8: launch_first<8>(d, L, a, s); break;
    case 16: launch_first<16>(d, L, a, s); break;
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(select_merge_kernel, dim3(d.n_kv_heads, d.batch), dim3(kBigThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace locks
