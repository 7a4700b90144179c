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
//  1. grid (chunk, KV head, sequence): every workgroup forms the keys of one
//     chunk of <= 1024 pages as 64-bit sort keys (order-preserving key bits
//     << 32 | ~page id, so one integer comparison applies "larger key, then
//     lower id") and keeps those at or above a lower bound on the k-th largest
//     key. The bound comes from the scoring pass's per-range maxima: every
//     64-page range holds a page whose key is at least
//     max_g(range max of s_hat_g - L_g) - log2 G, so the k-th largest of these
//     bounds cannot exceed the k-th largest key. Survivors are written in
//     page order (typically about k of them in total, not k per chunk).
//  2. one workgroup per (sequence, KV head) streams over the chunk lists in
//     page order, 8192 candidates per round, carrying the running top-k, and
//     writes the ids; kept candidates always precede the new ones in page
//     order, so the result comes out sorted without a sort. (A separate launch
//     instead of a last-workgroup merge: on this chip a device-scope release
//     from every workgroup costs an L2 write-back each.)
// Ranking = exact selection by bucket refinement on the key bits: a 256-bucket
// histogram over the live [lo, hi] key range picks the bucket holding the
// k-th key; everything above it is in, below it out; repeat inside that
// bucket (range shrinks ~256x per pass) until the count fits or all live keys
// are equal, where the lowest ids win.
#include "device_common.h"
#include "internal.h"

namespace locks {

namespace {

constexpr int kThreads = 256;
constexpr int kEpt = kSelectMaxElems / kThreads;  // 32 elements per thread at most (merge)
constexpr int kEpt1 = kSelectChunk / kThreads;     // 4 pages per thread (chunk pass)

struct SelectArgs {
  const float* scores;
  const float* score_part;
  const int32_t* seq_lens;
  unsigned long long* cand;
  int32_t* cand_count;
  int32_t* selected;
  int Hq, Hkv, N, k, n_score_wg, chunk, n_chunks;
};

struct TopkShared {
  uint32_t hist[256];
  uint32_t red[3][4];
  int scan[4];
  uint32_t bstar, above;
};

__device__ __forceinline__ uint32_t key_order_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // monotone in f
}

// Block-wide sum, min and max of three u32 values (all threads get the result).
__device__ void block_reduce3(uint32_t& sum, uint32_t& mn, uint32_t& mx, TopkShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    sum += __shfl_xor(sum, o);
    mn = min(mn, (uint32_t)__shfl_xor(mn, o));
    mx = max(mx, (uint32_t)__shfl_xor(mx, o));
  }
  if (lane == 0) {
    sh.red[0][wave] = sum;
    sh.red[1][wave] = mn;
    sh.red[2][wave] = mx;
  }
  __syncthreads();
  sum = sh.red[0][0] + sh.red[0][1] + sh.red[0][2] + sh.red[0][3];
  mn = min(min(sh.red[1][0], sh.red[1][1]), min(sh.red[1][2], sh.red[1][3]));
  mx = max(max(sh.red[2][0], sh.red[2][1]), max(sh.red[2][2], sh.red[2][3]));
  __syncthreads();
}

// Exclusive prefix over threads (thread order = element order); returns the
// offset of this thread and the block total in *total.
__device__ int block_exclusive_scan(int v, int* total, TopkShared& sh) {
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
  for (int w = 0; w < 4; ++w) {
    const int c = sh.scan[w];
    if (w < wave) before += c;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return before + incl - v;
}

// Marks (in `sel`) the `need` largest of the live elements (`live` bits) of
// x[0..ept) across the block; element order is thread-major.
__device__ void block_topk(const unsigned long long* x, int ept, uint32_t live, uint32_t& sel,
                           int need, TopkShared& sh) {
  for (int iter = 0; iter < 40; ++iter) {
    uint32_t cnt = __popc(live), lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int i = 0; i < kEpt; ++i) {
      if (i < ept && ((live >> i) & 1u)) {
        const uint32_t v = (uint32_t)(x[i] >> 32);
        lo = min(lo, v);
        hi = max(hi, v);
      }
    }
    block_reduce3(cnt, lo, hi, sh);
    if ((int)cnt <= need) { sel |= live; return; }
    if (need <= 0) return;
    if (lo == hi) {
      // all live keys equal: the lowest page ids (earliest elements) win
      int tot;
      int off = block_exclusive_scan(__popc(live), &tot, sh);
#pragma unroll
      for (int i = 0; i < kEpt; ++i)
        if (i < ept && ((live >> i) & 1u)) {
          if (off < need) sel |= 1u << i;
          ++off;
        }
      return;
    }
    // 256 buckets over [lo, hi]; lo -> 0 and hi -> >= 128, so every pass makes progress
    const float scale = 256.0f / ((float)(hi - lo) + 1.0f);
    for (int i = threadIdx.x; i < 256; i += kThreads) sh.hist[i] = 0;
    __syncthreads();
    uint32_t bk[kEpt];
#pragma unroll
    for (int i = 0; i < kEpt; ++i) {
      bk[i] = 0;
      if (i < ept && ((live >> i) & 1u)) {
        const uint32_t v = (uint32_t)(x[i] >> 32);
        bk[i] = min(255u, (uint32_t)((float)(v - lo) * scale));
        atomicAdd(&sh.hist[bk[i]], 1u);
      }
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      const int l = threadIdx.x;
      const uint32_t h0 = sh.hist[4 * l], h1 = sh.hist[4 * l + 1], h2 = sh.hist[4 * l + 2],
                     h3 = sh.hist[4 * l + 3];
      const uint32_t mine = h0 + h1 + h2 + h3;
      // suffix sum over lanes above this one
      uint32_t incl = mine;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_down(incl, o);
        if (l + o < 64) incl += y;
      }
      const uint32_t above_lane = incl - mine;  // buckets > 4l+3
      const uint32_t hb[4] = {h0, h1, h2, h3};
      uint32_t acc = above_lane;
#pragma unroll
      for (int q = 3; q >= 0; --q) {
        if (acc < (uint32_t)need && (uint32_t)need <= acc + hb[q]) {
          sh.bstar = 4 * l + q;
          sh.above = acc;
        }
        acc += hb[q];
      }
    }
    __syncthreads();
    const uint32_t bstar = sh.bstar, above = sh.above;
#pragma unroll
    for (int i = 0; i < kEpt; ++i) {
      if (i < ept && ((live >> i) & 1u)) {
        if (bk[i] > bstar) sel |= 1u << i;
        if (bk[i] != bstar) live &= ~(1u << i);
      }
    }
    need -= (int)above;
    __syncthreads();
  }
  // unreachable for 32-bit keys (the range shrinks every pass); keep it total
  int tot;
  int off = block_exclusive_scan(__popc(live), &tot, sh);
#pragma unroll
  for (int i = 0; i < kEpt; ++i)
    if (i < ept && ((live >> i) & 1u)) {
      if (off < need) sel |= 1u << i;
      ++off;
    }
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

__global__ __launch_bounds__(256) void select_kernel(SelectArgs a) {
  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.Hq / a.Hkv;
  const int N = a.N;
  const int nr = a.n_score_wg;
  const int n_b = full_pages(a.seq_lens, b, N);
  __shared__ float L_s[kMaxGroup];
  __shared__ float red_s[4][kMaxGroup][2];
  __shared__ TopkShared sh;
  const float* part = a.score_part + ((size_t)b * a.Hq + (size_t)kvh * G) * nr * 2;  // [g][range][2]

  // ---- every head's total mass L_g (base 2) from the per-range partials
  float lm[kMaxGroup], ls[kMaxGroup];
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) { lm[g] = -1e30f; ls[g] = 0.f; }
  for (int r = tid; r < nr; r += kThreads) {
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g)
      if (g < G) {
        const float m = part[((size_t)g * nr + r) * 2], sv = part[((size_t)g * nr + r) * 2 + 1];
        lse2_acc(lm[g], ls[g], sv > 0.f ? m : -1e30f, sv);
      }
  }
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g)
    if (g < G) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) lse2_acc(lm[g], ls[g], __shfl_xor(lm[g], o), __shfl_xor(ls[g], o));
      if (lane == 0) { red_s[wave][g][0] = lm[g]; red_s[wave][g][1] = ls[g]; }
    }
  __syncthreads();
  if (tid < G) {
    float m = red_s[0][tid][0], sv = red_s[0][tid][1];
    for (int w = 1; w < 4; ++w) lse2_acc(m, sv, red_s[w][tid][0], red_s[w][tid][1]);
    L_s[tid] = (sv > 0.f) ? m + fast_log2(sv) : -INFINITY;
  }
  __syncthreads();

  // ---- lower bound on the k-th largest key: range r holds a page whose key is
  // at least max_g(m_rg - L_g) - log2 G, so the k-th largest of these bounds
  // (over distinct ranges) is at most the k-th largest key
  const float log2G = log2f((float)G);
  float tlb = -INFINITY;
  {
    uint32_t cnt = 0, lo = 0xffffffffu, hi = 0u;
    for (int r = tid; r < nr; r += kThreads) {
      float v = -INFINITY;
      for (int g = 0; g < G; ++g) v = fmaxf(v, part[((size_t)g * nr + r) * 2] - L_s[g]);
      if (v > -INFINITY) {
        const uint32_t u = key_order_bits(v - log2G);
        ++cnt;
        lo = min(lo, u);
        hi = max(hi, u);
      }
    }
    block_reduce3(cnt, lo, hi, sh);
    if ((int)cnt >= a.k) {
      uint32_t best = lo;
      if (hi > lo) {
        const float scale = 256.0f / ((float)(hi - lo) + 1.0f);
        for (int i = tid; i < 256; i += kThreads) sh.hist[i] = 0;
        __syncthreads();
        for (int r = tid; r < nr; r += kThreads) {
          float v = -INFINITY;
          for (int g = 0; g < G; ++g) v = fmaxf(v, part[((size_t)g * nr + r) * 2] - L_s[g]);
          if (v > -INFINITY)
            atomicAdd(&sh.hist[min(255u, (uint32_t)((float)(key_order_bits(v - log2G) - lo) * scale))], 1u);
        }
        __syncthreads();
        if (tid < 64) {  // bucket holding the k-th largest bound
          const uint32_t h0 = sh.hist[4 * tid], h1 = sh.hist[4 * tid + 1], h2 = sh.hist[4 * tid + 2],
                         h3 = sh.hist[4 * tid + 3];
          const uint32_t mine = h0 + h1 + h2 + h3;
          uint32_t incl = mine;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_down(incl, o);
            if (tid + o < 64) incl += y;
          }
          const uint32_t hb[4] = {h0, h1, h2, h3};
          uint32_t acc = incl - mine;
#pragma unroll
          for (int q = 3; q >= 0; --q) {
            if (acc < (uint32_t)a.k && (uint32_t)a.k <= acc + hb[q]) sh.bstar = 4 * tid + q;
            acc += hb[q];
          }
        }
        __syncthreads();
        const uint32_t bstar = sh.bstar;
        // the smallest bound in buckets >= b*: at least k bounds are >= it
        uint32_t c2 = 0, mn = 0xffffffffu, mx = 0u;
        for (int r = tid; r < nr; r += kThreads) {
          float v = -INFINITY;
          for (int g = 0; g < G; ++g) v = fmaxf(v, part[((size_t)g * nr + r) * 2] - L_s[g]);
          if (v > -INFINITY) {
            const uint32_t u = key_order_bits(v - log2G);
            if (min(255u, (uint32_t)((float)(u - lo) * scale)) >= bstar) mn = min(mn, u);
          }
        }
        block_reduce3(c2, mn, mx, sh);
        best = mn;
      }
      // margin for fp32 rounding between these bounds and the keys recomputed below
      tlb = key_from_order_bits(best) - 1e-3f;
    }
  }

  // ---- keys of this chunk: thread t owns pages chunk*M + t*ept + [0, ept), ept <= 4
  const int ept = a.chunk / kThreads;
  const int p0 = chunk * a.chunk + tid * ept;
  float km[kEpt1], ks[kEpt1];
#pragma unroll
  for (int i = 0; i < kEpt1; ++i) { km[i] = -1e30f; ks[i] = 0.f; }
  for (int g = 0; g < G; ++g) {
    const float* srow = a.scores + ((size_t)b * a.Hq + (size_t)kvh * G + g) * N;
#pragma unroll
    for (int i = 0; i < kEpt1; ++i)
      if (i < ept && p0 + i < n_b) lse2_acc(km[i], ks[i], srow[p0 + i] * kLog2e - L_s[g], 1.0f);
  }
  unsigned long long x[kEpt1];
  int nlive = 0;
#pragma unroll
  for (int i = 0; i < kEpt1; ++i) {
    x[i] = 0;
    // log2 of the summed shares, then the group mean; absent pages score -inf
    const float key2 = (i < ept && p0 + i < n_b && ks[i] > 0.f && km[i] > -1e29f)
                           ? km[i] + fast_log2(ks[i]) - log2G : -INFINITY;
    if (key2 > -INFINITY && key2 >= tlb) {
      const uint32_t j = (uint32_t)(p0 + i);
      x[i] = ((unsigned long long)key_order_bits(key2) << 32) | (unsigned long long)(0xffffffffu - j);
      ++nlive;
    }
  }
  int tot;
  int off = block_exclusive_scan(nlive, &tot, sh);
  unsigned long long* dst = a.cand + ((size_t)(b * a.Hkv + kvh) * a.n_chunks + chunk) * a.chunk;
#pragma unroll
  for (int i = 0; i < kEpt1; ++i)
    if (x[i] != 0) dst[off++] = x[i];
  if (tid == 0) a.cand_count[(size_t)(b * a.Hkv + kvh) * a.n_chunks + chunk] = tot;
}

// Level 2: one workgroup per (sequence, KV head) streams over the chunk lists.
__global__ __launch_bounds__(256) void select_merge_kernel(SelectArgs a) {
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  __shared__ TopkShared sh;
  __shared__ int off_s[1025];
  __shared__ unsigned long long kept_s[kSelectMaxK];
  __shared__ int nkept_s;
  const int* counts = a.cand_count + (size_t)(b * a.Hkv + kvh) * a.n_chunks;
  // offsets of the chunk lists in the concatenation (n_chunks <= 1024)
  int tot_all = 0;
  {
    const int per = (a.n_chunks + kThreads - 1) / kThreads;  // <= 4
    int local = 0;
    for (int i = 0; i < per; ++i) {
      const int c = tid * per + i;
      if (c < a.n_chunks) local += counts[c];
    }
    int off = block_exclusive_scan(local, &tot_all, sh);
    for (int i = 0; i < per; ++i) {
      const int c = tid * per + i;
      if (c < a.n_chunks) {
        off_s[c] = off;
        off += counts[c];
      }
    }
    if (tid == 0) { off_s[a.n_chunks] = tot_all; nkept_s = 0; }
  }
  __syncthreads();
  const unsigned long long* src = a.cand + (size_t)(b * a.Hkv + kvh) * a.n_chunks * a.chunk;
  // rounds: [kept (earlier pages) | next candidates in page order], <= 8192 per round
  int consumed = 0;
  do {
    const int nkept = nkept_s;
    const int take = min(tot_all - consumed, kSelectMaxElems - nkept);
    const int n = nkept + take;
    const int ept = (n + kThreads - 1) / kThreads;  // <= 32
    unsigned long long x[kEpt];
    uint32_t live = 0;
    const int e0 = tid * ept;
    int c = 0;  // chunk of candidate (consumed + e0 - nkept)
    {
      const int g0 = consumed + max(0, e0 - nkept);
      for (int lo = 0, hi = a.n_chunks - 1; lo <= hi;) {
        const int mid = (lo + hi) >> 1;
        if (off_s[mid] <= g0) { c = mid; lo = mid + 1; } else hi = mid - 1;
      }
    }
#pragma unroll
    for (int i = 0; i < kEpt; ++i) {
      x[i] = 0;
      const int e = e0 + i;
      if (i < ept && e < n) {
        if (e < nkept) {
          x[i] = kept_s[e];
        } else {
          const int gidx = consumed + (e - nkept);
          while (c + 1 < a.n_chunks && off_s[c + 1] <= gidx) ++c;
          x[i] = src[(size_t)c * a.chunk + (gidx - off_s[c])];
        }
        live |= 1u << i;
      }
    }
    __syncthreads();  // every thread has read kept_s
    uint32_t sel = 0;
    block_topk(x, ept, live, sel, a.k, sh);
    int tot;
    int off = block_exclusive_scan(__popc(sel), &tot, sh);
#pragma unroll
    for (int i = 0; i < kEpt; ++i)
      if ((sel >> i) & 1u) kept_s[off++] = x[i];
    if (tid == 0) nkept_s = tot;
    consumed += take;
    __syncthreads();
  } while (consumed < tot_all);
  const int nk = nkept_s;
  int32_t* out = a.selected + (size_t)(b * a.Hkv + kvh) * a.k;
  for (int i = tid; i < a.k; i += kThreads)
    out[i] = (i < nk) ? (int32_t)(0xffffffffu - (uint32_t)(kept_s[i] & 0xffffffffu)) : -1;
}

}  // namespace

hipError_t launch_select(const locks_dims& d, const WsLayout& L, const DevPtrs& P,
                         const int32_t* pt, const int32_t* sl, int32_t* selected, hipStream_t s) {
  SelectArgs a;
  a.scores = P.scores;
  a.score_part = P.score_part;
  (void)pt;
  a.seq_lens = sl;
  a.cand = P.cand;
  a.cand_count = P.cand_count;
  a.selected = selected;
  a.Hq = d.n_q_heads;
  a.Hkv = d.n_kv_heads;
  a.N = d.max_pages_per_seq;
  a.k = L.k;
  a.n_score_wg = L.n_score_wg;
  a.chunk = L.sel_chunk;
  a.n_chunks = L.n_sel_chunks;
  hipLaunchKernelGGL(select_kernel, dim3(L.n_sel_chunks, d.n_kv_heads, d.batch), dim3(kThreads), 0,
                     s, a);
  hipLaunchKernelGGL(select_merge_kernel, dim3(d.n_kv_heads, d.batch), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace locks
