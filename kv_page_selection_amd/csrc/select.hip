// select.hip — group-shared page selection (gfx950).
//
// Group combine (technical summary, section 2 mechanism 3): each head g of a
// GQA group has total mass L_g = log sum_j exp(s_hat[g][j]) over the
// sequence's pages; a page's key is the log of the group-mean normalised mass
// share, key_j = log((1/G) sum_g exp(s_hat[g][j] - L_g)).
// Top-k (blog post, "Code": keep budget/16 pages with the largest score, ids
// ascending): the k largest keys, ties to the lower page id.
//
// Two levels, no float atomics:
//  1. grid (chunk, KV head, sequence): every workgroup forms the keys of one
//     chunk of pages and keeps the chunk's k best as 64-bit sort keys
//     (order-preserving key bits << 32 | ~page id, so one integer comparison
//     applies "larger key, then lower id");
//  2. the last workgroup of each (sequence, KV head) to finish (device-scope
//     counter) ranks the union of the chunk winners the same way and writes
//     the ids; chunks and in-chunk order are ascending in page id, so the
//     survivors come out sorted without a sort.
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
constexpr int kEpt = kSelectMaxElems / kThreads;  // 32 elements per thread at most

struct SelectArgs {
  const float* scores;
  const float* score_part;
  const int32_t* page_table;
  const int32_t* seq_lens;
  unsigned long long* cand;
  int32_t* cand_count;
  uint32_t* counters;
  int32_t* selected;
  int Hq, Hkv, N, num_blocks, k, n_score_wg, chunk, n_chunks, slots;
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

__global__ __launch_bounds__(256) void select_kernel(SelectArgs a) {
  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.Hq / a.Hkv;
  const int N = a.N;
  const int n_b = full_pages(a.seq_lens, b, N);
  __shared__ float L_s[kMaxGroup];
  __shared__ TopkShared sh;
  __shared__ int last_s;
  __shared__ int off_s[1024];

  // ---- every head's total mass L_g (log2 units) from the score partials
  for (int g = wave; g < G; g += 4) {
    const float* part = a.score_part + ((size_t)b * a.Hq + (size_t)kvh * G + g) * a.n_score_wg * 2;
    float m = -INFINITY, s = 0.f;
    for (int i = lane; i < a.n_score_wg; i += 64) lse2_merge(m, s, part[2 * i], part[2 * i + 1]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
      lse2_merge(m, s, m2, s2);
    }
    if (lane == 0) L_s[g] = (m == -INFINITY) ? -INFINITY : m + log2f(s);
  }
  __syncthreads();

  // ---- keys of this chunk: thread t owns pages chunk*M + t*ept + [0, ept)
  const int ept = a.chunk / kThreads;
  const int p0 = chunk * a.chunk + tid * ept;
  const float log2G = log2f((float)G);
  unsigned long long x[kEpt];
  uint32_t live = 0;
#pragma unroll
  for (int i = 0; i < kEpt; ++i) {
    x[i] = 0;
    if (i < ept) {
      const int j = p0 + i;
      if (j < n_b) {
        const int blk = a.page_table[(size_t)b * N + j];
        if (blk >= 0 && blk < a.num_blocks) {
          // log2 of the summed shares, then the group mean
          float m = -INFINITY, s = 0.f;
          for (int g = 0; g < G; ++g) {
            const float sg = a.scores[((size_t)b * a.Hq + (size_t)kvh * G + g) * N + j] * kLog2e;
            lse2_merge(m, s, sg - L_s[g], 1.0f);
          }
          if (m != -INFINITY) {
            const float key2 = m + log2f(s) - log2G;
            x[i] = ((unsigned long long)key_order_bits(key2) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)j);
            live |= 1u << i;
          }
        }
      }
    }
  }
  uint32_t sel = 0;
  block_topk(x, ept, live, sel, a.k, sh);
  {
    int tot;
    int off = block_exclusive_scan(__popc(sel), &tot, sh);
    unsigned long long* dst = a.cand + ((size_t)(b * a.Hkv + kvh) * a.n_chunks + chunk) * a.slots;
#pragma unroll
    for (int i = 0; i < kEpt; ++i)
      if ((sel >> i) & 1u) dst[off++] = x[i];
    if (tid == 0) a.cand_count[(size_t)(b * a.Hkv + kvh) * a.n_chunks + chunk] = tot;
  }

  // ---- the last chunk of this (sequence, KV head) merges
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = atomicAdd(&a.counters[b * a.Hkv + kvh], 1u);
    last_s = (prev == (uint32_t)(a.n_chunks - 1));
  }
  __syncthreads();
  if (!last_s) return;
  __threadfence();

  // compact offsets of the chunk lists (n_chunks <= 1024)
  const int* counts = a.cand_count + (size_t)(b * a.Hkv + kvh) * a.n_chunks;
  int tot_all = 0;
  {
    const int per = (a.n_chunks + kThreads - 1) / kThreads;  // <= 4
    int local = 0;
    for (int i = 0; i < per; ++i) {
      const int c = tid * per + i;
      if (c < a.n_chunks) local += __builtin_nontemporal_load(&counts[c]);
    }
    int off = block_exclusive_scan(local, &tot_all, sh);
    for (int i = 0; i < per; ++i) {
      const int c = tid * per + i;
      if (c < a.n_chunks) {
        off_s[c] = off;
        off += __builtin_nontemporal_load(&counts[c]);
      }
    }
  }
  __syncthreads();
  // thread t owns elements [t*ept2, (t+1)*ept2) of the concatenated lists
  const int ept2 = (tot_all + kThreads - 1) / kThreads;  // <= 32
  const unsigned long long* src = a.cand + (size_t)(b * a.Hkv + kvh) * a.n_chunks * a.slots;
  live = 0;
  {
    // locate the chunk of this thread's first element (chunks are few)
    int e0 = tid * ept2;
    int c = 0;
    for (int lo = 0, hi = a.n_chunks - 1; lo <= hi;) {
      const int mid = (lo + hi) >> 1;
      if (off_s[mid] <= e0) { c = mid; lo = mid + 1; } else hi = mid - 1;
    }
#pragma unroll
    for (int i = 0; i < kEpt; ++i) {
      x[i] = 0;
      const int e = e0 + i;
      if (i < ept2 && e < tot_all) {
        while (c + 1 < a.n_chunks && off_s[c + 1] <= e) ++c;
        x[i] = __builtin_nontemporal_load(&src[(size_t)c * a.slots + (e - off_s[c])]);
        live |= 1u << i;
      }
    }
  }
  sel = 0;
  block_topk(x, ept2, live, sel, a.k, sh);
  {
    int tot;
    int off = block_exclusive_scan(__popc(sel), &tot, sh);
    int32_t* out = a.selected + (size_t)(b * a.Hkv + kvh) * a.k;
#pragma unroll
    for (int i = 0; i < kEpt; ++i)
      if ((sel >> i) & 1u) out[off++] = (int32_t)(0xffffffffu - (uint32_t)(x[i] & 0xffffffffu));
    for (int i = tot + tid; i < a.k; i += kThreads) out[i] = -1;
  }
  if (tid == 0) a.counters[b * a.Hkv + kvh] = 0;
}

}  // namespace

hipError_t launch_select(const locks_dims& d, const WsLayout& L, const DevPtrs& P,
                         const int32_t* pt, const int32_t* sl, int32_t* selected, hipStream_t s) {
  SelectArgs a;
  a.scores = P.scores;
  a.score_part = P.score_part;
  a.page_table = pt;
  a.seq_lens = sl;
  a.cand = P.cand;
  a.cand_count = P.cand_count;
  a.counters = P.cnt_select;
  a.selected = selected;
  a.Hq = d.n_q_heads;
  a.Hkv = d.n_kv_heads;
  a.N = d.max_pages_per_seq;
  a.num_blocks = d.num_blocks;
  a.k = L.k;
  a.n_score_wg = L.n_score_wg;
  a.chunk = L.sel_chunk;
  a.n_chunks = L.n_sel_chunks;
  a.slots = L.cand_slots;
  dim3 grid(L.n_sel_chunks, d.n_kv_heads, d.batch);
  hipLaunchKernelGGL(select_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace locks
