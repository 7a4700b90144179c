// rank_device.h — exact top-k over the chunk pass's candidate lists of one
// (sequence, KV head): device code shared by the select merge launch and the
// sparse attention launch that ranks its own list.
//
// Top-k (blog post "LOCKS: per-page SVD cuts KV-cache reads 10x at 1M
// context", "Code": keep the budget/16 pages with the largest score, ids
// ascending). A candidate is a 64-bit sort key, the order bits of its page key
// above the complement of its page id, so one integer comparison applies
// "larger key, then lower id"; each chunk list holds its candidates in page
// order, and the ranking keeps that order, so the kept ids come out ascending
// without a sort.
//
// Register path: at most kFastCap candidates, spread over every wave of the
// workgroup. Gathered in one round trip with the list counts when every list
// fits kFastCap/n_lists speculative slots, entry 64 j + lane in lane `lane`
// (so each load instruction reads 64 consecutive slots; page order is (j,
// lane) order, j running over a wave's slots, then the next wave's); else (still at most kFastCap in all) after the counts,
// consecutive entries per lane (lane order is page order).
// Ranked by bucket refinement: a 512-bucket histogram over the live key range
// picks the bucket holding the k-th key; candidates above it are in, below it
// out; repeat inside it until the count fits or every live key is equal, where
// the lowest ids win.
// Workgroup path (any count): a radix select over the lists where they lie
// (in L2), then one pass in page order hands out the kept ones.
#pragma once

#include "device_common.h"

namespace locks {

constexpr int kRankBuckets = 2048;           // workgroup path: digits of up to 11 bits
constexpr int kFastPerLane = 16;
constexpr int kFastCap = 64 * kFastPerLane;  // candidates ranked in registers
// the register path's histogram: kFastBpl buckets per lane (512 in all; at
// most 1024 candidates, 2^9 of range per pass resolves the k-th key in about
// as many passes as 2048 buckets, with a quarter of the LDS clears and reads)
constexpr int kFastBpl = 8;
constexpr int kFastBuckets = 64 * kFastBpl;

// LDS slot of register-path bucket bk, lane l owning buckets [kFastBpl l, +kFastBpl):
// lane-major, so the lanes reading their q-th bucket hit different banks
__device__ __forceinline__ uint32_t fast_slot(uint32_t bk) { return ((bk % kFastBpl) << 6) | (bk / kFastBpl); }

// One (sequence, KV head)'s candidate lists: list c holds count[c] sort keys
// (and their physical blocks) at x[c * chunk ...], in page order.
struct CandLists {
  const unsigned long long* x;
  const int32_t* blk;
  const int32_t* count;
  int nc;     // lists, 1..1024
  int chunk;  // slots per list, >= 1024
};

// LDS of the workgroup path for NT threads.
template <int NT>
struct RankLds {
  uint32_t hist[kRankBuckets];
  int off[1025];  // off[c]: first entry of list c in the concatenation; off[nc]: total
  uint32_t red3[3][NT / 64];
  uint32_t scn[NT / 64];
  uint32_t kept[NT / 64];  // register path: kept candidates per wave
  int bstar;
  uint32_t babove;
};

// ------------------------------------------------------------ register path
//
// Every wave of the NT-thread workgroup takes part: wave w holds kFastCap / NT
// candidates per lane (KPL), and page order is wave order, then the order
// within the wave given below. A pass is two workgroup barriers; the
// per-candidate work, most of a pass's instructions, is split over the waves.

// log2 of the speculative slots per list: the largest power of two S with nc S <= kFastCap
__device__ __forceinline__ int fast_lg_slots(int nc) { return 31 - __builtin_clz(max(1, kFastCap / nc)); }

// Register-path loads are split from their use so that a caller issues all
// of them (the counts and the speculative slots) before it consumes any: one
// round trip. Every load is unconditional (indices clamped in range), so no
// branch holds one back.

// Counts of lists lane + 64 i (clamped: read but ignored past nc), in every wave.
__device__ __forceinline__ void fast_count_load(const CandLists& L, int (&cc)[16]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 16; ++i) cc[i] = L.count[min(lane + 64 * i, L.nc - 1)];
}

// Every wave: the candidates in all lists (*total) and whether some list
// holds more than its 2^lgS speculative slots (the same in every wave).
__device__ __forceinline__ bool fast_count_check(const CandLists& L, int lgS, const int (&cc)[16],
                                                 int* total) {
  const int lane = threadIdx.x & 63;
  int t = 0;
  bool over = false;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int v = (lane + 64 * i < L.nc) ? cc[i] : 0;
    t += v;
    over |= v > (1 << lgS);
  }
  *total = (int)wave_sum_u32((uint32_t)t);
  return __ballot(over) != 0;
}

// Speculative gather: entry e = 64 (KPL w + i) + lane (slot i of the lane in
// wave w) is slot e % S of list e / S, S = 2^lgS, with that list's count in
// cof; within a wave page order is (slot, lane) order.
template <int NT>
__device__ __forceinline__ void fast_slots_load(const CandLists& L, int lgS,
                                                unsigned long long (&x)[kFastCap / NT],
                                                int (&bl)[kFastCap / NT], int (&cof)[kFastCap / NT]) {
  constexpr int KPL = kFastCap / NT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int S = 1 << lgS;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int e = 64 * (KPL * wave + i) + lane;
    const int c = e >> lgS, sl = e & (S - 1);
    const int idx = (c < L.nc) ? c * L.chunk + sl : 0;
    x[i] = L.x[idx];
    bl[i] = L.blk[idx];
    cof[i] = L.count[min(c, L.nc - 1)];
  }
}

// The lane's live bits of a speculative gather: slots below their list's count.
template <int NT>
__device__ __forceinline__ uint32_t fast_slots_live(const CandLists& L, int lgS,
                                                    const int (&cof)[kFastCap / NT]) {
  constexpr int KPL = kFastCap / NT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t live = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int e = 64 * (KPL * wave + i) + lane;
    live |= ((e >> lgS) < L.nc && (e & ((1 << lgS) - 1)) < cof[i]) ? 1u << i : 0u;
  }
  return live;
}

// Exact gather of total <= kFastCap candidates when some list overflowed its
// speculative slots: wave 0 writes the list offsets (a wave scan) to off (LDS,
// nc + 1 words), a barrier, then entry e = KPL (64 w + lane) + i < total (lane
// order within a wave is page order: one search per lane, then consecutive
// entries) comes from the list holding it. Every wave calls it; returns the
// lane's live bits (entries below total).
template <int NT>
__device__ __forceinline__ uint32_t fast_gather_exact(const CandLists& L, int* off, int total,
                                                      unsigned long long (&x)[kFastCap / NT],
                                                      int (&bl)[kFastCap / NT]) {
  constexpr int KPL = kFastCap / NT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave == 0) {
    int cc[16];  // lane l: lists [16 l, 16 l + 16)
#pragma unroll
    for (int i = 0; i < 16; ++i) cc[i] = L.count[min(16 * lane + i, L.nc - 1)];  // unconditional
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (16 * lane + i >= L.nc) cc[i] = 0;
      s += (uint32_t)cc[i];
    }
    uint32_t o = wave_incl_scan(s) - s;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = 16 * lane + i;
      if (c < L.nc) off[c] = (int)o;
      o += (uint32_t)cc[i];
    }
    if (lane == 0) off[L.nc] = total;
  }
  __syncthreads();
  const int e0 = KPL * (64 * wave + lane);
  int c = 0;
  if (e0 < total)
    for (int lo = 0, hi = L.nc - 1; lo <= hi;) {  // last list starting at or before e0
      const int mid = (lo + hi) >> 1;
      if (off[mid] <= e0) { c = mid; lo = mid + 1; } else hi = mid - 1;
    }
  uint32_t live = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int e = e0 + i;
    int idx = 0;
    if (e < total) {
      while (off[c + 1] <= e) ++c;
      idx = c * L.chunk + (e - off[c]);
      live |= 1u << i;
    }
    x[i] = L.x[idx];
    bl[i] = L.blk[idx];
  }
  return live;
}

// Lanes below this one whose bit is set in the wave mask m.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The sum over the waves before this one (*before) and over all of them
// (return) of a wave-uniform count, through the NT / 64 words w. One barrier;
// w must not be written again before every wave has passed it.
template <int NT>
__device__ __forceinline__ int waves_prefix(uint32_t v, uint32_t* w, int* before) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) w[wave] = v;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const uint32_t c = w[i];
    pre += (i < wave) ? c : 0u;
    tot += c;
  }
  *before = (int)pre;
  return (int)tot;
}

// Ranks the live candidates and returns the lane's kept bits: the k largest
// sort keys, or every live one if fewer. imajor: page order within a wave is
// (slot, lane) order (the speculative gather), else lane order (the exact
// gather); it decides only which of several equal keys are kept. Every wave
// calls it with the same k; the decisions are workgroup-uniform.
// Each pass: the live count and key range (a barrier), a 512-bucket
// histogram of the live keys over that range (a barrier), read whole by every
// wave, which finds the bucket of the need-th key from the top. The histogram
// is double-buffered in R.hist (kFastBuckets + 64 words each; the last 64 take
// the increments of dead slots, one per lane, so that no branch skips them),
// each pass clearing the next one's buffer.
template <int NT>
__device__ __forceinline__ uint32_t fast_rank(const unsigned long long (&x)[kFastCap / NT], uint32_t live,
                                              int k, bool imajor, RankLds<NT>& R) {
  constexpr int KPL = kFastCap / NT, NW = NT / 64;
  constexpr int kWords = kFastBuckets + 64;
  static_assert(2 * kWords <= kRankBuckets, "two histograms fit R.hist");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int q = tid; q < kFastBuckets; q += NT) R.hist[q] = 0u;  // the first pass's buffer
  uint32_t sel = 0;
  int need = k;
  bool settled = false;  // every kept key found (else the live keys left are all equal)
  for (int iter = 0; iter < 8; ++iter) {
    uint32_t* const hc = R.hist + (iter & 1) * kWords;
    uint32_t* const hn = R.hist + (~iter & 1) * kWords;
    // every step is branch-free over the slots: dead slots take neutral
    // values and a private histogram word
    uint32_t cnt = __popc(live), lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const uint32_t v = (uint32_t)(x[i] >> 32);
      const bool on = (live >> i) & 1u;
      lo = min(lo, on ? v : 0xffffffffu);
      hi = max(hi, on ? v : 0u);
    }
    cnt = wave_sum_u32(cnt);
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    if (lane == 0) { R.red3[0][wave] = cnt; R.red3[1][wave] = lo; R.red3[2][wave] = hi; }
    __syncthreads();
    cnt = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      cnt += R.red3[0][w];
      lo = min(lo, R.red3[1][w]);
      hi = max(hi, R.red3[2][w]);
    }
    if ((int)cnt <= need) { sel |= live; live = 0; settled = true; break; }
    if (lo == hi) break;
    // any positive scale near kFastBuckets / range keeps the bucket map
    // monotone, which is all the selection needs (out-of-range results clamp)
    const float scale = (float)kFastBuckets * __builtin_amdgcn_rcpf((float)(hi - lo) + 1.0f);
    for (int q = tid; q < kFastBuckets; q += NT) hn[q] = 0u;  // read last in the previous pass
    uint32_t bk[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const bool on = (live >> i) & 1u;
      bk[i] = min((uint32_t)(kFastBuckets - 1), (uint32_t)((float)((uint32_t)(x[i] >> 32) - lo) * scale));
      atomicAdd(&hc[on ? fast_slot(bk[i]) : (uint32_t)(kFastBuckets + lane)], 1u);
    }
    __syncthreads();
    uint32_t hb[kFastBpl];
    uint32_t mine = 0;
#pragma unroll
    for (int q = 0; q < kFastBpl; ++q) {
      hb[q] = hc[(q << 6) | lane];
      mine += hb[q];
    }
    const uint32_t pre = wave_incl_scan(mine);
    const uint32_t tot = __builtin_amdgcn_readlane(pre, 63);
    uint32_t acc = tot - pre;
    int bstar = -1;
    uint32_t above = 0, inb = 0;
#pragma unroll
    for (int q = kFastBpl - 1; q >= 0; --q) {
      if (acc < (uint32_t)need && (uint32_t)need <= acc + hb[q]) {
        bstar = kFastBpl * lane + q;
        above = acc;
        inb = hb[q];
      }
      acc += hb[q];
    }
    const uint64_t owner = __ballot(bstar >= 0);
    if (owner == 0) break;  // unreachable: some bucket holds the need-th key
    const int srcl = __builtin_ctzll(owner);
    const uint32_t bs = (uint32_t)__builtin_amdgcn_readlane(bstar, srcl);
    above = __builtin_amdgcn_readlane(above, srcl);
    inb = __builtin_amdgcn_readlane(inb, srcl);
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      gt |= bk[i] > bs ? 1u << i : 0u;
      eq |= bk[i] == bs ? 1u << i : 0u;
    }
    need -= (int)above;
    if ((int)inb == need) {  // the bucket is exactly the rest: all of it is in, no further pass
      sel |= live & (gt | eq);
      live = 0;
      settled = true;
      break;
    }
    sel |= live & gt;
    live &= eq;
  }
  if (!settled) {  // workgroup-uniform
    // live keys all equal (or, unreachably, out of passes): the earliest
    // (lowest page ids) win
    int before;
    waves_prefix<NT>(wave_sum_u32(__popc(live)), R.scn, &before);
    if (imajor) {
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        const uint64_t m = __ballot((live >> i) & 1u);
        if (((live >> i) & 1u) && before + lanes_below(m) < need) sel |= 1u << i;
        before += __popcll(m);
      }
    } else {
      const uint32_t nl = __popc(live);
      before += (int)(wave_incl_scan(nl) - nl);
#pragma unroll
      for (int i = 0; i < KPL; ++i)
        if ((live >> i) & 1u) {
          if (before < need) sel |= 1u << i;
          ++before;
        }
    }
  }
  return sel;
}

// Hands out the kept candidates whose positions in the kept list (page
// order; imajor as for fast_rank) fall in [w0, w1): emit(pos, page id,
// block), and emit(pos, -1, -1) for the positions of [w0, w1) from the kept
// count up to k. Every wave calls it (one barrier).
template <int NT, class Emit>
__device__ __forceinline__ void fast_emit(const unsigned long long (&x)[kFastCap / NT],
                                          const int (&bl)[kFastCap / NT], uint32_t sel, int k, bool imajor,
                                          int w0, int w1, RankLds<NT>& R, Emit&& emit) {
  constexpr int KPL = kFastCap / NT;
  auto id_of = [](unsigned long long v) { return (int)(0xffffffffu - (uint32_t)(v & 0xffffffffu)); };
  int base;
  const int nk = waves_prefix<NT>(wave_sum_u32(__popc(sel)), R.kept, &base);
  if (imajor) {
    // slot i of every lane is one run of the list: a ballot places it
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const uint64_t m = __ballot((sel >> i) & 1u);
      const int n = __popcll(m);
      if (base < w1 && base + n > w0 && ((sel >> i) & 1u)) {
        const int pos = base + lanes_below(m);
        if (pos >= w0 && pos < w1) emit(pos, id_of(x[i]), bl[i]);
      }
      base += n;
    }
  } else {
    const uint32_t ns = __popc(sel);
    int o = base + (int)(wave_incl_scan(ns) - ns);
    if (o < w1 && o + (int)ns > w0) {
#pragma unroll
      for (int i = 0; i < KPL; ++i)
        if ((sel >> i) & 1u) {
          if (o >= w0 && o < w1) emit(o, id_of(x[i]), bl[i]);
          ++o;
        }
    }
  }
  for (int i = max(nk, w0) + (int)threadIdx.x; i < min(k, w1); i += NT) emit(i, -1, -1);
}

// ----------------------------------------------------------- workgroup path

// Exclusive prefix sum over the NT threads (thread order) of one u32; *total
// gets the workgroup total. One barrier; scn is free again after the next.
template <int NT>
__device__ __forceinline__ uint32_t rank_excl_scan(uint32_t v, uint32_t* scn, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) scn[wave] = inc;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t c = scn[w];
    pre += (w < wave) ? c : 0u;
    tot += c;
  }
  *total = tot;
  return pre + inc - v;
}

// R.off of the lists (1024 / NT counts per thread). Ends with a barrier.
template <int NT>
__device__ __forceinline__ void rank_list_offsets(RankLds<NT>& R, const CandLists& L) {
  constexpr int CPT = 1024 / NT;
  static_assert(CPT * NT == 1024, "thread count divides the list limit");
  const int tid = threadIdx.x;
  uint32_t c[CPT], s = 0;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int ci = CPT * tid + i;
    c[i] = (ci < L.nc) ? (uint32_t)L.count[ci] : 0u;
    s += c[i];
  }
  uint32_t total;
  uint32_t o = rank_excl_scan<NT>(s, R.scn, &total);
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int ci = CPT * tid + i;
    if (ci < L.nc) R.off[ci] = (int)o;
    o += c[i];
  }
  if (tid == 0) R.off[L.nc] = (int)total;
  __syncthreads();
}

// 2: above, 1: live, 0: out, for `plen` fixed high bits equal to `prefix`
__device__ __forceinline__ int global_class(uint32_t u, int plen, uint32_t prefix) {
  if (plen == 0) return 1;
  const uint32_t h = u >> (32 - plen);
  return h > prefix ? 2 : (h == prefix ? 1 : 0);
}

// Calls f(u) for the order bits of every candidate of this thread's
// contiguous slice of the concatenated lists, 8 loads in flight at a time.
template <int NT, class F>
__device__ __forceinline__ void rank_for_each(const RankLds<NT>& R, const CandLists& L, int total, F&& f) {
  const int per = (total + NT - 1) / NT;
  const int e_begin = min(total, (int)threadIdx.x * per), e_end = min(total, e_begin + per);
  int c = 0;
  if (e_begin < e_end)
    for (int lo = 0, hi = L.nc - 1; lo <= hi;) {
      const int mid = (lo + hi) >> 1;
      if (R.off[mid] <= e_begin) { c = mid; lo = mid + 1; } else hi = mid - 1;
    }
  for (int e = e_begin; e < e_end; e += 8) {
    int idx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      idx[i] = 0;
      if (e + i < e_end) {
        while (R.off[c + 1] <= e + i) ++c;
        idx[i] = c * L.chunk + (e + i - R.off[c]);
      }
    }
    uint32_t u[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) u[i] = (uint32_t)(L.x[idx[i]] >> 32);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (e + i < e_end) f(u[i]);
  }
}


// Radix select over every candidate where it lies: after the high bits all
// candidates share, digits of up to 11 bits of the key's 32 order bits, one
// histogram pass each; a candidate whose fixed high bits (prefix) exceed the
// chosen ones is kept, equal is live, lower is out; live ones left when all 32
// bits are fixed have equal keys, and the earliest (lowest page ids) take the
// remaining places. Then one pass in page order calls emit(pos, page id,
// block) for the kept ones and emit(pos, -1, -1) up to k. Every thread of the
// workgroup calls it. Not inlined: the register path around it keeps its own
// allocation.
template <int NT, class Emit>
__device__ __attribute__((noinline)) void rank_global(RankLds<NT>& R, const CandLists L, int k, Emit emit) {
  constexpr int NW = NT / 64;
  constexpr int BPT = kRankBuckets / NT;  // histogram buckets per thread
  // consecutive candidates per thread per output batch (8 below 512 threads:
  // the register allocation of a 256-thread caller stays under 128)
  constexpr int kGlobalEpt = NT >= 512 ? 16 : 8;
  const int tid = threadIdx.x;
  rank_list_offsets<NT>(R, L);
  const int total = R.off[L.nc];

  // the high bits every candidate shares are fixed at once (their keys lie
  // in a narrow range: a first digit over them would put nearly all into one
  // bucket, one LDS address)
  uint32_t mn = 0xffffffffu, mx = 0u;
  rank_for_each<NT>(R, L, total, [&](uint32_t u) {
    mn = min(mn, u);
    mx = max(mx, u);
  });
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  if ((tid & 63) == 0) { R.red3[1][tid >> 6] = mn; R.red3[2][tid >> 6] = mx; }
  __syncthreads();
  mn = 0xffffffffu;
  mx = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mn = min(mn, R.red3[1][w]);
    mx = max(mx, R.red3[2][w]);
  }
  __syncthreads();  // R.red3 free again
  int plen = (mn == mx) ? 32 : __builtin_clz(mn ^ mx);
  uint32_t prefix = (plen == 0) ? 0u : (plen == 32 ? mn : mn >> (32 - plen));
  int need = k;
  bool all_live = false;  // the live set is exactly the `need` still to take
  for (int level = 0; level < 3 && plen < 32; ++level) {
    const int width = min(11, 32 - plen), shift = 32 - plen - width;
#pragma unroll
    for (int q = 0; q < BPT; ++q) R.hist[BPT * tid + q] = 0u;
    __syncthreads();
    rank_for_each<NT>(R, L, total, [&](uint32_t u) {
      if (global_class(u, plen, prefix) == 1) atomicAdd(&R.hist[(u >> shift) & ((1u << width) - 1u)], 1u);
    });
    __syncthreads();
    // the digit holding the need-th live key, from the top
    uint32_t hb[BPT], mine = 0;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      hb[q] = R.hist[BPT * tid + q];
      mine += hb[q];
    }
    uint32_t tot;
    const uint32_t pre = rank_excl_scan<NT>(mine, R.scn, &tot);
    uint32_t acc = tot - pre - mine;
#pragma unroll
    for (int q = BPT - 1; q >= 0; --q) {
      if (acc < (uint32_t)need && (uint32_t)need <= acc + hb[q]) {
        R.bstar = BPT * tid + q;
        R.babove = acc;
        R.red3[0][0] = hb[q];
      }
      acc += hb[q];
    }
    __syncthreads();
    prefix = (prefix << width) | (uint32_t)R.bstar;
    plen += width;
    need -= (int)R.babove;
    const uint32_t in_digit = R.red3[0][0];
    __syncthreads();  // hist, bstar, red3 free again
    if ((int)in_digit == need) { all_live = true; break; }
  }

  // ---- output pass in page order: above, then live ones while `need` lasts
  int nsel = 0, nlive = 0;
  for (int base = 0; base < total; base += NT * kGlobalEpt) {
    const int e0 = base + tid * kGlobalEpt;
    int c = 0;
    if (e0 < total)
      for (int lo = 0, hi = L.nc - 1; lo <= hi;) {
        const int mid = (lo + hi) >> 1;
        if (R.off[mid] <= e0) { c = mid; lo = mid + 1; } else hi = mid - 1;
      }
    unsigned long long xv[kGlobalEpt];
    int bv[kGlobalEpt], cls[kGlobalEpt];
    uint32_t nl = 0;
#pragma unroll
    for (int i = 0; i < kGlobalEpt; ++i) {
      const int e = e0 + i;
      int sidx = 0;
      if (e < total) {
        while (R.off[c + 1] <= e) ++c;
        sidx = c * L.chunk + (e - R.off[c]);
      }
      xv[i] = L.x[sidx];
      bv[i] = L.blk[sidx];
      cls[i] = (e < total) ? global_class((uint32_t)(xv[i] >> 32), plen, prefix) : 0;
      nl += cls[i] == 1 ? 1u : 0u;
    }
    uint32_t live_tot;
    uint32_t lrank = (uint32_t)nlive + rank_excl_scan<NT>(nl, R.scn, &live_tot);
    uint32_t ns = 0;
#pragma unroll
    for (int i = 0; i < kGlobalEpt; ++i) {
      if (cls[i] == 1) {
        if (!all_live && lrank >= (uint32_t)need) cls[i] = 0;
        ++lrank;
      }
      ns += cls[i] != 0 ? 1u : 0u;
    }
    __syncthreads();  // R.scn read by every thread before it is reused
    uint32_t sel_tot;
    uint32_t pos = (uint32_t)nsel + rank_excl_scan<NT>(ns, R.scn, &sel_tot);
#pragma unroll
    for (int i = 0; i < kGlobalEpt; ++i)
      if (cls[i] != 0) {
        if (pos < (uint32_t)k) emit((int)pos, (int)(0xffffffffu - (uint32_t)(xv[i] & 0xffffffffu)), bv[i]);
        ++pos;
      }
    nlive += (int)live_tot;
    nsel += (int)sel_tot;
    __syncthreads();
  }
  for (int i = nsel + tid; i < k; i += NT) emit(i, -1, -1);
}

}  // namespace locks
