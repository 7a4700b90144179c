// score.hip — page scoring from compressed summaries (gfx950).
//
// For every (sequence b, KV head, page j) and each of the G query heads of the
// group, computes the page score of the LOCKS blog post ("How LOCKS works",
// page-score equation; technical summary, section 2 mechanism 2):
//   s_hat = log sum_{i<16} exp((q.mu + (V^T q).c_i) / sqrt(128))
// from the page's summary record alone (no key or value is read).
//
// Mapping. A workgroup is 4 waves of one KV head (and one slice of at most 8
// of its query heads); wave w scores 64 consecutive pages (4 tiles of 16), and
// the waves take 4 consecutive page ranges. The q prologue (fixed-point digits
// of the group's query heads) is split over the 4 waves and shared in LDS.
//
// Stage 1, mu.q and V^T q, on v_mfma_i32_16x16x64_i8, exact: the row operand is
// each query head as a 22-bit fixed-point integer in three signed int8 digits
// (rows = 4 heads x 4 digit slots, the 4th slot zero), the column operand is
// the record's codes as stored (mu bytes; V nibbles widened to 16*code with
// one shift and mask). A lane then holds all three digit sums of one value,
// which it combines in int32 and one fp32 rounding.
// Stage 2, the in-page contraction C p (16 tokens x 8 x G heads), on
// v_mfma_f32_16x16x{32,16}_f16: C codes are exact in f16 and p enters as an
// f16 hi + lo pair (about 22 significant bits); 16/G pages are packed
// block-diagonally along K so one pass fills the 16 output columns. The
// 16-token log-sum-exp is one in-lane step and two cross-row swaps, in base 2.
// The wave keeps its 64 x G scores in LDS; at the end it writes them once and
// leaves, per head, the (max, sum) of exp2 over its pages, which the group
// combine needs for every head's total mass, and the max of each 16-page tile,
// the units of the selection's pruning bound.
//
// Loads. Each wave turns its 64 page-table entries into record offsets once
// (an LDS table); every tile then issues its 13 record loads back to back in
// a fixed order (V rows first) and consumes them in that order, so the first
// MFMAs run while the tail of the tile is still arriving.
#include "device_common.h"
#include "internal.h"

namespace locks {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int kTiles = kScorePagesPerWave / 16;

struct ScoreArgs {
  const float* q;
  const uint8_t* summ;
  const int32_t* page_table;
  const int32_t* seq_lens;
  float* scores;
  float* partials;
  float* tile_max;
  int Hq, Hkv, N, num_blocks, n_ranges, tile_pages;
};

__device__ __forceinline__ int nib_lo(uint32_t x) { return (int)((x << 4) & 0xF0F0F0F0u); }
__device__ __forceinline__ int nib_hi(uint32_t x) { return (int)(x & 0xF0F0F0F0u); }

// Four int8 codes -> four exact f16 values: bias to u = code + 128, place u in
// the mantissa of 1024.0 (0x64uu), subtract 1152 with one packed f16 add.
__device__ __forceinline__ h4 codes_to_h4(uint32_t x) {
  const uint32_t u = x ^ 0x80808080u;
  const h2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  const h2 lo = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) + bias;
  const h2 hi = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) + bias;
  return h4{lo[0], lo[1], hi[0], hi[1]};
}

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Per-wave LDS staging of one 16-page tile.
template <int G>
struct TileLds {
  __align__(16) int8_t c[16][144];      // C codes per page (token-major), padded rows
  __align__(16) _Float16 ph[16][G][8];  // p (scaled by 2^-22) high part, [page][head][k]
  __align__(16) _Float16 pl[16][G][8];  // low part
  __align__(16) _Float16 zero[8];       // masked B operand
  float a[16][G + 1];                   // mu . q (exact integer), [page][head]; column G spare
  float sc[32][2];                      // s_mu, s_V/16 * s_C; rows 16.. take the other lanes' copies
  __align__(16) float out[kScorePagesPerWave][G];  // the wave's page scores, [page][head], base 2
};

template <int G>
struct ScoreLds {
  TileLds<G> w[4];
  union {
    __align__(16) int8_t dig[3][G][kDim];  // q digit planes of the workgroup's heads,
    uint32_t off[4][kScorePagesPerWave];   // then each wave's page record offsets
  } u;
  float esc[16];                           // per head: 2^-e log2(e) / sqrt(128)
};

// GROUP = query heads per KV head; a wave scores G = min(GROUP, 8) of them
// (larger groups are split into slices of 8 heads, one wave each, which share
// the record loads through the cache and fill the stage-2 MFMA columns)
template <int GROUP>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  constexpr int G = GROUP > 8 ? 8 : GROUP;
  constexpr int NS = GROUP / G;           // head slices per KV head
  constexpr int RB = G < 4 ? 1 : G / 4;   // stage-1 row blocks (4 heads each)
  constexpr int PG = 16 / G;              // pages per stage-2 pass
  __shared__ ScoreLds<G> S;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int b = blockIdx.z;
  // workgroup -> (KV head, head slice, 4 page ranges). Slices are the slow
  // grid dimension y = kvh * NS + slice over an x extent padded to a multiple
  // of 8: workgroups are dealt round-robin to the 8 XCDs, so every slice of a
  // range group lands on the XCD (and L2) that fetched its records first.
  const int kvh = blockIdx.y / NS;
  const int slice = blockIdx.y % NS;
  const int range = blockIdx.x * 4 + wave;
  const int hbase = kvh * GROUP + slice * G;  // first query head of this workgroup
  const int N = a.N;
  const int n_b = full_pages(a.seq_lens, b, N);
  TileLds<G>& T = S.w[wave];
  const int p0 = range * kScorePagesPerWave;

  // A range wholly past the sequence's full pages (shorter sequences of a
  // batch) has no work and writes nothing (its partials are never read);
  // the whole workgroup leaves at once when none of its ranges has a page.
  if (blockIdx.x * 4 * kScorePagesPerWave >= n_b) return;  // workgroup-uniform

  // page table of this wave's 64 pages, one entry per lane; issued first, so
  // its latency overlaps the q prologue below
  int myblk = -1;
  {
    const int j = p0 + lane;
    if (range < a.n_ranges && j < n_b) myblk = a.page_table[(size_t)b * N + j];
  }

  // ---- q of the group -> per-head exponent -> three int8 digit planes;
  // wave w converts heads w, w+4, ...
  {
    const float* qg = a.q + ((size_t)b * a.Hq + (size_t)hbase) * kDim;
    for (int h = wave; h < G; h += 4) {
      const float q0 = qg[h * kDim + lane], q1 = qg[h * kDim + 64 + lane];
      const float qm = wave_max(fmaxf(fabsf(q0), fabsf(q1)));
      int e = 0;
      if (qm > 0.f) {
        int E;
        frexpf(qm, &E);
        e = 22 - E;  // max |q| * 2^e in [2^21, 2^22)
      }
      const float qs[2] = {q0, q1};
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int qf = (int)rintf(ldexpf(qs[u], e));
        const int d0 = ((qf + 128) & 255) - 128;
        const int r1 = (qf - d0) / 256;
        const int d1 = ((r1 + 128) & 255) - 128;
        const int d2 = (r1 - d1) / 256;
        S.u.dig[0][h][lane + 64 * u] = (int8_t)d0;
        S.u.dig[1][h][lane + 64 * u] = (int8_t)d1;
        S.u.dig[2][h][lane + 64 * u] = (int8_t)d2;
      }
      if (lane == 0) S.esc[h] = ldexpf(1.0f, -e) * (kLog2e * kInvSqrtD);
    }
  }
  __syncthreads();
  // row operands: lane (row = (head 4rb + row/4, digit row%4), K group kg), d in [32kg+16m, +16)
  v4i aop[RB][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int h = 4 * rb + (row >> 2), dg = row & 3;
#pragma unroll
    for (int m = 0; m < 2; ++m)
      aop[rb][m] = (h < G && dg < 3)
                       ? *reinterpret_cast<const v4i*>(&S.u.dig[dg < 3 ? dg : 0][h < G ? h : 0][32 * kg + 16 * m])
                       : v4i{0, 0, 0, 0};
  }
  __syncthreads();  // digit planes consumed: the space takes the record offsets
  if (range >= a.n_ranges) return;  // whole wave; no workgroup barrier follows
  if (p0 >= n_b) return;            // whole wave: past the sequence's full pages
  if (lane < 8) T.zero[lane] = (_Float16)0.0f;

  // An absent page (past the sequence's full pages, or a table entry out of
  // range) reads block 0's record in its place, so every load is
  // unconditional; its score is replaced by -inf at the end.
  if (myblk < 0 || myblk >= a.num_blocks) myblk = -1;
  const unsigned long long present = __ballot(myblk >= 0);  // bit i: page p0 + i
  // the lane's page record, as an offset from summ in 16-byte units (the
  // library limits num_blocks * n_kv_heads * 49 to 32 bits)
  S.u.off[wave][lane] = (uint32_t)((myblk < 0 ? 0 : myblk) * a.Hkv + kvh) * (uint32_t)(kStride / 16);
  const uint8_t* vbase = a.summ + kVOff + (row & 7) * 64 + kg * 16;  // V row of the lane
  const uint8_t* rbase = a.summ + kg * 32;                           // mu, C slice of the lane

  // stage-2 output column col = (page pc of the pass, head hc)
  const int pc = row / G, hc = row % G;
  const float es = S.esc[hc];

  wave_lds_sync();

  // one tile's records as this lane holds them: V rows (page 2vt + row/8,
  // basis vector row%8), and the mu, C and scales of page row
  struct TileRec {
    uint4 v[8], mu1, mu0, c1, c0;
    uint2 scl;
  };
  // The 13 loads of tile t go out in a pinned order (the order is worth ~5%
  // of the gather rate at 4-head groups): issue_v the 8 V rows, issue_tail
  // the mu, C and scales after them. Offsets come from the wave's LDS table.
  auto issue_v = [&](int t, TileRec& r) {
    uint32_t ov[8];
#pragma unroll
    for (int vt = 0; vt < 8; ++vt) ov[vt] = S.u.off[wave][t * 16 + 2 * vt + (row >> 3)];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int vt = 0; vt < 8; ++vt) {
      r.v[vt] = *reinterpret_cast<const uint4*>(vbase + ((size_t)ov[vt] << 4));
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto issue_tail = [&](int t, TileRec& r) {
    const uint32_t om = S.u.off[wave][t * 16 + row];
    const uint8_t* rec = rbase + ((size_t)om << 4);  // page t*16 + row
    __builtin_amdgcn_sched_barrier(0);
    r.mu1 = *reinterpret_cast<const uint4*>(rec + kMuOff + 16);
    __builtin_amdgcn_sched_barrier(0);
    r.mu0 = *reinterpret_cast<const uint4*>(rec + kMuOff);
    __builtin_amdgcn_sched_barrier(0);
    r.c1 = *reinterpret_cast<const uint4*>(rec + kCOff + 16);
    __builtin_amdgcn_sched_barrier(0);
    r.c0 = *reinterpret_cast<const uint4*>(rec + kCOff);
    __builtin_amdgcn_sched_barrier(0);
    r.scl = *reinterpret_cast<const uint2*>(rec - kg * 32 + kSOff);
    __builtin_amdgcn_sched_barrier(0);
  };

  // With up to 4 heads per wave (little compute per byte), the next tile's V
  // rows are issued as soon as stage 1 has consumed the current ones, so they
  // travel during stage 2; 8-head waves are compute-bound and skip this (the
  // extra registers cost more than the overlap gains).
  constexpr bool kPrefetchV = G <= 4;
  TileRec cur;
  issue_v(0, cur);
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    if (!kPrefetchV && t > 0) issue_v(t, cur);
    issue_tail(t, cur);
    const uint4* vraw = cur.v;
    const uint4 mu0 = cur.mu0, mu1 = cur.mu1, c0 = cur.c0, c1 = cur.c1;
    const uint2 scl = cur.scl;
    // consumed in the order the loads were issued, so work starts on the
    // first records while the rest are still arriving
    // ---- stage 1: V tiles (columns = (page 2vt + row/8, basis vector row%8))
#pragma unroll
    for (int vt = 0; vt < 8; ++vt) {
      const uint4 v = vraw[vt];
      const v4i B0 = {nib_lo(v.x), nib_hi(v.x), nib_lo(v.y), nib_hi(v.y)};
      const v4i B1 = {nib_lo(v.z), nib_hi(v.z), nib_lo(v.w), nib_hi(v.w)};
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        v4i acc = mfma_i8(aop[rb][0], B0, v4i{0, 0, 0, 0});
        acc = mfma_i8(aop[rb][1], B1, acc);
        const int h = 4 * rb + kg;
        // exact integer (|.| < 2^37) -> fp32 -> scaled into f16 range, split hi + lo
        const float x = ((float)(acc[2] * 256 + acc[1]) * 256.0f + (float)acc[0]) * 0x1p-22f;
        const _Float16 xh = (_Float16)x;
        const _Float16 xl = (_Float16)(x - (float)xh);
        if (h < G) {
          T.ph[2 * vt + (row >> 3)][h < G ? h : 0][row & 7] = xh;
          T.pl[2 * vt + (row >> 3)][h < G ? h : 0][row & 7] = xl;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- stage 1: mu tile (columns = the 16 pages); lane (page row, kg) -> head 4rb + kg
    {
      const v4i B0 = {(int)mu0.x, (int)mu0.y, (int)mu0.z, (int)mu0.w};
      const v4i B1 = {(int)mu1.x, (int)mu1.y, (int)mu1.z, (int)mu1.w};
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        v4i acc = mfma_i8(aop[rb][0], B0, v4i{0, 0, 0, 0});
        acc = mfma_i8(aop[rb][1], B1, acc);
        const int h = 4 * rb + kg;
        T.a[row][h < G ? h : G] = (float)(acc[2] * 256 + acc[1]) * 256.0f + (float)acc[0];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    *reinterpret_cast<uint4*>(&T.c[row][kg * 32]) = c0;
    *reinterpret_cast<uint4*>(&T.c[row][kg * 32 + 16]) = c1;
    {
      // every lane stores (lanes kg > 0 into the spare rows), so that the
      // scale load is issued with the others rather than behind a branch
      const int r = kg == 0 ? row : 16 + row;
      T.sc[r][0] = f16bits_to_float(scl.x);
      T.sc[r][1] = f16bits_to_float(scl.x >> 16) * (1.0f / 16.0f) * f16bits_to_float(scl.y);
    }
    if (kPrefetchV && t + 1 < kTiles) issue_v(t + 1, cur);
    wave_lds_sync();

    // ---- stage 2 + LSE, one pass per PG pages
#pragma unroll
    for (int gp = 0; gp < G; ++gp) {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      const int pp = gp * PG + pc;  // tile page of this lane's output column
      if constexpr (PG >= 4) {
        // K = 32 per MFMA = 4 page slots x 8 basis vectors; lane group kg = slot
#pragma unroll
        for (int ch = 0; ch < PG / 4; ++ch) {
          const int slot = 4 * ch + kg;
          const uint2 cw = *reinterpret_cast<const uint2*>(&T.c[gp * PG + slot][row * 8]);
          const h4 c_lo = codes_to_h4(cw.x), c_hi = codes_to_h4(cw.y);
          const h8 A = {c_lo[0], c_lo[1], c_lo[2], c_lo[3], c_hi[0], c_hi[1], c_hi[2], c_hi[3]};
          const bool on = (pc == slot);
          const h8 Bh = *reinterpret_cast<const h8*>(on ? &T.ph[pp][hc][0] : &T.zero[0]);
          const h8 Bl = *reinterpret_cast<const h8*>(on ? &T.pl[pp][hc][0] : &T.zero[0]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bh, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bl, acc, 0, 0, 0);
        }
      } else {
        // K = 16 per MFMA = 2 page slots x 8; lane group kg = (slot kg/2, half kg%2)
        const int slot = kg >> 1, half = kg & 1;
        const int pg = gp * PG + (slot < PG ? slot : 0);
        const uint32_t cw = *reinterpret_cast<const uint32_t*>(&T.c[pg][row * 8 + 4 * half]);
        const h4 cv = codes_to_h4(cw);
        const h4 A = (slot < PG) ? cv : h4{0, 0, 0, 0};
        const bool on = (pc == slot);
        const h4 Bh = *reinterpret_cast<const h4*>(on ? &T.ph[pp][hc][4 * half] : &T.zero[0]);
        const h4 Bl = *reinterpret_cast<const h4*>(on ? &T.pl[pp][hc][4 * half] : &T.zero[0]);
        acc = __builtin_amdgcn_mfma_f32_16x16x16f16(A, Bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16f16(A, Bl, acc, 0, 0, 0);
      }
      // lane (col = row, kg) holds tokens 4kg .. 4kg+3 of (page pp, head hc)
      const float sa = T.sc[pp][0] * es, sv = T.sc[pp][1] * es * 0x1p22f;
      const float base = T.a[pp][hc] * sa;
      const float t0 = fmaf(acc[0], sv, base), t1 = fmaf(acc[1], sv, base);
      const float t2 = fmaf(acc[2], sv, base), t3 = fmaf(acc[3], sv, base);
      float mx = fmaxf(fmaxf(t0, t1), fmaxf(t2, t3));
      mx = xor32_max(xor16_max(mx));
      float ssum = fast_exp2(t0 - mx) + fast_exp2(t1 - mx) + fast_exp2(t2 - mx) + fast_exp2(t3 - mx);
      ssum = xor32_sum(xor16_sum(ssum));
      if (kg == 0) T.out[t * 16 + pp][hc] = mx + fast_log2(ssum);
    }
    wave_lds_sync();
  }

  // ---- the wave's scores, written once after its last loads: a store in
  // flight would hold up the wait for later loads (one in-order counter
  // covers both); whole 256-byte rows per head coalesce, and streaming
  // (non-temporal) stores keep them from sitting dirty in L2 until the end
  // of the launch
  const bool mine = (present >> lane) & 1ull;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float sc = mine ? T.out[lane][h] * kLn2 : -INFINITY;  // natural log; absent: -inf
    if (p0 + lane < n_b) __builtin_nontemporal_store(sc, &a.scores[((size_t)b * a.Hq + (size_t)hbase + h) * N + p0 + lane]);
  }

  // ---- per-head (max, sum) of exp2 over the wave's pages: lane takes head
  // lane % G and pages i * 64/G + lane / G, then lanes of one head merge
  constexpr int LPH = kScorePagesPerWave / G;
  float m = -INFINITY, v[G];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int pg = i * LPH + lane / G;
    v[i] = ((present >> pg) & 1ull) ? T.out[pg][lane % G] : -INFINITY;
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
    float* dst = a.partials + (((size_t)b * a.Hq + (size_t)hbase + lane) * a.n_ranges + range) * 2;
    dst[0] = (ssum > 0.f) ? m : -INFINITY;
    dst[1] = ssum;
  }
  // ---- per head and 16-page tile: the max of s_hat (base 2; -inf if no page),
  // for a sequence whose selection bounds by tiles
  if (n_b < a.tile_pages && lane < kTiles * G) {
    const int tt = lane / G, hh = lane % G;
    float tm = -INFINITY;
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int pg = tt * 16 + p;
      if ((present >> pg) & 1ull) tm = fmaxf(tm, T.out[pg][hh]);
    }
    a.tile_max[((size_t)b * a.Hq + (size_t)hbase + hh) * ((size_t)a.n_ranges * kTiles) +
               (size_t)range * kTiles + tt] = tm;
  }
}

template <int G>
hipError_t launch_g(const locks_dims& d, const WsLayout& L, const DevPtrs& P, const float* q,
                    const uint8_t* summ, const int32_t* pt, const int32_t* sl, hipStream_t s) {
  ScoreArgs a;
  a.q = q;
  a.summ = summ;
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
  constexpr int NS = G > 8 ? G / 8 : 1;
  const int nrg = (L.n_score_wg + 3) / 4;
  dim3 grid(NS == 1 ? nrg : (nrg + 7) / 8 * 8, d.n_kv_heads * NS, d.batch);
  hipLaunchKernelGGL(score_kernel<G>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const locks_dims& d, const WsLayout& L, const DevPtrs& P, const float* q,
                        const uint8_t* summ, const int32_t* pt, const int32_t* sl, hipStream_t s) {
  switch (d.n_q_heads / d.n_kv_heads) {
    case 1: return launch_g<1>(d, L, P, q, summ, pt, sl, s);
    case 2: return launch_g<2>(d, L, P, q, summ, pt, sl, s);
    case 4: return launch_g<4>(d, L, P, q, summ, pt, sl, s);
    case 8: return launch_g<8>(d, L, P, q, summ, pt, sl, s);
    case 16: return launch_g<16>(d, L, P, q, summ, pt, sl, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace locks
