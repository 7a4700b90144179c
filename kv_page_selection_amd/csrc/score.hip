// score.hip — page scoring from compressed summaries (gfx950).
//
// For every (sequence b, KV head, page j) and each of the G query heads of the
// group, computes the page score of the LOCKS blog post ("How LOCKS works",
// page-score equation; technical summary, section 2 mechanism 2):
//   s_hat = log sum_{i<16} exp((q.mu + (V^T q).c_i) / sqrt(128))
// from the page's summary record alone (no key or value is read).
//
// Mapping. A workgroup is 4 waves of one KV head and all G of its query heads;
// up to 8 heads, wave w scores 64 consecutive pages (4 tiles of 16) and the
// waves take 4 consecutive page ranges; with 16 heads two waves share a
// 64-page range (32 pages each) and a workgroup takes 2 ranges. Grids of at
// most 1024 (sequence, KV head, range) triples, which would leave SIMDs with
// one wave or none, split each range over four waves of 16 pages instead
// (a workgroup per range), still one round of resident waves. The waves of a
// range merge their per-head (max, sum) in LDS. The q prologue (fixed-point
// digits of the group's query heads) is split over the 4 waves and shared in
// LDS.
//
// Stage 1, mu.q and V^T q, on v_mfma_i32_16x16x64_i8, exact: the row operand is
// each query head as a 22-bit fixed-point integer in three signed int8 digits,
// the column operand is the record's codes as stored (mu bytes; V nibbles
// widened to 16*code with one shift and mask). Up to 8 heads, a row block is 4
// heads x 4 digit slots (the 4th zero), so a lane holds all three digit sums
// of one value; with 16 heads a row block is one digit plane of all 16 heads,
// and a lane finds the same 4 heads in the three planes' outputs. Either way
// it combines the digit sums in int32 and one fp32 rounding.
// Stage 2, the in-page contraction C p (16 tokens x 8 x G heads), on
// v_mfma_f32_16x16x{32,16}_f16: C codes are exact in f16 and p enters as an
// f16 hi + lo pair (about 22 significant bits). Up to 8 heads, 16/G pages are
// packed block-diagonally along K so one pass fills the 16 output columns;
// with 16 heads one page fills them, and hi and lo share one product (K =
// 8 basis vectors x {hi, lo}). The 16-token log-sum-exp is one in-lane step
// and two cross-row swaps, in base 2.
// The wave keeps its 64 x G scores in LDS; at the end it writes them once and
// leaves, per head, the (max, sum) of exp2 over its pages, which the group
// combine needs for every head's total mass, and the max of each 16-page tile,
// the units of the selection's pruning bound.
//
// Loads. Each wave turns its page-table entries into record offsets once (an
// LDS table); every tile then issues its 13 record loads back to back in a
// fixed order (V rows first) and consumes them in that order, so the first
// MFMAs run while the tail of the tile is still arriving.
#include "build_device.h"

namespace locks {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int kTiles = kScorePagesPerWave / 16;
constexpr long long kScoreRoundWaves = 4096;  // 4 waves per SIMD x 1024 SIMDs: one round of a scorer grid

struct ScoreArgs {
  const float* q;
  const uint8_t* summ;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* fill;  // nullable: pages that filled in this step (attended as the tail)
  float* scores;
  float* partials;
  float* tile_max;
  int Hq, Hkv, N, num_blocks, n_ranges, tile_pages;
  // with a fill (1-D grid): the first fill_wgs workgroups build the records
  // of the pages that filled in this step (fb); the rest score, as workgroup
  // (x, y, z) of a gx x Hkv x B grid in x-fastest order
  BuildArgs fb;
  int fill_wgs, gx;
};

// A scoring kernel's LDS; with a fill, shared with the build waves' LDS.
template <class SL, bool Fill>
struct KernelLds {
  SL s;
};
template <class SL>
struct KernelLds<SL, true> {
  union {
    SL s;
    WaveLds b[4];
  };
};

// The workgroup's scoring coordinates (bx, by, bz); with a fill, false for a
// workgroup that built records instead (one page-head per wave).
template <bool Fill, class U>
__device__ __forceinline__ bool score_workgroup(const ScoreArgs& a, U& lds, int wave, int lane, int& bx,
                                                int& by, int& bz) {
  bx = blockIdx.x;
  by = blockIdx.y;
  bz = blockIdx.z;
  if constexpr (Fill) {
    int lid = blockIdx.x;
    if (lid < a.fill_wgs) {
      build_wave<1>(a.fb, lds.b[wave], (long long)lid * 4 + wave, lane);
      return false;
    }
    lid -= a.fill_wgs;
    bx = lid % a.gx;
    lid /= a.gx;
    by = lid % a.Hkv;
    bz = lid / a.Hkv;
  }
  return true;
}

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

// Per-wave LDS staging of one 16-page tile; the wave's P page scores.
template <int G, int P>
struct TileLds {
  __align__(16) int8_t c[16][144];      // C codes per page (token-major), padded rows
  __align__(16) _Float16 ph[16][G][8];  // p (scaled by 2^-22) high part, [page][head][k]
  __align__(16) _Float16 pl[16][G][8];  // low part
  __align__(16) _Float16 zero[8];       // masked B operand
  float a[16][G + 1];                   // mu . q (exact integer), [page][head]; column G spare
  float sc[32][2];                      // s_mu, s_V/16 * s_C; rows 16.. take the other lanes' copies
  __align__(16) float out[P][G];        // the wave's page scores, [page][head], base 2
};

template <int G, class TileT>
struct ScoreLds {
  TileT w[4];
  union {
    __align__(16) int8_t dig[3][G][kDim];  // q digit planes of the workgroup's heads,
    uint32_t off[4][kScorePagesPerWave];   // then each wave's page record offsets
  } u;
  float esc[16];                           // per head: 2^-e log2(e) / sqrt(128)
  float2 ms[4][8];                         // per wave and head: (max, sum of exp2) over its pages
};

// q of the G heads at qg -> per-head exponent e (max |q| * 2^e in [2^21,
// 2^22)) -> three signed int8 digit planes, q * 2^e = d0 + 256 d1 + 65536 d2;
// wave w converts heads w, w+4, ... All of the wave's q loads are issued
// before any is used: one memory round trip at launch, before the grid's
// record loads queue up (a trip per head, the later ones behind those loads,
// cost 16-head launches ~1 us).
template <int G>
__device__ __forceinline__ void q_digit_planes(const float* qg, int8_t (&dig)[3][G][kDim],
                                               float* esc, int wave, int lane) {
  constexpr int HPW = (G + 3) / 4;  // heads per wave
  float qv[HPW][2];
#pragma unroll
  for (int i = 0; i < HPW; ++i) {
    const int h = wave + 4 * i;
    qv[i][0] = h < G ? qg[h * kDim + lane] : 0.f;
    qv[i][1] = h < G ? qg[h * kDim + 64 + lane] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < HPW; ++i) {
    const int h = wave + 4 * i;
    if (h >= G) break;
    const float q0 = qv[i][0], q1 = qv[i][1];
    const float qm = wave_max(fmaxf(fabsf(q0), fabsf(q1)));
    int e = 0;
    if (qm > 0.f) {
      int E;
      frexpf(qm, &E);
      e = 22 - E;
    }
    const float qs[2] = {q0, q1};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int qf = (int)rintf(ldexpf(qs[u], e));
      const int d0 = ((qf + 128) & 255) - 128;
      const int r1 = (qf - d0) / 256;
      const int d1 = ((r1 + 128) & 255) - 128;
      const int d2 = (r1 - d1) / 256;
      dig[0][h][lane + 64 * u] = (int8_t)d0;
      dig[1][h][lane + 64 * u] = (int8_t)d1;
      dig[2][h][lane + 64 * u] = (int8_t)d2;
    }
    if (lane == 0) esc[h] = ldexpf(1.0f, -e) * (kLog2e * kInvSqrtD);
  }
}

// The three digit sums of one value -> fp32 (|value| < 2^37; the top two
// digits combine exactly in int32)
__device__ __forceinline__ float digits_to_float(int s0, int s1, int s2) {
  return (float)(s2 * 256 + s1) * 256.0f + (float)s0;
}

// Reduce-scatter of 4 passes' per-lane partial sums over the 4 lane groups (16
// lanes each) of a wave: one v_permlane16_swap pairs groups (0, 1) and (2, 3),
// one v_permlane32_swap pairs the halves, and each swap leaves a lane two
// copies of one pass, its own and its partner's. A lane ends with the total of
// pass reduce_scatter4_pass() of the four.
__device__ __forceinline__ float swap16_sum(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_sum(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float reduce_scatter4(float s0, float s1, float s2, float s3) {
  return swap32_sum(swap16_sum(s0, s1), swap16_sum(s2, s3));
}
// the pass a lane keeps: the same two swaps applied to pass tags
__device__ __forceinline__ int reduce_scatter4_pass() {
  const auto a = __builtin_amdgcn_permlane16_swap(0u, 1u, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(0u, 1u, false, false);
  return (int)a[0] + 2 * (int)b[0];
}

// A wave's outputs from its base-2 scores out[page][head] (pages p0 .. p0+P-1
// of sequence b, query heads hbase ..): page scores in natural log (-inf for
// an absent page), the per-head (max, sum of exp2) over the range, and, for a
// sequence bounded by tiles, the max of each 16-page tile. With W waves per
// 64-page range (P = 64 / W), waves part > 0 leave their (max, sum) in LDS
// and part 0 merges them; every wave of the workgroup calls this (the merge
// has a barrier), those without pages with present = 0. Nothing but page
// scores is written for a range without pages (live = false).
template <int G, int P, class Lds>
__device__ __forceinline__ void write_wave_outputs(const ScoreArgs& a, const float (&out)[P][G], Lds& S,
                                                   unsigned long long present, bool live, int b, int hbase,
                                                   int range, int part, int p0, int n_b, int wave,
                                                   int lane) {
  constexpr int W = kScorePagesPerWave / P;
  constexpr int HP = 64 / P;  // heads per store pass
  const int N = a.N;
  // written once after the wave's last loads: a store in flight would hold
  // up the wait for later loads (one in-order counter covers both); lane =
  // page lane % P of head group lane / P, so whole runs of 4P bytes per head
  // coalesce, and streaming (non-temporal) stores keep them from sitting
  // dirty in L2 until the end of the launch
  {
    const int pg = lane % P;
    const bool mine = (present >> pg) & 1ull;
    if (p0 + pg < n_b) {
#pragma unroll
      for (int j = 0; j < (G + HP - 1) / HP; ++j) {
        const int h = HP * j + lane / P;
        if (HP * j + HP <= G || h < G) {
          const float sc = mine ? out[pg][h < G ? h : 0] * kLn2 : -INFINITY;
          __builtin_nontemporal_store(sc, &a.scores[((size_t)b * a.Hq + (size_t)hbase + h) * N + p0 + pg]);
        }
      }
    }
  }

  // per-head (max, sum) of exp2 over the wave's pages: lane takes head
  // lane % G and pages i * 64/G + lane / G, then lanes of one head merge
  constexpr int LPH = kScorePagesPerWave / G;
  constexpr int PPL = (P + LPH - 1) / LPH;  // pages per lane
  float m = -INFINITY, v[PPL];
#pragma unroll
  for (int i = 0; i < PPL; ++i) {
    const int pg = i * LPH + lane / G;
    v[i] = (pg < P && ((present >> pg) & 1ull)) ? out[pg < P ? pg : 0][lane % G] : -INFINITY;
    m = fmaxf(m, v[i]);
  }
  float ssum = 0.f;
  {
    const float ms = m == -INFINITY ? 0.f : m;
#pragma unroll
    for (int i = 0; i < PPL; ++i) ssum += fast_exp2(v[i] - ms);
  }
#pragma unroll
  for (int off = G; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(ssum, off);
    const float mn = fmaxf(m, m2);
    const float ms = mn == -INFINITY ? 0.f : mn;
    ssum = ssum * fast_exp2(m - ms) + s2 * fast_exp2(m2 - ms);
    m = mn;
  }
  if constexpr (W > 1) {
    if (part > 0 && lane < G) S.ms[wave][lane] = make_float2(m, ssum);
    __syncthreads();
    if (part == 0 && lane < G) {
#pragma unroll
      for (int w = 1; w < W; ++w) {
        const float2 o = S.ms[wave + w][lane];
        const float mn = fmaxf(m, o.x);
        const float ms = mn == -INFINITY ? 0.f : mn;
        ssum = ssum * fast_exp2(m - ms) + o.y * fast_exp2(o.x - ms);
        m = mn;
      }
    }
  }
  if (live && part == 0 && lane < G) {
    float* dst = a.partials + (((size_t)b * a.Hq + (size_t)hbase + lane) * a.n_ranges + range) * 2;
    dst[0] = (ssum > 0.f) ? m : -INFINITY;
    dst[1] = ssum;
  }
  // per head and 16-page tile: the max of s_hat (base 2; -inf if no page)
  constexpr int TPW = P / 16;  // tiles per wave
  if (live && n_b < a.tile_pages && lane < TPW * G) {
    const int tt = lane / G, hh = lane % G;
    float tm = -INFINITY;
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int pg = tt * 16 + p;
      if ((present >> pg) & 1ull) tm = fmaxf(tm, out[pg][hh]);
    }
    a.tile_max[((size_t)b * a.Hq + (size_t)hbase + hh) * ((size_t)a.n_ranges * kTiles) +
               (size_t)range * kTiles + part * TPW + tt] = tm;
  }
}

// One tile's records as a lane holds them: V rows (page 2vt + row/8, basis
// vector row%8), and the mu, C and scales of page row
struct TileRec {
  uint4 v[8], mu1, mu0, c1, c0;
  uint2 scl;
};

// G = query heads per KV head (at most 8); P = pages per wave: 64 (a range
// per wave, four per workgroup) or, for grids that would leave SIMDs idle,
// 16 (a range over four waves). 8-head waves are held to 128 VGPRs (4 waves
// per SIMD; left alone they take a few more and drop to 3).
template <int G, int P, bool Fill>
__global__ __launch_bounds__(256, G == 8 ? 4 : 1) void score_kernel(ScoreArgs a) {
  static_assert(G <= 8, "16-head groups use score16_kernel");
  constexpr int RB = G < 4 ? 1 : G / 4;   // stage-1 row blocks (4 heads each)
  constexpr int PG = 16 / G;              // pages per stage-2 pass
  constexpr int W = kScorePagesPerWave / P;  // waves per range
  constexpr int TPW = P / 16;                // tiles per wave
  __shared__ KernelLds<ScoreLds<G, TileLds<G, P>>, Fill> U;
  auto& S = U.s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  int bx, by, bz;
  if (!score_workgroup<Fill>(a, U, wave, lane, bx, by, bz)) return;  // workgroup-uniform
  const int b = bz;
  const int kvh = by;
  const int range = bx * (4 / W) + wave / W;
  const int part = wave % W;  // the wave's part of its range
  const int hbase = kvh * G;  // first query head of the group
  const int N = a.N;
  const int n_b = full_pages(a.seq_lens, a.fill, b, N);
  TileLds<G, P>& T = S.w[wave];
  const int p0 = range * kScorePagesPerWave + part * P;

  // A range wholly past the sequence's full pages (shorter sequences of a
  // batch) has no work and writes nothing (its partials are never read);
  // the whole workgroup leaves at once when none of its ranges has a page.
  if (bx * (4 / W) * kScorePagesPerWave >= n_b) return;  // workgroup-uniform

  // page table of this wave's P pages, one entry per lane; issued first, so
  // its latency overlaps the q prologue below
  int myblk = -1;
  {
    const int j = p0 + lane;
    if (range < a.n_ranges && lane < P && j < n_b) myblk = a.page_table[(size_t)b * N + j];
  }
  q_digit_planes<G>(a.q + ((size_t)b * a.Hq + (size_t)hbase) * kDim, S.u.dig, S.esc, wave, lane);
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
  // A wave past the ranges or the sequence's full pages has no work. With one
  // wave per range it leaves here (no workgroup barrier follows); with
  // several, it still reaches the merge barrier at the end.
  const bool live = range < a.n_ranges && range * kScorePagesPerWave < n_b;  // the range has pages
  const bool active = live && p0 < n_b;                                      // this wave has pages
  if (W == 1 && !active) return;
  if (lane < 8) T.zero[lane] = (_Float16)0.0f;

  // An absent page (past the sequence's full pages, or a table entry out of
  // range) reads block 0's record in its place, so every load is
  // unconditional; its score is replaced by -inf at the end.
  if (myblk < 0 || myblk >= a.num_blocks) myblk = -1;
  const unsigned long long present = __ballot(myblk >= 0);  // bit i: page p0 + i
  if (active) {
    // the lane's page record, as an offset from summ in 16-byte units (the
    // library limits num_blocks * n_kv_heads * 49 to 32 bits)
    S.u.off[wave][lane] = (uint32_t)((myblk < 0 ? 0 : myblk) * a.Hkv + kvh) * (uint32_t)(kStride / 16);
    const uint8_t* vbase = a.summ + kVOff + (row & 7) * 64 + kg * 16;  // V row of the lane
    const uint8_t* rbase = a.summ + kg * 32;                           // mu, C slice of the lane

    // stage-2 output column col = (page pc of the pass, head hc)
    const int pc = row / G, hc = row % G;
    const float es = S.esc[hc], es22 = es * 0x1p22f;
    const int jpass = reduce_scatter4_pass();  // with G >= 4: which pass of each 4 this lane finishes

    wave_lds_sync();

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
    for (int t = 0; t < TPW; ++t) {
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
          // exact integer (|.| < 2^37) -> fp32 -> split hi + lo, both scaled by
          // 2^-22 into f16 range as they are rounded (the scaling is exact)
          const float x = digits_to_float(acc[0], acc[1], acc[2]);
          const _Float16 xh = (_Float16)(x * 0x1p-22f);
          const _Float16 xl = (_Float16)fmaf(x, 0x1p-22f, -(float)xh);
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
      if (kPrefetchV && t + 1 < TPW) issue_v(t + 1, cur);
      wave_lds_sync();

      // ---- stage 2 + LSE, one pass per PG pages, as one branch-free block.
      // The LSE sums exp2 of the deviation term alone and adds the centroid
      // term after the log; a non-finite result (an overflowed sum) redoes the
      // tile's passes with the page max subtracted. With 4 or more passes, each
      // 4 share one reduce-scatter over the lane groups and each lane group
      // finishes one of them; with fewer, every lane of a column reduces and
      // stores the same value.
      auto deviations = [&](int gp) -> v4f {
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
        const float sv = T.sc[pp][1] * es22;
        return v4f{acc[0] * sv, acc[1] * sv, acc[2] * sv, acc[3] * sv};
      };
      auto part_sum = [&](int gp) -> float {
        const v4f d = deviations(gp);
        return (fast_exp2(d[0]) + fast_exp2(d[1])) + (fast_exp2(d[2]) + fast_exp2(d[3]));
      };
      // pass gp's score (every lane of the column); safe: page max subtracted first
      auto score_full = [&](int gp, bool safe) -> float {
        const v4f d = deviations(gp);
        const int pp = gp * PG + pc;
        float mx = 0.f;
        if (safe) {
          mx = fmaxf(fmaxf(d[0], d[1]), fmaxf(d[2], d[3]));
          mx = xor32_max(xor16_max(mx));
        }
        float ssum = (fast_exp2(d[0] - mx) + fast_exp2(d[1] - mx)) + (fast_exp2(d[2] - mx) + fast_exp2(d[3] - mx));
        ssum = xor32_sum(xor16_sum(ssum));
        return fmaf(T.a[pp][hc], T.sc[pp][0] * es, mx + fast_log2(ssum));
      };
      bool redo = false;
      if constexpr (G >= 4) {
  #pragma unroll
        for (int g = 0; g < G / 4; ++g) {
          const float s0 = part_sum(4 * g), s1 = part_sum(4 * g + 1);
          const float s2 = part_sum(4 * g + 2), s3 = part_sum(4 * g + 3);
          const float tot = reduce_scatter4(s0, s1, s2, s3);
          const int pp = (4 * g + jpass) * PG + pc;
          const float r = fmaf(T.a[pp][hc], T.sc[pp][0] * es, fast_log2(tot));
          redo |= !__builtin_isfinite(r);
          T.out[t * 16 + pp][hc] = r;
        }
      } else {
  #pragma unroll
        for (int gp = 0; gp < G; ++gp) {
          const float r = score_full(gp, false);
          redo |= !__builtin_isfinite(r);
          T.out[t * 16 + gp * PG + pc][hc] = r;
        }
      }
      if (__builtin_expect(__ballot(redo) != 0ull, 0)) {
  #pragma unroll 1
        for (int gp = 0; gp < G; ++gp) T.out[t * 16 + gp * PG + pc][hc] = score_full(gp, true);
      }
      wave_lds_sync();
    }

  }

  write_wave_outputs<G, P>(a, T.out, S, present, live, b, hbase, range, part, p0, n_b, wave, lane);
}

// ---- 16 query heads per KV head: one wave decodes each record once for all
// 16 heads.
//
// Work split. A 64-page range is two waves of 32 pages (2 tiles each), and a
// workgroup takes two ranges: a 1M-token sequence with 2 KV heads then gives
// every SIMD four waves, one round. Smaller grids (B * Hkv * ranges <= 1024)
// run 16 pages per wave, a range per workgroup, for twice the waves: at 7000
// pages that scores in 9.6 us instead of 11.8, while at 65536 pages the
// second round costs more than it hides (33.3 us against 29.0). LDS per wave
// stays under 10 KB (V^T q staged half a tile at a time; the q digit planes
// share their space with the tile buffers, which are not in use yet), so four
// workgroups fit a CU. The waves of a range merge their per-head (max, sum)
// through LDS at the end.
//
// Stage 1 row blocks are the digit planes (rows = the 16 heads): lane (column
// j, group kg) finds heads 4kg .. 4kg+3 of column j in each plane's output.
// V^T q goes to LDS as one word per (page, basis vector k, head) holding the
// f16 hi part and, above it, the lo part, so the lane's 4 heads are one
// 16-byte store. Stage 2 is one v_mfma_f32_16x16x16_f16 per page over K = 16
// = (k, part): lane group kg supplies (k = kg, hi), (kg, lo), (kg + 4, hi),
// (kg + 4, lo), so A repeats two C codes and B is two LDS words.
// The 16-token log-sum-exp runs on the deviation term alone: the centroid
// term is the same for the page's 16 tokens and is added after the log. A
// page's deviations sum to about zero (its coefficients are centred), so the
// sum of their exp2 is at least about 1 and does not underflow; a sum that
// overflows gives a non-finite score, and that half tile is redone with the
// max subtracted.

template <int PPW>
struct Tile16Lds {
  __align__(16) int8_t c[16][128];          // C codes + 128 per page (token-major)
  __align__(16) uint32_t p[8][kRank][16];   // V^T q * 2^-22 of half a tile, [page][k][head]: f16 hi | lo << 16
  __align__(16) float a[16][16];            // mu . q per (page, head), digit units
  float sc[32][2];                          // s_mu, s_V/16 * s_C; rows 16.. take the other lanes' copies
  float out[PPW][17];                       // the wave's page scores, [page][head] (+1 pad), base 2
};
template <int PPW>
struct Score16Lds {
  union {
    __align__(16) int8_t dig[3][16][kDim];  // q digit planes (prologue only)
    Tile16Lds<PPW> w[4];
  } u;
  uint32_t off[4][PPW];                     // each wave's page record offsets, 16-byte units
  float2 ms[4][16];                         // per wave and head: (max, sum of exp2) over its pages
  float esc[16];                            // per head: 2^-e log2(e) / sqrt(128)
};

template <int PPW, bool Fill>
__global__ __launch_bounds__(256, 4) void score16_kernel(ScoreArgs a) {
  constexpr int G = 16;
  constexpr int k16PagesPerWave = PPW;
  constexpr int k16Tiles = PPW / 16;
  constexpr int k16WavesPerRange = kScorePagesPerWave / PPW;  // 2 or 4
  constexpr int k16RangesPerWg = 4 / k16WavesPerRange;
  __shared__ KernelLds<Score16Lds<PPW>, Fill> U;
  auto& S = U.s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  int bx, by, bz;
  if (!score_workgroup<Fill>(a, U, wave, lane, bx, by, bz)) return;  // workgroup-uniform
  const int b = bz;
  const int kvh = by;
  const int range = bx * k16RangesPerWg + wave / k16WavesPerRange;
  const int half = wave % k16WavesPerRange;  // the wave's part of its range
  const int hbase = kvh * G;
  const int N = a.N;
  const int n_b = full_pages(a.seq_lens, a.fill, b, N);
  const int p0 = range * kScorePagesPerWave + half * k16PagesPerWave;  // the wave's first page

  if (bx * k16RangesPerWg * kScorePagesPerWave >= n_b) return;  // workgroup-uniform

  // A wave past the ranges or the sequence's full pages has no work but still
  // reaches the workgroup barriers below (no wave returns after this point).
  const bool active = range < a.n_ranges && p0 < n_b;  // wave-uniform
  int myblk = -1;
  if (active && lane < k16PagesPerWave && p0 + lane < n_b) myblk = a.page_table[(size_t)b * N + p0 + lane];
  q_digit_planes<G>(a.q + ((size_t)b * a.Hq + (size_t)hbase) * kDim, S.u.dig, S.esc, wave, lane);
  __syncthreads();
  // row operands: digit plane dg, lane (row = head, kg), d in [32kg+16m, +16)
  v4i aop[3][2];
#pragma unroll
  for (int dg = 0; dg < 3; ++dg)
#pragma unroll
    for (int m = 0; m < 2; ++m) aop[dg][m] = *reinterpret_cast<const v4i*>(&S.u.dig[dg][row][32 * kg + 16 * m]);
  // stage-2 scales of this lane's head (column row)
  const float es = S.esc[row], es22 = es * 0x1p22f;
  const int jpass = reduce_scatter4_pass();  // which page of each 4 this lane finishes
  __syncthreads();  // digit planes consumed: their space becomes the tile buffers

  Tile16Lds<PPW>& T = S.u.w[wave];
  if (myblk < 0 || myblk >= a.num_blocks) myblk = -1;
  const unsigned long long present = __ballot(myblk >= 0);  // bit i: page p0 + i
  if (active) {
    if (lane < k16PagesPerWave)
      S.off[wave][lane] = (uint32_t)((myblk < 0 ? 0 : myblk) * a.Hkv + kvh) * (uint32_t)(kStride / 16);
    const uint8_t* vbase = a.summ + kVOff + (row & 7) * 64 + kg * 16;
    const uint8_t* rbase = a.summ + kg * 32;
    wave_lds_sync();

    // a tile's loads in three groups, in the order they are consumed: V rows
    // of pages 0-7, the mu, C and scales, V rows of pages 8-15
    auto issue_v = [&](int t, int h, TileRec& r) {
      uint32_t ov[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[i] = S.off[wave][t * 16 + 2 * (4 * h + i) + (row >> 3)];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        r.v[4 * h + i] = *reinterpret_cast<const uint4*>(vbase + ((size_t)ov[i] << 4));
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto issue_tail = [&](int t, TileRec& r) {
      const uint8_t* rec = rbase + ((size_t)S.off[wave][t * 16 + row] << 4);  // page t*16 + row
      __builtin_amdgcn_sched_barrier(0);
      r.mu1 = *reinterpret_cast<const uint4*>(rec + kMuOff + 16);
      r.mu0 = *reinterpret_cast<const uint4*>(rec + kMuOff);
      r.c1 = *reinterpret_cast<const uint4*>(rec + kCOff + 16);
      r.c0 = *reinterpret_cast<const uint4*>(rec + kCOff);
      r.scl = *reinterpret_cast<const uint2*>(rec - kg * 32 + kSOff);
      __builtin_amdgcn_sched_barrier(0);
    };

    // stage 1 for the V rows of half h of the tile -> T.p (pages 8h .. 8h+7)
    auto stage1 = [&](const TileRec& r, int h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = r.v[4 * h + i];
        const v4i B0 = {nib_lo(v.x), nib_hi(v.x), nib_lo(v.y), nib_hi(v.y)};
        const v4i B1 = {nib_lo(v.z), nib_hi(v.z), nib_lo(v.w), nib_hi(v.w)};
        v4i s[3];
#pragma unroll
        for (int dg = 0; dg < 3; ++dg) s[dg] = mfma_i8(aop[dg][1], B1, mfma_i8(aop[dg][0], B0, v4i{0, 0, 0, 0}));
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // hi + lo, both scaled by 2^-22 into f16 range as they are rounded;
          // lo goes straight into the high half
          const float x = digits_to_float(s[0][j], s[1][j], s[2][j]);
          const _Float16 xh = (_Float16)(x * 0x1p-22f);
          const h2 hl = {xh, (_Float16)fmaf(x, 0x1p-22f, -(float)xh)};
          w[j] = __builtin_bit_cast(uint32_t, hl);
        }
        *reinterpret_cast<uint4*>(&T.p[2 * i + (row >> 3)][row & 7][4 * kg]) = uint4{w[0], w[1], w[2], w[3]};
      }
    };

    // stage 2 of tile page pp (T.p holds its half): lane (head row, kg) gets
    // the deviation terms of tokens 4kg .. 4kg+3
    const h2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const uint32_t csel = 0x04000400u | (uint32_t)kg | ((uint32_t)kg << 16);  // bytes kg, 0x64, kg, 0x64
    auto deviations = [&](int pp) -> v4f {
      const uint2 cw = *reinterpret_cast<const uint2*>(&T.c[pp][row * 8]);  // token row, k = 0..7
      const h2 clo = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, cw.x, csel)) + bias;
      const h2 chi = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, cw.y, csel)) + bias;
      const h4 A = {clo[0], clo[1], chi[0], chi[1]};
      const h2 p0v = __builtin_bit_cast(h2, T.p[pp & 7][kg][row]);
      const h2 p1v = __builtin_bit_cast(h2, T.p[pp & 7][kg + 4][row]);
      const h4 B = {p0v[0], p0v[1], p1v[0], p1v[1]};
      const v4f acc = __builtin_amdgcn_mfma_f32_16x16x16f16(A, B, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      const float sv = T.sc[pp][1] * es22;
      return v4f{acc[0] * sv, acc[1] * sv, acc[2] * sv, acc[3] * sv};
    };
    // the lane's part of sum_i exp2(deviation_i) for page pp
    auto part_sum = [&](int pp) -> float {
      const v4f d = deviations(pp);
      return (fast_exp2(d[0]) + fast_exp2(d[1])) + (fast_exp2(d[2]) + fast_exp2(d[3]));
    };
    // page pp's score with the page max subtracted first (every lane of the head)
    auto score_safe = [&](int pp) -> float {
      const v4f d = deviations(pp);
      float mx = fmaxf(fmaxf(d[0], d[1]), fmaxf(d[2], d[3]));
      mx = xor32_max(xor16_max(mx));
      float ssum = (fast_exp2(d[0] - mx) + fast_exp2(d[1] - mx)) + (fast_exp2(d[2] - mx) + fast_exp2(d[3] - mx));
      ssum = xor32_sum(xor16_sum(ssum));
      return fmaf(T.a[pp][row], T.sc[pp][0] * es, mx + fast_log2(ssum));
    };
    // the 8 pages of half h of tile t, 4 at a time: one reduce-scatter leaves
    // each lane group the sum of one page, whose score it finishes and stores
    auto stage2 = [&](int t, int h) {
      bool redo = false;
#pragma unroll
      for (int g = 2 * h; g < 2 * h + 2; ++g) {
        const float s0 = part_sum(4 * g), s1 = part_sum(4 * g + 1);
        const float s2 = part_sum(4 * g + 2), s3 = part_sum(4 * g + 3);
        const float tot = reduce_scatter4(s0, s1, s2, s3);
        const int pp = 4 * g + jpass;
        const float r = fmaf(T.a[pp][row], T.sc[pp][0] * es, fast_log2(tot));
        redo |= !__builtin_isfinite(r);
        T.out[t * 16 + pp][row] = r;
      }
      if (__builtin_expect(__ballot(redo) != 0ull, 0)) {
#pragma unroll 1
        for (int pp = 8 * h; pp < 8 * h + 8; ++pp) T.out[t * 16 + pp][row] = score_safe(pp);
      }
    };

    TileRec cur, nxt;
    issue_v(0, 0, cur);
    issue_tail(0, cur);
    issue_v(0, 1, cur);
#pragma unroll
    for (int t = 0; t < k16Tiles; ++t) {
      const bool more = t + 1 < k16Tiles;
      stage1(cur, 0);
      if (more) issue_v(t + 1, 0, nxt);
      __builtin_amdgcn_sched_barrier(0);
      // ---- stage 1: mu tile (columns = the 16 pages); lane (page row, kg) -> heads 4kg ..
      {
        const uint4 mu0 = cur.mu0, mu1 = cur.mu1;
        const v4i B0 = {(int)mu0.x, (int)mu0.y, (int)mu0.z, (int)mu0.w};
        const v4i B1 = {(int)mu1.x, (int)mu1.y, (int)mu1.z, (int)mu1.w};
        v4i s[3];
#pragma unroll
        for (int dg = 0; dg < 3; ++dg) s[dg] = mfma_i8(aop[dg][1], B1, mfma_i8(aop[dg][0], B0, v4i{0, 0, 0, 0}));
        float4 av;
        av.x = digits_to_float(s[0][0], s[1][0], s[2][0]);
        av.y = digits_to_float(s[0][1], s[1][1], s[2][1]);
        av.z = digits_to_float(s[0][2], s[1][2], s[2][2]);
        av.w = digits_to_float(s[0][3], s[1][3], s[2][3]);
        *reinterpret_cast<float4*>(&T.a[row][4 * kg]) = av;
        const uint4 c0 = cur.c0, c1 = cur.c1;
        *reinterpret_cast<uint4*>(&T.c[row][kg * 32]) =
            uint4{c0.x ^ 0x80808080u, c0.y ^ 0x80808080u, c0.z ^ 0x80808080u, c0.w ^ 0x80808080u};
        *reinterpret_cast<uint4*>(&T.c[row][kg * 32 + 16]) =
            uint4{c1.x ^ 0x80808080u, c1.y ^ 0x80808080u, c1.z ^ 0x80808080u, c1.w ^ 0x80808080u};
        const uint2 scl = cur.scl;
        const int r = kg == 0 ? row : 16 + row;
        T.sc[r][0] = f16bits_to_float(scl.x);
        T.sc[r][1] = f16bits_to_float(scl.x >> 16) * (1.0f / 16.0f) * f16bits_to_float(scl.y);
      }
      if (more) issue_tail(t + 1, nxt);
      wave_lds_sync();
      stage2(t, 0);
      wave_lds_sync();  // half 0 of T.p read: half 1 takes its place
      stage1(cur, 1);
      if (more) issue_v(t + 1, 1, nxt);
      wave_lds_sync();
      stage2(t, 1);
      wave_lds_sync();
      if (more) cur = nxt;
    }
  }

  // ---- per-head (max, sum of exp2) over the wave's present pages: lane
  // (head row, kg) takes pages 4i + kg, then the 4 lanes of a head merge
  float m = -INFINITY, ssum = 0.f;
  if (active) {
    float v[k16PagesPerWave / 4];
#pragma unroll
    for (int i = 0; i < k16PagesPerWave / 4; ++i) {
      const int pg = 4 * i + kg;
      v[i] = ((present >> pg) & 1ull) ? T.out[pg][row] : -INFINITY;
      m = fmaxf(m, v[i]);
    }
    const float ms = m == -INFINITY ? 0.f : m;
#pragma unroll
    for (int i = 0; i < k16PagesPerWave / 4; ++i) ssum += fast_exp2(v[i] - ms);
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
      const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(ssum, off);
      const float mn = fmaxf(m, m2);
      const float mz = mn == -INFINITY ? 0.f : mn;
      ssum = ssum * fast_exp2(m - mz) + s2 * fast_exp2(m2 - mz);
      m = mn;
    }
  }
  if constexpr (k16WavesPerRange > 1) {
    if (half > 0 && lane < 16) S.ms[wave][row] = make_float2(m, ssum);
    __syncthreads();
  }
  if (!active) return;
  if (half == 0 && lane < 16) {
    float mn = m, st = ssum;
#pragma unroll
    for (int w = 1; w < k16WavesPerRange; ++w) {
      const float2 o = S.ms[wave + w][row];
      const float mx = fmaxf(mn, o.x);
      const float mz = mx == -INFINITY ? 0.f : mx;
      st = st * fast_exp2(mn - mz) + o.y * fast_exp2(o.x - mz);
      mn = mx;
    }
    float* dst = a.partials + (((size_t)b * a.Hq + (size_t)hbase + row) * a.n_ranges + range) * 2;
    dst[0] = (st > 0.f) ? mn : -INFINITY;
    dst[1] = st;
  }
  // ---- page scores (natural log; -inf for an absent page): lane = page
  // lane % P, heads HP j + lane / P (P pages per wave, HP = 64 / P heads per
  // store), so each store covers HP runs of 4P bytes
  {
    constexpr int HP = 64 / k16PagesPerWave;
    const int pg = lane % k16PagesPerWave;
    const bool mine = (present >> pg) & 1ull;
    if (p0 + pg < n_b) {
#pragma unroll
      for (int j = 0; j < G / HP; ++j) {
        const int h = HP * j + lane / k16PagesPerWave;
        const float sc = mine ? T.out[pg][h] * kLn2 : -INFINITY;
        __builtin_nontemporal_store(sc, &a.scores[((size_t)b * a.Hq + (size_t)hbase + h) * N + p0 + pg]);
      }
    }
  }
  // ---- per head and 16-page tile: the max of s_hat (base 2; -inf if no page)
  if (n_b < a.tile_pages && lane < k16Tiles * 16) {
    const int tt = lane >> 4;
    float tm = -INFINITY;
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int pg = tt * 16 + p;
      if ((present >> pg) & 1ull) tm = fmaxf(tm, T.out[pg][row]);
    }
    a.tile_max[((size_t)b * a.Hq + (size_t)hbase + row) * ((size_t)a.n_ranges * kTiles) +
               (size_t)range * kTiles + k16Tiles * half + tt] = tm;
  }
}

// Launches kernel K over grid (gx, Hkv, B); with a fill, as a 1-D grid whose
// first workgroups build the records of the pages that filled in this step.
template <class K>
void launch_scorer(K kernel, K fill_kernel, ScoreArgs& a, const locks_dims& d, int gx, hipStream_t s) {
  if (!a.fill) {
    hipLaunchKernelGGL(kernel, dim3(gx, d.n_kv_heads, d.batch), dim3(256), 0, s, a);
    return;
  }
  a.gx = gx;
  a.fill_wgs = (int)((a.fb.items + 3) / 4);  // one page-head per wave
  const long long wgs = (long long)a.fill_wgs + (long long)gx * d.n_kv_heads * d.batch;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)wgs), dim3(256), 0, s, a);
}

template <int G>
hipError_t launch_g(const locks_dims& d, const WsLayout& L, const DevPtrs& P, const float* q,
                    const uint8_t* summ, const int32_t* pt, const int32_t* sl, const int32_t* fill,
                    const uint16_t* kc, hipStream_t s) {
  ScoreArgs a;
  a.q = q;
  a.summ = summ;
  a.page_table = pt;
  a.seq_lens = sl;
  a.fill = fill;
  a.scores = P.scores;
  a.partials = P.score_part;
  a.tile_max = P.tile_max;
  a.tile_pages = kTileBoundPages * L.k;
  a.Hq = d.n_q_heads;
  a.Hkv = d.n_kv_heads;
  a.N = d.max_pages_per_seq;
  a.num_blocks = d.num_blocks;
  a.n_ranges = L.n_score_wg;
  a.fill_wgs = 0;
  a.gx = 0;
  a.fb.kc = kc;
  a.fb.page_table = pt;
  a.fb.seq_lens = sl;
  a.fb.blocks = nullptr;
  a.fb.fill = fill;
  // the records of the pages that filled are written by this launch and read
  // by none of its scoring workgroups (those pages are not scored this step)
  a.fb.summ = const_cast<uint8_t*>(summ);
  a.fb.B = d.batch;
  a.fb.Hkv = d.n_kv_heads;
  a.fb.N = d.max_pages_per_seq;
  a.fb.num_blocks = d.num_blocks;
  a.fb.items = (long long)d.batch * d.n_kv_heads;
  if constexpr (G == 16) {
    // 32 pages per wave (two ranges per workgroup); 16 (one range per
    // workgroup) when that grid still fits one round of resident waves
    if ((long long)d.batch * d.n_kv_heads * L.n_score_wg * 4 <= kScoreRoundWaves)
      launch_scorer(score16_kernel<16, false>, score16_kernel<16, true>, a, d, L.n_score_wg, s);
    else
      launch_scorer(score16_kernel<32, false>, score16_kernel<32, true>, a, d, (L.n_score_wg + 1) / 2, s);
  } else {
    // 64 pages per wave (four ranges per workgroup); 16 (a range over four
    // waves) when that grid still fits one round of resident waves: four
    // times the waves to hide latency with where the 64-page grid leaves a
    // SIMD one wave or none
    const long long units = (long long)d.batch * d.n_kv_heads * L.n_score_wg;  // (seq, KV head, range)
    if (units * 4 <= kScoreRoundWaves)
      launch_scorer(score_kernel<G, 16, false>, score_kernel<G, 16, true>, a, d, L.n_score_wg, s);
    else
      launch_scorer(score_kernel<G, 64, false>, score_kernel<G, 64, true>, a, d, (L.n_score_wg + 3) / 4, s);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const locks_dims& d, const WsLayout& L, const DevPtrs& P, const float* q,
                        const uint8_t* summ, const int32_t* pt, const int32_t* sl,
                        const int32_t* fill, const uint16_t* kc, hipStream_t s) {
  switch (d.n_q_heads / d.n_kv_heads) {
    case 1: return launch_g<1>(d, L, P, q, summ, pt, sl, fill, kc, s);
    case 2: return launch_g<2>(d, L, P, q, summ, pt, sl, fill, kc, s);
    case 4: return launch_g<4>(d, L, P, q, summ, pt, sl, fill, kc, s);
    case 8: return launch_g<8>(d, L, P, q, summ, pt, sl, fill, kc, s);
    case 16: return launch_g<16>(d, L, P, q, summ, pt, sl, fill, kc, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace locks
