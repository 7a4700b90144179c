// attend.hip — split-K flash-decode over a list of pages (gfx950).
//
// Sparse mode: exact attention of each query head over only the kept pages of
// its (sequence, KV head) (blog post, "Code": attention over the gathered
// tokens of the selected pages; softmax scale 1/sqrt(128), renormalised over
// those tokens). Dense mode: the same over every full page, the full-KV
// comparison of the same section. Both modes also attend the sequence's tail,
// the tokens of its partly filled last page (no summary exists for it until
// it fills: "How LOCKS works"), as one more list entry whose rows past the
// tail are neither read nor weighted.
//
// Grid (split, KV head, sequence); a split is a run of pages of the list and a
// wave handles one page at a time for all G heads of the group:
//   QK: lane (token i = lane%16, d-chunk c = lane/16) reads 64 contiguous bytes
//       of key row i and dots them with the LDS-resident query chunk; two
//       permlane swaps (lanes l^16, l^32) finish each logit;
//   online softmax in base 2 over the page's 16 tokens (DPP row butterflies);
//   PV: lane owns d = 2*lane, 2*lane+1, reads one bf16 pair per token row
//       (coalesced 256-byte rows) and takes each token's weight by readlane.
// Waves merge in LDS into one (max, sum, o[128]) partial per head and split; a
// second launch, one workgroup per (sequence, query head), merges the splits
// in fixed order and writes the output. No float atomics. For G >= 8 (and the
// dense comparator at G = 4) the per-page products run on MFMA instead
// (attend_mfma_kernel below).
#include "device_common.h"
#include "internal.h"
#include "rank_device.h"

namespace locks {

namespace {

struct AttnArgs {
  const float* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* fill;  // nullable: pages that filled in this step (attended as the tail)
  const int32_t* sel;      // nullptr: dense (every full page)
  const int32_t* sel_blk;  // physical blocks of sel's pages (nullptr: look them up)
  float* partials;
  float* out;
  int Hq, Hkv, N, num_blocks, k, pages_per_split, n_split;
  // ranking launches only: the chunk pass's candidate lists, and where split 0
  // writes the kept ids
  const unsigned long long* cand;
  const int32_t* cand_blk;
  const int32_t* cand_count;
  int32_t* sel_out;
  int n_chunks, chunk;
};

// LDS of a launch that ranks its own list: the workgroup path's space and
// the blocks of this split's entries (at most 64 pages per split).
template <bool RANK>
struct RankSpace {
  RankLds<256> r;
  int sblk[64];
};
template <>
struct RankSpace<false> {
  int sblk[1];
};

// The kept list of this workgroup's (sequence, KV head), ranked here from the
// chunk lists exactly as the select merge launch does; of it, this split's
// entries [s0, s0 + pages_per_split): their blocks go to sblk and their ids
// to the step's selection output (-1 past the kept pages), so the splits
// together write the whole list. Every thread calls it; the caller's next
// barrier publishes sblk.
__device__ __forceinline__ void rank_split(const AttnArgs& a, RankSpace<true>& RS, size_t head, int split) {
  const size_t lists = head * a.n_chunks;
  const CandLists L{a.cand + lists * a.chunk, a.cand_blk + lists * a.chunk, a.cand_count + lists,
                    a.n_chunks, a.chunk};
  const int s0 = split * a.pages_per_split, pps = a.pages_per_split;
  int32_t* ids = a.sel_out + head * a.k;
  int* sblk = RS.sblk;
  auto emit = [ids, sblk, s0, pps](int pos, int id, int blk) {
    const unsigned r = (unsigned)(pos - s0);
    if (r < (unsigned)pps) {
      ids[pos] = id;
      sblk[r] = blk;
    }
  };
  // the counts and the speculative slots, in one round trip
  const int lgS = fast_lg_slots(L.nc);
  int cc[16];
  fast_count_load(L, cc);
  constexpr int KPL = kFastCap / 256;
  unsigned long long x[KPL];
  int bl[KPL], cof[KPL];
  fast_slots_load<256>(L, lgS, x, bl, cof);
  int total;
  const bool over = fast_count_check(L, lgS, cc, &total);  // the same in every wave
  if (over && total > kFastCap) {
    rank_global<256>(RS.r, L, a.k, emit);
    return;
  }
  const uint32_t live = over ? fast_gather_exact<256>(L, RS.r.off, total, x, bl) : fast_slots_live<256>(L, lgS, cof);
  fast_emit<256>(x, bl, fast_rank<256>(x, live, a.k, !over, RS.r), a.k, !over, s0, s0 + pps, RS.r, emit);
}

// RANK: the list is ranked here (rank_split) instead of read from sel_blk.
template <int G, bool RANK>
__global__ __launch_bounds__(256) void attend_kernel(AttnArgs a) {
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tok = lane & 15, c = lane >> 4;
  const int N = a.N;
  const int n_b = full_pages(a.seq_lens, a.fill, b, N);
  const int tail = tail_tokens(a.seq_lens, a.fill, b, N);
  const int base_len = a.sel ? a.k : n_b;  // entry base_len is the tail, if any
  const int list_len = base_len + (tail > 0 ? 1 : 0);
  const int s0 = split * a.pages_per_split;
  __shared__ RankSpace<RANK> RS;
  // q of the group, base-2 logit scale: loaded first, so that a ranking
  // launch finds it arrived when its waves stage their shares after ranking
  constexpr int QPT = (G * kDim + 255) / 256;  // q values per thread
  const float qscale = kLog2e * kInvSqrtD;
  float qv[QPT];
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int i = tid + 256 * j;
    qv[j] = (i < G * kDim) ? a.q[((size_t)b * a.Hq + (size_t)kvh * G) * kDim + i] * qscale : 0.f;
  }
  if constexpr (RANK) rank_split(a, RS, (size_t)b * a.Hkv + kvh, split);
  // the first entry's block id: a selected page (entry < k) needs no sequence
  // length, so its load goes out together with the length's
  int blk_first = -1;
  if (!RANK && a.sel_blk && s0 + wave < a.k) {
    const int blk = a.sel_blk[((size_t)b * a.Hkv + kvh) * a.k + s0 + wave];
    blk_first = (blk >= 0 && blk < a.num_blocks) ? blk : -1;
  }
  const int s1 = min(s0 + a.pages_per_split, list_len);

  __shared__ __align__(16) float q_s[G][kDim];
  __shared__ float wm_s[4][G], wl_s[4][G];
  __shared__ float wo_s[4][G][kDim];

  // physical block of list entry s (-1: skip): from this launch's ranking, the
  // selection's block list, through the page table, or (dense) page s itself
  auto page_block = [&](int s) -> int {
    int blk;
    if (s == base_len) {
      blk = a.page_table[(size_t)b * N + n_b];  // the tail page (n_b < N here)
    } else if constexpr (RANK) {
      blk = RS.sblk[s - s0];
    } else if (a.sel_blk) {
      blk = a.sel_blk[((size_t)b * a.Hkv + kvh) * a.k + s];
    } else {
      const int j = a.sel ? a.sel[((size_t)b * a.Hkv + kvh) * a.k + s] : s;
      if (j < 0 || j >= n_b) return -1;
      blk = a.page_table[(size_t)b * N + j];
    }
    return (blk >= 0 && blk < a.num_blocks) ? blk : -1;
  };
  // a selected entry's block id was loaded above; others (the tail, dense
  // lists, caller-given ids) are looked up here
  int blk_next = blk_first;
  if (!RANK && !(a.sel_blk && s0 + wave < a.k)) blk_next = (s0 + wave < s1) ? page_block(s0 + wave) : -1;

  // a page's K and V rows for this lane (rows >= ntok: not read, zero)
  uint4 kr[4];
  uint32_t vr[kPage];
  auto load_page = [&](int s, int blk) {
    const int ntok = (s == base_len) ? tail : kPage;
    const size_t tile = ((size_t)blk * a.Hkv + kvh) * (kPage * kDim);
    const uint4* krow = reinterpret_cast<const uint4*>(a.kc + tile + tok * kDim + c * 32);
#pragma unroll
    for (int u = 0; u < 4; ++u) kr[u] = (tok < ntok) ? krow[u] : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t* vbase = reinterpret_cast<const uint32_t*>(a.vc + tile) + lane;
#pragma unroll
    for (int i = 0; i < kPage; ++i) vr[i] = (i < ntok) ? vbase[i * (kDim / 2)] : 0u;
  };
  // the wave's first page goes out before q is staged: its rows need only the
  // block id, and travel during the q load and the barrier (a ranking launch
  // knows its blocks only after that barrier)
  int blk = -1;
  if constexpr (!RANK) {
    blk = blk_next;
    if (s0 + wave < s1 && blk >= 0) load_page(s0 + wave, blk);
    blk_next = (s0 + wave + 4 < s1) ? page_block(s0 + wave + 4) : -1;
  }

#pragma unroll
  for (int j = 0; j < QPT; ++j) {  // logits in base-2 units
    const int i = tid + 256 * j;
    if (i < G * kDim) q_s[i / kDim][i % kDim] = qv[j];
  }
  __syncthreads();
  if constexpr (RANK) {
    blk = (s0 + wave < s1) ? page_block(s0 + wave) : -1;
    if (blk >= 0) load_page(s0 + wave, blk);
    blk_next = (s0 + wave + 4 < s1) ? page_block(s0 + wave + 4) : -1;
  }

  float m[G], l[G], o0[G], o1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) { m[h] = -INFINITY; l[h] = 0.f; o0[h] = 0.f; o1[h] = 0.f; }

  for (int s = s0 + wave; s < s1; s += 4) {
    if (s > s0 + wave) {  // later pages of a long split: loaded in turn
      blk = blk_next;
      blk_next = (s + 4 < s1) ? page_block(s + 4) : -1;
      if (blk >= 0) load_page(s, blk);
    }
    if (blk < 0) continue;
    const int ntok = (s == base_len) ? tail : kPage;  // rows >= ntok: not read, not weighted

    // ---- logits of token `tok`, partial over d in [32c, 32c+32)
    float lg[G];
#pragma unroll
    for (int h = 0; h < G; ++h) lg[h] = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t w[4] = {kr[u].x, kr[u].y, kr[u].z, kr[u].w};
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float4 qa = *reinterpret_cast<const float4*>(&q_s[h][c * 32 + u * 8]);
        const float4 qb = *reinterpret_cast<const float4*>(&q_s[h][c * 32 + u * 8 + 4]);
        float acc = lg[h];
        acc = fmaf(bf16lo(w[0]), qa.x, acc);
        acc = fmaf(bf16hi(w[0]), qa.y, acc);
        acc = fmaf(bf16lo(w[1]), qa.z, acc);
        acc = fmaf(bf16hi(w[1]), qa.w, acc);
        acc = fmaf(bf16lo(w[2]), qb.x, acc);
        acc = fmaf(bf16hi(w[2]), qb.y, acc);
        acc = fmaf(bf16lo(w[3]), qb.z, acc);
        acc = fmaf(bf16hi(w[3]), qb.w, acc);
        lg[h] = acc;
      }
    }
    float pw[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float x = xor16_sum(lg[h]);  // the four d-chunks of token `tok`
      x = xor32_sum(x);
      if (tok >= ntok) x = -INFINITY;
      const float pm = row16_reduce(x, [](float u, float v) { return fmaxf(u, v); });
      const float mn = fmaxf(m[h], pm);
      const float alpha = exp2f(m[h] - mn);  // m = -inf -> 0
      const float p = exp2f(x - mn);
      const float ps = row16_reduce(p, [](float u, float v) { return u + v; });
      l[h] = l[h] * alpha + ps;
      m[h] = mn;
      o0[h] *= alpha;
      o1[h] *= alpha;
      pw[h] = p;
    }
    // ---- o += sum_i p_i v_i for d = 2*lane, 2*lane+1
#pragma unroll
    for (int i = 0; i < kPage; ++i) {
      const float v0 = bf16lo(vr[i]), v1 = bf16hi(vr[i]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pf = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pw[h]), i));
        o0[h] = fmaf(pf, v0, o0[h]);
        o1[h] = fmaf(pf, v1, o1[h]);
      }
    }
  }

  // ---- merge the 4 waves of this split
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (lane == 0) { wm_s[wave][h] = m[h]; wl_s[wave][h] = l[h]; }
    wo_s[wave][h][2 * lane] = o0[h];
    wo_s[wave][h][2 * lane + 1] = o1[h];
  }
  __syncthreads();
  float* part = a.partials + (((size_t)b * a.Hq + (size_t)kvh * G) * a.n_split + split) * kPartialFloats;
  for (int i = tid; i < G * kDim; i += 256) {
    const int h = i / kDim, d = i % kDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm_s[w][h]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = exp2f(wm_s[w][h] - M);
        L += wl_s[w][h] * f;
        O += wo_s[w][h][d] * f;
      }
    }
    float* ph = part + (size_t)h * a.n_split * kPartialFloats;
    ph[2 + d] = O;
    if (d == 0) { ph[0] = M; ph[1] = L; }
  }
}

typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef short s4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ short bf16_bits(float x) {
  return __builtin_bit_cast(short, (__bf16)x);
}

// MFMA flash-decode for G >= 4 query heads per KV head: each page is a
// (16 tokens x 128) x (128 x G heads) contraction and back.
//   S^T = K Q^T on v_mfma_f32_16x16x32_bf16: A = the key rows as stored
//     (lane: token l%16, dims 8(l/16)+e of a 32-wide chunk), B = q as bf16
//     hi + lo (~16 significant bits), heads padded to 16 with zeros; a lane
//     then holds the base-2 logits of tokens 4(l/16)+r for head l%16.
//   softmax over the page's tokens: in-lane over r, then two permlane swaps.
//   O += P V on v_mfma_f32_16x16x16_bf16: those same registers are the A
//     operand (P[head][token]) as bf16 hi + lo; B = V[token][dim], read from a
//     per-wave LDS copy of the tile whose 272-byte rows make the 4-token
//     column reads bank-conflict free; a lane accumulates O[head 4(l/16)+r]
//     [dim 16 blk + l%16].
template <int G, bool RANK>
__global__ __launch_bounds__(256) void attend_mfma_kernel(AttnArgs a) {
  static_assert(G >= 4 && G <= 16, "MFMA rows are the query heads of a group");
  constexpr int kVRow = kDim + 8;  // staged V row in bf16 (272 bytes)
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lj = lane >> 4;
  const int N = a.N;
  const int n_b = full_pages(a.seq_lens, a.fill, b, N);
  const int tail = tail_tokens(a.seq_lens, a.fill, b, N);
  const int base_len = a.sel ? a.k : n_b;  // entry base_len is the tail, if any
  const int list_len = base_len + (tail > 0 ? 1 : 0);
  const int s0 = split * a.pages_per_split;
  // the first entry's block id: a selected page (entry < k) needs no sequence
  // length, so its load goes out together with the length's
  int blk_first = -1;
  if (!RANK && a.sel_blk && s0 + wave < a.k) {
    const int blk = a.sel_blk[((size_t)b * a.Hkv + kvh) * a.k + s0 + wave];
    blk_first = (blk >= 0 && blk < a.num_blocks) ? blk : -1;
  }
  const int s1 = min(s0 + a.pages_per_split, list_len);

  // V staging during the page loop; the waves' O rows for the merge after it
  union AttnLds {
    __bf16 v[4][kPage][kVRow];
    float wo[4][G][kDim];
  };
  __shared__ __align__(16) AttnLds U;
  __shared__ float wm_s[4][G], wl_s[4][G];
  __shared__ RankSpace<RANK> RS;

  auto page_block = [&](int s) -> int {
    int blk;
    if (s == base_len) {
      blk = a.page_table[(size_t)b * N + n_b];  // the tail page (n_b < N here)
    } else if constexpr (RANK) {
      blk = RS.sblk[s - s0];
    } else if (a.sel_blk) {
      blk = a.sel_blk[((size_t)b * a.Hkv + kvh) * a.k + s];
    } else {
      const int j = a.sel ? a.sel[((size_t)b * a.Hkv + kvh) * a.k + s] : s;
      if (j < 0 || j >= n_b) return -1;
      blk = a.page_table[(size_t)b * N + j];
    }
    return (blk >= 0 && blk < a.num_blocks) ? blk : -1;
  };
  int blk_next = blk_first;
  if (!RANK && !(a.sel_blk && s0 + wave < a.k)) blk_next = (s0 + wave < s1) ? page_block(s0 + wave) : -1;

  // q of head li (zero for li >= G), base-2 logit scale, bf16 hi + lo
  bf8_t qh[4], ql[4];
  {
    const float qscale = kLog2e * kInvSqrtD;
    const float* qrow = a.q + ((size_t)b * a.Hq + (size_t)kvh * G + (li < G ? li : 0)) * kDim;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float4 x0 = *reinterpret_cast<const float4*>(qrow + 32 * c + 8 * lj);
      const float4 x1 = *reinterpret_cast<const float4*>(qrow + 32 * c + 8 * lj + 4);
      const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (li < G) ? xs[e] * qscale : 0.f;
        const __bf16 h = (__bf16)x;
        qh[c][e] = h;
        ql[c][e] = (__bf16)(x - (float)h);
      }
    }
  }

  if constexpr (RANK) {  // the list, ranked here, after q's loads went out
    rank_split(a, RS, (size_t)b * a.Hkv + kvh, split);
    __syncthreads();
    blk_next = (s0 + wave < s1) ? page_block(s0 + wave) : -1;
  }

  float m_run = -INFINITY, l_run = 0.f;  // head li
  v4f oacc[8];
#pragma unroll
  for (int k8 = 0; k8 < 8; ++k8) oacc[k8] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int s = s0 + wave; s < s1; s += 4) {
    const int blk = blk_next;
    blk_next = (s + 4 < s1) ? page_block(s + 4) : -1;
    if (blk < 0) continue;
    const int ntok = (s == base_len) ? tail : kPage;  // rows >= ntok: not read, not weighted
    const size_t tile = ((size_t)blk * a.Hkv + kvh) * (kPage * kDim);
    const uint4* krow = reinterpret_cast<const uint4*>(a.kc + tile + li * kDim + 8 * lj);
    const uint4* vrow = reinterpret_cast<const uint4*>(a.vc + tile + li * kDim + 8 * lj);
    uint4 kr[4], vr[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      kr[c] = (li < ntok) ? krow[4 * c] : make_uint4(0u, 0u, 0u, 0u);
      vr[c] = (li < ntok) ? vrow[4 * c] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) *reinterpret_cast<uint4*>(&U.v[wave][li][32 * c + 8 * lj]) = vr[c];

    v4f sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf8_t kk = __builtin_bit_cast(bf8_t, kr[c]);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qh[c], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, ql[c], sacc, 0, 0, 0);
    }
    // online softmax for head li over the page's 16 tokens (4lj + r)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * lj + r >= ntok) sacc[r] = -INFINITY;
    float mx = fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3]));
    mx = xor32_max(xor16_max(mx));
    const float mn = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - mn);  // m_run = -inf -> 0
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sacc[r] - mn);
    float ps = (pr[0] + pr[1]) + (pr[2] + pr[3]);
    ps = xor32_sum(xor16_sum(ps));
    l_run = fmaf(l_run, alpha, ps);
    m_run = mn;
    // O rows are heads 4lj + r: their rescale factors sit in lanes 4lj + r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float al = __shfl(alpha, 4 * lj + r);
#pragma unroll
      for (int k8 = 0; k8 < 8; ++k8) oacc[k8][r] *= al;
    }
    s4_t ph, pl;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const __bf16 h = (__bf16)pr[r];
      ph[r] = __builtin_bit_cast(short, h);
      pl[r] = bf16_bits(pr[r] - (float)h);
    }
    wave_lds_sync();  // the V tile is staged
#pragma unroll
    for (int k8 = 0; k8 < 8; ++k8) {
      s4_t vb;
#pragma unroll
      for (int e = 0; e < 4; ++e) vb[e] = __builtin_bit_cast(short, U.v[wave][4 * lj + e][16 * k8 + li]);
      oacc[k8] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, vb, oacc[k8], 0, 0, 0);
      oacc[k8] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, vb, oacc[k8], 0, 0, 0);
    }
    wave_lds_sync();  // every lane has read the tile before the next one lands
  }

  // ---- merge the 4 waves of this split (the V staging area becomes O rows)
  __syncthreads();
  if (lj == 0 && li < G) { wm_s[wave][li] = m_run; wl_s[wave][li] = l_run; }
#pragma unroll
  for (int k8 = 0; k8 < 8; ++k8)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * lj + r < G) U.wo[wave][4 * lj + r][16 * k8 + li] = oacc[k8][r];
  __syncthreads();
  float* part = a.partials + (((size_t)b * a.Hq + (size_t)kvh * G) * a.n_split + split) * kPartialFloats;
  for (int i = tid; i < G * kDim; i += 256) {
    const int h = i / kDim, d = i % kDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm_s[w][h]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = exp2f(wm_s[w][h] - M);
        L += wl_s[w][h] * f;
        O += U.wo[w][h][d] * f;
      }
    }
    float* ph2 = part + (size_t)h * a.n_split * kPartialFloats;
    ph2[2 + d] = O;
    if (d == 0) { ph2[0] = M; ph2[1] = L; }
  }
}

// Merge of the split partials of one (sequence, query head): 256 threads =
// 128 output dims x 2 halves of the split list. Each half folds its splits in
// fixed order with an online rescale, 8 splits' loads in flight at a time;
// then half 1 is folded into half 0. Base-2 units throughout.
__global__ __launch_bounds__(256) void attend_merge_kernel(const float* partials, float* out,
                                                           int Hq, int n_split) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, d = tid & 127, half = tid >> 7;
  __shared__ float m_s, l_s, o_s[kDim];
  const float* ph = partials + ((size_t)b * Hq + h) * n_split * kPartialFloats;
  const int per = (n_split + 1) / 2;
  const int s0 = half * per, s1 = min(n_split, s0 + per);
  constexpr int MB = 8;  // splits' loads in flight at a time (16 or 32 measured slower)
  float M = -1e30f, L = 0.f, O = 0.f;  // (-1e30, 0, 0) = empty
  for (int sb = s0; sb < s1; sb += MB) {
    float mv[MB], lv[MB], ov[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int sp = (sb + i < s1) ? sb + i : s0;
      const float* p = ph + (size_t)sp * kPartialFloats;
      mv[i] = p[0];
      lv[i] = p[1];
      ov[i] = p[2 + d];
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const float mi = (sb + i < s1) ? fmaxf(mv[i], -1e30f) : -1e30f;
      const float mn = fmaxf(M, mi);
      const float fa = fast_exp2(M - mn), fb = (sb + i < s1) ? fast_exp2(mi - mn) : 0.f;
      L = L * fa + lv[i] * fb;
      O = O * fa + ov[i] * fb;
      M = mn;
    }
  }
  if (half == 1) {
    if (d == 0) { m_s = M; l_s = L; }
    o_s[d] = O;
  }
  __syncthreads();
  if (half == 0) {
    const float M1 = m_s, mn = fmaxf(M, M1);
    const float fa = fast_exp2(M - mn), fb = fast_exp2(M1 - mn);
    const float Lt = L * fa + l_s * fb;
    const float Ot = O * fa + o_s[d] * fb;
    out[((size_t)b * Hq + h) * kDim + d] = (Lt > 0.f) ? Ot / Lt : 0.f;
  }
}

template <int G>
hipError_t launch_g(const locks_dims& d, const WsLayout& L, const DevPtrs& P, const float* q,
                    const uint16_t* kc, const uint16_t* vc, const int32_t* pt, const int32_t* sl,
                    const int32_t* fill, const int32_t* sel, const int32_t* sel_blk, float* out,
                    bool dense, bool rank, hipStream_t s) {
  AttnArgs a;
  a.q = q;
  a.kc = kc;
  a.vc = vc;
  a.page_table = pt;
  a.seq_lens = sl;
  a.fill = fill;
  a.sel = dense ? nullptr : sel;
  a.sel_blk = (dense || rank) ? nullptr : sel_blk;
  a.partials = dense ? P.dense_part : P.att_part;
  a.out = out;
  a.Hq = d.n_q_heads;
  a.Hkv = d.n_kv_heads;
  a.N = d.max_pages_per_seq;
  a.num_blocks = d.num_blocks;
  a.k = L.k;
  a.pages_per_split = dense ? L.dense_pages_per_split : L.att_pages_per_split;
  a.n_split = dense ? L.n_dense_split : L.n_att_split;
  a.cand = P.cand;
  a.cand_blk = P.cand_blk;
  a.cand_count = P.cand_count;
  a.sel_out = rank ? const_cast<int32_t*>(sel) : nullptr;
  a.n_chunks = L.n_sel_chunks;
  a.chunk = L.sel_chunk;
  if (rank && (dense || a.pages_per_split > 64)) return hipErrorInvalidValue;
  // MFMA where a query group fills enough of the 16 rows: G >= 8 always, and
  // G = 4 for the long dense splits; a sparse split at G = 4 (one page per
  // wave, 3/4 of the rows padding) stays on VALU: MFMA there showed no clear
  // gain (1.0 us per step faster at one 1M-token sequence, 0.5 slower at
  // eight of 256K tokens)
  const dim3 grid(a.n_split, d.n_kv_heads, d.batch);
  if constexpr (G >= 8) {
    if (rank) hipLaunchKernelGGL((attend_mfma_kernel<G, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attend_mfma_kernel<G, false>), grid, dim3(256), 0, s, a);
  } else if constexpr (G == 4) {
    if (dense) hipLaunchKernelGGL((attend_mfma_kernel<G, false>), grid, dim3(256), 0, s, a);
    else if (rank) hipLaunchKernelGGL((attend_kernel<G, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attend_kernel<G, false>), grid, dim3(256), 0, s, a);
  } else {
    if (rank) hipLaunchKernelGGL((attend_kernel<G, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attend_kernel<G, false>), grid, dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL(attend_merge_kernel, dim3(d.n_q_heads, d.batch), dim3(256), 0, s, a.partials,
                     out, d.n_q_heads, a.n_split);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend(const locks_dims& d, const WsLayout& L, const DevPtrs& P, const float* q,
                         const uint16_t* kc, const uint16_t* vc, const int32_t* pt,
                         const int32_t* sl, const int32_t* fill, const int32_t* sel,
                         const int32_t* sel_blk, float* out, bool dense, bool rank, hipStream_t s) {
  switch (d.n_q_heads / d.n_kv_heads) {
    case 1: return launch_g<1>(d, L, P, q, kc, vc, pt, sl, fill, sel, sel_blk, out, dense, rank, s);
    case 2: return launch_g<2>(d, L, P, q, kc, vc, pt, sl, fill, sel, sel_blk, out, dense, rank, s);
    case 4: return launch_g<4>(d, L, P, q, kc, vc, pt, sl, fill, sel, sel_blk, out, dense, rank, s);
    case 8: return launch_g<8>(d, L, P, q, kc, vc, pt, sl, fill, sel, sel_blk, out, dense, rank, s);
    case 16: return launch_g<16>(d, L, P, q, kc, vc, pt, sl, fill, sel, sel_blk, out, dense, rank, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace locks
