// attend.hip — split-K flash-decode over a list of pages (gfx950).
//
// Sparse mode: exact attention of each query head over only the kept pages of
// its (sequence, KV head) (blog post, "Code": attention over the gathered
// tokens of the selected pages; softmax scale 1/sqrt(128), renormalised over
// those tokens). Dense mode: the same over every full page, the full-KV
// comparison of the same section.
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
// in fixed order and writes the output. No float atomics.
#include "device_common.h"
#include "internal.h"

namespace locks {

namespace {

struct AttnArgs {
  const float* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* sel;      // nullptr: dense (every full page)
  const int32_t* sel_blk;  // physical blocks of sel's pages (nullptr: look them up)
  float* partials;
  float* out;
  int Hq, Hkv, N, num_blocks, k, pages_per_split, n_split;
};

template <int G>
__global__ __launch_bounds__(256) void attend_kernel(AttnArgs a) {
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tok = lane & 15, c = lane >> 4;
  const int N = a.N;
  const int n_b = full_pages(a.seq_lens, b, N);
  const int list_len = a.sel ? a.k : n_b;
  const int s0 = split * a.pages_per_split;
  const int s1 = min(s0 + a.pages_per_split, list_len);

  __shared__ __align__(16) float q_s[G][kDim];
  __shared__ float wm_s[4][G], wl_s[4][G];
  __shared__ float wo_s[4][G][kDim];

  // physical block of list entry s (-1: skip): from the selection's block
  // list, through the page table, or (dense) page s itself
  auto page_block = [&](int s) -> int {
    int blk;
    if (a.sel_blk) {
      blk = a.sel_blk[((size_t)b * a.Hkv + kvh) * a.k + s];
    } else {
      const int j = a.sel ? a.sel[((size_t)b * a.Hkv + kvh) * a.k + s] : s;
      if (j < 0 || j >= n_b) return -1;
      blk = a.page_table[(size_t)b * N + j];
    }
    return (blk >= 0 && blk < a.num_blocks) ? blk : -1;
  };
  int blk_next = (s0 + wave < s1) ? page_block(s0 + wave) : -1;  // in flight during q staging

  const float qscale = kLog2e * kInvSqrtD;  // logits in base-2 units
  for (int i = tid; i < G * kDim; i += 256)
    q_s[i / kDim][i % kDim] = a.q[((size_t)b * a.Hq + (size_t)kvh * G) * kDim + i] * qscale;
  __syncthreads();

  float m[G], l[G], o0[G], o1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) { m[h] = -INFINITY; l[h] = 0.f; o0[h] = 0.f; o1[h] = 0.f; }

  for (int s = s0 + wave; s < s1; s += 4) {
    const int blk = blk_next;
    blk_next = (s + 4 < s1) ? page_block(s + 4) : -1;
    if (blk < 0) continue;
    const size_t tile = ((size_t)blk * a.Hkv + kvh) * (kPage * kDim);
    const uint4* krow = reinterpret_cast<const uint4*>(a.kc + tile + tok * kDim + c * 32);
    uint4 kr[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) kr[u] = krow[u];
    uint32_t vr[kPage];
    const uint32_t* vbase = reinterpret_cast<const uint32_t*>(a.vc + tile) + lane;
#pragma unroll
    for (int i = 0; i < kPage; ++i) vr[i] = vbase[i * (kDim / 2)];

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
  float M = -1e30f, L = 0.f, O = 0.f;  // (-1e30, 0, 0) = empty
  for (int sb = s0; sb < s1; sb += 8) {
    float mv[8], lv[8], ov[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int sp = (sb + i < s1) ? sb + i : s0;
      const float* p = ph + (size_t)sp * kPartialFloats;
      mv[i] = p[0];
      lv[i] = p[1];
      ov[i] = p[2 + d];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
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
                    const int32_t* sel, const int32_t* sel_blk, float* out, bool dense,
                    hipStream_t s) {
  AttnArgs a;
  a.q = q;
  a.kc = kc;
  a.vc = vc;
  a.page_table = pt;
  a.seq_lens = sl;
  a.sel = dense ? nullptr : sel;
  a.sel_blk = dense ? nullptr : sel_blk;
  a.partials = dense ? P.dense_part : P.att_part;
  a.out = out;
  a.Hq = d.n_q_heads;
  a.Hkv = d.n_kv_heads;
  a.N = d.max_pages_per_seq;
  a.num_blocks = d.num_blocks;
  a.k = L.k;
  a.pages_per_split = dense ? L.dense_pages_per_split : kSparsePagesPerSplit;
  a.n_split = dense ? L.n_dense_split : L.n_att_split;
  hipLaunchKernelGGL(attend_kernel<G>, dim3(a.n_split, d.n_kv_heads, d.batch), dim3(256), 0, s, a);
  hipLaunchKernelGGL(attend_merge_kernel, dim3(d.n_q_heads, d.batch), dim3(256), 0, s, a.partials,
                     out, d.n_q_heads, a.n_split);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend(const locks_dims& d, const WsLayout& L, const DevPtrs& P, const float* q,
                         const uint16_t* kc, const uint16_t* vc, const int32_t* pt,
                         const int32_t* sl, const int32_t* sel, const int32_t* sel_blk,
                         float* out, bool dense, hipStream_t s) {
  switch (d.n_q_heads / d.n_kv_heads) {
    case 1: return launch_g<1>(d, L, P, q, kc, vc, pt, sl, sel, sel_blk, out, dense, s);
    case 2: return launch_g<2>(d, L, P, q, kc, vc, pt, sl, sel, sel_blk, out, dense, s);
    case 4: return launch_g<4>(d, L, P, q, kc, vc, pt, sl, sel, sel_blk, out, dense, s);
    case 8: return launch_g<8>(d, L, P, q, kc, vc, pt, sl, sel, sel_blk, out, dense, s);
    case 16: return launch_g<16>(d, L, P, q, kc, vc, pt, sl, sel, sel_blk, out, dense, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace locks
