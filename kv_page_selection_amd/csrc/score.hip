// score.hip — page scoring from compressed summaries (gfx950).
//
// For every (sequence b, KV head, page j) and each of the G query heads of the
// group, computes the page score of the LOCKS blog post ("How LOCKS works",
// page-score equation; technical summary, section 2 mechanism 2):
//   s_hat = log sum_{i<16} exp((q.mu + (V^T q).c_i) / sqrt(128))
// from the page's 832-byte summary record alone (no key or value is read).
//
// Mapping. One workgroup = 4 waves = 256 consecutive pages of one (b, KV head).
// A wave handles 16 pages per tile. The two contractions with q, mu^T q and
// V^T q, run on int8 MFMA (v_mfma_i32_16x16x64_i8): the A operand is the
// record's codes exactly as stored (mu bytes as they are; V nibbles widened to
// 16*code bytes with one shift and mask), the B operand is each query head as a
// 22-bit fixed-point integer split into three signed int8 digits, so every
// product and sum is exact in int32 and one fp32 rounding combines the digits.
// Tile rows: 16 pages' mu rows in one MFMA tile; 2 pages x 8 basis vectors in
// each of 8 V tiles. Columns: the G query heads. The in-page part (C p and the
// 16-token log-sum-exp) runs on VALU from LDS, in base-2 units.
// Each workgroup also leaves, per head, the (max, sum) of exp over its pages,
// which the group combine needs for every head's total mass.
#include "device_common.h"
#include "internal.h"

namespace locks {

namespace {

struct ScoreArgs {
  const float* q;
  const uint8_t* summ;
  const int32_t* page_table;
  const int32_t* seq_lens;
  float* scores;
  float* partials;
  uint32_t* reset;
  int n_reset;
  int Hq, Hkv, N, num_blocks, n_wg;
};

__device__ __forceinline__ int nib_lo(uint32_t x) { return (int)((x << 4) & 0xF0F0F0F0u); }
__device__ __forceinline__ int nib_hi(uint32_t x) { return (int)(x & 0xF0F0F0F0u); }

// acc2*2^16 + acc1*2^8 + acc0, exact in int arithmetic up to the last fp32 rounding.
__device__ __forceinline__ float digits_value(int a2, int a1, int a0) {
  return (float)(a2 * 256 + a1) * 256.0f + (float)a0;
}

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

template <int G>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  constexpr int kPairs = 16 * G;  // (page, head) pairs of a tile
  constexpr int kSlots = (kPairs + 63) / 64;
  const int wg = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int N = a.N;
  const int n_b = full_pages(a.seq_lens, b, N);

  __shared__ float q_s[G * kDim];
  __shared__ int qmax_s[G];
  __shared__ __align__(16) int8_t dig_s[3][G][kDim];
  __shared__ float esc_s[G];
  __shared__ float pv_s[4][16][kRank][G];
  __shared__ float a_s[4][16][G];
  __shared__ __align__(16) uint8_t c_s[4][16][128];
  __shared__ float sc_s[4][16][3];
  __shared__ float red_s[4][G][2];

  // Counters of the later phases start every step at zero.
  if (wg == 0 && kvh == 0 && b == 0)
    for (int i = tid; i < a.n_reset; i += 256) a.reset[i] = 0;

  // ---- q of the group -> per-head exponent -> three int8 digit planes
  if (tid < G) qmax_s[tid] = 0;
  const float* qg = a.q + ((size_t)b * a.Hq + (size_t)kvh * G) * kDim;
  for (int i = tid; i < G * kDim; i += 256) q_s[i] = qg[i];
  __syncthreads();
  for (int i = tid; i < G * kDim; i += 256)
    atomicMax(&qmax_s[i / kDim], __float_as_int(fabsf(q_s[i])));
  __syncthreads();
  for (int i = tid; i < G * kDim; i += 256) {
    const int h = i / kDim, d = i % kDim;
    const float qm = __int_as_float(qmax_s[h]);
    int e = 0;
    if (qm > 0.f) {
      int E;
      frexpf(qm, &E);
      e = 22 - E;  // max |q| * 2^e in [2^21, 2^22)
    }
    const int qf = (int)rintf(ldexpf(q_s[i], e));
    const int d0 = ((qf + 128) & 255) - 128;
    const int r1 = (qf - d0) / 256;
    const int d1 = ((r1 + 128) & 255) - 128;
    const int d2 = (r1 - d1) / 256;
    dig_s[0][h][d] = (int8_t)d0;
    dig_s[1][h][d] = (int8_t)d1;
    dig_s[2][h][d] = (int8_t)d2;
    if (d == 0) esc_s[h] = ldexpf(1.0f, -e);
  }
  __syncthreads();

  // B operands: lane (column = head `row`, K group kg) holds d in [32kg+16m, +16).
  v4i bop[2][3];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int dg = 0; dg < 3; ++dg)
      bop[m][dg] = (row < G) ? *reinterpret_cast<const v4i*>(&dig_s[dg][row < G ? row : 0][32 * kg + 16 * m])
                             : v4i{0, 0, 0, 0};

  float run_m = -INFINITY, run_s = 0.f;  // this lane's head, log2 units

  for (int t = 0; t < 4; ++t) {
    const int pbase = wg * kScorePagesPerWG + wave * 64 + t * 16;
    const int j = pbase + row;
    int blk = -1;
    if (j < n_b) {
      blk = a.page_table[(size_t)b * N + j];
      if (blk < 0 || blk >= a.num_blocks) blk = -1;
    }
    // ---- loads: V rows (page 2vt + row/8, basis vector row%8), mu, C, scales
    uint4 vraw[8];
#pragma unroll
    for (int vt = 0; vt < 8; ++vt) {
      const int blk2 = __shfl(blk, 2 * vt + (row >> 3));
      vraw[vt] = make_uint4(0, 0, 0, 0);
      if (blk2 >= 0)
        vraw[vt] = *reinterpret_cast<const uint4*>(
            a.summ + ((size_t)blk2 * a.Hkv + kvh) * kStride + kVOff + (row & 7) * 64 + kg * 16);
    }
    uint4 mu0 = make_uint4(0, 0, 0, 0), mu1 = mu0, c0 = mu0, c1 = mu0;
    uint2 scl = make_uint2(0, 0);
    if (blk >= 0) {
      const uint8_t* rec = a.summ + ((size_t)blk * a.Hkv + kvh) * kStride;
      mu0 = *reinterpret_cast<const uint4*>(rec + kMuOff + kg * 32);
      mu1 = *reinterpret_cast<const uint4*>(rec + kMuOff + kg * 32 + 16);
      c0 = *reinterpret_cast<const uint4*>(rec + kCOff + kg * 32);
      c1 = *reinterpret_cast<const uint4*>(rec + kCOff + kg * 32 + 16);
      if (kg == 0) scl = *reinterpret_cast<const uint2*>(rec + kSOff);
    }
    *reinterpret_cast<uint4*>(&c_s[wave][row][kg * 32]) = c0;
    *reinterpret_cast<uint4*>(&c_s[wave][row][kg * 32 + 16]) = c1;
    if (kg == 0) {
      sc_s[wave][row][0] = f16bits_to_float(scl.x);
      sc_s[wave][row][1] = f16bits_to_float(scl.x >> 16) * (1.0f / 16.0f) * f16bits_to_float(scl.y);
      sc_s[wave][row][2] = (blk >= 0) ? 1.0f : 0.0f;
    }

    // ---- mu tile: rows = the 16 pages
    {
      v4i acc[3] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
      const v4i A0 = {(int)mu0.x, (int)mu0.y, (int)mu0.z, (int)mu0.w};
      const v4i A1 = {(int)mu1.x, (int)mu1.y, (int)mu1.z, (int)mu1.w};
#pragma unroll
      for (int dg = 0; dg < 3; ++dg) {
        acc[dg] = mfma_i8(A0, bop[0][dg], acc[dg]);
        acc[dg] = mfma_i8(A1, bop[1][dg], acc[dg]);
      }
      if (row < G) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a_s[wave][4 * kg + i][row < G ? row : 0] = digits_value(acc[2][i], acc[1][i], acc[0][i]);
      }
    }
    // ---- V tiles: rows = (page 2vt + r/8, basis vector r%8)
#pragma unroll
    for (int vt = 0; vt < 8; ++vt) {
      const uint4 v = vraw[vt];
      const v4i A0 = {nib_lo(v.x), nib_hi(v.x), nib_lo(v.y), nib_hi(v.y)};
      const v4i A1 = {nib_lo(v.z), nib_hi(v.z), nib_lo(v.w), nib_hi(v.w)};
      v4i acc[3] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
      for (int dg = 0; dg < 3; ++dg) {
        acc[dg] = mfma_i8(A0, bop[0][dg], acc[dg]);
        acc[dg] = mfma_i8(A1, bop[1][dg], acc[dg]);
      }
      if (row < G) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pv_s[wave][2 * vt + (kg >> 1)][4 * (kg & 1) + i][row < G ? row : 0] =
              digits_value(acc[2][i], acc[1][i], acc[0][i]);
      }
    }
    wave_lds_sync();

    // ---- in-page logits and their log-sum-exp; lane <-> (page, head) pairs
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
      const int pi = lane + 64 * s;
      if (pi < kPairs) {
        const int p = pi / G, h = pi % G;
        if (sc_s[wave][p][2] != 0.0f) {
          const float es = esc_s[h] * (kLog2e * kInvSqrtD);
          const float cs = sc_s[wave][p][1] * es;
          float pk[kRank], psum = 0.f;
#pragma unroll
          for (int k = 0; k < kRank; ++k) {
            pk[k] = pv_s[wave][p][k][h] * cs;
            psum += pk[k];
          }
          // C codes are read as unsigned bytes (code + 128); the offset is removed once.
          const float base = a_s[wave][p][h] * sc_s[wave][p][0] * es - 128.0f * psum;
          float t2[kPage], m = -INFINITY;
#pragma unroll
          for (int i = 0; i < kPage; ++i) {
            const uint2 cw = *reinterpret_cast<const uint2*>(&c_s[wave][p][i * 8]);
            const uint32_t u0 = cw.x ^ 0x80808080u, u1 = cw.y ^ 0x80808080u;
            float acc = base;
            acc = fmaf((float)(u0 & 0xffu), pk[0], acc);
            acc = fmaf((float)((u0 >> 8) & 0xffu), pk[1], acc);
            acc = fmaf((float)((u0 >> 16) & 0xffu), pk[2], acc);
            acc = fmaf((float)(u0 >> 24), pk[3], acc);
            acc = fmaf((float)(u1 & 0xffu), pk[4], acc);
            acc = fmaf((float)((u1 >> 8) & 0xffu), pk[5], acc);
            acc = fmaf((float)((u1 >> 16) & 0xffu), pk[6], acc);
            acc = fmaf((float)(u1 >> 24), pk[7], acc);
            t2[i] = acc;
            m = fmaxf(m, acc);
          }
          float ssum = 0.f;
#pragma unroll
          for (int i = 0; i < kPage; ++i) ssum += exp2f(t2[i] - m);
          const float shat2 = m + log2f(ssum);
          a.scores[((size_t)b * a.Hq + (size_t)kvh * G + h) * N + pbase + p] = shat2 * kLn2;
          lse2_merge(run_m, run_s, shat2, 1.0f);
        }
      }
    }
    wave_lds_sync();
  }

  // ---- per-head (max, sum) over this workgroup's pages
#pragma unroll
  for (int off = G; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(run_m, off), s2 = __shfl_xor(run_s, off);
    lse2_merge(run_m, run_s, m2, s2);
  }
  if (lane < G) {
    red_s[wave][lane < G ? lane : 0][0] = run_m;
    red_s[wave][lane < G ? lane : 0][1] = run_s;
  }
  __syncthreads();
  if (tid < G) {
    float m = red_s[0][tid][0], s = red_s[0][tid][1];
    for (int w = 1; w < 4; ++w) lse2_merge(m, s, red_s[w][tid][0], red_s[w][tid][1]);
    float* dst = a.partials + (((size_t)b * a.Hq + (size_t)kvh * G + tid) * a.n_wg + wg) * 2;
    dst[0] = m;
    dst[1] = s;
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
  a.reset = P.cnt_select;  // select and sparse-attention counters are adjacent
  a.n_reset = 2 * d.batch * d.n_kv_heads;
  a.Hq = d.n_q_heads;
  a.Hkv = d.n_kv_heads;
  a.N = d.max_pages_per_seq;
  a.num_blocks = d.num_blocks;
  a.n_wg = L.n_score_wg;
  dim3 grid(L.n_score_wg, d.n_kv_heads, d.batch);
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
