// build_device.h — the summary build's per-wave device code (gfx950), shared
// by the build kernels and by the scoring kernel of a decode step that builds
// the pages which filled in that step inside its own launch.
//
// Steps (blog post, "How LOCKS works" and "Code" build loop; technical summary,
// section 2 mechanism 1): centroid, centred deviations, eigendecomposition of
// the 16x16 Gram D D^T, rank-8 basis and coefficients, fp16 absmax scales,
// int8 / int4 codes, the packed record. The phases are described in build.hip.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace locks {

namespace {


constexpr int kWaves = 4;
constexpr int kPagesPerWave = 4;
constexpr int kMaxSweeps = 12;
// converged when the off-diagonal energy is below this fraction of the total
// (off-diagonal norm ~1e-5 of the Frobenius norm; the codes keep 4-8 bits)
constexpr float kOffTol = 1e-10f;

struct BuildArgs {
  const uint16_t* kc;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* blocks;  // non-null: build these blocks (every KV head) instead
  const int32_t* fill;    // non-null: item b * Hkv + kvh builds (b, kvh)'s page that
                          // filled in this step (see full_pages()), if any
  uint8_t* summ;
  int B, Hkv, N, num_blocks;
  long long items;
};

// Per-wave LDS; RecBytes = the record being assembled (the shipped 784 bytes,
// or a variant format's).
template <int RecBytes>
struct WaveLdsT {
  // Gram rows, slot-permuted (slot t = column i ^ t), until phase 2 has them in
  // registers; then the eigenvectors, transposed: [column][row]
  union {
    float A[kPagesPerWave][kPage][kPage];
    float UT[kPagesPerWave][kPage][kPage];
  };
  float2 rot[kPagesPerWave][kPage];      // this round's (cos, signed sin) per column
  float lam[kPagesPerWave][kPage];       // eigenvalues, descending
  int perm[kPagesPerWave][kPage];        // column of U holding the r-th eigenvector
  float diag[kPagesPerWave][kPage];
  float energy[kPagesPerWave];           // sum of squared deviations per page
  int8_t vq[kRank][kDim];
  __align__(16) uint8_t rec[RecBytes];
};
using WaveLds = WaveLdsT<kStride>;

__device__ __forceinline__ int quant(float x, float s, int qmax) {
  if (!(s > 0.f) || isinf(s)) return 0;
  const float c = rintf(__fdiv_rn(x, s));
  return (int)fminf(fmaxf(c, (float)-qmax), (float)qmax);
}

__device__ __forceinline__ float f16_round(float x) { return (float)(_Float16)x; }

__device__ __forceinline__ uint32_t f16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// value of lane (lane ^ M) (M < 16: stays in the lane's 16-lane group)
template <int M>
__device__ __forceinline__ float swz(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (M << 10) | 0x1F));
}

// One Jacobi round: rotate the pairs (i, i ^ M) of every page of the wave.
// J[p][p] = J[q][q] = c, J[p][q] = s, J[q][p] = -s (p < q); A <- J^T A J,
// U <- U J; the rotated element becomes exactly zero. The angle table is read
// per slot at column i ^ t: those 16 addresses are the same in every round
// (a per-pair read would need different addresses in each of the 15
// unrolled rounds, all kept live across the sweep loop).
// `live` is false for the lanes of a page that has converged: its rotations
// are the identity and its rows stay as they are, so each page gets the
// same sweeps whether it shares its wave with other pages or not.
template <int M>
__device__ __forceinline__ void jacobi_round(float (&a)[kPage], float (&u)[kPage], int i, bool live,
                                             float2* rot) {
  const bool lower = i < (i ^ M);
  // the partner row, slot-permuted: pa[t] = partner's slot t ^ M (column i ^ t).
  // All 16 swizzles go out before any is used, so the round waits on LDS
  // latency once rather than once per element.
  float pa[kPage];
#pragma unroll
  for (int tt = 0; tt < kPage; ++tt) pa[tt] = swz<M>(a[tt ^ M]);
  __builtin_amdgcn_sched_barrier(0);
  const float d_me = a[0], d_other = pa[M];
  const float o_me = a[M], o_other = pa[0];
  // both lanes of a pair take the same inputs, hence the same angle
  const float app = lower ? d_me : d_other, aqq = lower ? d_other : d_me;
  const float apq = lower ? o_me : o_other;
  // hardware reciprocal / square root (about 1 ulp): any rotation keeps the
  // matrix orthogonally similar, a slightly inexact angle only leaves a tiny
  // residual for the next sweep
  const float safe = (apq != 0.f) ? apq : 1.f;
  const float tau = (aqq - app) * __builtin_amdgcn_rcpf(2.f * safe);
  const float t = copysignf(1.0f, tau) *
                  __builtin_amdgcn_rcpf(fabsf(tau) + __builtin_amdgcn_sqrtf(fmaf(tau, tau, 1.f)));
  const bool rotate = live && apq != 0.f;
  const float c = rotate ? __builtin_amdgcn_rsqf(fmaf(t, t, 1.f)) : 1.f;
  const float s = rotate ? t * c : 0.f;
  const float sg = lower ? -s : s;
  // rows: row_i <- c row_i + sg row_partner; the partner's slot t ^ M is column i ^ t
  float ar[kPage];
#pragma unroll
  for (int tt = 0; tt < kPage; ++tt) ar[tt] = fmaf(c, a[tt], sg * pa[tt]);
  rot[i] = make_float2(c, sg);
  wave_lds_sync();
  // the angles of all 16 columns this lane's slots hold, read together
  float2 rc[kPage];
#pragma unroll
  for (int tt = 0; tt < kPage; ++tt) rc[tt] = rot[i ^ tt];
  __builtin_amdgcn_sched_barrier(0);
  // columns: slot t is column x = i ^ t, rotated with column x ^ M (slot t ^ M);
  // updated in place one slot pair at a time
#pragma unroll
  for (int tt = 0; tt < kPage; ++tt) {
    if (tt < (tt ^ M)) {
      const int t2 = tt ^ M;
      const float2 r1 = rc[tt], r2 = rc[t2];
      a[tt] = fmaf(r1.x, ar[tt], r1.y * ar[t2]);
      a[t2] = fmaf(r2.x, ar[t2], r2.y * ar[tt]);
      const float u1 = u[tt], u2 = u[t2];
      u[tt] = fmaf(r1.x, u1, r1.y * u2);
      u[t2] = fmaf(r2.x, u2, r2.y * u1);
      // pin the update to this round (an empty asm consuming the value): nothing
      // reads U until the end, and sinking the rotations would keep every
      // round's angles live
      asm volatile("" : "+v"(u[tt]), "+v"(u[t2]));
    }
  }
  a[M] = live ? 0.f : a[M];
  wave_lds_sync();  // every lane has read this round's angles
}

// The same round for a wave that holds one page: lanes 0-15 hold the rows of
// A and lanes 16-31 the rows of U (slot-permuted alike), so one column
// rotation updates both. Rows of U skip the row rotation (c = 1, s = 0) and
// only rows of A publish their angles; lanes 32-63 hold zeros.
template <int M>
__device__ __forceinline__ void jacobi_round_shared(float (&x)[kPage], int i, bool arow, float2* rot) {
  const bool lower = i < (i ^ M);
  float pa[kPage];
#pragma unroll
  for (int tt = 0; tt < kPage; ++tt) pa[tt] = swz<M>(x[tt ^ M]);
  __builtin_amdgcn_sched_barrier(0);
  const float d_me = x[0], d_other = pa[M];
  const float o_me = x[M], o_other = pa[0];
  const float app = lower ? d_me : d_other, aqq = lower ? d_other : d_me;
  const float apq = lower ? o_me : o_other;
  const float safe = (apq != 0.f) ? apq : 1.f;
  const float tau = (aqq - app) * __builtin_amdgcn_rcpf(2.f * safe);
  const float t = copysignf(1.0f, tau) *
                  __builtin_amdgcn_rcpf(fabsf(tau) + __builtin_amdgcn_sqrtf(fmaf(tau, tau, 1.f)));
  const float c = (apq != 0.f) ? __builtin_amdgcn_rsqf(fmaf(t, t, 1.f)) : 1.f;
  const float s = (apq != 0.f) ? t * c : 0.f;
  const float sg = lower ? -s : s;
  const float cr = arow ? c : 1.f, sr = arow ? sg : 0.f;
  float ar[kPage];
#pragma unroll
  for (int tt = 0; tt < kPage; ++tt) ar[tt] = fmaf(cr, x[tt], sr * pa[tt]);
  if (arow) rot[i] = make_float2(c, sg);
  wave_lds_sync();
  float2 rc[kPage];
#pragma unroll
  for (int tt = 0; tt < kPage; ++tt) rc[tt] = rot[i ^ tt];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int tt = 0; tt < kPage; ++tt) {
    if (tt < (tt ^ M)) {
      const int t2 = tt ^ M;
      const float2 r1 = rc[tt], r2 = rc[t2];
      x[tt] = fmaf(r1.x, ar[tt], r1.y * ar[t2]);
      x[t2] = fmaf(r2.x, ar[t2], r2.y * ar[tt]);
    }
  }
  x[M] = arow ? 0.f : x[M];
  wave_lds_sync();  // every lane has read this round's angles
}

__device__ __forceinline__ void jacobi_sweep_shared(float (&x)[kPage], int i, bool arow, float2* rot) {
  jacobi_round_shared<1>(x, i, arow, rot);
  jacobi_round_shared<2>(x, i, arow, rot);
  jacobi_round_shared<3>(x, i, arow, rot);
  jacobi_round_shared<4>(x, i, arow, rot);
  jacobi_round_shared<5>(x, i, arow, rot);
  jacobi_round_shared<6>(x, i, arow, rot);
  jacobi_round_shared<7>(x, i, arow, rot);
  jacobi_round_shared<8>(x, i, arow, rot);
  jacobi_round_shared<9>(x, i, arow, rot);
  jacobi_round_shared<10>(x, i, arow, rot);
  jacobi_round_shared<11>(x, i, arow, rot);
  jacobi_round_shared<12>(x, i, arow, rot);
  jacobi_round_shared<13>(x, i, arow, rot);
  jacobi_round_shared<14>(x, i, arow, rot);
  jacobi_round_shared<15>(x, i, arow, rot);
}

__device__ __forceinline__ void jacobi_sweep(float (&a)[kPage], float (&u)[kPage], int i, bool live,
                                             float2* rot) {
  jacobi_round<1>(a, u, i, live, rot);
  jacobi_round<2>(a, u, i, live, rot);
  jacobi_round<3>(a, u, i, live, rot);
  jacobi_round<4>(a, u, i, live, rot);
  jacobi_round<5>(a, u, i, live, rot);
  jacobi_round<6>(a, u, i, live, rot);
  jacobi_round<7>(a, u, i, live, rot);
  jacobi_round<8>(a, u, i, live, rot);
  jacobi_round<9>(a, u, i, live, rot);
  jacobi_round<10>(a, u, i, live, rot);
  jacobi_round<11>(a, u, i, live, rot);
  jacobi_round<12>(a, u, i, live, rot);
  jacobi_round<13>(a, u, i, live, rot);
  jacobi_round<14>(a, u, i, live, rot);
  jacobi_round<15>(a, u, i, live, rot);
}

// (b, j, kvh) of work item `item` (or (list entry, kvh) for a block list);
// blk < 0 when there is nothing to build
__device__ __forceinline__ int item_block(const BuildArgs& a, long long item, int* kvh) {
  *kvh = 0;
  if (item >= a.items) return -1;
  *kvh = (int)(item % a.Hkv);
  if (a.blocks) {
    const int blk = a.blocks[item / a.Hkv];
    return (blk >= 0 && blk < a.num_blocks) ? blk : -1;
  }
  if (a.fill) {
    // the last full page of sequence b, when it filled in this step
    const int b = (int)(item / a.Hkv);
    const int n = full_pages(a.seq_lens, nullptr, b, a.N);
    if (n == full_pages(a.seq_lens, a.fill, b, a.N)) return -1;  // nothing filled
    const int blk = a.page_table[(size_t)b * a.N + n - 1];
    return (blk >= 0 && blk < a.num_blocks) ? blk : -1;
  }
  const long long bj = item / a.Hkv;
  const int j = (int)(bj % a.N);
  const int b = (int)(bj / a.N);
  if (j >= full_pages(a.seq_lens, nullptr, b, a.N)) return -1;
  const int blk = a.page_table[(size_t)b * a.N + j];
  return (blk >= 0 && blk < a.num_blocks) ? blk : -1;
}

// Phases 1 and 2 for the PPW pages of a wave (items item0 .. item0 + PPW - 1):
// per page the centroid, the deviation energy and the Gram rows into LDS, then
// the eigenproblems; leaves S.lam, S.perm, S.UT, S.energy.
template <int PPW, class LdsT>
__device__ __forceinline__ void eigen_phases(const BuildArgs& a, LdsT& S, long long item0, int lane) {
  const int ti = lane & 15, kg = lane >> 4;
  // ================================================ 1. centroid, deviations, Gram
#pragma unroll 1
  for (int pg = 0; pg < PPW; ++pg) {
    int kvh;
    const int blk = item_block(a, item0 + pg, &kvh);
    float kf[32];
    if (blk >= 0) {
      const uint4* src = reinterpret_cast<const uint4*>(
          a.kc + ((size_t)blk * a.Hkv + kvh) * (kPage * kDim) + ti * kDim + kg * 32);
#pragma unroll
      for (int uu = 0; uu < 4; ++uu) {
        const uint4 w = src[uu];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kf[uu * 8 + 2 * e] = bf16lo(ws[e]);
          kf[uu * 8 + 2 * e + 1] = bf16hi(ws[e]);
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < 32; ++s) kf[s] = 0.f;
    }
    // centroid of d = 32kg + s: sum over the 16 token lanes of the group
    float en = 0.f;
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      const float mu = row16_reduce(kf[s], [](float x, float y) { return x + y; }) * (1.0f / kPage);
      kf[s] -= mu;
      en = fmaf(kf[s], kf[s], en);
    }
    en = wave_sum(en);
    if (lane == 0) S.energy[pg] = en;
    v4f g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 32; ++s) g = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[s], kf[s], g, 0, 0, 0);
    // lane holds G[4kg + r][ti]; row i stores column ti at slot i ^ ti
#pragma unroll
    for (int r = 0; r < 4; ++r) S.A[pg][4 * kg + r][(4 * kg + r) ^ ti] = g[r];
  }
  wave_lds_sync();

  // ================================================ 2. four eigenproblems, 16 lanes each
  {
    const int pg = lane >> 4, i = lane & 15;
    const auto add = [](float x, float y) { return x + y; };
    float a_[kPage];
    if constexpr (PPW == 1) {
      // one page: A in lanes 0-15, U in lanes 16-31 (identity: U[i][i ^ t] =
      // (t == 0)), rotated by the same instructions; lanes 32-63 hold zeros
      const bool arow = lane < 16;
#pragma unroll
      for (int tt = 0; tt < kPage; ++tt)
        a_[tt] = arow ? S.A[0][i][tt] : ((lane < 32 && tt == 0) ? 1.0f : 0.0f);
      for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
        float off = 0.f, tot = a_[0] * a_[0];
#pragma unroll
        for (int tt = 1; tt < kPage; ++tt) off = fmaf(a_[tt], a_[tt], off);
        tot += off;
        off = row16_reduce(off, add);
        tot = row16_reduce(tot, add);
        if (__ballot(arow && off > kOffTol * tot) == 0) break;  // converged
        jacobi_sweep_shared(a_, i, arow, S.rot[0]);
      }
      if (arow) S.diag[0][i] = a_[0];
      // (storage shared with the Gram rows read above: one wave's LDS
      // operations complete in order, and the union keeps the compiler from
      // reordering them)
      if (lane >= 16 && lane < 32) {
#pragma unroll
        for (int tt = 0; tt < kPage; ++tt) S.UT[0][i ^ tt][i] = a_[tt];
      }
    } else {
      float u_[kPage];
#pragma unroll
      for (int tt = 0; tt < kPage; ++tt) {
        a_[tt] = S.A[pg][i][tt];
        u_[tt] = (tt == 0) ? 1.0f : 0.0f;  // identity: U[i][i ^ t] = (t == 0)
      }
      for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
        float off = 0.f, tot = a_[0] * a_[0];
#pragma unroll
        for (int tt = 1; tt < kPage; ++tt) off = fmaf(a_[tt], a_[tt], off);
        tot += off;
        off = row16_reduce(off, add);
        tot = row16_reduce(tot, add);
        // a converged page stays as it is (as a wave with one page stops there)
        const bool live = off > kOffTol * tot;
        if (__ballot(live) == 0) break;  // every page converged
        jacobi_sweep(a_, u_, i, live, S.rot[pg]);
      }
      S.diag[pg][i] = a_[0];
      // (storage shared with the Gram rows this wave read above: one wave's LDS
      // operations complete in order, and the union keeps the compiler from
      // reordering them)
#pragma unroll
      for (int tt = 0; tt < kPage; ++tt) S.UT[pg][i ^ tt][i] = u_[tt];
    }
    wave_lds_sync();
    // eigenvalues in descending order, equal values keep index order
    if (pg < PPW) {
      const float lx = a_[0];
      int rank = 0;
#pragma unroll
      for (int y = 0; y < kPage; ++y) {
        const float ly = S.diag[pg][y];
        rank += (ly > lx) || (ly == lx && y < i);
      }
      S.perm[pg][rank] = i;
      S.lam[pg][rank] = lx;
    }
  }
  wave_lds_sync();

}
// Phase 3, shared part, for page pg of the wave (block blk, KV head kvh):
// the lane's key dims d = 2*lane, 2*lane+1 of the 16 tokens are reloaded and
// centred (mu0, mu1), and the first R basis vectors V[:,k] = D^T u_k /
// sqrt(lambda_k) are formed with the sign rule applied (sgn[k] = the flip).
template <int R, class LdsT>
__device__ __forceinline__ void lane_basis(const BuildArgs& a, const LdsT& S, int pg, int blk, int kvh,
                                           int lane, float& mu0, float& mu1, float (&v)[R][2],
                                           float (&sgn)[R], float& lam0, float& en) {
    // keys d = 2*lane, 2*lane+1 of all 16 tokens
    const uint32_t* kw = reinterpret_cast<const uint32_t*>(
        a.kc + ((size_t)blk * a.Hkv + kvh) * (kPage * kDim)) + lane;
    float d0[kPage], d1[kPage];
    float m0 = 0.f, m1 = 0.f;
#pragma unroll
    for (int i = 0; i < kPage; ++i) {
      const uint32_t w = kw[i * (kDim / 2)];
      d0[i] = bf16lo(w);
      d1[i] = bf16hi(w);
      m0 += d0[i];
      m1 += d1[i];
    }
    mu0 = m0 * (1.0f / kPage);
    mu1 = m1 * (1.0f / kPage);
#pragma unroll
    for (int i = 0; i < kPage; ++i) {
      d0[i] -= mu0;
      d1[i] -= mu1;
    }
    lam0 = S.lam[pg][0];
    en = S.energy[pg];
    // ---- basis V[:,k] = D^T u_k / sqrt(lambda_k) for d = 2*lane, 2*lane+1
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const float lk = S.lam[pg][k];
      const bool keep = lam0 > 0.f && lk > 1e-6f * lam0 && lk > 1e-10f * en;
      const int col = S.perm[pg][k];
      float s0 = 0.f, s1 = 0.f;
      if (keep) {
        const float4* uc = reinterpret_cast<const float4*>(&S.UT[pg][col][0]);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 uq = uc[q4];
          const float us[4] = {uq.x, uq.y, uq.z, uq.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s0 = fmaf(d0[4 * q4 + e], us[e], s0);
            s1 = fmaf(d1[4 * q4 + e], us[e], s1);
          }
        }
        const float inv = 1.0f / sqrtf(lk);
        s0 *= inv;
        s1 *= inv;
      }
      v[k][0] = s0;
      v[k][1] = s1;
    }
    // ---- sign: largest-|.| entry of each basis vector positive (lowest d on ties)
#pragma unroll
    for (int k = 0; k < R; ++k) {
      float best = fabsf(v[k][0]);
      int bd = 2 * lane;
      float bv = v[k][0];
      if (fabsf(v[k][1]) > best) { best = fabsf(v[k][1]); bd = 2 * lane + 1; bv = v[k][1]; }
      // wave argmax of |v| (lowest d on ties); every step pairs lanes
      // symmetrically, so all lanes end with the same winner
      auto take = [&](float ob, int od, float ov) {
        if (ob > best || (ob == best && od < bd)) { best = ob; bd = od; bv = ov; }
      };
      take(dpp_mov<kDppXor1>(best), (int)dpp_mov<kDppXor1>((uint32_t)bd), dpp_mov<kDppXor1>(bv));
      take(dpp_mov<kDppXor2>(best), (int)dpp_mov<kDppXor2>((uint32_t)bd), dpp_mov<kDppXor2>(bv));
      take(dpp_mov<kDppHalfMirror>(best), (int)dpp_mov<kDppHalfMirror>((uint32_t)bd),
           dpp_mov<kDppHalfMirror>(bv));
      take(dpp_mov<kDppMirror>(best), (int)dpp_mov<kDppMirror>((uint32_t)bd), dpp_mov<kDppMirror>(bv));
      {
        const auto rb = __builtin_amdgcn_permlane16_swap(__float_as_uint(best), __float_as_uint(best), false, false);
        const auto rd = __builtin_amdgcn_permlane16_swap((uint32_t)bd, (uint32_t)bd, false, false);
        const auto rv = __builtin_amdgcn_permlane16_swap(__float_as_uint(bv), __float_as_uint(bv), false, false);
        best = __uint_as_float(rb[0]); bd = (int)rd[0]; bv = __uint_as_float(rv[0]);
        take(__uint_as_float(rb[1]), (int)rd[1], __uint_as_float(rv[1]));
      }
      {
        const auto rb = __builtin_amdgcn_permlane32_swap(__float_as_uint(best), __float_as_uint(best), false, false);
        const auto rd = __builtin_amdgcn_permlane32_swap((uint32_t)bd, (uint32_t)bd, false, false);
        const auto rv = __builtin_amdgcn_permlane32_swap(__float_as_uint(bv), __float_as_uint(bv), false, false);
        best = __uint_as_float(rb[0]); bd = (int)rd[0]; bv = __uint_as_float(rv[0]);
        take(__uint_as_float(rb[1]), (int)rd[1], __uint_as_float(rv[1]));
      }
      sgn[k] = (bv < 0.f) ? -1.0f : 1.0f;
      v[k][0] *= sgn[k];
      v[k][1] *= sgn[k];
    }
}

// PPW pages per wave: 4 for throughput; 1 when there are few items (a list of
// pages that just filled), so phases 1 and 3, which walk a wave's pages one
// after another, take a quarter of the time and more waves share the work.
// Phases 1-3 for the PPW pages of one wave (items item0 .. item0 + PPW - 1):
// every record of those items written to a.summ. Waves are independent (no
// workgroup barrier), so a kernel may run this in any of its waves.
template <int PPW>
__device__ __forceinline__ void build_wave(const BuildArgs& a, WaveLds& S, long long item0, int lane) {
  static_assert(PPW == 1 || PPW == kPagesPerWave, "pages per wave");
  eigen_phases<PPW>(a, S, item0, lane);

  // ================================================ 3. basis, coefficients, codes, record
#pragma unroll 1
  for (int pg = 0; pg < PPW; ++pg) {
    int kvh;
    const int blk = item_block(a, item0 + pg, &kvh);
    if (blk < 0) continue;  // wave-uniform
    float mu0, mu1, v[kRank][2], sgn[kRank], lam0, en;
    lane_basis<kRank>(a, S, pg, blk, kvh, lane, mu0, mu1, v, sgn, lam0, en);
    // ---- coefficients C[i][k] = sqrt(lambda_k) u_k[i]: lane owns (i, k) pairs lane, lane+64
    float cval[2];
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
      const int e = lane + 64 * uu, i = e >> 3, k = e & 7;
      const float lk = S.lam[pg][k];
      const bool keep = lam0 > 0.f && lk > 1e-6f * lam0 && lk > 1e-10f * en;
      cval[uu] = keep ? sqrtf(lk) * S.UT[pg][S.perm[pg][k]][i] * sgn[k] : 0.f;
    }
    // ---- absmax scales
    float am_mu = fmaxf(fabsf(mu0), fabsf(mu1));
    float am_v = 0.f;
#pragma unroll
    for (int k = 0; k < kRank; ++k) am_v = fmaxf(am_v, fmaxf(fabsf(v[k][0]), fabsf(v[k][1])));
    float am_c = fmaxf(fabsf(cval[0]), fabsf(cval[1]));
    am_mu = wave_max(am_mu);
    am_v = wave_max(am_v);
    am_c = wave_max(am_c);
    const float s_mu = f16_round(am_mu / 127.0f), s_v = f16_round(am_v / 7.0f),
                s_c = f16_round(am_c / 127.0f);

    // ---- codes into the LDS record
#pragma unroll
    for (int k = 0; k < kRank; ++k) {
      S.vq[k][2 * lane] = (int8_t)quant(v[k][0], s_v, 7);
      S.vq[k][2 * lane + 1] = (int8_t)quant(v[k][1], s_v, 7);
    }
    S.rec[kMuOff + 2 * lane] = (uint8_t)(int8_t)quant(mu0, s_mu, 127);
    S.rec[kMuOff + 2 * lane + 1] = (uint8_t)(int8_t)quant(mu1, s_mu, 127);
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) S.rec[kCOff + lane + 64 * uu] = (uint8_t)(int8_t)quant(cval[uu], s_c, 127);
    if (lane < (kStride - kSOff) / 4) {  // bytes [768, 784): scales then zero padding, as dwords
      uint32_t w = 0;
      if (lane == 0) w = f16_bits(s_mu) | (f16_bits(s_v) << 16);
      if (lane == 1) w = f16_bits(s_c);
      *reinterpret_cast<uint32_t*>(&S.rec[kSOff + 4 * lane]) = w;
    }
    wave_lds_sync();
    // V words: word w of row k, byte b = V[8w+b][k] (low nibble) | V[8w+4+b][k] (high nibble)
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
      const int e = lane + 64 * uu, k = e >> 4, w = e & 15;
      uint32_t word = 0;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const uint32_t lo = (uint32_t)S.vq[k][8 * w + bb] & 0xFu;
        const uint32_t hi = (uint32_t)S.vq[k][8 * w + 4 + bb] & 0xFu;
        word |= (lo | (hi << 4)) << (8 * bb);
      }
      *reinterpret_cast<uint32_t*>(&S.rec[kVOff + k * 64 + w * 4]) = word;
    }
    wave_lds_sync();
    uint32_t* dst = reinterpret_cast<uint32_t*>(a.summ + ((size_t)blk * a.Hkv + kvh) * kStride);
    const uint32_t* srcw = reinterpret_cast<const uint32_t*>(S.rec);
    for (int e = lane; e < kStride / 4; e += 64) dst[e] = srcw[e];
    wave_lds_sync();  // the record buffer is reused by the next page
  }
}


}  // namespace

}  // namespace locks
