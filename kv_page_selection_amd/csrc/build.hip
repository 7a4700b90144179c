// build.hip — summary build, one wave per (block, KV head) page (gfx950).
//
// Steps (blog post, "How LOCKS works" and "Code" build loop; technical summary,
// section 2 mechanism 1): centroid mu = mean of the page's 16 keys; centred
// deviations D = K - 1 mu^T; eigendecomposition of the 16x16 Gram D D^T;
// the 8 leading eigenpairs give the basis V[:,k] = D^T u_k / sqrt(lambda_k) and
// coefficients C[:,k] = sqrt(lambda_k) u_k (= D V); fp16 absmax scales; codes
// int8 (mu, C, +-127) and int4 (V, +-7), round half to even; pack the record.
//
// Mapping: lane (token i = lane%16, K group kg = lane/16) holds key row i,
// d in [32kg, 32kg+32). The Gram is 32 chained v_mfma_f32_16x16x4_f32 with the
// same register as A and B (lane (i, kg) holds D[i][32kg+s]; for a sum over d
// only the pairing of A and B lanes matters, which is symmetric). The
// eigensolver is cyclic Jacobi in parallel (round-robin) order: 15 rounds of 8
// disjoint rotations per sweep, applied to LDS copies of the Gram and the
// eigenvector matrix. Waves are independent (wave-scope LDS ordering only).
#include "device_common.h"
#include "internal.h"

namespace locks {

namespace {

constexpr int kWaves = 4;
constexpr int kMaxSweeps = 12;

struct BuildArgs {
  const uint16_t* kc;
  const int32_t* page_table;
  const int32_t* seq_lens;
  uint8_t* summ;
  int B, Hkv, N, num_blocks;
};

struct WaveLds {
  float D[kPage][kDim];
  float A[kPage][kPage + 1];
  float U[kPage][kPage + 1];
  float mu[kDim];
  int mate[kPage];
  float cx[kPage], sx[kPage];
  int perm[kPage];
  float lam[kPage];
  int8_t vq[kRank][kDim];
  __align__(16) uint8_t rec[kStride];
};

__device__ __forceinline__ int quant(float x, float s, int qmax) {
  if (!(s > 0.f) || isinf(s)) return 0;
  const float c = rintf(__fdiv_rn(x, s));
  return (int)fminf(fmaxf(c, (float)-qmax), (float)qmax);
}

__device__ __forceinline__ float f16_round(float x) { return (float)(_Float16)x; }

__device__ __forceinline__ uint32_t f16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

__global__ __launch_bounds__(256) void build_kernel(BuildArgs a) {
  __shared__ WaveLds lds_all[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  WaveLds& S = lds_all[wave];
  const long long item = (long long)blockIdx.x * kWaves + wave;  // (b, j, kvh)
  const int kvh = (int)(item % a.Hkv);
  const long long bj = item / a.Hkv;
  const int j = (int)(bj % a.N);
  const int b = (int)(bj / a.N);
  if (b >= a.B) return;
  if (j >= full_pages(a.seq_lens, b, a.N)) return;
  const int blk = a.page_table[(size_t)b * a.N + j];
  if (blk < 0 || blk >= a.num_blocks) return;

  const int ti = lane & 15, kg = lane >> 4;
  // ---- keys: row ti, d in [32kg, 32kg+32)
  float kf[32];
  {
    const uint4* src = reinterpret_cast<const uint4*>(
        a.kc + ((size_t)blk * a.Hkv + kvh) * (kPage * kDim) + ti * kDim + kg * 32);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 w = src[u];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[u * 8 + 2 * e] = bf16lo(ws[e]);
        kf[u * 8 + 2 * e + 1] = bf16hi(ws[e]);
      }
    }
  }
  float energy = 0.f;
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    S.D[ti][kg * 32 + s] = kf[s];
    energy = fmaf(kf[s], kf[s], energy);
  }
  energy = wave_sum(energy);
  wave_lds_sync();
  // ---- centroid (lane owns d = 2*lane, 2*lane+1)
  {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < kPage; ++i) {
      s0 += S.D[i][2 * lane];
      s1 += S.D[i][2 * lane + 1];
    }
    S.mu[2 * lane] = s0 * (1.0f / kPage);
    S.mu[2 * lane + 1] = s1 * (1.0f / kPage);
  }
  wave_lds_sync();
  // ---- deviations, in registers and in LDS
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    kf[s] -= S.mu[kg * 32 + s];
    S.D[ti][kg * 32 + s] = kf[s];
  }
  // ---- Gram = D D^T (16x16) on MFMA
  v4f g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 32; ++s) g = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[s], kf[s], g, 0, 0, 0);
  // lane (col ti, row group kg) holds G[4kg + r][ti]
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    S.A[4 * kg + r][ti] = g[r];
    S.U[4 * kg + r][ti] = (4 * kg + r == ti) ? 1.0f : 0.0f;
  }
  wave_lds_sync();

  // ---- parallel cyclic Jacobi
  for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
    float off = 0.f, tot = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = lane + 64 * u, r = e >> 4, c = e & 15;
      const float v = S.A[r][c];
      tot = fmaf(v, v, tot);
      if (r != c) off = fmaf(v, v, off);
    }
    off = wave_sum(off);
    tot = wave_sum(tot);
    if (!(off > 1.6e-13f * tot)) break;  // off-diagonal norm below ~4e-7 of the whole
    for (int round = 0; round < 15; ++round) {
      if (lane < 8) {
        const int p = (lane == 0) ? 15 : (round + lane) % 15;
        const int q = (lane == 0) ? round : (round - lane + 15) % 15;
        const float app = S.A[p][p], aqq = S.A[q][q], apq = S.A[p][q];
        float c = 1.f, s = 0.f;
        if (apq != 0.f) {
          const float tau = (aqq - app) / (2.f * apq);
          const float t = copysignf(1.0f, tau) / (fabsf(tau) + sqrtf(fmaf(tau, tau, 1.f)));
          c = 1.0f / sqrtf(fmaf(t, t, 1.f));
          s = t * c;
        }
        S.mate[p] = q; S.cx[p] = c; S.sx[p] = -s;
        S.mate[q] = p; S.cx[q] = c; S.sx[q] = s;
      }
      wave_lds_sync();
      // columns: A <- A J, U <- U J
      float na[4], nu[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = lane + 64 * u, r = e >> 4, x = e & 15;
        const int mt = S.mate[x];
        const float cxv = S.cx[x], sxv = S.sx[x];
        na[u] = cxv * S.A[r][x] + sxv * S.A[r][mt];
        nu[u] = cxv * S.U[r][x] + sxv * S.U[r][mt];
      }
      wave_lds_sync();
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = lane + 64 * u, r = e >> 4, x = e & 15;
        S.A[r][x] = na[u];
        S.U[r][x] = nu[u];
      }
      wave_lds_sync();
      // rows: A <- J^T A
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = lane + 64 * u, x = e >> 4, c = e & 15;
        const int mt = S.mate[x];
        na[u] = S.cx[x] * S.A[x][c] + S.sx[x] * S.A[mt][c];
      }
      wave_lds_sync();
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = lane + 64 * u, x = e >> 4, c = e & 15;
        S.A[x][c] = (S.mate[x] == c) ? 0.0f : na[u];  // the rotated pair is exactly zeroed
      }
      wave_lds_sync();
    }
  }

  // ---- eigenvalues in descending order, equal values keep index order
  if (lane < kPage) {
    const float lx = S.A[lane][lane];
    int rank = 0;
    for (int y = 0; y < kPage; ++y) {
      const float ly = S.A[y][y];
      rank += (ly > lx) || (ly == lx && y < lane);
    }
    S.perm[rank] = lane;
    S.lam[rank] = lx;
  }
  wave_lds_sync();
  const float lam0 = S.lam[0];
  // ---- basis V[:,k] = D^T u_k / sqrt(lambda_k) for d = 2*lane, 2*lane+1
  float v[kRank][2];
#pragma unroll
  for (int k = 0; k < kRank; ++k) {
    const float lk = S.lam[k];
    const bool keep = lam0 > 0.f && lk > 1e-6f * lam0 && lk > 1e-10f * energy;
    const int col = S.perm[k];
    float s0 = 0.f, s1 = 0.f;
    if (keep) {
#pragma unroll
      for (int i = 0; i < kPage; ++i) {
        const float uik = S.U[i][col];
        s0 = fmaf(S.D[i][2 * lane], uik, s0);
        s1 = fmaf(S.D[i][2 * lane + 1], uik, s1);
      }
      const float inv = 1.0f / sqrtf(lk);
      s0 *= inv;
      s1 *= inv;
    }
    v[k][0] = s0;
    v[k][1] = s1;
  }
  // ---- sign: largest-|.| entry of each basis vector positive (lowest d on ties)
  float sgn[kRank];
#pragma unroll
  for (int k = 0; k < kRank; ++k) {
    float best = fabsf(v[k][0]);
    int bd = 2 * lane;
    float bv = v[k][0];
    if (fabsf(v[k][1]) > best) { best = fabsf(v[k][1]); bd = 2 * lane + 1; bv = v[k][1]; }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ob = __shfl_xor(best, o);
      const int od = __shfl_xor(bd, o);
      const float ov = __shfl_xor(bv, o);
      if (ob > best || (ob == best && od < bd)) { best = ob; bd = od; bv = ov; }
    }
    sgn[k] = (bv < 0.f) ? -1.0f : 1.0f;
    v[k][0] *= sgn[k];
    v[k][1] *= sgn[k];
  }
  // ---- coefficients C[i][k] = sqrt(lambda_k) u_k[i]: lane owns (i, k) pairs lane, lane+64
  float cval[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = lane + 64 * u, i = e >> 3, k = e & 7;
    const float lk = S.lam[k];
    const bool keep = lam0 > 0.f && lk > 1e-6f * lam0 && lk > 1e-10f * energy;
    cval[u] = keep ? sqrtf(lk) * S.U[i][S.perm[k]] * sgn[k] : 0.f;
  }
  // ---- absmax scales
  float am_mu = fmaxf(fabsf(S.mu[2 * lane]), fabsf(S.mu[2 * lane + 1]));
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
  S.rec[kMuOff + 2 * lane] = (uint8_t)(int8_t)quant(S.mu[2 * lane], s_mu, 127);
  S.rec[kMuOff + 2 * lane + 1] = (uint8_t)(int8_t)quant(S.mu[2 * lane + 1], s_mu, 127);
#pragma unroll
  for (int u = 0; u < 2; ++u) S.rec[kCOff + lane + 64 * u] = (uint8_t)(int8_t)quant(cval[u], s_c, 127);
  if (lane < (kStride - kSOff) / 4) {  // bytes [768, 784): scales then zero padding, as dwords
    uint32_t w = 0;
    if (lane == 0) w = f16_bits(s_mu) | (f16_bits(s_v) << 16);
    if (lane == 1) w = f16_bits(s_c);
    *reinterpret_cast<uint32_t*>(&S.rec[kSOff + 4 * lane]) = w;
  }
  wave_lds_sync();
  // V words: word w of row k, byte b = V[8w+b][k] (low nibble) | V[8w+4+b][k] (high nibble)
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = lane + 64 * u, k = e >> 4, w = e & 15;
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
}

}  // namespace

hipError_t launch_build(const locks_dims& d, const uint16_t* kc, const int32_t* pt,
                        const int32_t* sl, uint8_t* summ, hipStream_t s) {
  BuildArgs a;
  a.kc = kc;
  a.page_table = pt;
  a.seq_lens = sl;
  a.summ = summ;
  a.B = d.batch;
  a.Hkv = d.n_kv_heads;
  a.N = d.max_pages_per_seq;
  a.num_blocks = d.num_blocks;
  const long long items = (long long)d.batch * d.max_pages_per_seq * d.n_kv_heads;
  const long long wgs = (items + kWaves - 1) / kWaves;
  if (wgs <= 0) return hipSuccess;
  hipLaunchKernelGGL(build_kernel, dim3((unsigned)wgs), dim3(64 * kWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace locks
