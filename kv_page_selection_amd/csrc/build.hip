// build.hip — summary build (gfx950): 4 pages per wave (1 for a short list
// of pages that just filled).
//
// Steps (blog post, "How LOCKS works" and "Code" build loop; technical summary,
// section 2 mechanism 1): centroid mu = mean of the page's 16 keys; centred
// deviations D = K - 1 mu^T; eigendecomposition of the 16x16 Gram D D^T;
// the 8 leading eigenpairs give the basis V[:,k] = D^T u_k / sqrt(lambda_k) and
// coefficients C[:,k] = sqrt(lambda_k) u_k (= D V); fp16 absmax scales; codes
// int8 (mu, C, +-127) and int4 (V, +-7), round half to even; pack the record.
//
// A wave builds 4 page records in three phases:
//  1. per page, all 64 lanes: lane (token i = lane%16, group kg = lane/16)
//     holds key row i, d in [32kg, 32kg+32); the centroid comes from 16-lane
//     row sums, and the Gram is 32 chained v_mfma_f32_16x16x4_f32 with the
//     same register as A and B (for a sum over d only the pairing of A and B
//     lanes matters, which is symmetric).
//  2. the 4 eigenproblems at once, 16 lanes each: lane i holds row i of the
//     Gram and of the eigenvector matrix in registers, column-permuted by XOR
//     (slot t = column i ^ t). Cyclic Jacobi with XOR pairings: round m of a
//     sweep rotates the 8 pairs (i, i ^ m), m = 1..15, so every pair is
//     rotated once per sweep. In this layout the diagonal is slot 0, the
//     rotated element is slot m, the partner row is one ds_swizzle (XOR m)
//     away and reads slot-permuted by XOR m, and the column rotation of slot
//     t uses the angle of column i ^ t, published through a 16-entry LDS
//     table: no register is indexed per lane. A wave with one page holds the
//     eigenvector rows in lanes 16-31 instead, so the same instructions
//     rotate both matrices.
//  3. per page, all 64 lanes: lane owns d = 2*lane, 2*lane+1 of all 16 keys
//     (reloaded, L2-resident), forms V, the sign rule, C, the scales and the
//     codes, and writes the record.
#include "build_device.h"

namespace locks {

namespace {

template <int PPW>
__global__ __launch_bounds__(64 * kWaves) void build_kernel(BuildArgs a) {
  __shared__ WaveLds lds_all[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  build_wave<PPW>(a, lds_all[wave], ((long long)blockIdx.x * kWaves + wave) * PPW, lane);
}

// ---------------------------------------------------------------------------
// Variant record formats (the precision / rank ablation; blog post "Caveats":
// Theorem 1 covers unquantised summaries, int4 loses a few recall points, int2
// collapses). Rank R in {4, 8, 16}; V stored in VB in {2, 4} bits (signed codes,
// range +-(2^(VB-1) - 1)) or 16 (fp16 values); mu and C as int8 codes, or fp16
// values when VB = 16. Layout: V [d][k] row-major, element e = d*R + k in bits
// [e*VB, (e+1)*VB), little-endian; mu[128]; C[16][R]; fp16 scales
// {s_mu, s_V, s_C, 0} (1.0 for fp16 tensors); zero padding to 16 bytes.
template <int R, int VB>
struct VariantFmt {
  static constexpr int MB = VB == 16 ? 16 : 8;
  static constexpr int kV = kDim * R * VB / 8;        // V bytes
  static constexpr int kMu = kV;                      // offset of mu
  static constexpr int kC = kMu + kDim * MB / 8;      // offset of C
  static constexpr int kS = kC + kPage * R * MB / 8;  // offset of the scales
  static constexpr int kBytes = (kS + 8 + 15) / 16 * 16;
};

__device__ __forceinline__ uint32_t variant_code(float x, float s, int bits) {
  if (bits == 16) return f16_bits(x);
  return (uint32_t)quant(x, s, (1 << (bits - 1)) - 1) & ((1u << bits) - 1u);
}

template <int R, int VB>
__global__ __launch_bounds__(64 * kWaves) void build_variant_kernel(BuildArgs a) {
  using F = VariantFmt<R, VB>;
  constexpr int MB = F::MB;
  __shared__ WaveLdsT<F::kBytes> lds_all[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  WaveLdsT<F::kBytes>& S = lds_all[wave];
  const long long item0 = ((long long)blockIdx.x * kWaves + wave) * kPagesPerWave;
  eigen_phases<kPagesPerWave>(a, S, item0, lane);
#pragma unroll 1
  for (int pg = 0; pg < kPagesPerWave; ++pg) {
    int kvh;
    const int blk = item_block(a, item0 + pg, &kvh);
    if (blk < 0) continue;  // wave-uniform
    float mu0, mu1, v[R][2], sgn[R], lam0, en;
    lane_basis<R>(a, S, pg, blk, kvh, lane, mu0, mu1, v, sgn, lam0, en);
    // coefficients C[i][k] = sqrt(lambda_k) u_k[i] (= D V): lane takes e = lane + 64 t
    constexpr int kCpl = (kPage * R + 63) / 64;
    float cval[kCpl];
#pragma unroll
    for (int t = 0; t < kCpl; ++t) {
      const int e = lane + 64 * t, i = e / R, k = e % R;
      cval[t] = 0.f;
      if (e < kPage * R) {
        const float lk = S.lam[pg][k];
        const bool keep = lam0 > 0.f && lk > 1e-6f * lam0 && lk > 1e-10f * en;
        cval[t] = keep ? sqrtf(lk) * S.UT[pg][S.perm[pg][k]][i] * sgn[k] : 0.f;
      }
    }
    // scales: fp16(absmax / qmax) for codes, 1.0 for fp16 values
    float am_mu = fmaxf(fabsf(mu0), fabsf(mu1)), am_v = 0.f, am_c = 0.f;
#pragma unroll
    for (int k = 0; k < R; ++k) am_v = fmaxf(am_v, fmaxf(fabsf(v[k][0]), fabsf(v[k][1])));
#pragma unroll
    for (int t = 0; t < kCpl; ++t) am_c = fmaxf(am_c, fabsf(cval[t]));
    am_mu = wave_max(am_mu);
    am_v = wave_max(am_v);
    am_c = wave_max(am_c);
    const float s_v = VB == 16 ? 1.0f : f16_round(am_v / (float)((1 << (VB - 1)) - 1));
    const float s_mu = MB == 16 ? 1.0f : f16_round(am_mu / 127.0f);
    const float s_c = MB == 16 ? 1.0f : f16_round(am_c / 127.0f);
    // ---- the record in LDS: zero it, then each lane writes its own bytes
    for (int e = lane; e < F::kBytes / 4; e += 64) reinterpret_cast<uint32_t*>(S.rec)[e] = 0u;
    wave_lds_sync();
    {
      // V rows d = 2*lane, 2*lane+1: elements (2 lane) R + k and (2 lane + 1) R + k,
      // one contiguous run of 2 R VB bits (a whole number of bytes) per lane
      constexpr int kBits = 2 * R * VB, kWords = (kBits + 31) / 32, kLaneBytes = kBits / 8;
      uint32_t w[kWords];
#pragma unroll
      for (int x = 0; x < kWords; ++x) w[x] = 0u;
#pragma unroll
      for (int j = 0; j < 2 * R; ++j) {
        const uint32_t c = variant_code(j < R ? v[j][0] : v[j - R][1], s_v, VB);
        w[(j * VB) / 32] |= c << ((j * VB) % 32);
      }
#pragma unroll
      for (int bb = 0; bb < kLaneBytes; ++bb)
        S.rec[lane * kLaneBytes + bb] = (uint8_t)(w[bb / 4] >> (8 * (bb % 4)));
    }
    if (MB == 8) {
      S.rec[F::kMu + 2 * lane] = (uint8_t)variant_code(mu0, s_mu, 8);
      S.rec[F::kMu + 2 * lane + 1] = (uint8_t)variant_code(mu1, s_mu, 8);
    } else {
      const uint32_t h0 = variant_code(mu0, s_mu, 16), h1 = variant_code(mu1, s_mu, 16);
      *reinterpret_cast<uint32_t*>(&S.rec[F::kMu + 4 * lane]) = h0 | (h1 << 16);
    }
#pragma unroll
    for (int t = 0; t < kCpl; ++t) {
      const int e = lane + 64 * t;
      if (e < kPage * R) {
        const uint32_t c = variant_code(cval[t], s_c, MB);
        if (MB == 8) {
          S.rec[F::kC + e] = (uint8_t)c;
        } else {
          S.rec[F::kC + 2 * e] = (uint8_t)c;
          S.rec[F::kC + 2 * e + 1] = (uint8_t)(c >> 8);
        }
      }
    }
    if (lane < 3) {
      const float sc = lane == 0 ? s_mu : (lane == 1 ? s_v : s_c);
      const uint32_t h = f16_bits(sc);
      S.rec[F::kS + 2 * lane] = (uint8_t)h;
      S.rec[F::kS + 2 * lane + 1] = (uint8_t)(h >> 8);
    }
    wave_lds_sync();
    uint32_t* dst = reinterpret_cast<uint32_t*>(a.summ + ((size_t)blk * a.Hkv + kvh) * F::kBytes);
    const uint32_t* srcw = reinterpret_cast<const uint32_t*>(S.rec);
    for (int e = lane; e < F::kBytes / 4; e += 64) dst[e] = srcw[e];
    wave_lds_sync();  // the record buffer is reused by the next page
  }
}

template <int R, int VB>
hipError_t launch_variant(const BuildArgs& a, hipStream_t s) {
  const long long per_wg = (long long)kWaves * kPagesPerWave;
  const long long wgs = (a.items + per_wg - 1) / per_wg;
  if (wgs <= 0) return hipSuccess;
  hipLaunchKernelGGL((build_variant_kernel<R, VB>), dim3((unsigned)wgs), dim3(64 * kWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace

size_t variant_record_bytes(int rank, int v_bits) {
#define LOCKS_VARIANT_BYTES(R, VB) \
  if (rank == R && v_bits == VB) return (size_t)VariantFmt<R, VB>::kBytes;
  LOCKS_VARIANT_BYTES(4, 2) LOCKS_VARIANT_BYTES(4, 4) LOCKS_VARIANT_BYTES(4, 16)
  LOCKS_VARIANT_BYTES(8, 2) LOCKS_VARIANT_BYTES(8, 4) LOCKS_VARIANT_BYTES(8, 16)
  LOCKS_VARIANT_BYTES(16, 2) LOCKS_VARIANT_BYTES(16, 4) LOCKS_VARIANT_BYTES(16, 16)
#undef LOCKS_VARIANT_BYTES
  return 0;
}

hipError_t launch_build_variant(const locks_dims& d, const uint16_t* kc, const int32_t* pt,
                                const int32_t* sl, int rank, int v_bits, uint8_t* summ,
                                hipStream_t s) {
  BuildArgs a;
  a.kc = kc;
  a.page_table = pt;
  a.seq_lens = sl;
  a.blocks = nullptr;
  a.fill = nullptr;
  a.summ = summ;
  a.B = d.batch;
  a.Hkv = d.n_kv_heads;
  a.N = d.max_pages_per_seq;
  a.num_blocks = d.num_blocks;
  a.items = (long long)d.batch * d.max_pages_per_seq * d.n_kv_heads;
#define LOCKS_VARIANT_LAUNCH(R, VB) \
  if (rank == R && v_bits == VB) return launch_variant<R, VB>(a, s);
  LOCKS_VARIANT_LAUNCH(4, 2) LOCKS_VARIANT_LAUNCH(4, 4) LOCKS_VARIANT_LAUNCH(4, 16)
  LOCKS_VARIANT_LAUNCH(8, 2) LOCKS_VARIANT_LAUNCH(8, 4) LOCKS_VARIANT_LAUNCH(8, 16)
  LOCKS_VARIANT_LAUNCH(16, 2) LOCKS_VARIANT_LAUNCH(16, 4) LOCKS_VARIANT_LAUNCH(16, 16)
#undef LOCKS_VARIANT_LAUNCH
  return hipErrorInvalidValue;
}

hipError_t launch_build(const locks_dims& d, const uint16_t* kc, const int32_t* pt,
                        const int32_t* sl, const int32_t* blocks, int n_blocks, uint8_t* summ,
                        hipStream_t s) {
  BuildArgs a;
  a.kc = kc;
  a.page_table = pt;
  a.seq_lens = sl;
  a.blocks = blocks;
  a.fill = nullptr;
  a.summ = summ;
  a.B = d.batch;
  a.Hkv = d.n_kv_heads;
  a.N = d.max_pages_per_seq;
  a.num_blocks = d.num_blocks;
  a.items = blocks ? (long long)n_blocks * d.n_kv_heads
                   : (long long)d.batch * d.max_pages_per_seq * d.n_kv_heads;
  // few items (up to one page per wave of a full chip): latency mode
  const bool few = a.items <= 4096;
  const long long per_wg = (long long)kWaves * (few ? 1 : kPagesPerWave);
  const long long wgs = (a.items + per_wg - 1) / per_wg;
  if (wgs <= 0) return hipSuccess;
  if (few)
    hipLaunchKernelGGL(build_kernel<1>, dim3((unsigned)wgs), dim3(64 * kWaves), 0, s, a);
  else
    hipLaunchKernelGGL(build_kernel<kPagesPerWave>, dim3((unsigned)wgs), dim3(64 * kWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace locks
