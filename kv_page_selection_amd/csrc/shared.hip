// shared.hip — records of the shared-basis comparison (gfx950).
//
// Proposition 1 of the LOCKS pages (blog post, "Why shared-basis sparse
// attention is structurally broken"; technical summary, section 3): a fixed
// projection shared by all pages of a sequence has a null space, and page
// content there is invisible to it. To measure that on the GPU, this kernel
// writes each page's record in the page-score form of LOCKS but with a
// caller-given shared basis W (128 x 8, one per sequence and KV head) in place
// of the page's own: centroid mu = mean of the 16 keys, coefficients
// C = (K - 1 mu^T) W, V = W, all as fp16 values in the variant record layout
// (rank 8, v_bits 16). The variant scorer then scores them unchanged.
//
// One wave per page-head. Lane (token i = lane % 16, group g = lane / 16)
// holds key row i, d in [32g, 32g+32); centroids come from 16-lane row sums;
// the lane's partial projections onto the 8 columns of W are summed over the
// four groups with two cross-row swaps.
#include "device_common.h"
#include "internal.h"

namespace locks {

namespace {

constexpr int kSharedRank = 8;
// variant layout at rank 8 with fp16 values: V [128][8], mu [128], C [16][8],
// scales {1, 1, 1, 0}, zero padding to 16 bytes
constexpr int kShV = 0, kShMu = kDim * kSharedRank * 2, kShC = kShMu + kDim * 2,
              kShS = kShC + kPage * kSharedRank * 2;
constexpr int kShBytes = (kShS + 8 + 15) / 16 * 16;

struct SharedArgs {
  const uint16_t* kc;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const float* basis;  // [B][Hkv][128][8]
  uint8_t* summ;
  int Hkv, N, num_blocks;
  long long items;     // B * N * Hkv
};

__device__ __forceinline__ uint32_t half2_bits(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

__global__ __launch_bounds__(256) void build_shared_kernel(SharedArgs a) {
  __shared__ float mu_s[4][kDim];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long item = (long long)blockIdx.x * 4 + wave;
  if (item >= a.items) return;  // wave-uniform; no workgroup barrier below
  const int kvh = (int)(item % a.Hkv);
  const long long bj = item / a.Hkv;
  const int j = (int)(bj % a.N), b = (int)(bj / a.N);
  if (j >= full_pages(a.seq_lens, nullptr, b, a.N)) return;
  const int blk = a.page_table[(size_t)b * a.N + j];
  if (blk < 0 || blk >= a.num_blocks) return;
  const int ti = lane & 15, g = lane >> 4;

  float kf[32];
  {
    const uint4* src = reinterpret_cast<const uint4*>(
        a.kc + ((size_t)blk * a.Hkv + kvh) * (kPage * kDim) + ti * kDim + g * 32);
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
  }
  const float* W = a.basis + ((size_t)b * a.Hkv + kvh) * (kDim * kSharedRank);
  // centroid and deviations of d = 32g + s; partial coefficients over those d
  float c[kSharedRank];
#pragma unroll
  for (int k = 0; k < kSharedRank; ++k) c[k] = 0.f;
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    const float mu = row16_reduce(kf[s], [](float x, float y) { return x + y; }) * (1.0f / kPage);
    if (ti == 0) mu_s[wave][32 * g + s] = mu;
    const float dev = kf[s] - mu;
    const float4 w0 = *reinterpret_cast<const float4*>(W + (32 * g + s) * kSharedRank);
    const float4 w1 = *reinterpret_cast<const float4*>(W + (32 * g + s) * kSharedRank + 4);
    c[0] = fmaf(dev, w0.x, c[0]);
    c[1] = fmaf(dev, w0.y, c[1]);
    c[2] = fmaf(dev, w0.z, c[2]);
    c[3] = fmaf(dev, w0.w, c[3]);
    c[4] = fmaf(dev, w1.x, c[4]);
    c[5] = fmaf(dev, w1.y, c[5]);
    c[6] = fmaf(dev, w1.z, c[6]);
    c[7] = fmaf(dev, w1.w, c[7]);
  }
#pragma unroll
  for (int k = 0; k < kSharedRank; ++k) c[k] = xor32_sum(xor16_sum(c[k]));  // over the 4 groups
  wave_lds_sync();

  uint8_t* rec = a.summ + ((size_t)blk * a.Hkv + kvh) * kShBytes;
  {
    // V = W as fp16, rows d = 2 lane, 2 lane + 1
    const float4* wr = reinterpret_cast<const float4*>(W + 2 * lane * kSharedRank);
    const float4 r0 = wr[0], r1 = wr[1], r2 = wr[2], r3 = wr[3];
    uint4* dst = reinterpret_cast<uint4*>(rec + kShV + 32 * lane);
    dst[0] = make_uint4(half2_bits(r0.x, r0.y), half2_bits(r0.z, r0.w), half2_bits(r1.x, r1.y),
                        half2_bits(r1.z, r1.w));
    dst[1] = make_uint4(half2_bits(r2.x, r2.y), half2_bits(r2.z, r2.w), half2_bits(r3.x, r3.y),
                        half2_bits(r3.z, r3.w));
  }
  *reinterpret_cast<uint32_t*>(rec + kShMu + 4 * lane) =
      half2_bits(mu_s[wave][2 * lane], mu_s[wave][2 * lane + 1]);
  if (g == 0)
    *reinterpret_cast<uint4*>(rec + kShC + 16 * ti) =
        make_uint4(half2_bits(c[0], c[1]), half2_bits(c[2], c[3]), half2_bits(c[4], c[5]),
                   half2_bits(c[6], c[7]));
  if (lane == 0)  // scales {1, 1, 1, 0} (fp16), then the zero padding
    *reinterpret_cast<uint4*>(rec + kShS) = make_uint4(0x3C003C00u, 0x00003C00u, 0u, 0u);
}

}  // namespace

size_t shared_record_bytes() { return (size_t)kShBytes; }

hipError_t launch_build_shared(const locks_dims& d, const uint16_t* kc, const int32_t* pt,
                               const int32_t* sl, const float* basis, uint8_t* summ,
                               hipStream_t s) {
  SharedArgs a;
  a.kc = kc;
  a.page_table = pt;
  a.seq_lens = sl;
  a.basis = basis;
  a.summ = summ;
  a.Hkv = d.n_kv_heads;
  a.N = d.max_pages_per_seq;
  a.num_blocks = d.num_blocks;
  a.items = (long long)d.batch * d.max_pages_per_seq * d.n_kv_heads;
  const long long wgs = (a.items + 3) / 4;
  if (wgs <= 0) return hipSuccess;
  hipLaunchKernelGGL(build_shared_kernel, dim3((unsigned)wgs), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace locks
