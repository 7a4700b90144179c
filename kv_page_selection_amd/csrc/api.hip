// api.hip — the C ABI of liblocks.so: argument checks, workspace layout and
// the launch sequence of each entry point. See include/locks.h for the
// contract of every call.
#include <stdint.h>
#include <string.h>

#include <string>

#include "device_common.h"
#include "internal.h"

#include <algorithm>
#include <atomic>
#include <mutex>
#include "locks.h"

namespace locks {

namespace {

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

bool ws_layout(const locks_dims& d, int k, WsLayout* L, const char** why) {
  const long long B = d.batch, Hq = d.n_q_heads, Hkv = d.n_kv_heads, N = d.max_pages_per_seq;
  L->k = k;
  L->n_score_wg = (int)((N + kScorePagesPerWave - 1) / kScorePagesPerWave);
  {
    const int G = d.n_q_heads / d.n_kv_heads;
    // bound units, pooled into super-ranges of S units so that every head's
    // unit maxima fit the LDS slots: 64-page ranges, or (for a sequence of
    // fewer than kTileBoundPages * k pages, where a bound over its ranges
    // would prune little) 16-page tiles, at most 8k of them
    auto pool = [&](long long units) {
      int S = 1;
      while ((long long)G * ((units + S - 1) / S) > kBoundSlots) S *= 2;
      return S;
    };
    L->sup_r = pool(L->n_score_wg);
    L->sup_t = pool(std::min(4LL * L->n_score_wg, (long long)kTileBoundPages / 16 * k));
  }
  // select chunks of up to 1024 pages; every page's sort key fits the chunk's slots
  if (k > kSelectMaxK) {
    *why = "budget/16 above 4096 pages";
    return false;
  }
  long long M = 1024;
  while (M < kSelectChunk && M < N) M *= 2;
  {
    // each chunk workgroup folds G heads per page: while the chunk grid has
    // fewer than 64G workgroups (few sequences and KV heads), smaller chunks
    // spread that work over more CUs; below it, the merge's extra lists cost
    // more than they save (measured: the 1M-token layer of 8 KV heads takes
    // 2048-page chunks, -1.2 us per step against 4096; 1024 costs +4.7 us)
    const long long G = d.n_q_heads / d.n_kv_heads;
    while (M > 1024 && B * Hkv * ((N + M - 1) / M) < 64 * G) M /= 2;
  }
  if ((N + M - 1) / M > 1024) {
    *why = "more than 1024 select chunks (max_pages_per_seq above 2^22)";
    return false;
  }
  L->sel_chunk = (int)M;
  L->n_sel_chunks = (int)((N + M - 1) / M);
  // list entries: k selected pages, then the tail (tokens of the partly filled page)
  // sparse list: 4-page splits (one page per wave) while a (sequence, KV
  // head) has at most 128 of them; longer lists (large budgets) double the
  // split, up to 64 pages, so the partials the merge folds stay few
  long long app = kSparsePagesPerSplit;
  while (app < 64 && (k + 1 + app - 1) / app > 128) app *= 2;
  L->att_pages_per_split = (int)app;
  L->n_att_split = (int)((k + 1 + app - 1) / app);
  if (L->n_att_split > kMaxSplits) {
    *why = "budget/16 above the sparse-attention split capacity";
    return false;
  }
  // dense list: N pages, then the tail, in splits of kDensePagesPerSplit
  // pages; halved (down to one page per wave) while the grid has fewer than
  // kDenseMinWgs workgroups, so short contexts and small batches still fill
  // the GPU (the MFMA kernel of 8- and 16-head groups holds 3 workgroups per
  // CU and does more work per page: a quarter of that). Filled grids keep the
  // long splits, which ragged batches need (measured).
  const long long min_wgs = (d.n_q_heads / d.n_kv_heads) >= 8 ? kDenseMinWgs / 4 : kDenseMinWgs;
  long long dps = kDensePagesPerSplit;
  while (dps > 4 && B * Hkv * ((N + 1 + dps - 1) / dps) < min_wgs) dps /= 2;
  while ((N + 1 + dps - 1) / dps > kMaxSplits) dps *= 2;
  L->dense_pages_per_split = (int)dps;
  L->n_dense_split = (int)((N + 1 + dps - 1) / dps);
  size_t off = 0;
  L->dense_part = off; off = align_up(off + (size_t)(B * Hq) * L->n_dense_split * kPartialFloats * 4);
  L->score_part = off; off = align_up(off + (size_t)(B * Hq * L->n_score_wg) * 2 * 4);
  L->tile_max = off;   off = align_up(off + (size_t)(B * Hq * L->n_score_wg) * 4 * 4);
  L->scores = off;     off = align_up(off + (size_t)(B * Hq * N) * 4);
  L->cand = off;       off = align_up(off + (size_t)(B * Hkv * L->n_sel_chunks) * L->sel_chunk * 8);
  L->cand_blk = off;   off = align_up(off + (size_t)(B * Hkv * L->n_sel_chunks) * L->sel_chunk * 4);
  L->cand_count = off; off = align_up(off + (size_t)(B * Hkv * L->n_sel_chunks) * 4);
  L->sel_blk = off;    off = align_up(off + (size_t)(B * Hkv) * k * 4);
  L->att_part = off;   off = align_up(off + (size_t)(B * Hq) * L->n_att_split * kPartialFloats * 4);
  L->total = off;
  return true;
}

DevPtrs ws_ptrs(const locks_dims& d, const WsLayout& L, void* ws, float* page_scores) {
  (void)d;
  uint8_t* w = static_cast<uint8_t*>(ws);
  DevPtrs P;
  P.ws = w;
  P.scores = page_scores ? page_scores : reinterpret_cast<float*>(w + L.scores);
  P.score_part = reinterpret_cast<float*>(w + L.score_part);
  P.tile_max = reinterpret_cast<float*>(w + L.tile_max);
  P.cand = reinterpret_cast<unsigned long long*>(w + L.cand);
  P.cand_blk = reinterpret_cast<int32_t*>(w + L.cand_blk);
  P.cand_count = reinterpret_cast<int32_t*>(w + L.cand_count);
  P.sel_blk = reinterpret_cast<int32_t*>(w + L.sel_blk);
  P.att_part = reinterpret_cast<float*>(w + L.att_part);
  P.dense_part = reinterpret_cast<float*>(w + L.dense_part);
  return P;
}

}  // namespace locks

using namespace locks;

namespace {

thread_local std::string g_err;

locks_status fail(locks_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

locks_status check_dims(const locks_dims* d) {
  if (!d) return fail(LOCKS_ERR_INVALID_ARG, "dims is NULL");
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->max_pages_per_seq < 1 ||
      d->num_blocks < 1)
    return fail(LOCKS_ERR_INVALID_ARG, "batch, head counts, max_pages_per_seq and num_blocks must be >= 1");
  if (d->head_dim != kDim || d->page_size != kPage || d->rank != kRank)
    return fail(LOCKS_ERR_UNSUPPORTED, "only head_dim 128, page_size 16, rank 8 are supported");
  if (d->n_q_heads % d->n_kv_heads != 0)
    return fail(LOCKS_ERR_INVALID_ARG, "n_q_heads must be a multiple of n_kv_heads");
  const int G = d->n_q_heads / d->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(LOCKS_ERR_UNSUPPORTED, "GQA group size must be 1, 2, 4, 8 or 16");
  if (d->max_pages_per_seq > (1 << 20))
    return fail(LOCKS_ERR_UNSUPPORTED, "max_pages_per_seq above 2^20");
  if ((long long)d->batch * d->n_kv_heads > 65535 || d->batch > 65535)
    return fail(LOCKS_ERR_UNSUPPORTED, "batch * n_kv_heads above 65535");
  if ((long long)d->num_blocks * d->n_kv_heads * (kStride / 16) > 0xFFFFFFFFLL)
    return fail(LOCKS_ERR_UNSUPPORTED, "num_blocks * n_kv_heads above 87652393 (summaries above 64 GiB)");
  return LOCKS_OK;
}

locks_status check_budget(int32_t budget) {
  if (budget < kPage || budget % kPage != 0)
    return fail(LOCKS_ERR_INVALID_ARG, "budget_tokens must be a positive multiple of 16");
  return LOCKS_OK;
}

locks_status layout(const locks_dims* d, int32_t budget, WsLayout* L) {
  const char* why = nullptr;
  if (!ws_layout(*d, budget / kPage, L, &why)) return fail(LOCKS_ERR_UNSUPPORTED, why);
  return LOCKS_OK;
}

locks_status check_ws(const WsLayout& L, const void* ws, size_t bytes) {
  if (!ws) return fail(LOCKS_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(LOCKS_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (bytes < L.total)
    return fail(LOCKS_ERR_WORKSPACE, "workspace too small: need " + std::to_string(L.total) +
                                         " bytes, got " + std::to_string(bytes));
  return LOCKS_OK;
}

locks_status need(const void* p, size_t align, const char* name) {
  if (!p) return fail(LOCKS_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!aligned(p, align))
    return fail(LOCKS_ERR_INVALID_ARG, std::string(name) + " must be " + std::to_string(align) +
                                           "-byte aligned");
  return LOCKS_OK;
}

locks_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(LOCKS_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return LOCKS_OK;
}

// Library-owned workspace of locks_decode_step_noalloc: one copy per GPU (the
// runtime places a __device__ array on every device the library runs on),
// held until the process ends. In host code `scratch` names a host-side
// stand-in, never the device memory: its device address is looked up once per
// device with hipGetSymbolAddress and kept in scratch_dev.
__device__ __align__(256) uint8_t scratch[LOCKS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::atomic<void*> scratch_dev[kMaxDevices];
std::mutex scratch_mu;

// Device address of `scratch` on the device `stream` runs on; the first call
// for a device looks it up with that device current.
locks_status scratch_for(hipStream_t stream, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(LOCKS_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  int dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess)
      return fail(LOCKS_ERR_HIP, std::string("hipStreamGetDevice: ") + hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(LOCKS_ERR_UNSUPPORTED, "device ordinal above 255");
  void* p = scratch_dev[dev].load(std::memory_order_acquire);
  if (p) {
    *out = p;
    return LOCKS_OK;
  }
  std::lock_guard<std::mutex> lock(scratch_mu);
  p = scratch_dev[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(LOCKS_ERR_HIP, std::string("hipSetDevice: ") + hipGetErrorString(e));
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p)
      return fail(LOCKS_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                     (e != hipSuccess ? hipGetErrorString(e) : "null address"));
    scratch_dev[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return LOCKS_OK;
}

#define LOCKS_TRY(x)                  \
  do {                                \
    const locks_status st_ = (x);     \
    if (st_ != LOCKS_OK) return st_;  \
  } while (0)

}  // namespace

namespace {

// The three phases of a decode step on one workspace; fill (nullable) marks,
// per sequence, a last full page that filled in this step (attended as the
// tail, not scored).
locks_status decode_step_impl(const locks_dims* dims, const float* q, const void* summaries,
                              const void* k_cache, const void* v_cache,
                              const int32_t* page_table, const int32_t* seq_lens,
                              const int32_t* fill, int32_t budget_tokens, float* out,
                              int32_t* selected, float* page_scores, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  LOCKS_TRY(check_dims(dims));
  LOCKS_TRY(check_budget(budget_tokens));
  LOCKS_TRY(need(q, 4, "q"));
  LOCKS_TRY(need(summaries, 16, "summaries"));
  LOCKS_TRY(need(k_cache, 16, "k_cache"));
  LOCKS_TRY(need(v_cache, 16, "v_cache"));
  LOCKS_TRY(need(page_table, 4, "page_table"));
  LOCKS_TRY(need(seq_lens, 4, "seq_lens"));
  LOCKS_TRY(need(out, 4, "out"));
  LOCKS_TRY(need(selected, 4, "selected"));
  if (page_scores) LOCKS_TRY(need(page_scores, 4, "page_scores"));
  WsLayout L;
  LOCKS_TRY(layout(dims, budget_tokens, &L));
  LOCKS_TRY(check_ws(L, workspace, workspace_bytes));
  const DevPtrs P = ws_ptrs(*dims, L, workspace, page_scores);
  (void)hipGetLastError();
  LOCKS_TRY(hip_status(launch_score(*dims, L, P, q, static_cast<const uint8_t*>(summaries),
                                    page_table, seq_lens, fill,
                                    static_cast<const uint16_t*>(k_cache), stream),
                       "score launch"));
  // small budgets on small grids: no merge launch, the attention workgroups
  // rank the lists (each (sequence, KV head)'s ranking repeats in all its
  // splits, which pays only while the grid fits the GPU about once)
  const bool rank_in_attend =
      L.k <= kRankInAttendMaxK &&
      (long long)dims->batch * dims->n_kv_heads * L.n_att_split <= kRankInAttendMaxWgs;
  LOCKS_TRY(hip_status(launch_select(*dims, L, P, page_table, seq_lens, fill, selected,
                                     !rank_in_attend, stream),
                       "select launch"));
  return hip_status(launch_attend(*dims, L, P, q, static_cast<const uint16_t*>(k_cache),
                                  static_cast<const uint16_t*>(v_cache), page_table, seq_lens,
                                  fill, selected, P.sel_blk, out, false, rank_in_attend, stream),
                    "sparse attention launch");
}

}  // namespace

extern "C" {

size_t locks_summary_record_bytes(void) { return kStride; }

const char* locks_last_error(void) { return g_err.c_str(); }

locks_status locks_workspace_bytes(const locks_dims* dims, int32_t budget_tokens, size_t* out_bytes) {
  g_err.clear();
  LOCKS_TRY(check_dims(dims));
  LOCKS_TRY(check_budget(budget_tokens));
  if (!out_bytes) return fail(LOCKS_ERR_INVALID_ARG, "out_bytes is NULL");
  WsLayout L;
  LOCKS_TRY(layout(dims, budget_tokens, &L));
  *out_bytes = L.total;
  return LOCKS_OK;
}

locks_status locks_build_summaries(const locks_dims* dims, const void* k_cache,
                                   const int32_t* page_table, const int32_t* seq_lens,
                                   void* summaries, hipStream_t stream) {
  g_err.clear();
  LOCKS_TRY(check_dims(dims));
  LOCKS_TRY(need(k_cache, 16, "k_cache"));
  LOCKS_TRY(need(page_table, 4, "page_table"));
  LOCKS_TRY(need(seq_lens, 4, "seq_lens"));
  LOCKS_TRY(need(summaries, 16, "summaries"));
  if ((long long)dims->batch * dims->max_pages_per_seq * dims->n_kv_heads > (1LL << 35))
    return fail(LOCKS_ERR_UNSUPPORTED, "batch * max_pages_per_seq * n_kv_heads above 2^35");
  (void)hipGetLastError();
  return hip_status(launch_build(*dims, static_cast<const uint16_t*>(k_cache), page_table, seq_lens,
                                 nullptr, 0, static_cast<uint8_t*>(summaries), stream),
                    "summary build launch");
}

locks_status locks_build_blocks(const locks_dims* dims, const void* k_cache, const int32_t* blocks,
                                int32_t n_blocks, void* summaries, hipStream_t stream) {
  g_err.clear();
  LOCKS_TRY(check_dims(dims));
  if (n_blocks < 0) return fail(LOCKS_ERR_INVALID_ARG, "n_blocks must be >= 0");
  LOCKS_TRY(need(k_cache, 16, "k_cache"));
  LOCKS_TRY(need(summaries, 16, "summaries"));
  if ((long long)n_blocks * dims->n_kv_heads > (1LL << 35))
    return fail(LOCKS_ERR_UNSUPPORTED, "n_blocks * n_kv_heads above 2^35");
  if (n_blocks == 0) return LOCKS_OK;
  LOCKS_TRY(need(blocks, 4, "blocks"));
  (void)hipGetLastError();
  return hip_status(launch_build(*dims, static_cast<const uint16_t*>(k_cache), nullptr, nullptr,
                                 blocks, n_blocks, static_cast<uint8_t*>(summaries), stream),
                    "block build launch");
}

locks_status locks_score_pages(const locks_dims* dims, const float* q, const void* summaries,
                               const int32_t* page_table, const int32_t* seq_lens,
                               int32_t budget_tokens, float* page_scores, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  LOCKS_TRY(check_dims(dims));
  LOCKS_TRY(check_budget(budget_tokens));
  LOCKS_TRY(need(q, 4, "q"));
  LOCKS_TRY(need(summaries, 16, "summaries"));
  LOCKS_TRY(need(page_table, 4, "page_table"));
  LOCKS_TRY(need(seq_lens, 4, "seq_lens"));
  if (page_scores) LOCKS_TRY(need(page_scores, 4, "page_scores"));
  WsLayout L;
  LOCKS_TRY(layout(dims, budget_tokens, &L));
  LOCKS_TRY(check_ws(L, workspace, workspace_bytes));
  const DevPtrs P = ws_ptrs(*dims, L, workspace, page_scores);
  (void)hipGetLastError();
  return hip_status(launch_score(*dims, L, P, q, static_cast<const uint8_t*>(summaries), page_table,
                                 seq_lens, nullptr, nullptr, stream),
                    "score launch");
}

locks_status locks_exact_score_pages(const locks_dims* dims, const float* q, const void* k_cache,
                                     const int32_t* page_table, const int32_t* seq_lens,
                                     int32_t budget_tokens, float* page_scores, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  LOCKS_TRY(check_dims(dims));
  LOCKS_TRY(check_budget(budget_tokens));
  LOCKS_TRY(need(q, 16, "q"));
  LOCKS_TRY(need(k_cache, 16, "k_cache"));
  LOCKS_TRY(need(page_table, 4, "page_table"));
  LOCKS_TRY(need(seq_lens, 4, "seq_lens"));
  if (page_scores) LOCKS_TRY(need(page_scores, 4, "page_scores"));
  WsLayout L;
  LOCKS_TRY(layout(dims, budget_tokens, &L));
  LOCKS_TRY(check_ws(L, workspace, workspace_bytes));
  const DevPtrs P = ws_ptrs(*dims, L, workspace, page_scores);
  (void)hipGetLastError();
  return hip_status(launch_exact_score(*dims, L, P, q, static_cast<const uint16_t*>(k_cache),
                                       page_table, seq_lens, stream),
                    "exact score launch");
}

locks_status locks_variant_record_bytes(int32_t rank, int32_t v_bits, size_t* out_bytes) {
  g_err.clear();
  if (!out_bytes) return fail(LOCKS_ERR_INVALID_ARG, "out_bytes is NULL");
  const size_t n = variant_record_bytes(rank, v_bits);
  if (!n) return fail(LOCKS_ERR_UNSUPPORTED, "variant format: rank must be 4, 8 or 16 and v_bits 2, 4 or 16");
  *out_bytes = n;
  return LOCKS_OK;
}

locks_status locks_build_summaries_variant(const locks_dims* dims, const void* k_cache,
                                           const int32_t* page_table, const int32_t* seq_lens,
                                           int32_t rank, int32_t v_bits, void* summaries,
                                           hipStream_t stream) {
  g_err.clear();
  LOCKS_TRY(check_dims(dims));
  size_t n = 0;
  LOCKS_TRY(locks_variant_record_bytes(rank, v_bits, &n));
  LOCKS_TRY(need(k_cache, 16, "k_cache"));
  LOCKS_TRY(need(page_table, 4, "page_table"));
  LOCKS_TRY(need(seq_lens, 4, "seq_lens"));
  LOCKS_TRY(need(summaries, 16, "summaries"));
  if ((long long)dims->batch * dims->max_pages_per_seq * dims->n_kv_heads > (1LL << 35))
    return fail(LOCKS_ERR_UNSUPPORTED, "batch * max_pages_per_seq * n_kv_heads above 2^35");
  (void)hipGetLastError();
  return hip_status(launch_build_variant(*dims, static_cast<const uint16_t*>(k_cache), page_table,
                                         seq_lens, rank, v_bits, static_cast<uint8_t*>(summaries),
                                         stream),
                    "variant build launch");
}

locks_status locks_build_summaries_shared(const locks_dims* dims, const void* k_cache,
                                          const int32_t* page_table, const int32_t* seq_lens,
                                          const float* basis, void* summaries,
                                          hipStream_t stream) {
  g_err.clear();
  LOCKS_TRY(check_dims(dims));
  LOCKS_TRY(need(k_cache, 16, "k_cache"));
  LOCKS_TRY(need(page_table, 4, "page_table"));
  LOCKS_TRY(need(seq_lens, 4, "seq_lens"));
  LOCKS_TRY(need(basis, 16, "basis"));
  LOCKS_TRY(need(summaries, 16, "summaries"));
  if ((long long)dims->batch * dims->max_pages_per_seq * dims->n_kv_heads > (1LL << 35))
    return fail(LOCKS_ERR_UNSUPPORTED, "batch * max_pages_per_seq * n_kv_heads above 2^35");
  if ((unsigned long long)dims->num_blocks * dims->n_kv_heads * shared_record_bytes() > (1ULL << 40))
    return fail(LOCKS_ERR_UNSUPPORTED, "shared-basis records above 1 TiB");
  (void)hipGetLastError();
  return hip_status(launch_build_shared(*dims, static_cast<const uint16_t*>(k_cache), page_table,
                                        seq_lens, basis, static_cast<uint8_t*>(summaries), stream),
                    "shared-basis build launch");
}

locks_status locks_score_pages_variant(const locks_dims* dims, const float* q, const void* summaries,
                                       const int32_t* page_table, const int32_t* seq_lens,
                                       int32_t budget_tokens, int32_t rank, int32_t v_bits,
                                       float* page_scores, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  LOCKS_TRY(check_dims(dims));
  LOCKS_TRY(check_budget(budget_tokens));
  size_t n = 0;
  LOCKS_TRY(locks_variant_record_bytes(rank, v_bits, &n));
  LOCKS_TRY(need(q, 4, "q"));
  LOCKS_TRY(need(summaries, 16, "summaries"));
  LOCKS_TRY(need(page_table, 4, "page_table"));
  LOCKS_TRY(need(seq_lens, 4, "seq_lens"));
  if (page_scores) LOCKS_TRY(need(page_scores, 4, "page_scores"));
  if ((unsigned long long)dims->num_blocks * dims->n_kv_heads * n > (1ULL << 40))
    return fail(LOCKS_ERR_UNSUPPORTED, "variant summaries above 1 TiB");
  WsLayout L;
  LOCKS_TRY(layout(dims, budget_tokens, &L));
  LOCKS_TRY(check_ws(L, workspace, workspace_bytes));
  const DevPtrs P = ws_ptrs(*dims, L, workspace, page_scores);
  (void)hipGetLastError();
  return hip_status(launch_score_variant(*dims, L, P, q, static_cast<const uint8_t*>(summaries),
                                         page_table, seq_lens, rank, v_bits, stream),
                    "variant score launch");
}

locks_status locks_select_pages(const locks_dims* dims, const int32_t* page_table,
                                const int32_t* seq_lens, int32_t budget_tokens, int32_t* selected,
                                const float* page_scores, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  g_err.clear();
  LOCKS_TRY(check_dims(dims));
  LOCKS_TRY(check_budget(budget_tokens));
  LOCKS_TRY(need(page_table, 4, "page_table"));
  LOCKS_TRY(need(seq_lens, 4, "seq_lens"));
  LOCKS_TRY(need(selected, 4, "selected"));
  if (page_scores) LOCKS_TRY(need(page_scores, 4, "page_scores"));
  WsLayout L;
  LOCKS_TRY(layout(dims, budget_tokens, &L));
  LOCKS_TRY(check_ws(L, workspace, workspace_bytes));
  const DevPtrs P = ws_ptrs(*dims, L, workspace, const_cast<float*>(page_scores));
  (void)hipGetLastError();
  return hip_status(launch_select(*dims, L, P, page_table, seq_lens, nullptr, selected, true, stream),
                    "select launch");
}

locks_status locks_sparse_attention(const locks_dims* dims, const float* q, const void* k_cache,
                                    const void* v_cache, const int32_t* page_table,
                                    const int32_t* seq_lens, int32_t budget_tokens,
                                    const int32_t* selected, float* out, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  LOCKS_TRY(check_dims(dims));
  LOCKS_TRY(check_budget(budget_tokens));
  LOCKS_TRY(need(q, 4, "q"));
  LOCKS_TRY(need(k_cache, 16, "k_cache"));
  LOCKS_TRY(need(v_cache, 16, "v_cache"));
  LOCKS_TRY(need(page_table, 4, "page_table"));
  LOCKS_TRY(need(seq_lens, 4, "seq_lens"));
  LOCKS_TRY(need(selected, 4, "selected"));
  LOCKS_TRY(need(out, 4, "out"));
  WsLayout L;
  LOCKS_TRY(layout(dims, budget_tokens, &L));
  LOCKS_TRY(check_ws(L, workspace, workspace_bytes));
  const DevPtrs P = ws_ptrs(*dims, L, workspace, nullptr);
  (void)hipGetLastError();
  return hip_status(launch_attend(*dims, L, P, q, static_cast<const uint16_t*>(k_cache),
                                  static_cast<const uint16_t*>(v_cache), page_table, seq_lens,
                                  nullptr, selected, nullptr, out, false, false, stream),
                    "sparse attention launch");
}

locks_status locks_decode_step(const locks_dims* dims, const float* q, const void* summaries,
                               const void* k_cache, const void* v_cache,
                               const int32_t* page_table, const int32_t* seq_lens,
                               int32_t budget_tokens, float* out, int32_t* selected,
                               float* page_scores, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  return decode_step_impl(dims, q, summaries, k_cache, v_cache, page_table, seq_lens, nullptr,
                          budget_tokens, out, selected, page_scores, workspace, workspace_bytes,
                          stream);
}

locks_status locks_decode_step_fill(const locks_dims* dims, const float* q, void* summaries,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* page_table, const int32_t* seq_lens,
                                    const int32_t* filled, int32_t budget_tokens, float* out,
                                    int32_t* selected, float* page_scores, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  LOCKS_TRY(need(filled, 4, "filled"));
  if (dims && (long long)dims->batch * dims->n_kv_heads > (1LL << 30))
    return fail(LOCKS_ERR_UNSUPPORTED, "batch * n_kv_heads above 2^30");
  return decode_step_impl(dims, q, summaries, k_cache, v_cache, page_table, seq_lens, filled,
                          budget_tokens, out, selected, page_scores, workspace, workspace_bytes,
                          stream);
}

locks_status locks_decode_step_noalloc(const locks_dims* dims, const float* q,
                                       const void* summaries, const void* k_cache,
                                       const void* v_cache, const int32_t* page_table,
                                       const int32_t* seq_lens, int32_t budget_tokens, float* out,
                                       int32_t* selected, float* page_scores, hipStream_t stream) {
  g_err.clear();
  LOCKS_TRY(check_dims(dims));
  LOCKS_TRY(check_budget(budget_tokens));
  WsLayout L;
  LOCKS_TRY(layout(dims, budget_tokens, &L));
  if (L.total > (size_t)LOCKS_NOALLOC_SCRATCH_BYTES)
    return fail(LOCKS_ERR_WORKSPACE,
                "these dims and budget need " + std::to_string(L.total) +
                    " bytes of workspace, above the library's no-allocation scratch of " +
                    std::to_string((size_t)LOCKS_NOALLOC_SCRATCH_BYTES) +
                    " bytes: use locks_decode_step with a caller workspace");
  LOCKS_TRY(need(q, 4, "q"));
  LOCKS_TRY(need(summaries, 16, "summaries"));
  LOCKS_TRY(need(k_cache, 16, "k_cache"));
  LOCKS_TRY(need(v_cache, 16, "v_cache"));
  LOCKS_TRY(need(page_table, 4, "page_table"));
  LOCKS_TRY(need(seq_lens, 4, "seq_lens"));
  LOCKS_TRY(need(out, 4, "out"));
  LOCKS_TRY(need(selected, 4, "selected"));
  if (page_scores) LOCKS_TRY(need(page_scores, 4, "page_scores"));
  void* ws = nullptr;
  LOCKS_TRY(scratch_for(stream, &ws));
  return locks_decode_step(dims, q, summaries, k_cache, v_cache, page_table, seq_lens,
                           budget_tokens, out, selected, page_scores, ws,
                           (size_t)LOCKS_NOALLOC_SCRATCH_BYTES, stream);
}

locks_status locks_dense_attention(const locks_dims* dims, const float* q, const void* k_cache,
                                   const void* v_cache, const int32_t* page_table,
                                   const int32_t* seq_lens, float* out, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  LOCKS_TRY(check_dims(dims));
  LOCKS_TRY(need(q, 4, "q"));
  LOCKS_TRY(need(k_cache, 16, "k_cache"));
  LOCKS_TRY(need(v_cache, 16, "v_cache"));
  LOCKS_TRY(need(page_table, 4, "page_table"));
  LOCKS_TRY(need(seq_lens, 4, "seq_lens"));
  LOCKS_TRY(need(out, 4, "out"));
  WsLayout L;
  LOCKS_TRY(layout(dims, kPage, &L));
  LOCKS_TRY(check_ws(L, workspace, workspace_bytes));
  const DevPtrs P = ws_ptrs(*dims, L, workspace, nullptr);
  (void)hipGetLastError();
  return hip_status(launch_attend(*dims, L, P, q, static_cast<const uint16_t*>(k_cache),
                                  static_cast<const uint16_t*>(v_cache), page_table, seq_lens,
                                  nullptr, nullptr, nullptr, out, true, false, stream),
                    "dense attention launch");
}

}  // extern "C"
