// internal.h — host-side pieces shared by the library's translation units:
// workspace layout and the kernel launchers behind the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "locks.h"

namespace locks {

constexpr int kScorePagesPerWave = 64;  // 4 tiles x 16 pages per wave and KV head
constexpr int kSelectMaxK = 4096;       // budget/16 limit (the merge keeps up to k between rounds)
constexpr int kSelectChunk = 4096;      // pages per select workgroup at most (4 per thread)
constexpr int kBoundSlots = 16384;      // (head, super-range) maxima the bound pass holds in LDS
constexpr int kSparsePagesPerSplit = 4; // one page per wave (longer for large budgets)
constexpr int kDensePagesPerSplit = 256; // usual dense split; smaller for small grids, larger past kMaxSplits
constexpr int kDenseMinWgs = 1024;       // dense splits shrink while the grid has fewer workgroups
constexpr int kMaxSplits = 2048;        // split partials one merge workgroup combines
constexpr int kPartialFloats = 130;     // (m, l, o[128]) per head and split
constexpr int kTileBoundPages = 128;    // per selected page: sequences with fewer pages bound by tiles
// decode steps with budget/16 up to this rank their lists inside the sparse
// attention launch instead of a merge launch of their own
constexpr int kRankInAttendMaxK = 256;
constexpr int kRankInAttendMaxWgs = 1024;  // and with at most this many attention workgroups

// Byte offsets of the regions of the caller's workspace (each 256-aligned).
struct WsLayout {
  size_t scores = 0;       // f32 [B][Hq][N]   page scores when the caller passes none
  size_t score_part = 0;   // f32 [B][Hq][n_score_wg][2]  (max, sum) per 64-page range, base 2
  size_t tile_max = 0;     // f32 [B][Hq][4 n_score_wg]   max per 16-page tile, base 2
  size_t cand = 0;         // u64 [B][Hkv][n_sel_chunks][chunk] survivors of each chunk
  size_t cand_blk = 0;     // i32 [B][Hkv][n_sel_chunks][chunk] their physical blocks
  size_t cand_count = 0;   // i32 [B][Hkv][n_sel_chunks]
  size_t sel_blk = 0;      // i32 [B][Hkv][k]  physical blocks of the selected pages
  size_t att_part = 0;     // f32 [B][Hq][n_att_split][130]
  size_t dense_part = 0;   // f32 [B][Hq][n_dense_split][130]
  size_t total = 0;
  int k = 0;
  int n_score_wg = 0;
  // selection bound units, chosen per sequence on the device: 16-page tiles
  // when the sequence has fewer than 2k ranges (< kTileBoundRanges * k
  // pages), else 64-page ranges; units per super-range for each kind
  int sup_r = 1, sup_t = 1;
  int sel_chunk = 0, n_sel_chunks = 0;
  int n_att_split = 0, n_dense_split = 0, dense_pages_per_split = 0, att_pages_per_split = 0;
};

// Returns false (and sets *why) when the dims/budget exceed the kernels' limits.
bool ws_layout(const locks_dims& d, int k, WsLayout* L, const char** why);

struct DevPtrs {
  uint8_t* ws;
  float* scores;
  float* score_part;
  float* tile_max;
  unsigned long long* cand;
  int32_t* cand_blk;
  int32_t* cand_count;
  int32_t* sel_blk;
  float* att_part;
  float* dense_part;
};
DevPtrs ws_ptrs(const locks_dims& d, const WsLayout& L, void* ws, float* page_scores);

// Kernel launchers (enqueue only; return hipGetLastError()).
// fill (nullable): per sequence, nonzero when its last full page filled in
// this step; that page is attended as the tail instead of scored (see
// full_pages()), and this launch also builds its records (every KV head) from
// kc into summ, in workgroups of its own.
hipError_t launch_score(const locks_dims& d, const WsLayout& L, const DevPtrs& P, const float* q,
                        const uint8_t* summ, const int32_t* page_table, const int32_t* seq_lens,
                        const int32_t* fill, const uint16_t* kc, hipStream_t s);
// Variant record formats (precision / rank ablation): bytes per record (0 if
// unsupported), whole-cache build, and scores (same workspace outputs as
// launch_score).
size_t variant_record_bytes(int rank, int v_bits);
hipError_t launch_build_variant(const locks_dims& d, const uint16_t* kc, const int32_t* page_table,
                                const int32_t* seq_lens, int rank, int v_bits, uint8_t* summ,
                                hipStream_t s);
hipError_t launch_score_variant(const locks_dims& d, const WsLayout& L, const DevPtrs& P,
                                const float* q, const uint8_t* summ, const int32_t* page_table,
                                const int32_t* seq_lens, int rank, int v_bits, hipStream_t s);
// Exact-mass scores from the keys themselves (the reference selector); same
// workspace outputs as launch_score.
hipError_t launch_exact_score(const locks_dims& d, const WsLayout& L, const DevPtrs& P,
                              const float* q, const uint16_t* kc, const int32_t* page_table,
                              const int32_t* seq_lens, hipStream_t s);
// merge == false: the chunk pass only (the attention launch then ranks the
// candidate lists itself: launch_attend with rank == true).
hipError_t launch_select(const locks_dims& d, const WsLayout& L, const DevPtrs& P,
                         const int32_t* page_table, const int32_t* seq_lens, const int32_t* fill,
                         int32_t* selected, bool merge, hipStream_t s);
// rank == true (sparse only): every workgroup ranks its (sequence, KV head)'s
// candidate lists left by launch_select(merge = false) and split 0 writes the
// kept ids to `selected`; selected_blocks is unused.
hipError_t launch_attend(const locks_dims& d, const WsLayout& L, const DevPtrs& P, const float* q,
                         const uint16_t* kc, const uint16_t* vc, const int32_t* page_table,
                         const int32_t* seq_lens, const int32_t* fill, const int32_t* selected,
                         const int32_t* selected_blocks, float* out, bool dense, bool rank,
                         hipStream_t s);
// Shared-basis comparison records (variant layout, rank 8, fp16 values) of
// every full page, under basis [B][Hkv][128][8].
size_t shared_record_bytes();
hipError_t launch_build_shared(const locks_dims& d, const uint16_t* kc, const int32_t* page_table,
                               const int32_t* seq_lens, const float* basis, uint8_t* summ,
                               hipStream_t s);
// Whole cache (blocks == nullptr: every full page through the page table) or
// the n_blocks listed blocks, every KV head of each.
hipError_t launch_build(const locks_dims& d, const uint16_t* kc, const int32_t* page_table,
                        const int32_t* seq_lens, const int32_t* blocks, int n_blocks,
                        uint8_t* summ, hipStream_t s);

}  // namespace locks
