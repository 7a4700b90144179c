/*
 * locks.h — C ABI of liblocks.so, the MI355X (gfx950) LOCKS decode path.
 *
 * Sources cited below:
 *   (A) blog post "LOCKS: per-page SVD cuts KV-cache reads 10x at 1M context"
 *       (sections "How LOCKS works", "Code", "Results", "Caveats");
 *   (B) technical summary "LOCKS – 효율적인 롱 컨텍스트 디코딩을 위한 페이지 로컬
 *       압축 키 요약" on gist.science, paper 2607.24555 (section 2 "방법론",
 *       mechanisms 1-4).
 *
 * What the library computes (one decode step, one query token per sequence):
 *   1. score every 16-token KV page from its compressed key summary alone
 *      (A "How LOCKS works", page-score equation; B mechanism 2);
 *   2. turn the per-head scores into one key per (sequence, KV head) by
 *      averaging each head's normalised mass share over the GQA group
 *      (B mechanism 3);
 *   3. keep the k = budget/16 pages with the largest key (A "Code", top-k);
 *   4. run exact softmax attention over the kept pages only, renormalised
 *      over the kept tokens (A "Code", sparse attention), plus the tokens of
 *      the sequence's partly filled last page, which has no summary yet.
 * The summary build (A "How LOCKS works", summary list; B mechanism 1) is a
 * separate, off-critical-path call, for the whole cache or for the pages that
 * just filled.
 *
 * Conventions for every entry point:
 *  - All array arguments are DEVICE pointers owned by the caller; the library
 *    never allocates, frees, copies host<->device or synchronises inside a
 *    call. Work is enqueued on `stream` and is asynchronous; results are
 *    valid once the stream reaches that point.
 *  - Arguments are checked on the host before anything is enqueued. A failed
 *    check returns a negative locks_status and enqueues nothing;
 *    locks_last_error() then describes it. Nothing is thrown across the ABI.
 *  - Identical inputs give bitwise-identical outputs (no float atomics).
 *  - Supported shape: head_dim 128, page_size 16, rank 8, and a GQA group
 *    size G = n_q_heads / n_kv_heads in {1, 2, 4, 8, 16}; budget/16 <= 4096
 *    pages; max_pages_per_seq <= 2^20; batch * n_kv_heads <= 65535;
 *    num_blocks * n_kv_heads <= 87652393 (summary records within 64 GiB).
 *    Other values return LOCKS_ERR_UNSUPPORTED.
 *  - q must be finite.
 *  - Page table: page_table[b*max_pages_per_seq + j] is the physical block
 *    that holds logical page j of sequence b. Sequence b has
 *    n_b = min(seq_lens[b] / 16, max_pages_per_seq) full pages. Only full
 *    pages have summaries (a page's summary is built when its 16th token
 *    lands, A "How LOCKS works"), so only they are scored and selected. The
 *    t_b = seq_lens[b] - 16 n_b tokens after them (when n_b <
 *    max_pages_per_seq) sit in logical page n_b, the tail page: attention
 *    always includes them, and reads nothing of that page past token t_b.
 *    A block id outside [0, num_blocks) marks an absent page: it is never
 *    read, never scored, never selected and never attended.
 *  - Query head h uses KV head h / G, G = n_q_heads / n_kv_heads.
 *
 * Layouts (row-major, C order):
 *   k_cache, v_cache  bf16  [num_blocks][n_kv_heads][16][128]
 *   summaries         u8    [num_blocks][n_kv_heads][LOCKS_SUMMARY_STRIDE]
 *   q                 f32   [batch][n_q_heads][128]
 *   out               f32   [batch][n_q_heads][128]
 *   selected          i32   [batch][n_kv_heads][budget/16]
 *   page_scores       f32   [batch][n_q_heads][max_pages_per_seq]
 *
 * Summary record (one per physical block and KV head, A "How LOCKS works",
 * B mechanism 1; every scale is an fp16 per-page absmax scale):
 *   bytes [  0, 512)  V codes, k-major: for k in 0..7, 16 little-endian u32
 *                     words w = 0..15; byte b (0..3) of word w holds
 *                     V[8w+b][k] in its low nibble and V[8w+4+b][k] in its
 *                     high nibble, 4-bit two's complement, range -7..7.
 *   bytes [512, 640)  mu codes, int8[128], range -127..127.
 *   bytes [640, 768)  C codes, int8[16][8] (token-major), range -127..127.
 *   bytes [768, 776)  fp16 scales {s_mu, s_V, s_C, 0}.
 *   bytes [776, 784)  zero padding (keeps every record 16-byte aligned).
 *   Dequantised: mu = s_mu*mu_code, V = s_V*V_code, C = s_C*C_code.
 */
#ifndef LOCKS_H
#define LOCKS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOCKS_HEAD_DIM 128
#define LOCKS_PAGE_SIZE 16
#define LOCKS_RANK 8
#define LOCKS_SUMMARY_STRIDE 784
#define LOCKS_SUMMARY_PAYLOAD 776
#define LOCKS_MAX_GROUP 16

typedef struct locks_dims {
  int32_t batch;             /* B, sequences (one query token each) */
  int32_t n_q_heads;         /* Hq */
  int32_t n_kv_heads;        /* Hkv; G = Hq / Hkv query heads share a KV head */
  int32_t head_dim;          /* must be 128 */
  int32_t page_size;         /* must be 16 */
  int32_t rank;              /* must be 8 */
  int32_t max_pages_per_seq; /* row length of page_table */
  int32_t num_blocks;        /* physical blocks in k_cache / v_cache / summaries */
} locks_dims;

typedef enum locks_status {
  LOCKS_OK = 0,
  LOCKS_ERR_INVALID_ARG = -1, /* NULL/misaligned pointer, bad size or budget */
  LOCKS_ERR_UNSUPPORTED = -2, /* shape outside the supported set */
  LOCKS_ERR_WORKSPACE = -3,   /* workspace smaller than locks_workspace_bytes */
  LOCKS_ERR_HIP = -4          /* a launch failed; see locks_last_error() */
} locks_status;

/* Bytes per summary record (LOCKS_SUMMARY_STRIDE = 784; payload 776). */
size_t locks_summary_record_bytes(void);

/* Message for the last failed call on this thread ("" if none). The pointer
 * stays valid until the next call on the same thread. */
const char* locks_last_error(void);

/* Workspace bytes that locks_decode_step (and its three phases) and
 * locks_dense_attention need for these dims and budget. Pure host call.
 * budget_tokens must be a positive multiple of 16 (A "Code": the page count
 * is the token budget divided by the page size); pass 16 when sizing for
 * locks_dense_attention alone. */
locks_status locks_workspace_bytes(const locks_dims* dims, int32_t budget_tokens,
                                   size_t* out_bytes);

/* Builds the summary record of every full page of every sequence (A "How LOCKS
 * works": centroid, rank-8 basis of the centred keys, per-token coefficients;
 * B mechanism 1: eigendecomposition of the page's small Gram matrix, int4
 * basis, int8 centroid and coefficients). For each (b, j < n_b, kv head) it
 * reads the 16x128 key tile of block page_table[b][j] and writes that block's
 * record. Records of blocks no sequence references are left untouched; a block
 * referenced twice is written twice with identical bytes.
 * k_cache: bf16 keys; summaries: 16-byte aligned output. */
locks_status locks_build_summaries(const locks_dims* dims, const void* k_cache,
                                   const int32_t* page_table, const int32_t* seq_lens,
                                   void* summaries, hipStream_t stream);

/* Builds the records of an explicit list of physical blocks, every KV head of
 * each: the pages that just filled (A "How LOCKS works": a page's summary is
 * built once, when its 16th token lands; B mechanism 1: when a page is
 * finalised). Same record as locks_build_summaries writes for that block.
 *  blocks    device i32[n_blocks]; an entry outside [0, num_blocks) is
 *            skipped (e.g. -1 for "no page filled in this sequence"), so a
 *            captured decode graph can pass a fixed-length list. A block
 *            listed twice is written twice with identical bytes.
 *  n_blocks  >= 0 (0: nothing is enqueued); blocks may be NULL only then.
 * Records of unlisted blocks are left untouched. */
locks_status locks_build_blocks(const locks_dims* dims, const void* k_cache,
                                const int32_t* blocks, int32_t n_blocks, void* summaries,
                                hipStream_t stream);

/* One LOCKS decode step = locks_score_pages + locks_select_pages +
 * locks_sparse_attention on the same workspace, with the same results (for
 * budgets up to 4096 tokens on small grids the selection's final ranking runs
 * inside the attention launch instead of a launch of its own).
 *  q            f32 queries, one token per sequence.
 *  summaries    records written by locks_build_summaries (or any records in
 *               the documented format).
 *  budget_tokens  positive multiple of 16; k = budget_tokens / 16 pages are
 *               kept per (sequence, KV head).
 *  out          f32 attention output over the kept pages and the tail; heads of
 *               a sequence with no token (seq_lens[b] == 0) get 0.
 *  selected     kept logical page ids per (sequence, KV head) in ascending
 *               order; when fewer than k pages exist, the tail is -1.
 *  page_scores  optional (NULL = not written): per-head page score s_hat
 *               (A page-score equation); entries j >= n_b are not written.
 *  workspace    >= locks_workspace_bytes(dims, budget_tokens) bytes of device
 *               memory, 256-byte aligned; its contents need no initialisation.
 *               Calls sharing a workspace must be stream-ordered. */
locks_status locks_decode_step(const locks_dims* dims, const float* q, const void* summaries,
                               const void* k_cache, const void* v_cache,
                               const int32_t* page_table, const int32_t* seq_lens,
                               int32_t budget_tokens, float* out, int32_t* selected,
                               float* page_scores, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Phase 1 of the step: per-head page scores s_hat[b][h][j] (A "How LOCKS
 * works", page-score equation; B mechanism 2) computed from the summaries
 * only — no key or value byte is read — plus the per-head partial
 * log-sum-exp terms the group combine needs. Results stay in the workspace
 * (and in page_scores when it is not NULL). */
locks_status locks_score_pages(const locks_dims* dims, const float* q, const void* summaries,
                               const int32_t* page_table, const int32_t* seq_lens,
                               int32_t budget_tokens, float* page_scores, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* Reference selector: the exact page masses, s*[b][h][j] = log sum_i
 * exp(q_h . k_i / sqrt(128)) over the 16 real keys of every full page — the
 * exact mass selection that Theorem 1 bounds LOCKS's coverage against (A "How
 * LOCKS works", Theorem 1; B section 3). It reads every key (4 KiB per
 * page-head), so it is a quality reference, not a decode path. It leaves the
 * workspace as locks_score_pages does, so locks_select_pages and
 * locks_sparse_attention can follow it unchanged (then selecting by exact
 * mass). Same arguments as locks_score_pages with k_cache (bf16, 16-byte
 * aligned) in place of the summaries; q must be 16-byte aligned. */
locks_status locks_exact_score_pages(const locks_dims* dims, const float* q, const void* k_cache,
                                     const int32_t* page_table, const int32_t* seq_lens,
                                     int32_t budget_tokens, float* page_scores, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/* Precision / rank ablation (A "Caveats": Theorem 1 covers unquantised
 * summaries; int4 loses a few recall points; int2 collapses). Variant records
 * hold the same summary at rank in {4, 8, 16} with V as int2 or int4 codes
 * (v_bits = 2, 4; range +-(2^(v_bits-1) - 1)) or fp16 values (v_bits = 16),
 * and mu, C as int8 codes (fp16 values when v_bits = 16). Layout per record:
 * V [d][k] row-major, element e = d*rank + k in bits [e*v_bits, (e+1)*v_bits),
 * little-endian, two's complement codes; mu[128]; C[16][rank]; fp16 scales
 * {s_mu, s_V, s_C, 0} (1.0 for fp16 tensors); zero padding to a multiple of
 * 16 bytes. Records are [num_blocks][n_kv_heads][locks_variant_record_bytes].
 * A measurement path: locks_score_pages_variant leaves the workspace as
 * locks_score_pages does, so locks_select_pages and locks_sparse_attention
 * follow it unchanged; it is not tuned like the shipped format's scorer.
 * Unsupported (rank, v_bits) return LOCKS_ERR_UNSUPPORTED. */
locks_status locks_variant_record_bytes(int32_t rank, int32_t v_bits, size_t* out_bytes);
locks_status locks_build_summaries_variant(const locks_dims* dims, const void* k_cache,
                                           const int32_t* page_table, const int32_t* seq_lens,
                                           int32_t rank, int32_t v_bits, void* summaries,
                                           hipStream_t stream);
locks_status locks_score_pages_variant(const locks_dims* dims, const float* q, const void* summaries,
                                       const int32_t* page_table, const int32_t* seq_lens,
                                       int32_t budget_tokens, int32_t rank, int32_t v_bits,
                                       float* page_scores, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/* Shared-basis comparison (A "Why shared-basis sparse attention is
 * structurally broken"; B section 3, Proposition 1: a fixed projection shared
 * by all pages is blind to page content in its null space). Writes, for every
 * full page, the record a shared-basis selector scores with, in the LOCKS
 * page-score form: centroid mu = mean of the page's 16 keys, coefficients
 * C = (K - 1 mu^T) W, V = W, where W = basis[b][kvh] is the one 128 x 8
 * projection of sequence b and KV head kvh (row-major [d][k], f32, 16-byte
 * aligned; the caller builds it, e.g. from the sequence's keys). Records use
 * the variant layout at rank 8 with fp16 values (locks_variant_record_bytes(8,
 * 16) bytes each), so locks_score_pages_variant(rank 8, v_bits 16) scores them
 * and locks_select_pages / locks_sparse_attention follow unchanged. A
 * measurement path, not a decode path. */
locks_status locks_build_summaries_shared(const locks_dims* dims, const void* k_cache,
                                          const int32_t* page_table, const int32_t* seq_lens,
                                          const float* basis, void* summaries,
                                          hipStream_t stream);

/* Phase 2: group combine (B mechanism 3: every head's mass share averaged over
 * the GQA group) and top-k (A "Code": top-k by score, ids sorted ascending).
 * Ties between equal keys go to the lower page id. Must follow
 * locks_score_pages on the same workspace, budget and page_scores argument. */
locks_status locks_select_pages(const locks_dims* dims, const int32_t* page_table,
                                const int32_t* seq_lens, int32_t budget_tokens,
                                int32_t* selected, const float* page_scores, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* Phase 3: exact attention over the selected pages only (A "Code": attention
 * over the gathered tokens of the kept pages, softmax scale 1/sqrt(128)),
 * plus the tail page's t_b tokens. `selected` may come from
 * locks_select_pages or from the caller: entries < 0 or >= n_b are skipped;
 * ids should be distinct. */
locks_status locks_sparse_attention(const locks_dims* dims, const float* q,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* page_table, const int32_t* seq_lens,
                                    int32_t budget_tokens, const int32_t* selected, float* out,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* A decode step in which some sequences' last page has just filled (its 16th
 * token landed in this step): the step also builds that page's summary, off
 * its critical path (A "How LOCKS works": the summary is built once, when a
 * page fills; B mechanism 4: summary building stays off the decode critical
 * path, the whole step in one graph). Same arguments and results as
 * locks_decode_step, plus:
 *  filled     device i32[batch]; filled[b] != 0 marks that page n_b - 1 of
 *             sequence b filled in this step (seq_lens[b] = 16 n_b, n_b >= 1;
 *             marks on other sequences are ignored). A marked page has no
 *             summary yet: it is not scored or selected, and all 16 of its
 *             tokens are attended like a partly filled tail page.
 *  summaries  also written: the records of every marked page (block
 *             page_table[b][n_b - 1], every KV head), the bytes
 *             locks_build_blocks writes for that block. They are built by
 *             workgroups of the scoring launch itself, which run first and
 *             alongside the scoring (no scoring workgroup reads them), so the
 *             build costs the step little time; from the next step on the page
 *             is scored as usual. A marked page's block must not also be a
 *             scored page of another sequence in the same step. */
locks_status locks_decode_step_fill(const locks_dims* dims, const float* q, void* summaries,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* page_table, const int32_t* seq_lens,
                                    const int32_t* filled, int32_t budget_tokens, float* out,
                                    int32_t* selected, float* page_scores, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * locks_decode_step with its workspace in a library-owned device array of
 * LOCKS_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, which the library looks up on
 * its first call on a device and holds until the process ends. The call
 * allocates nothing. Arguments, layouts and results are those of
 * locks_decode_step. Dims and budgets whose locks_workspace_bytes exceed the
 * scratch return LOCKS_ERR_WORKSPACE before anything is enqueued. Every call
 * on a GPU shares that GPU's scratch, so calls that may overlap on one GPU
 * (different streams, threads or processes' graphs replayed concurrently)
 * race and must be serialised by the caller; the scratch needs no
 * initialisation between calls. */
#define LOCKS_NOALLOC_SCRATCH_BYTES (64u << 20)
locks_status locks_decode_step_noalloc(const locks_dims* dims, const float* q,
                                       const void* summaries, const void* k_cache,
                                       const void* v_cache, const int32_t* page_table,
                                       const int32_t* seq_lens, int32_t budget_tokens, float* out,
                                       int32_t* selected, float* page_scores, hipStream_t stream);

/* Dense decode attention over all seq_lens[b] tokens: every full page and the
 * tail (A "Code": the full-KV comparison; A "Results": the dense baseline the
 * speed-ups are quoted against). Same layouts and workspace rules as locks_decode_step; size the
 * workspace with budget_tokens = 16. */
locks_status locks_dense_attention(const locks_dims* dims, const float* q, const void* k_cache,
                                   const void* v_cache, const int32_t* page_table,
                                   const int32_t* seq_lens, float* out, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LOCKS_H */
