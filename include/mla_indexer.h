/* Lightning indexer and top-k pick for sparse MLA decode, gfx950.
 *
 * The two calls produce the per-request index lists that mla_decode_attn
 * consumes in its sparse mode ("DeepSeek's KV Cache: From 3.9 MB to 890 B per
 * Token", sections "DSA: three things the indexer builds" and "The score that
 * picks positions", Figures 8 and 9):
 *
 *   1. mla_indexer_scores   I(b, s) = sum_j w[b][j] * ReLU(q[b][j] . k[s])
 *                           for every cached position s of request b, with the
 *                           search key k[s] stored as E4M3 values times one
 *                           float32 scale per position (section "Calculating
 *                           V3.2's KV cache": the 132-byte search-key item);
 *   2. mla_topk_select      per request, up to k of the highest-scoring
 *                           positions 0 .. seq_lens[b]-1, sorted by position.
 *
 * mla_indexer_topk runs both in one call.
 *
 * Same conventions as mla_absorb.h: every buffer belongs to the caller and
 * lives in device memory unless stated; the library allocates nothing, keeps
 * no state and never synchronises; every call checks its host-visible
 * arguments and enqueues nothing on error; device metadata (block table,
 * lengths) is never trusted to be in range.
 */
#ifndef MLA_INDEXER_H_
#define MLA_INDEXER_H_

#include <stddef.h>
#include <stdint.h>

#include "mla_absorb.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The dims with a kernel: 64 indexer heads of width 128 (V3.2). */
#define MLA_INDEXER_HEADS 64
#define MLA_INDEXER_DIM 128

/* Byte layout of one search-key page (64 positions, sections 16-byte
 * aligned): keys [64][dim] e4m3, then scales [64] f32.  For dim = 128 that is
 * 8,448 bytes, 132 per position.  Host only. */
mla_status mla_indexer_page_layout(int32_t dim, size_t* page_bytes, size_t* scale_offset);

/* Step 1: indexer scores of every cached position.
 *   n_heads, dim: must be MLA_INDEXER_HEADS and MLA_INDEXER_DIM
 *                 (MLA_ERR_UNSUPPORTED otherwise).
 *   q_idx [batch][n_heads][dim] BF16 (16-byte aligned): indexer queries.
 *   w_idx [batch][n_heads] float32: head weights (any sign).
 *   key_pool: num_pages pages in the layout above (16-byte aligned); page
 *             block_table[b][i] holds positions 64i .. 64i+63 of request b
 *             (int32 [batch][block_table_stride]).
 *   seq_lens [batch] int32: cached positions per request.
 *   scores [batch][score_stride] float32: scores[b][s] is written for
 *             0 <= s < min(seq_lens[b], score_stride, 64 * block_table_stride);
 *             other entries are left alone.  A position whose page id is out
 *             of range gets -infinity.
 * The FP8 keys are widened exactly to BF16 and contracted with the queries on
 * the matrix cores in float32; the scale is applied after the ReLU, which is
 * exact for positive scales (ReLU(s x) = s ReLU(x)).  Errors: null or
 * misaligned pointers, batch < 1, strides < 1 -> MLA_ERR_INVALID_ARG. */
mla_status mla_indexer_scores(int32_t n_heads, int32_t dim, const void* q_idx, const float* w_idx,
                              const void* key_pool, int64_t num_pages, const int32_t* block_table,
                              int32_t block_table_stride, const int32_t* seq_lens, int32_t batch,
                              float* scores, int64_t score_stride, void* stream);

/* Workspace bytes mla_topk_select needs for `batch` score rows of
 * `score_stride` entries: per request a histogram, per-chunk counters and
 * room to gather up to a whole row of candidates (8 bytes per entry).  The
 * call clears what must start at zero itself.  0 for batch < 1 or
 * score_stride < 1. */
size_t mla_topk_workspace_bytes(int32_t batch, int64_t score_stride);

/* Step 2: pick, per request b, min(k, T_b) positions among 0 .. T_b - 1
 * (T_b = min(seq_lens[b], score_stride); negative lengths count as 0) with the
 * highest scores[b][s]; among equal scores the lower position comes first.
 * idx_out [batch][k] int32 receives them in increasing position order, then
 * -1 up to k: the index-list format mla_decode_attn takes.
 *   -0 and +0 count as equal; NaN ranks below every other value.
 *   workspace: mla_topk_workspace_bytes(batch, score_stride) bytes,
 *   16-byte aligned.  Calls that share a workspace must not overlap.
 * Errors: null or misaligned pointers, batch < 1, k < 1, score_stride < 1, a
 * too small workspace -> MLA_ERR_INVALID_ARG; score_stride above 8,388,608
 * -> MLA_ERR_UNSUPPORTED. */
mla_status mla_topk_select(const float* scores, int64_t score_stride, const int32_t* seq_lens, int32_t batch,
                           int32_t k, int32_t* idx_out, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Steps 1 and 2 in one call: the scores of mla_indexer_scores, then the pick
 * of mla_topk_select over them, with the pick's first radix histogram built
 * while the scores are computed (one pass over the score rows fewer).  The
 * arguments are those of the two calls; T_b here is
 * min(seq_lens[b], score_stride, 64 * block_table_stride), the positions that
 * get a score, so idx_out equals what the two calls give whenever
 * seq_lens[b] <= 64 * block_table_stride.  scores is written as by step 1.
 *   workspace: mla_topk_workspace_bytes(batch, score_stride) bytes, 16-byte
 *   aligned; calls that share a workspace must not overlap.
 * Errors: those of the two calls. */
mla_status mla_indexer_topk(int32_t n_heads, int32_t dim, const void* q_idx, const float* w_idx,
                            const void* key_pool, int64_t num_pages, const int32_t* block_table,
                            int32_t block_table_stride, const int32_t* seq_lens, int32_t batch,
                            float* scores, int64_t score_stride, int32_t k, int32_t* idx_out, void* workspace,
                            size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_INDEXER_H_ */
