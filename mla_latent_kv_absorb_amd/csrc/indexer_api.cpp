// Host side of the indexer calls (mla_indexer.h): argument checks and
// launches.  Nothing here allocates device memory or synchronises a stream.
#include "../../include/mla_indexer.h"
#include "mla_internal.h"
#include "side_calls.h"

#include <cstdint>

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
size_t al16(size_t x) { return (x + 15) / 16 * 16; }
mla_status launch_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH; }

void key_layout(int32_t dim, size_t* page, size_t* scale_off) {
  *scale_off = al16((size_t)MLA_PAGE_TOKENS * dim);
  *page = al16(*scale_off + (size_t)MLA_PAGE_TOKENS * 4);
}

}  // namespace

extern "C" {

mla_status mla_indexer_page_layout(int32_t dim, size_t* page_bytes, size_t* scale_offset) {
  if (dim < 1 || page_bytes == nullptr || scale_offset == nullptr) return MLA_ERR_INVALID_ARG;
  key_layout(dim, page_bytes, scale_offset);
  return MLA_OK;
}

mla_status mla_indexer_scores(int32_t n_heads, int32_t dim, const void* q_idx, const float* w_idx,
                              const void* key_pool, int64_t num_pages, const int32_t* block_table,
                              int32_t block_table_stride, const int32_t* seq_lens, int32_t batch,
                              float* scores, int64_t score_stride, void* stream) {
  if (n_heads < 1 || dim < 1) return MLA_ERR_INVALID_ARG;
  if (n_heads != MLA_INDEXER_HEADS || dim != MLA_INDEXER_DIM) return MLA_ERR_UNSUPPORTED;
  if (q_idx == nullptr || w_idx == nullptr || key_pool == nullptr || block_table == nullptr ||
      seq_lens == nullptr || scores == nullptr)
    return MLA_ERR_INVALID_ARG;
  if (batch < 1 || batch > 65535 || num_pages < 1 || block_table_stride < 1 || score_stride < 1)
    return MLA_ERR_INVALID_ARG;
  if (!aligned(q_idx, 16) || !aligned(w_idx, 4) || !aligned(key_pool, 16) || !aligned(block_table, 4) ||
      !aligned(seq_lens, 4) || !aligned(scores, 4))
    return MLA_ERR_INVALID_ARG;
  size_t page, scale_off;
  key_layout(dim, &page, &scale_off);
  mla::IndexerArgs a{};
  a.q = q_idx;
  a.w = w_idx;
  a.pool = (const uint8_t*)key_pool;
  a.num_pages = num_pages;
  a.page_bytes = (int64_t)page;
  a.scale_off = (int64_t)scale_off;
  a.block_table = block_table;
  a.bt_stride = block_table_stride;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.scores = scores;
  a.score_stride = score_stride;
  return launch_status(mla::launch_indexer_scores(a, (hipStream_t)stream));
}

size_t mla_topk_workspace_bytes(int32_t batch, int64_t score_stride) {
  return batch < 1 || score_stride < 1 ? 0 : mla::topk_workspace_bytes(batch, score_stride);
}

mla_status mla_topk_select(const float* scores, int64_t score_stride, const int32_t* seq_lens, int32_t batch,
                           int32_t k, int32_t* idx_out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (scores == nullptr || seq_lens == nullptr || idx_out == nullptr || workspace == nullptr)
    return MLA_ERR_INVALID_ARG;
  if (batch < 1 || batch > 65535 || k < 1 || score_stride < 1) return MLA_ERR_INVALID_ARG;
  if (!aligned(scores, 4) || !aligned(seq_lens, 4) || !aligned(idx_out, 4) || !aligned(workspace, 16))
    return MLA_ERR_INVALID_ARG;
  if (score_stride > mla::topk_max_stride()) return MLA_ERR_UNSUPPORTED;
  if (workspace_bytes < mla::topk_workspace_bytes(batch, score_stride)) return MLA_ERR_INVALID_ARG;
  mla::TopkArgs a{};
  a.scores = scores;
  a.score_stride = score_stride;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.k = k;
  a.idx_out = idx_out;
  a.hist = (uint32_t*)workspace;
  a.len_cap = INT64_MAX;
  return launch_status(mla::launch_topk_select(a, (hipStream_t)stream));
}

mla_status mla_indexer_topk(int32_t n_heads, int32_t dim, const void* q_idx, const float* w_idx,
                            const void* key_pool, int64_t num_pages, const int32_t* block_table,
                            int32_t block_table_stride, const int32_t* seq_lens, int32_t batch,
                            float* scores, int64_t score_stride, int32_t k, int32_t* idx_out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (n_heads < 1 || dim < 1) return MLA_ERR_INVALID_ARG;
  if (n_heads != MLA_INDEXER_HEADS || dim != MLA_INDEXER_DIM) return MLA_ERR_UNSUPPORTED;
  if (q_idx == nullptr || w_idx == nullptr || key_pool == nullptr || block_table == nullptr ||
      seq_lens == nullptr || scores == nullptr || idx_out == nullptr || workspace == nullptr)
    return MLA_ERR_INVALID_ARG;
  if (batch < 1 || batch > 65535 || num_pages < 1 || block_table_stride < 1 || score_stride < 1 || k < 1)
    return MLA_ERR_INVALID_ARG;
  if (!aligned(q_idx, 16) || !aligned(w_idx, 4) || !aligned(key_pool, 16) || !aligned(block_table, 4) ||
      !aligned(seq_lens, 4) || !aligned(scores, 4) || !aligned(idx_out, 4) || !aligned(workspace, 16))
    return MLA_ERR_INVALID_ARG;
  if (score_stride > mla::topk_max_stride()) return MLA_ERR_UNSUPPORTED;
  if (workspace_bytes < mla::topk_workspace_bytes(batch, score_stride)) return MLA_ERR_INVALID_ARG;
  size_t page, scale_off;
  key_layout(dim, &page, &scale_off);
  mla::IndexerArgs a{};
  a.q = q_idx;
  a.w = w_idx;
  a.pool = (const uint8_t*)key_pool;
  a.num_pages = num_pages;
  a.page_bytes = (int64_t)page;
  a.scale_off = (int64_t)scale_off;
  a.block_table = block_table;
  a.bt_stride = block_table_stride;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.scores = scores;
  a.score_stride = score_stride;
  a.hist = (uint32_t*)workspace;
  a.topk = k;
  mla::TopkArgs t{};
  t.scores = scores;
  t.score_stride = score_stride;
  t.seq_lens = seq_lens;
  t.batch = batch;
  t.k = k;
  t.idx_out = idx_out;
  t.hist = (uint32_t*)workspace;
  t.len_cap = (int64_t)block_table_stride * MLA_PAGE_TOKENS;
  return launch_status(mla::launch_indexer_topk(a, t, (hipStream_t)stream));
}

}  // extern "C"
