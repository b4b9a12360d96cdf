// Launching calls of the indexer ABI (mla_indexer.h): each checks its
// arguments with the HIP-free host checks (host_checks.cpp), then enqueues
// its kernels.  Nothing here allocates device memory or synchronises a stream.
#include "../../include/mla_indexer.h"
#include "host_checks.h"
#include "mla_internal.h"
#include "side_calls.h"

using namespace mla_host;

namespace {
mla_status launch_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH; }

mla::IndexerArgs indexer_args(int32_t dim, const void* q_idx, const float* w_idx, const void* key_pool,
                              int64_t num_pages, const int32_t* block_table, int32_t block_table_stride,
                              const int32_t* seq_lens, int32_t batch, float* scores, int64_t score_stride) {
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
  return a;
}

mla::TopkArgs topk_args(const float* scores, int64_t score_stride, const int32_t* seq_lens, int32_t batch, int32_t k,
                        int32_t* idx_out, void* workspace, int64_t len_cap) {
  mla::TopkArgs t{};
  t.scores = scores;
  t.score_stride = score_stride;
  t.seq_lens = seq_lens;
  t.batch = batch;
  t.k = k;
  t.idx_out = idx_out;
  t.hist = (uint32_t*)workspace;
  t.len_cap = len_cap;
  return t;
}
}  // namespace

extern "C" {

mla_status mla_indexer_scores(int32_t n_heads, int32_t dim, const void* q_idx, const float* w_idx,
                              const void* key_pool, int64_t num_pages, const int32_t* block_table,
                              int32_t block_table_stride, const int32_t* seq_lens, int32_t batch,
                              float* scores, int64_t score_stride, void* stream) {
  mla_status st = check_indexer_scores(n_heads, dim, q_idx, w_idx, key_pool, num_pages, block_table,
                                       block_table_stride, seq_lens, batch, scores, score_stride);
  if (st != MLA_OK) return st;
  const mla::IndexerArgs a = indexer_args(dim, q_idx, w_idx, key_pool, num_pages, block_table, block_table_stride,
                                          seq_lens, batch, scores, score_stride);
  return launch_status(mla::launch_indexer_scores(a, (hipStream_t)stream));
}

size_t mla_topk_workspace_bytes(int32_t batch, int64_t score_stride) {
  return batch < 1 || score_stride < 1 ? 0 : mla::topk_workspace_bytes(batch, score_stride);
}

mla_status mla_topk_select(const float* scores, int64_t score_stride, const int32_t* seq_lens, int32_t batch,
                           int32_t k, int32_t* idx_out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  const size_t need = batch < 1 || score_stride < 1 ? 0 : mla::topk_workspace_bytes(batch, score_stride);
  mla_status st = check_topk_select(scores, score_stride, seq_lens, batch, k, idx_out, workspace, workspace_bytes,
                                    need, mla::topk_max_stride());
  if (st != MLA_OK) return st;
  const mla::TopkArgs t = topk_args(scores, score_stride, seq_lens, batch, k, idx_out, workspace, INT64_MAX);
  return launch_status(mla::launch_topk_select(t, (hipStream_t)stream));
}

mla_status mla_indexer_topk(int32_t n_heads, int32_t dim, const void* q_idx, const float* w_idx,
                            const void* key_pool, int64_t num_pages, const int32_t* block_table,
                            int32_t block_table_stride, const int32_t* seq_lens, int32_t batch,
                            float* scores, int64_t score_stride, int32_t k, int32_t* idx_out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  mla_status st = check_indexer_scores(n_heads, dim, q_idx, w_idx, key_pool, num_pages, block_table,
                                       block_table_stride, seq_lens, batch, scores, score_stride);
  if (st != MLA_OK) return st;
  const size_t need = mla::topk_workspace_bytes(batch, score_stride);
  st = check_topk_select(scores, score_stride, seq_lens, batch, k, idx_out, workspace, workspace_bytes, need,
                         mla::topk_max_stride());
  if (st != MLA_OK) return st;
  mla::IndexerArgs a = indexer_args(dim, q_idx, w_idx, key_pool, num_pages, block_table, block_table_stride,
                                    seq_lens, batch, scores, score_stride);
  a.hist = (uint32_t*)workspace;
  a.topk = k;
  const mla::TopkArgs t = topk_args(scores, score_stride, seq_lens, batch, k, idx_out, workspace,
                                    (int64_t)block_table_stride * MLA_PAGE_TOKENS);
  return launch_status(mla::launch_indexer_topk(a, t, (hipStream_t)stream));
}

}  // extern "C"
