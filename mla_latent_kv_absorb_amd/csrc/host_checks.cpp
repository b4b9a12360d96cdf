// Host-side logic of the C ABI that needs no GPU (see host_checks.h): the
// host-only ABI calls, and the argument checks of every call.  Plain C++.
#include "host_checks.h"

#include <math.h>

namespace mla_host {

mla_status check_config(const mla_config* c, Path* path) {
  if (c == nullptr) return MLA_ERR_INVALID_ARG;
  if (c->num_heads < 1 || c->d_latent < 1 || c->d_rope < 0 || c->d_nope < 1 || c->d_v < 1)
    return MLA_ERR_INVALID_ARG;
  if (c->block_size != MLA_PAGE_TOKENS) return MLA_ERR_INVALID_ARG;
  if (!isfinite(c->softmax_scale) || !(c->softmax_scale > 0.f)) return MLA_ERR_INVALID_ARG;
  if (c->cache_dtype == MLA_F32 && c->act_dtype == MLA_F32) {
    if ((size_t)c->num_heads * c->d_latent > 8192 || c->d_latent > 512 || c->d_rope > 512)
      return MLA_ERR_UNSUPPORTED;
    if (mla::decode_f32_lds_bytes(c->num_heads, c->d_latent, c->d_rope) > 65536) return MLA_ERR_UNSUPPORTED;
    *path = Path::kF32;
    return MLA_OK;
  }
  if ((c->cache_dtype == MLA_BF16 || c->cache_dtype == MLA_FP8_E4M3 || c->cache_dtype == MLA_FP8_E4M3_G128) &&
      c->act_dtype == MLA_BF16) {
    if (c->num_heads != mla::kHeads || c->d_latent != mla::kLatent || c->d_rope != mla::kRope)
      return MLA_ERR_UNSUPPORTED;
    if (c->d_nope % 16 != 0 || c->d_v % 32 != 0) return MLA_ERR_UNSUPPORTED;
    *path = c->cache_dtype == MLA_BF16       ? Path::kMfmaBf16
            : c->cache_dtype == MLA_FP8_E4M3 ? Path::kMfmaFp8
                                             : Path::kMfmaFp8G128;
    return MLA_OK;
  }
  if (c->cache_dtype < MLA_F32 || c->cache_dtype > MLA_FP8_E4M3_G128 || c->act_dtype < MLA_F32 ||
      c->act_dtype > MLA_BF16)
    return MLA_ERR_INVALID_ARG;
  return MLA_ERR_UNSUPPORTED;
}

void page_layout(const mla_config* c, size_t* page, size_t* rope_off, size_t* scale_off) {
  size_t cb, rb, sb;
  if (c->cache_dtype == MLA_F32) {
    cb = (size_t)MLA_PAGE_TOKENS * c->d_latent * 4;
    rb = (size_t)MLA_PAGE_TOKENS * c->d_rope * 4;
    sb = 0;
  } else if (c->cache_dtype == MLA_BF16) {
    cb = (size_t)MLA_PAGE_TOKENS * c->d_latent * 2;
    rb = (size_t)MLA_PAGE_TOKENS * c->d_rope * 2;
    sb = 0;
  } else {
    // FP8: one float32 scale per position, or one per 128 latent channels
    cb = (size_t)MLA_PAGE_TOKENS * c->d_latent;
    rb = (size_t)MLA_PAGE_TOKENS * c->d_rope * 2;
    const size_t groups = c->cache_dtype == MLA_FP8_E4M3_G128 ? (size_t)(c->d_latent + 127) / 128 : 1;
    sb = (size_t)MLA_PAGE_TOKENS * groups * 4;
  }
  *rope_off = al16(cb);
  *scale_off = al16(*rope_off + rb);
  *page = al16(*scale_off + sb);
}

size_t workspace_bytes(const mla_config* c, int64_t slots) {
  return al16((size_t)slots * c->num_heads * c->d_latent * 4) + al16((size_t)slots * c->num_heads * 4);
}

size_t packed_partials_bytes(const mla_config* c, Path path, int64_t slots) {
  const size_t elem = partials_bf16(path) ? 2 : 4;
  return al16((size_t)slots * c->num_heads * c->d_latent * elem) + al16((size_t)slots * c->num_heads * 4);
}

void partials_at(const mla_config* c, Path path, void* base, int64_t slots, bool packed, void** part_o,
                 float** part_lse) {
  const size_t elem = packed && partials_bf16(path) ? 2 : 4;
  *part_o = base;
  *part_lse = (float*)((char*)base + al16((size_t)slots * c->num_heads * c->d_latent * elem));
}

mla::CacheKind cache_kind(Path path) {
  return path == Path::kMfmaFp8       ? mla::CacheKind::kFp8Token
         : path == Path::kMfmaFp8G128 ? mla::CacheKind::kFp8Group128
                                      : mla::CacheKind::kBf16;
}

mla_status prepare_head_gemm(const mla_config* cfg, const void* x, const void* w, void* y, int32_t batch,
                             bool absorb, mla::HeadGemmArgs* a, Path* path) {
  mla_status st = check_config(cfg, path);
  if (st != MLA_OK) return st;
  if (x == nullptr || w == nullptr || y == nullptr || batch < 1) return MLA_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16)) return MLA_ERR_INVALID_ARG;
  if (batch > 65535 * 32) return MLA_ERR_UNSUPPORTED;
  if (absorb)
    *a = mla::HeadGemmArgs{x, w, y, batch, cfg->num_heads, cfg->d_latent, cfg->d_nope};
  else
    *a = mla::HeadGemmArgs{x, w, y, batch, cfg->num_heads, cfg->d_v, cfg->d_latent};
  return MLA_OK;
}

mla_status prepare_decode(const mla_config* cfg, const void* q_lat, const void* q_rope, const void* kv_pool,
                          int64_t num_pages, const int32_t* block_table, int32_t block_table_stride,
                          const int32_t* seq_lens, const int32_t* topk_idx, int32_t topk, int32_t batch,
                          const mla_plan* plan, void* workspace, size_t ws_bytes, void* o_lat,
                          float* lse_out, mla::DecodeArgs* a, Path* path) {
  mla_status st = check_config(cfg, path);
  if (st != MLA_OK) return st;
  if (q_lat == nullptr || q_rope == nullptr || kv_pool == nullptr || block_table == nullptr ||
      seq_lens == nullptr)
    return MLA_ERR_INVALID_ARG;
  if (batch < 1 || num_pages < 1 || block_table_stride < 1) return MLA_ERR_INVALID_ARG;
  if (topk_idx == nullptr ? topk != 0 : topk < 1) return MLA_ERR_INVALID_ARG;
  if (!aligned(q_lat, 16) || !aligned(q_rope, 16) || !aligned(kv_pool, 16) || !aligned(block_table, 4) ||
      !aligned(seq_lens, 4) || (topk_idx && !aligned(topk_idx, 4)))
    return MLA_ERR_INVALID_ARG;
  if (num_pages >= (int64_t)1 << 24) return MLA_ERR_UNSUPPORTED;  // row codes page * 64 + slot fit int32
  size_t page, rope_off, scale_off;
  page_layout(cfg, &page, &rope_off, &scale_off);
  *a = mla::DecodeArgs{};
  a->q_lat = q_lat;
  a->q_rope = q_rope;
  a->pool = (const uint8_t*)kv_pool;
  a->num_pages = num_pages;
  a->page_bytes = (int64_t)page;
  a->rope_off = (int64_t)rope_off;
  a->scale_off = (int64_t)scale_off;
  a->block_table = block_table;
  a->bt_stride = block_table_stride;
  a->seq_lens = seq_lens;
  a->topk_idx = topk_idx;
  a->topk = topk;
  a->batch = batch;
  a->H = cfg->num_heads;
  a->D_C = cfg->d_latent;
  a->D_R = cfg->d_rope;
  a->scale = cfg->softmax_scale;
  if (o_lat != nullptr) {
    if (!aligned(o_lat, 16) || (lse_out && !aligned(lse_out, 4))) return MLA_ERR_INVALID_ARG;
    a->num_workers = 0;
    a->o_lat = o_lat;
    a->lse_out = lse_out;
    return MLA_OK;
  }
  if (plan == nullptr || plan->num_workers < 1 || plan->num_workers > kMaxWorkers || workspace == nullptr ||
      !aligned(workspace, 16))
    return MLA_ERR_INVALID_ARG;
  const int64_t slots = (int64_t)plan->num_workers + batch - 1;
  if (ws_bytes < workspace_bytes(cfg, slots)) return MLA_ERR_INVALID_ARG;
  a->num_workers = plan->num_workers;
  partials_at(cfg, *path, workspace, slots, false, &a->part_o, &a->part_lse);
  a->part_bf16 = partials_bf16(*path);
  return MLA_OK;
}

namespace {
// checks shared by the two merge calls; fills the merge arguments
mla_status prepare_merge(const mla_config* cfg, const void* workspace, size_t ws_bytes, const int32_t* seq_lens,
                         int32_t topk, int32_t batch, const mla_plan* plan, float* lse_out, mla::CombineArgs* a,
                         Path* path) {
  mla_status st = check_config(cfg, path);
  if (st != MLA_OK) return st;
  if (workspace == nullptr || seq_lens == nullptr || plan == nullptr) return MLA_ERR_INVALID_ARG;
  if (batch < 1 || batch > 65535 || topk < 0 || plan->num_workers < 1 || plan->num_workers > kMaxWorkers)
    return MLA_ERR_INVALID_ARG;
  if (!aligned(workspace, 16) || (lse_out && !aligned(lse_out, 4))) return MLA_ERR_INVALID_ARG;
  const int64_t slots = (int64_t)plan->num_workers + batch - 1;
  if (ws_bytes < workspace_bytes(cfg, slots)) return MLA_ERR_INVALID_ARG;
  *a = mla::CombineArgs{};
  void* po;
  float* pl;
  partials_at(cfg, *path, (void*)workspace, slots, false, &po, &pl);
  a->part_o = po;
  a->part_lse = pl;
  a->part_bf16 = partials_bf16(*path);
  a->seq_lens = seq_lens;
  a->topk = topk;
  a->batch = batch;
  a->num_workers = plan->num_workers;
  a->lse_out = lse_out;
  a->H = cfg->num_heads;
  a->D_C = cfg->d_latent;
  return MLA_OK;
}
}  // namespace

mla_status prepare_combine(const mla_config* cfg, const void* workspace, size_t ws_bytes, const int32_t* seq_lens,
                           int32_t topk, int32_t batch, const mla_plan* plan, void* o_lat, float* lse_out,
                           mla::CombineArgs* a) {
  Path path;
  if (o_lat == nullptr) {
    mla_status st = check_config(cfg, &path);
    return st != MLA_OK ? st : MLA_ERR_INVALID_ARG;
  }
  mla_status st = prepare_merge(cfg, workspace, ws_bytes, seq_lens, topk, batch, plan, lse_out, a, &path);
  if (st != MLA_OK) return st;
  if (!aligned(o_lat, 16)) return MLA_ERR_INVALID_ARG;
  if (cfg->d_latent % 4 != 0) return MLA_ERR_UNSUPPORTED;
  a->o_lat = o_lat;
  a->out_bf16 = cfg->act_dtype == MLA_BF16;
  return MLA_OK;
}

mla_status prepare_combine_up(const mla_config* cfg, const void* workspace, size_t ws_bytes,
                              const int32_t* seq_lens, int32_t topk, int32_t batch, const mla_plan* plan,
                              const void* w_uv, void* out, float* lse_out, mla::CombineUpArgs* u) {
  Path path;
  if (w_uv == nullptr || out == nullptr) {
    mla_status st = check_config(cfg, &path);
    return st != MLA_OK ? st : MLA_ERR_INVALID_ARG;
  }
  *u = mla::CombineUpArgs{};
  mla_status st = prepare_merge(cfg, workspace, ws_bytes, seq_lens, topk, batch, plan, lse_out, &u->c, &path);
  if (st != MLA_OK) return st;
  if (!aligned(w_uv, 16) || !aligned(out, 16)) return MLA_ERR_INVALID_ARG;
  if (path == Path::kF32 || cfg->d_v != 128) return MLA_ERR_UNSUPPORTED;  // H, D_C fixed by the MFMA paths
  u->c.o_lat = nullptr;
  u->c.out_bf16 = 1;
  u->w_uv = w_uv;
  u->out = out;
  return MLA_OK;
}

mla_status check_cache_append(const mla_config* cfg, const void* c_new, const void* k_new, const float* rope_cos,
                              const float* rope_sin, int32_t rope_rows, const int32_t* positions,
                              const void* kv_pool, int64_t num_pages, const int32_t* block_table,
                              int32_t block_table_stride, int32_t batch, Path* path) {
  mla_status st = check_config(cfg, path);
  if (st != MLA_OK) return st;
  if (c_new == nullptr || k_new == nullptr || positions == nullptr || kv_pool == nullptr || block_table == nullptr)
    return MLA_ERR_INVALID_ARG;
  if ((rope_cos == nullptr) != (rope_sin == nullptr)) return MLA_ERR_INVALID_ARG;
  if (rope_cos != nullptr && rope_rows < 1) return MLA_ERR_INVALID_ARG;
  if (batch < 1 || num_pages < 1 || block_table_stride < 1) return MLA_ERR_INVALID_ARG;
  if (!aligned(c_new, 16) || !aligned(k_new, 16) || !aligned(positions, 4) || !aligned(kv_pool, 16) ||
      !aligned(block_table, 4) || (rope_cos && (!aligned(rope_cos, 4) || !aligned(rope_sin, 4))))
    return MLA_ERR_INVALID_ARG;
  if (cfg->d_rope % 2 != 0) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

namespace {
mla_status check_prefill_config(const mla_config* cfg) {
  Path path;
  mla_status st = check_config(cfg, &path);
  if (st != MLA_OK) return st;
  if (path == Path::kF32 || cfg->d_nope != 128 || cfg->d_v != 128) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}
}  // namespace

mla_status check_prepare_w_uk_t(const mla_config* cfg, const void* w_uk, const void* w_uk_t) {
  mla_status st = check_prefill_config(cfg);
  if (st != MLA_OK) return st;
  if (w_uk == nullptr || w_uk_t == nullptr || !aligned(w_uk, 16) || !aligned(w_uk_t, 16)) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

mla_status check_prefill_expand(const mla_config* cfg, const void* kv_pool, int64_t num_pages,
                                const int32_t* block_table, int32_t T, const void* w_uk_t, const void* w_uv,
                                const void* k_nope, const void* v, const void* k_rope) {
  mla_status st = check_prefill_config(cfg);
  if (st != MLA_OK) return st;
  if (kv_pool == nullptr || block_table == nullptr || w_uk_t == nullptr || w_uv == nullptr || k_nope == nullptr ||
      v == nullptr || k_rope == nullptr)
    return MLA_ERR_INVALID_ARG;
  if (T < 1 || num_pages < 1) return MLA_ERR_INVALID_ARG;
  if (!aligned(kv_pool, 16) || !aligned(block_table, 4) || !aligned(w_uk_t, 16) || !aligned(w_uv, 16) ||
      !aligned(k_nope, 16) || !aligned(v, 16) || !aligned(k_rope, 16))
    return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

mla_status check_prefill_attn(const mla_config* cfg, const void* q_nope, const void* q_rope, const void* k_nope,
                              const void* v, const void* k_rope, int32_t T, int32_t q_start, int32_t n_queries,
                              const void* out, const float* lse_out) {
  mla_status st = check_prefill_config(cfg);
  if (st != MLA_OK) return st;
  if (q_nope == nullptr || q_rope == nullptr || k_nope == nullptr || v == nullptr || k_rope == nullptr ||
      out == nullptr)
    return MLA_ERR_INVALID_ARG;
  if (n_queries < 1 || q_start < 0 || T < 1 || (int64_t)q_start + n_queries > T || n_queries > 65535 * 128)
    return MLA_ERR_INVALID_ARG;
  if (!aligned(q_nope, 16) || !aligned(q_rope, 16) || !aligned(k_nope, 16) || !aligned(v, 16) ||
      !aligned(k_rope, 16) || !aligned(out, 16) || (lse_out && !aligned(lse_out, 4)))
    return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

void key_layout(int32_t dim, size_t* page, size_t* scale_off) {
  *scale_off = al16((size_t)MLA_PAGE_TOKENS * dim);
  *page = al16(*scale_off + (size_t)MLA_PAGE_TOKENS * 4);
}

mla_status check_indexer_scores(int32_t n_heads, int32_t dim, const void* q_idx, const float* w_idx,
                                const void* key_pool, int64_t num_pages, const int32_t* block_table,
                                int32_t block_table_stride, const int32_t* seq_lens, int32_t batch,
                                const float* scores, int64_t score_stride) {
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
  return MLA_OK;
}

mla_status check_topk_select(const float* scores, int64_t score_stride, const int32_t* seq_lens, int32_t batch,
                             int32_t k, const int32_t* idx_out, const void* workspace, size_t ws_bytes,
                             size_t need_bytes, int64_t max_stride) {
  if (scores == nullptr || seq_lens == nullptr || idx_out == nullptr || workspace == nullptr)
    return MLA_ERR_INVALID_ARG;
  if (batch < 1 || batch > 65535 || k < 1 || score_stride < 1) return MLA_ERR_INVALID_ARG;
  if (!aligned(scores, 4) || !aligned(seq_lens, 4) || !aligned(idx_out, 4) || !aligned(workspace, 16))
    return MLA_ERR_INVALID_ARG;
  if (score_stride > max_stride) return MLA_ERR_UNSUPPORTED;
  if (ws_bytes < need_bytes) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

}  // namespace mla_host

using namespace mla_host;

extern "C" {

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported dimensions or data types";
    case MLA_ERR_LAUNCH: return "kernel launch failed";
    case MLA_ERR_SCRATCH: return "the call needs more than the library's static scratch";
  }
  return "unknown status";
}

mla_status mla_page_layout(const mla_config* cfg, size_t* page_bytes, size_t* rope_offset,
                           size_t* scale_offset) {
  Path path;
  mla_status st = check_config(cfg, &path);
  if (st != MLA_OK) return st;
  if (page_bytes == nullptr || rope_offset == nullptr || scale_offset == nullptr) return MLA_ERR_INVALID_ARG;
  page_layout(cfg, page_bytes, rope_offset, scale_offset);
  return MLA_OK;
}

mla_status mla_decode_plan(const mla_config* cfg, int32_t batch, const int32_t* seq_lens_host,
                           int32_t max_len, int32_t topk, int32_t num_cus, mla_plan* plan) {
  Path path;
  mla_status st = check_config(cfg, &path);
  if (st != MLA_OK) return st;
  if (plan == nullptr || batch < 1 || topk < 0 || num_cus < 1) return MLA_ERR_INVALID_ARG;
  if (seq_lens_host == nullptr && topk == 0 && max_len < 1) return MLA_ERR_INVALID_ARG;
  int64_t W = 0;  // tiles of the batch
  for (int32_t b = 0; b < batch; ++b) {
    int32_t len = topk > 0 ? topk : (seq_lens_host ? seq_lens_host[b] : max_len);
    if (len < 0) return MLA_ERR_INVALID_ARG;
    W += mla::tiles_of(len);
  }
  if (W < 1) W = 1;
  // As many workers as CUs (one 4-wave work-group fills a CU), but at least
  // two tiles each: a worker's fixed cost (queries, pipeline fill, partial
  // write) is several tiles' worth, so short batches gain little from more,
  // and each extra partial is read again by the merge.
  const int64_t kMinTilesPerWorker = 2;
  int64_t P = (W + kMinTilesPerWorker - 1) / kMinTilesPerWorker;
  if (P > num_cus) P = num_cus;
  if (P > kMaxWorkers) P = kMaxWorkers;
  // Index lists give every request the same tile count and no lead: with a
  // multiple of the batch as worker count every worker covers tiles of one
  // request only, so it starts one segment and writes one partial.
  if (topk > 0 && P >= batch) P -= P % batch;
  if (P < 1) P = 1;
  plan->num_workers = (int32_t)P;
  plan->num_slots = (int32_t)(P + batch - 1);
  plan->workspace_bytes = workspace_bytes(cfg, P + batch - 1);
  return MLA_OK;
}

mla_status mla_check_decode_inputs_host(const mla_config* cfg, int32_t batch, const int32_t* seq_lens,
                                        const int32_t* block_table, int32_t block_table_stride,
                                        int64_t num_pages, const int32_t* topk_idx, int32_t topk,
                                        int32_t* err_index) {
  Path path;
  mla_status st = check_config(cfg, &path);
  if (st != MLA_OK) return st;
  if (err_index) *err_index = -1;
  if (batch < 1 || seq_lens == nullptr || block_table == nullptr || block_table_stride < 1 || num_pages < 1)
    return MLA_ERR_INVALID_ARG;
  if (topk_idx == nullptr ? topk != 0 : topk < 1) return MLA_ERR_INVALID_ARG;
  for (int32_t b = 0; b < batch; ++b) {
    auto fail = [&]() {
      if (err_index) *err_index = b;
      return MLA_ERR_INVALID_ARG;
    };
    const int32_t T = seq_lens[b];
    if (T < 1) return fail();
    const int64_t pages = (T + MLA_PAGE_TOKENS - 1) / MLA_PAGE_TOKENS;
    if (pages > block_table_stride) return fail();
    for (int64_t i = 0; i < pages; ++i) {
      const int32_t pg = block_table[(int64_t)b * block_table_stride + i];
      if (pg < 0 || pg >= num_pages) return fail();
    }
    if (topk_idx) {
      const int32_t* row = topk_idx + (int64_t)b * topk;
      bool padding = false;
      int32_t prev = -1;
      for (int32_t i = 0; i < topk; ++i) {
        const int32_t v = row[i];
        if (v == -1) {
          padding = true;
          continue;
        }
        if (padding || v < 0 || v >= T || v <= prev) return fail();
        prev = v;
      }
    }
  }
  return MLA_OK;
}

mla_status mla_indexer_page_layout(int32_t dim, size_t* page_bytes, size_t* scale_offset) {
  if (dim < 1 || page_bytes == nullptr || scale_offset == nullptr) return MLA_ERR_INVALID_ARG;
  key_layout(dim, page_bytes, scale_offset);
  return MLA_OK;
}

}  // extern "C"
