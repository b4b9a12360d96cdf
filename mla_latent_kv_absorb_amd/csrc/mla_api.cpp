// Host side of the C ABI: argument validation, split planning, workspace
// layout and kernel launches.  Nothing here allocates device memory or
// synchronises a stream.
#include <math.h>
#include <string.h>

#include "../../include/mla_absorb.h"
#include "mla_internal.h"
#include "side_calls.h"

namespace {

using mla::kHeads;
using mla::kLatent;
using mla::kRope;

enum class Path { kF32, kMfmaBf16, kMfmaFp8, kMfmaFp8G128 };

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

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
    if (c->num_heads != kHeads || c->d_latent != kLatent || c->d_rope != kRope) return MLA_ERR_UNSUPPORTED;
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

size_t al16(size_t x) { return (x + 15) / 16 * 16; }

// Upper bound on split workers (the combine kernel's empty-worker test works
// in 32-bit products of worker index and tile count below this bound).
constexpr int64_t kMaxWorkers = 65536;

void layout(const mla_config* c, size_t* page, size_t* rope_off, size_t* scale_off) {
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

size_t workspace_bytes_for(const mla_config* c, int64_t slots) {
  return al16((size_t)slots * c->num_heads * c->d_latent * 4) + al16((size_t)slots * c->num_heads * 4);
}

// Split partials (normalised weighted latents) are kept in BF16 when the
// activations are BF16: the combined output is rounded to BF16 anyway, so one
// more BF16 rounding of each partial stays at the output's own precision,
// and the partials cost half the bytes to write and to read back.  The FP32
// path keeps FP32 partials.
bool partials_bf16(Path p) { return p != Path::kF32; }

mla_status launch_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH; }

}  // namespace

extern "C" {

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported dimensions or data types";
    case MLA_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

mla_status mla_page_layout(const mla_config* cfg, size_t* page_bytes, size_t* rope_offset,
                           size_t* scale_offset) {
  Path path;
  mla_status st = check_config(cfg, &path);
  if (st != MLA_OK) return st;
  if (page_bytes == nullptr || rope_offset == nullptr || scale_offset == nullptr) return MLA_ERR_INVALID_ARG;
  layout(cfg, page_bytes, rope_offset, scale_offset);
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
  if (P < 1) P = 1;
  plan->num_workers = (int32_t)P;
  plan->num_slots = (int32_t)(P + batch - 1);
  plan->workspace_bytes = workspace_bytes_for(cfg, P + batch - 1);
  return MLA_OK;
}

mla_status mla_cache_append(const mla_config* cfg, const void* c_new, const void* k_new, const float* rope_cos,
                            const float* rope_sin, int32_t rope_rows, const int32_t* positions, void* kv_pool,
                            int64_t num_pages, const int32_t* block_table, int32_t block_table_stride,
                            int32_t batch, void* stream) {
  Path path;
  mla_status st = check_config(cfg, &path);
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
  size_t page, rope_off, scale_off;
  layout(cfg, &page, &rope_off, &scale_off);
  mla::AppendArgs a{};
  a.c_new = c_new;
  a.k_new = k_new;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.rope_rows = rope_rows;
  a.positions = positions;
  a.pool = (uint8_t*)kv_pool;
  a.num_pages = num_pages;
  a.page_bytes = (int64_t)page;
  a.rope_off = (int64_t)rope_off;
  a.scale_off = (int64_t)scale_off;
  a.block_table = block_table;
  a.bt_stride = block_table_stride;
  a.batch = batch;
  a.D_C = cfg->d_latent;
  a.D_R = cfg->d_rope;
  const int kind = path == Path::kF32 ? 0 : path == Path::kMfmaBf16 ? 1 : path == Path::kMfmaFp8 ? 2 : 3;
  return launch_status(mla::launch_cache_append(a, kind, (hipStream_t)stream));
}

namespace {
mla_status check_prefill(const mla_config* cfg) {
  Path path;
  mla_status st = check_config(cfg, &path);
  if (st != MLA_OK) return st;
  if (path != Path::kMfmaBf16 || cfg->d_nope != 128 || cfg->d_v != 128) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}
}  // namespace

mla_status mla_prepare_w_uk_t(const mla_config* cfg, const void* w_uk, void* w_uk_t, void* stream) {
  mla_status st = check_prefill(cfg);
  if (st != MLA_OK) return st;
  if (w_uk == nullptr || w_uk_t == nullptr || !aligned(w_uk, 16) || !aligned(w_uk_t, 16)) return MLA_ERR_INVALID_ARG;
  return launch_status(mla::launch_transpose_w_uk(w_uk, w_uk_t, cfg->num_heads, cfg->d_latent, cfg->d_nope,
                                                  (hipStream_t)stream));
}

mla_status mla_prefill_expand(const mla_config* cfg, const void* kv_pool, int64_t num_pages,
                              const int32_t* block_table, int32_t T, const void* w_uk_t, const void* w_uv,
                              void* k_nope, void* v, void* k_rope, void* stream) {
  mla_status st = check_prefill(cfg);
  if (st != MLA_OK) return st;
  if (kv_pool == nullptr || block_table == nullptr || w_uk_t == nullptr || w_uv == nullptr || k_nope == nullptr ||
      v == nullptr || k_rope == nullptr)
    return MLA_ERR_INVALID_ARG;
  if (T < 1 || num_pages < 1) return MLA_ERR_INVALID_ARG;
  if (!aligned(kv_pool, 16) || !aligned(block_table, 4) || !aligned(w_uk_t, 16) || !aligned(w_uv, 16) ||
      !aligned(k_nope, 16) || !aligned(v, 16) || !aligned(k_rope, 16))
    return MLA_ERR_INVALID_ARG;
  size_t page, rope_off, scale_off;
  layout(cfg, &page, &rope_off, &scale_off);
  mla::ExpandArgs a{};
  a.pool = (const uint8_t*)kv_pool;
  a.page_bytes = (int64_t)page;
  a.rope_off = (int64_t)rope_off;
  a.num_pages = num_pages;
  a.block_table = block_table;
  a.T = T;
  a.N = (int64_t)cfg->num_heads * cfg->d_nope;
  hipStream_t s = (hipStream_t)stream;
  a.w = (const __bf16*)w_uk_t;
  a.out = (__bf16*)k_nope;
  a.k_rope = (__bf16*)k_rope;
  hipError_t e = mla::launch_expand(a, s);
  if (e != hipSuccess) return MLA_ERR_LAUNCH;
  a.w = (const __bf16*)w_uv;
  a.out = (__bf16*)v;
  a.k_rope = nullptr;
  return launch_status(mla::launch_expand(a, s));
}

mla_status mla_prefill_attn(const mla_config* cfg, const void* q_nope, const void* q_rope, const void* k_nope,
                            const void* v, const void* k_rope, int32_t T, int32_t q_start, int32_t n_queries,
                            void* out, float* lse_out, void* stream) {
  mla_status st = check_prefill(cfg);
  if (st != MLA_OK) return st;
  if (q_nope == nullptr || q_rope == nullptr || k_nope == nullptr || v == nullptr || k_rope == nullptr ||
      out == nullptr)
    return MLA_ERR_INVALID_ARG;
  if (n_queries < 1 || q_start < 0 || T < 1 || (int64_t)q_start + n_queries > T || n_queries > 65535 * 128)
    return MLA_ERR_INVALID_ARG;
  if (!aligned(q_nope, 16) || !aligned(q_rope, 16) || !aligned(k_nope, 16) || !aligned(v, 16) ||
      !aligned(k_rope, 16) || !aligned(out, 16) || (lse_out && !aligned(lse_out, 4)))
    return MLA_ERR_INVALID_ARG;
  mla::PrefillArgs a{};
  a.qn = (const __bf16*)q_nope;
  a.qr = (const __bf16*)q_rope;
  a.kn = (const __bf16*)k_nope;
  a.v = (const __bf16*)v;
  a.kr = (const __bf16*)k_rope;
  a.out = (__bf16*)out;
  a.lse = lse_out;
  a.H = cfg->num_heads;
  a.T = T;
  a.q_start = q_start;
  a.N = n_queries;
  a.scale = cfg->softmax_scale;
  return launch_status(mla::launch_prefill_attn(a, (hipStream_t)stream));
}

mla_status mla_absorb_q(const mla_config* cfg, const void* q_nope, const void* w_uk, void* q_lat,
                        int32_t batch, void* stream) {
  Path path;
  mla_status st = check_config(cfg, &path);
  if (st != MLA_OK) return st;
  if (q_nope == nullptr || w_uk == nullptr || q_lat == nullptr || batch < 1) return MLA_ERR_INVALID_ARG;
  if (!aligned(q_nope, 16) || !aligned(w_uk, 16) || !aligned(q_lat, 16)) return MLA_ERR_INVALID_ARG;
  if (batch > 65535 * 32) return MLA_ERR_UNSUPPORTED;
  mla::HeadGemmArgs a{q_nope, w_uk, q_lat, batch, cfg->num_heads, cfg->d_latent, cfg->d_nope};
  hipStream_t s = (hipStream_t)stream;
  if (path == Path::kF32) return launch_status(mla::launch_head_gemm_f32(a, s));
  return launch_status(mla::launch_head_gemm_bf16(a, s));
}

mla_status mla_out_up(const mla_config* cfg, const void* o_lat, const void* w_uv, void* out,
                      int32_t batch, void* stream) {
  Path path;
  mla_status st = check_config(cfg, &path);
  if (st != MLA_OK) return st;
  if (o_lat == nullptr || w_uv == nullptr || out == nullptr || batch < 1) return MLA_ERR_INVALID_ARG;
  if (!aligned(o_lat, 16) || !aligned(w_uv, 16) || !aligned(out, 16)) return MLA_ERR_INVALID_ARG;
  if (batch > 65535 * 32) return MLA_ERR_UNSUPPORTED;
  mla::HeadGemmArgs a{o_lat, w_uv, out, batch, cfg->num_heads, cfg->d_v, cfg->d_latent};
  hipStream_t s = (hipStream_t)stream;
  if (path == Path::kF32) return launch_status(mla::launch_head_gemm_f32(a, s));
  return launch_status(mla::launch_head_gemm_bf16(a, s));
}

mla_status mla_decode_attn(const mla_config* cfg, const void* q_lat, const void* q_rope,
                           const void* kv_pool, int64_t num_pages, const int32_t* block_table,
                           int32_t block_table_stride, const int32_t* seq_lens,
                           const int32_t* topk_idx, int32_t topk, int32_t batch,
                           const mla_plan* plan, void* workspace, size_t workspace_bytes,
                           void* o_lat, float* lse_out, void* stream) {
  Path path;
  mla_status st = check_config(cfg, &path);
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
  layout(cfg, &page, &rope_off, &scale_off);
  mla::DecodeArgs a{};
  a.q_lat = q_lat;
  a.q_rope = q_rope;
  a.pool = (const uint8_t*)kv_pool;
  a.num_pages = num_pages;
  a.page_bytes = (int64_t)page;
  a.rope_off = (int64_t)rope_off;
  a.scale_off = (int64_t)scale_off;
  a.block_table = block_table;
  a.bt_stride = block_table_stride;
  a.seq_lens = seq_lens;
  a.topk_idx = topk_idx;
  a.topk = topk;
  a.batch = batch;
  a.H = cfg->num_heads;
  a.D_C = cfg->d_latent;
  a.D_R = cfg->d_rope;
  a.scale = cfg->softmax_scale;
  if (o_lat != nullptr) {
    if (!aligned(o_lat, 16) || (lse_out && !aligned(lse_out, 4))) return MLA_ERR_INVALID_ARG;
    a.num_workers = 0;
    a.o_lat = o_lat;
    a.lse_out = lse_out;
  } else {
    if (plan == nullptr || plan->num_workers < 1 || plan->num_workers > kMaxWorkers || workspace == nullptr ||
        !aligned(workspace, 16))
      return MLA_ERR_INVALID_ARG;
    const int64_t slots = (int64_t)plan->num_workers + batch - 1;
    if (workspace_bytes < workspace_bytes_for(cfg, slots)) return MLA_ERR_INVALID_ARG;
    a.num_workers = plan->num_workers;
    a.part_o = workspace;
    a.part_lse = (float*)((char*)workspace + al16((size_t)slots * cfg->num_heads * cfg->d_latent * 4));
    a.part_bf16 = partials_bf16(path);
  }
  hipStream_t s = (hipStream_t)stream;
  if (path == Path::kF32) return launch_status(mla::launch_decode_f32(a, s));
  if (path == Path::kMfmaBf16 && topk_idx == nullptr) return launch_status(mla::launch_decode_bf16(a, s));
  const mla::CacheKind kind = path == Path::kMfmaFp8       ? mla::CacheKind::kFp8Token
                              : path == Path::kMfmaFp8G128 ? mla::CacheKind::kFp8Group128
                                                           : mla::CacheKind::kBf16;
  return launch_status(mla::launch_decode_mfma(a, kind, s));
}

mla_status mla_combine(const mla_config* cfg, const void* workspace, size_t workspace_bytes,
                       const int32_t* seq_lens, int32_t topk, int32_t batch, const mla_plan* plan,
                       void* o_lat, float* lse_out, void* stream) {
  Path path;
  mla_status st = check_config(cfg, &path);
  if (st != MLA_OK) return st;
  if (workspace == nullptr || seq_lens == nullptr || plan == nullptr || o_lat == nullptr) return MLA_ERR_INVALID_ARG;
  if (batch < 1 || batch > 65535 || topk < 0 || plan->num_workers < 1 || plan->num_workers > kMaxWorkers)
    return MLA_ERR_INVALID_ARG;
  if (!aligned(workspace, 16) || !aligned(o_lat, 16) || (lse_out && !aligned(lse_out, 4))) return MLA_ERR_INVALID_ARG;
  const int64_t slots = (int64_t)plan->num_workers + batch - 1;
  if (workspace_bytes < workspace_bytes_for(cfg, slots)) return MLA_ERR_INVALID_ARG;
  if (cfg->d_latent % 4 != 0) return MLA_ERR_UNSUPPORTED;
  mla::CombineArgs a{};
  a.part_o = workspace;
  a.part_lse = (const float*)((const char*)workspace + al16((size_t)slots * cfg->num_heads * cfg->d_latent * 4));
  a.part_bf16 = partials_bf16(path);
  a.seq_lens = seq_lens;
  a.topk = topk;
  a.batch = batch;
  a.num_workers = plan->num_workers;
  a.o_lat = o_lat;
  a.lse_out = lse_out;
  a.H = cfg->num_heads;
  a.D_C = cfg->d_latent;
  a.out_bf16 = cfg->act_dtype == MLA_BF16;
  return launch_status(mla::launch_combine(a, (hipStream_t)stream));
}

mla_status mla_combine_out_up(const mla_config* cfg, const void* workspace, size_t workspace_bytes,
                              const int32_t* seq_lens, int32_t topk, int32_t batch, const mla_plan* plan,
                              const void* w_uv, void* out, float* lse_out, void* stream) {
  Path path;
  mla_status st = check_config(cfg, &path);
  if (st != MLA_OK) return st;
  if (workspace == nullptr || seq_lens == nullptr || plan == nullptr || w_uv == nullptr || out == nullptr)
    return MLA_ERR_INVALID_ARG;
  if (batch < 1 || batch > 65535 || topk < 0 || plan->num_workers < 1 || plan->num_workers > kMaxWorkers)
    return MLA_ERR_INVALID_ARG;
  if (!aligned(workspace, 16) || !aligned(w_uv, 16) || !aligned(out, 16) || (lse_out && !aligned(lse_out, 4)))
    return MLA_ERR_INVALID_ARG;
  const int64_t slots = (int64_t)plan->num_workers + batch - 1;
  if (workspace_bytes < workspace_bytes_for(cfg, slots)) return MLA_ERR_INVALID_ARG;
  if (path == Path::kF32 || cfg->d_v != 128) return MLA_ERR_UNSUPPORTED;  // H, D_C fixed by the MFMA paths
  mla::CombineUpArgs u{};
  u.c.part_o = workspace;
  u.c.part_lse = (const float*)((const char*)workspace + al16((size_t)slots * cfg->num_heads * cfg->d_latent * 4));
  u.c.part_bf16 = partials_bf16(path);
  u.c.seq_lens = seq_lens;
  u.c.topk = topk;
  u.c.batch = batch;
  u.c.num_workers = plan->num_workers;
  u.c.o_lat = nullptr;
  u.c.lse_out = lse_out;
  u.c.H = cfg->num_heads;
  u.c.D_C = cfg->d_latent;
  u.c.out_bf16 = 1;
  u.w_uv = w_uv;
  u.out = out;
  return launch_status(mla::launch_combine_up(u, (hipStream_t)stream));
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

}  // extern "C"
