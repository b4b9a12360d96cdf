// Launching calls of the C ABI (mla_absorb.h): each checks its arguments with
// the HIP-free host checks (host_checks.cpp), then enqueues its kernels.
// Nothing here allocates device memory or synchronises a stream.
#include "../../include/mla_absorb.h"
#include "host_checks.h"
#include "mla_internal.h"
#include "side_calls.h"

using namespace mla_host;

namespace {
mla_status launch_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH; }
}  // namespace

extern "C" {

mla_status mla_cache_append(const mla_config* cfg, const void* c_new, const void* k_new, const float* rope_cos,
                            const float* rope_sin, int32_t rope_rows, const int32_t* positions, void* kv_pool,
                            int64_t num_pages, const int32_t* block_table, int32_t block_table_stride,
                            int32_t batch, void* stream) {
  Path path;
  mla_status st = check_cache_append(cfg, c_new, k_new, rope_cos, rope_sin, rope_rows, positions, kv_pool,
                                     num_pages, block_table, block_table_stride, batch, &path);
  if (st != MLA_OK) return st;
  size_t page, rope_off, scale_off;
  page_layout(cfg, &page, &rope_off, &scale_off);
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

mla_status mla_prepare_w_uk_t(const mla_config* cfg, const void* w_uk, void* w_uk_t, void* stream) {
  mla_status st = check_prepare_w_uk_t(cfg, w_uk, w_uk_t);
  if (st != MLA_OK) return st;
  return launch_status(mla::launch_transpose_w_uk(w_uk, w_uk_t, cfg->num_heads, cfg->d_latent, cfg->d_nope,
                                                  (hipStream_t)stream));
}

mla_status mla_prefill_expand(const mla_config* cfg, const void* kv_pool, int64_t num_pages,
                              const int32_t* block_table, int32_t T, const void* w_uk_t, const void* w_uv,
                              void* k_nope, void* v, void* k_rope, void* stream) {
  mla_status st = check_prefill_expand(cfg, kv_pool, num_pages, block_table, T, w_uk_t, w_uv, k_nope, v, k_rope);
  if (st != MLA_OK) return st;
  size_t page, rope_off, scale_off;
  page_layout(cfg, &page, &rope_off, &scale_off);
  mla::ExpandArgs a{};
  a.pool = (const uint8_t*)kv_pool;
  a.page_bytes = (int64_t)page;
  a.rope_off = (int64_t)rope_off;
  a.scale_off = (int64_t)scale_off;
  a.fmt = cfg->cache_dtype == MLA_FP8_E4M3        ? mla::kExpandFp8Token
          : cfg->cache_dtype == MLA_FP8_E4M3_G128 ? mla::kExpandFp8Group
                                                  : mla::kExpandBf16;
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
  mla_status st = check_prefill_attn(cfg, q_nope, q_rope, k_nope, v, k_rope, T, q_start, n_queries, out, lse_out);
  if (st != MLA_OK) return st;
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
  mla::HeadGemmArgs a;
  Path path;
  mla_status st = prepare_head_gemm(cfg, q_nope, w_uk, q_lat, batch, true, &a, &path);
  if (st != MLA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (path == Path::kF32) return launch_status(mla::launch_head_gemm_f32(a, s));
  return launch_status(mla::launch_head_gemm_bf16(a, s));
}

mla_status mla_out_up(const mla_config* cfg, const void* o_lat, const void* w_uv, void* out,
                      int32_t batch, void* stream) {
  mla::HeadGemmArgs a;
  Path path;
  mla_status st = prepare_head_gemm(cfg, o_lat, w_uv, out, batch, false, &a, &path);
  if (st != MLA_OK) return st;
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
  mla::DecodeArgs a;
  Path path;
  mla_status st = prepare_decode(cfg, q_lat, q_rope, kv_pool, num_pages, block_table, block_table_stride, seq_lens,
                                 topk_idx, topk, batch, plan, workspace, workspace_bytes, o_lat, lse_out, &a, &path);
  if (st != MLA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (path == Path::kF32) return launch_status(mla::launch_decode_f32(a, s));
  if (path == Path::kMfmaBf16 && topk_idx == nullptr) return launch_status(mla::launch_decode_bf16(a, s));
  return launch_status(mla::launch_decode_mfma(a, cache_kind(path), s));
}

mla_status mla_combine(const mla_config* cfg, const void* workspace, size_t workspace_bytes,
                       const int32_t* seq_lens, int32_t topk, int32_t batch, const mla_plan* plan,
                       void* o_lat, float* lse_out, void* stream) {
  mla::CombineArgs a;
  mla_status st = prepare_combine(cfg, workspace, workspace_bytes, seq_lens, topk, batch, plan, o_lat, lse_out, &a);
  if (st != MLA_OK) return st;
  return launch_status(mla::launch_combine(a, (hipStream_t)stream));
}

mla_status mla_combine_out_up(const mla_config* cfg, const void* workspace, size_t workspace_bytes,
                              const int32_t* seq_lens, int32_t topk, int32_t batch, const mla_plan* plan,
                              const void* w_uv, void* out, float* lse_out, void* stream) {
  mla::CombineUpArgs u;
  mla_status st =
      prepare_combine_up(cfg, workspace, workspace_bytes, seq_lens, topk, batch, plan, w_uv, out, lse_out, &u);
  if (st != MLA_OK) return st;
  return launch_status(mla::launch_combine_up(u, (hipStream_t)stream));
}

}  // extern "C"
