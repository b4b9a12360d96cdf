// Host-side logic of the C ABI that needs no GPU: configuration checks, page
// layout, split planning, the device-metadata contract check on host copies,
// and the validation of every call's arguments, which fills the kernels'
// launch arguments for the decode path.  Built without HIP (plain C++), so
// it also builds and runs under host sanitizers.  The HIP translation units
// (mla_api.cpp, indexer_api.cpp, noalloc.hip) call these, then launch.
// Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/mla_absorb.h"
#include "../../include/mla_indexer.h"
#include "mla_args.h"

namespace mla_host {

enum class Path { kF32, kMfmaBf16, kMfmaFp8, kMfmaFp8G128 };

// Upper bound on split workers (the combine kernel's empty-worker test works
// in 32-bit products of worker index and tile count below this bound).
constexpr int64_t kMaxWorkers = 65536;

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
inline size_t al16(size_t x) { return (x + 15) / 16 * 16; }

// The configuration is one the library has kernels for; *path says which.
mla_status check_config(const mla_config* c, Path* path);
void page_layout(const mla_config* c, size_t* page, size_t* rope_off, size_t* scale_off);

// Split partials (normalised weighted latents) are kept in BF16 when the
// activations are BF16: the combined output is rounded to BF16 anyway, so one
// more BF16 rounding of each partial stays at the output's own precision,
// and the partials cost half the bytes to write and to read back.  The FP32
// path keeps FP32 partials.
inline bool partials_bf16(Path p) { return p != Path::kF32; }

// Bytes of a caller's split workspace for `slots` partials: a section sized
// for float32 partials (BF16 partials use its first half), then the float32
// log-sum-exps, each 16-byte aligned.
size_t workspace_bytes(const mla_config* c, int64_t slots);
// The same partials and log-sum-exps packed tightly (BF16 partials take half
// the float32 size): the layout of the library's own static scratch.
size_t packed_partials_bytes(const mla_config* c, Path path, int64_t slots);
// Where the partials and their log-sum-exps of `slots` slots sit in a buffer
// at `base` (packed: the tight layout; else the caller-workspace layout).
void partials_at(const mla_config* c, Path path, void* base, int64_t slots, bool packed, void** part_o,
                 float** part_lse);

// ---- decode path: validate and fill the launch arguments ----
// absorb (x = q_nope, w = w_uk, y = q_lat) or up-projection (x = o_lat,
// w = w_uv, y = out)
mla_status prepare_head_gemm(const mla_config* cfg, const void* x, const void* w, void* y, int32_t batch,
                             bool absorb, mla::HeadGemmArgs* a, Path* path);
// The checks of mla_decode_attn and its launch arguments.  In split mode
// (o_lat == NULL) the partials go to `workspace` (caller layout), whose size
// is checked against the plan.
mla_status prepare_decode(const mla_config* cfg, const void* q_lat, const void* q_rope, const void* kv_pool,
                          int64_t num_pages, const int32_t* block_table, int32_t block_table_stride,
                          const int32_t* seq_lens, const int32_t* topk_idx, int32_t topk, int32_t batch,
                          const mla_plan* plan, void* workspace, size_t workspace_bytes, void* o_lat,
                          float* lse_out, mla::DecodeArgs* a, Path* path);
mla_status prepare_combine(const mla_config* cfg, const void* workspace, size_t workspace_bytes,
                           const int32_t* seq_lens, int32_t topk, int32_t batch, const mla_plan* plan,
                           void* o_lat, float* lse_out, mla::CombineArgs* a);
mla_status prepare_combine_up(const mla_config* cfg, const void* workspace, size_t workspace_bytes,
                              const int32_t* seq_lens, int32_t topk, int32_t batch, const mla_plan* plan,
                              const void* w_uv, void* out, float* lse_out, mla::CombineUpArgs* u);
// The cache kind the MFMA attention kernel takes for a path.
mla::CacheKind cache_kind(Path path);

// ---- the calls around the decode path: argument checks only ----
mla_status check_cache_append(const mla_config* cfg, const void* c_new, const void* k_new, const float* rope_cos,
                              const float* rope_sin, int32_t rope_rows, const int32_t* positions,
                              const void* kv_pool, int64_t num_pages, const int32_t* block_table,
                              int32_t block_table_stride, int32_t batch, Path* path);
mla_status check_prepare_w_uk_t(const mla_config* cfg, const void* w_uk, const void* w_uk_t);
mla_status check_prefill_expand(const mla_config* cfg, const void* kv_pool, int64_t num_pages,
                                const int32_t* block_table, int32_t T, const void* w_uk_t, const void* w_uv,
                                const void* k_nope, const void* v, const void* k_rope);
mla_status check_prefill_attn(const mla_config* cfg, const void* q_nope, const void* q_rope, const void* k_nope,
                              const void* v, const void* k_rope, int32_t T, int32_t q_start, int32_t n_queries,
                              const void* out, const float* lse_out);

void key_layout(int32_t dim, size_t* page, size_t* scale_off);
mla_status check_indexer_scores(int32_t n_heads, int32_t dim, const void* q_idx, const float* w_idx,
                                const void* key_pool, int64_t num_pages, const int32_t* block_table,
                                int32_t block_table_stride, const int32_t* seq_lens, int32_t batch,
                                const float* scores, int64_t score_stride);
// need_bytes / max_stride: the pick workspace size for (batch, stride) and the
// longest score row the pick kernels take
mla_status check_topk_select(const float* scores, int64_t score_stride, const int32_t* seq_lens, int32_t batch,
                             int32_t k, const int32_t* idx_out, const void* workspace, size_t workspace_bytes,
                             size_t need_bytes, int64_t max_stride);

}  // namespace mla_host
