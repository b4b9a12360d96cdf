// Internal declarations of the calls around the decode path (prefill,
// cache append, lightning indexer and top-k pick), shared by their host API
// and kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// prefill: per-head expansion of one request's latent (NT GEMM over D_C)
// cache formats of the expansion
constexpr int kExpandBf16 = 0, kExpandFp8Token = 1, kExpandFp8Group = 2;

struct ExpandArgs {
  const uint8_t* pool;
  int64_t page_bytes, rope_off, scale_off, num_pages;
  int32_t fmt;                 // kExpandBf16, kExpandFp8Token or kExpandFp8Group
  const int32_t* block_table;  // the request's pages
  int64_t T;
  const __bf16* w;             // [N][512]
  __bf16* out;                 // [T][N]
  int64_t N;                   // H * 128
  __bf16* k_rope;              // [T][64] or null
};

// prefill: causal attention over the expanded keys and values
struct PrefillArgs {
  const __bf16* qn;            // [N][H][128]
  const __bf16* qr;            // [N][H][64]
  const __bf16* kn;            // [T][H][128]
  const __bf16* v;             // [T][H][128]
  const __bf16* kr;            // [T][64]
  __bf16* out;                 // [N][H][128]
  float* lse;                  // [N][H] or null
  int64_t H, T, q_start, N;
  float scale;
};

hipError_t launch_expand(const ExpandArgs& a, hipStream_t s);
hipError_t launch_transpose_w_uk(const void* w_uk, void* w_uk_t, int H, int D_C, int D_N, hipStream_t s);
hipError_t launch_prefill_attn(const PrefillArgs& a, hipStream_t s);

// one new token per request written into its page slot
struct AppendArgs {
  const void* c_new;        // [batch][D_C], activation dtype
  const void* k_new;        // [batch][D_R], activation dtype, before rotation
  const float* rope_cos;    // [rope_rows][D_R / 2] or null
  const float* rope_sin;
  int32_t rope_rows;
  const int32_t* positions; // [batch]
  uint8_t* pool;
  int64_t num_pages, page_bytes, rope_off, scale_off;
  const int32_t* block_table;
  int32_t bt_stride;
  int32_t batch, D_C, D_R;
};

// kind: 0 F32 cache, 1 BF16, 2 FP8 with one scale per token, 3 FP8 with one
// scale per 128 latent channels
hipError_t launch_cache_append(const AppendArgs& a, int kind, hipStream_t s);

// lightning indexer scores: 64 heads x 128, FP8 search keys with one
// float32 scale per position
struct IndexerArgs {
  const void* q;            // [batch][64][128] BF16
  const float* w;           // [batch][64]
  const uint8_t* pool;      // search-key pages
  int64_t num_pages, page_bytes, scale_off;
  const int32_t* block_table;
  int32_t bt_stride;
  const int32_t* seq_lens;
  int32_t batch;
  float* scores;            // [batch][score_stride]
  int64_t score_stride;
  // fused pick: when set, each score's first radix digit is also counted
  // into this request's histogram of the pick workspace (requests with more
  // than topk positions only)
  uint32_t* hist;
  int32_t topk;
};

// top-k pick over score rows
struct TopkArgs {
  const float* scores;
  int64_t score_stride;
  const int32_t* seq_lens;
  int32_t batch;
  int32_t k;
  int32_t* idx_out;         // [batch][k]
  uint32_t* hist;           // workspace (layout in the pick kernels)
  int64_t len_cap;          // positions at or past it are not candidates
};

hipError_t launch_indexer_scores(const IndexerArgs& a, hipStream_t s);
hipError_t launch_topk_select(const TopkArgs& a, hipStream_t s);
// scores, with the pick's first histogram built by the score kernel, then the
// rest of the pick (a.hist and t.hist are the same workspace)
hipError_t launch_indexer_topk(const IndexerArgs& a, const TopkArgs& t, hipStream_t s);
size_t topk_workspace_bytes(int32_t batch, int64_t score_stride);
int64_t topk_max_stride();

}  // namespace mla
