// Internal declarations shared by the host API and the kernel translation
// units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kPageTokens = 64;
constexpr int kTile = 32;  // positions per attention tile (split granularity)

// V2 dimensions served by the MFMA kernels.
constexpr int kHeads = 128;
constexpr int kLatent = 512;
constexpr int kRope = 64;

struct DecodeArgs {
  const void* q_lat;
  const void* q_rope;
  const uint8_t* pool;
  int64_t num_pages;
  int64_t page_bytes;
  int64_t rope_off;
  int64_t scale_off;
  const int32_t* block_table;
  int32_t bt_stride;
  const int32_t* seq_lens;
  const int32_t* topk_idx;  // nullptr = dense
  int32_t topk;
  int32_t batch;
  int32_t num_workers;      // 0 = one work-group per request, final output
  void* part_o;             // [slots][H][D_C], BF16 if part_bf16 else FP32
  float* part_lse;          // [slots][H]
  int32_t part_bf16;
  void* o_lat;              // final output (direct mode)
  float* lse_out;           // optional
  int32_t H, D_C, D_R;
  float scale;
};

struct CombineArgs {
  const void* part_o;       // [slots][H][D_C], BF16 if part_bf16 else FP32
  const float* part_lse;
  int32_t part_bf16;
  const int32_t* seq_lens;
  int32_t topk;
  int32_t batch;
  int32_t num_workers;
  void* o_lat;
  float* lse_out;
  int32_t H, D_C;
  int32_t out_bf16;
};

// merge + value up-projection in one launch
struct CombineUpArgs {
  CombineArgs c;            // o_lat unused
  const void* w_uv;         // [H][D_V][D_C] BF16
  void* out;                // [batch][H][D_V] BF16
};

struct HeadGemmArgs {
  // y[b][h][m] = sum_k w[h][m][k] * x[b][h][k]
  const void* x;
  const void* w;
  void* y;
  int32_t batch, H, M, K;
};

// prefill: per-head expansion of one request's latent (NT GEMM over D_C)
struct ExpandArgs {
  const uint8_t* pool;
  int64_t page_bytes, rope_off, num_pages;
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
};

hipError_t launch_indexer_scores(const IndexerArgs& a, hipStream_t s);
hipError_t launch_topk_select(const TopkArgs& a, hipStream_t s);
size_t topk_workspace_bytes(int32_t batch, int64_t score_stride);
int64_t topk_max_stride();

// latent storage of the MFMA attention kernels
enum class CacheKind { kBf16, kFp8Token, kFp8Group128 };

hipError_t launch_decode_mfma(const DecodeArgs& a, CacheKind kind, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s);  // BF16 cache, dense
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_combine_up(const CombineUpArgs& u, hipStream_t s);  // V2 dims, BF16
hipError_t launch_head_gemm_bf16(const HeadGemmArgs& a, hipStream_t s);
hipError_t launch_head_gemm_f32(const HeadGemmArgs& a, hipStream_t s);

// LDS bytes the generic fp32 attention kernel needs for these dims.
size_t decode_f32_lds_bytes(int H, int D_C, int D_R);

}  // namespace mla

// ---------------------------------------------------------------------------
// Split partition shared by the attention kernels and the combine kernel.
// Every request with at least one tile occupies span_of(nt) = kLeadTiles + nt
// units of a concatenated space (requests in order, W units in total): a
// lead of kLeadTiles units that carry no work, then its nt tiles.  Worker p
// takes units [lo(p), lo(p+1)) with lo(p) = floor(p*W/P) and processes the
// tiles among them.  The lead stands for the fixed cost of starting a request
// (query loads, pipeline fill, one more partial to write): a worker whose
// range crosses into a new request gets that many fewer tiles, which evens
// out the finishing times.  A worker that covers tiles of several requests
// emits one partial per request into slot p + b, which is unique because p
// and b never both stay the same from one piece to the next.
// ---------------------------------------------------------------------------
namespace mla {
constexpr int32_t kLeadTiles = 12;
__host__ __device__ inline int64_t worker_lo(int64_t p, int64_t W, int64_t P) { return (p * W) / P; }
// Worker whose range contains unit x (0 <= x < W).
__host__ __device__ inline int64_t worker_of(int64_t x, int64_t W, int64_t P) {
  return ((x + 1) * P - 1) / W;
}
__host__ __device__ inline int32_t tiles_of(int32_t len) { return (len + kTile - 1) / kTile; }
// Units of the split space taken by a request with nt tiles.
__host__ __device__ inline int64_t span_of(int32_t nt) { return nt > 0 ? (int64_t)nt + kLeadTiles : 0; }
}  // namespace mla
