// Launch arguments of the decode-path kernels, and the split partition the
// attention and merge kernels share.  Plain C++ with no HIP types, so the
// host-side checks that fill these structs build without HIP (and under host
// sanitizers).  constexpr functions here are usable in device code too.
// Not part of the public ABI.
#pragma once

#include <stddef.h>
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

// latent storage of the MFMA attention kernels
enum class CacheKind { kBf16, kFp8Token, kFp8Group128 };

// LDS layout of the generic float32 attention kernel (offsets in floats).
struct F32Layout {
  int q = 0, qr = 0, c = 0, r = 0, s = 0, o = 0, m = 0, l = 0, al = 0, valid = 0, total = 0;
  constexpr F32Layout(int H, int DC, int DR) {
    q = 0;
    qr = q + H * DC;
    c = qr + H * DR;
    r = c + kTile * DC;
    s = r + kTile * DR;
    o = s + H * kTile;
    m = o + H * DC;
    l = m + H;
    al = l + H;
    valid = al + H;
    total = valid + kTile;
  }
};

constexpr size_t decode_f32_lds_bytes(int H, int D_C, int D_R) {
  return (size_t)F32Layout(H, D_C, D_R).total * sizeof(float);
}

// ---------------------------------------------------------------------------
// Split partition shared by the attention kernels and the combine kernel.
// Every request with at least one tile occupies span_of(nt) = lead + nt units
// of a concatenated space (requests in order, W units in total): a lead of
// kLeadTiles units that carry no work (dense requests only), then its nt
// tiles.  Worker p
// takes units [lo(p), lo(p+1)) with lo(p) = floor(p*W/P) and processes the
// tiles among them.  The lead stands for the fixed cost of starting a request
// (query loads, pipeline fill, one more partial to write): a worker whose
// range crosses into a new request gets that many fewer tiles, which evens
// out the finishing times.  A worker that covers tiles of several requests
// emits one partial per request into slot p + b, which is unique because p
// and b never both stay the same from one piece to the next.
// ---------------------------------------------------------------------------
constexpr int32_t kLeadTiles = 12;
// With index lists every request has the same number of tiles and there is no
// lead: a plan whose worker count is a multiple of the batch then gives every
// worker tiles of one request only (one segment, one partial).
constexpr int32_t lead_of(int32_t topk) { return topk > 0 ? 0 : kLeadTiles; }
constexpr int64_t worker_lo(int64_t p, int64_t W, int64_t P) { return (p * W) / P; }
// Worker whose range contains unit x (0 <= x < W).
constexpr int64_t worker_of(int64_t x, int64_t W, int64_t P) { return ((x + 1) * P - 1) / W; }
constexpr int32_t tiles_of(int32_t len) { return (len + kTile - 1) / kTile; }
// Units of the split space taken by a request with nt tiles.
constexpr int64_t span_of(int32_t nt, int32_t topk) { return nt > 0 ? (int64_t)nt + lead_of(topk) : 0; }

}  // namespace mla
