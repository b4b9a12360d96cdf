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
// takes units [lo(p), lo(p+1)) (worker_lo: floor(p*W/P), or weighted by XCD
// as below) and processes the tiles among them.  The lead stands for the fixed cost of starting a request
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
//
// Unequal shares by XCD.  The attention kernels give worker p to a
// work-group of XCD p / (P / 8) (consecutive workers share requests, and each
// XCD has its own L2), and under this load the odd-numbered XCDs of an
// MI355X run 2-5% slower than the even ones (per-XCD shader clocks measured
// with s_memtime / s_memrealtime pairs on every box used; the slowest XCD
// was an odd one every time).  The launch ends with its slowest XCD, so for
// dense batches with enough units per worker (at least 64, where one tile is
// under 1.6% of a share) a worker's share is weighted 65 on an even XCD and
// 63 on an odd one, instead of 64 each.  The weights are constants: the
// partition depends only on (W, P, topk), so results are the same on every
// run.  Index lists keep equal shares (with a worker count that is a
// multiple of the batch every worker then stays inside one request).  The
// weighted form needs P a power of two (the weight total 64 P then divides
// by a shift), as the one-worker-per-CU plan gives on 256 CUs.
constexpr int64_t kShareWeight = 64, kShareSkew = 1;
constexpr bool xcd_weighted(int64_t W, int64_t P, int32_t topk) {
  return topk <= 0 && P >= 16 && (P & (P - 1)) == 0 && W >= 64 * P;
}
// Weight of workers [0, p) for P a power of two: kShareWeight p plus
// kShareSkew times (workers on even XCDs - workers on odd XCDs) among them.
constexpr int64_t share_weight_below(int64_t p, int64_t P) {
  const int sh = __builtin_ctzll((uint64_t)P) - 3;  // P / 8 workers per XCD
  const int64_t k = p >> sh, r = p & ((P >> 3) - 1);
  return kShareWeight * p + kShareSkew * ((k & 1) ? (P >> 3) - r : r);
}
// First unit of worker p's range.  Equal shares: floor(p W / P), from an
// estimate in double precision and exact steps (no 64-bit integer division,
// which is a long software routine on the GPU).
constexpr int64_t worker_lo(int64_t p, int64_t W, int64_t P, int32_t topk) {
  if (xcd_weighted(W, P, topk)) return (W * share_weight_below(p, P)) >> (6 + __builtin_ctzll((uint64_t)P));
  const int64_t n = p * W;
  int64_t q = (int64_t)((double)n / (double)P);
  while (q > 0 && q * P > n) --q;
  while ((q + 1) * P <= n) ++q;
  return q;
}
// Worker whose range contains unit x (0 <= x < W): the last worker whose
// range starts at or before x.  An estimate in double precision (the
// weighted bounds lie within P / 512 workers of the equal ones), then exact
// steps on the bounds; no 64-bit integer division.
constexpr int64_t worker_of(int64_t x, int64_t W, int64_t P, int32_t topk) {
  int64_t p = (int64_t)((double)x * (double)P / (double)W);
  if (p < 0) p = 0;
  if (p > P - 1) p = P - 1;
  if (xcd_weighted(W, P, topk)) {
    while (p > 0 && worker_lo(p, W, P, topk) > x) --p;
    while (p + 1 < P && worker_lo(p + 1, W, P, topk) <= x) ++p;
  } else {
    // equal shares: worker_lo(p) <= x exactly when p W <= x P + P - 1
    while (p > 0 && p * W > x * P + P - 1) --p;
    while (p + 1 < P && (p + 1) * W <= x * P + P - 1) ++p;
  }
  return p;
}
constexpr int32_t tiles_of(int32_t len) { return (len + kTile - 1) / kTile; }
// Units of the split space taken by a request with nt tiles.
constexpr int64_t span_of(int32_t nt, int32_t topk) { return nt > 0 ? (int64_t)nt + lead_of(topk) : 0; }

}  // namespace mla
