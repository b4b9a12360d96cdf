// Lightning indexer scores and top-k pick, gfx950.
//
// Score ("DeepSeek's KV Cache", section "The score that picks positions",
// Figure 9): I(s) = sum_j w_j ReLU(q_j . k_s) over 64 indexer heads of width
// 128, with the search key k_s stored as E4M3 values times one float32 scale
// per position (section "Calculating V3.2's KV cache").
//
// Per work-group: 64 pages (4,096 positions) of one request, 4 waves, each
// wave 32 positions at a time.  The 64 x 128 query block of the request is the
// MFMA A operand (two 32-head blocks, held in registers for the whole
// work-group); the keys of 32 positions are the B operand, widened exactly
// from E4M3 to BF16 in registers.  D[head][position] comes out with one
// position per lane column, so ReLU, the head weights and the sum over the 32
// heads a lane holds are plain VALU work, and one lane swap adds the other 32.
// The scale multiplies the sum (ReLU is positively homogeneous).  The K index
// of the MFMA is permuted (lane half h, block kb covers dims 64h + 8kb .. +7)
// so each lane reads 64 contiguous key bytes; the query uses the same
// permutation, which leaves every dot product unchanged.
//
// Pick: radix selection on an order-preserving 32-bit image of the scores
// (11 + 11 + 10 bits from the top), spread over the chip in chunks of 4,096
// positions: (1) each chunk adds its first-digit histogram into the
// request's; (2) each chunk finds the digit holding the k-th largest score,
// counts its keys above that digit and gathers the keys in that digit's bin;
// (3) one work-group per request refines the two lower digits among the
// gathered keys -- the threshold key -- and turns per-chunk counts into
// per-chunk output offsets (equal keys are taken by position); (4) each chunk
// writes its picks in increasing order with a block prefix sum.  No work-group
// walks a whole row.
#include "attn_common.h"
#include "side_calls.h"

namespace mla {
namespace {

constexpr int kIdxHeads = 64;
constexpr int kIdxDim = 128;
constexpr int kIdxKeyRow = kIdxDim;          // bytes of one E4M3 key
constexpr int kIdxChunkPages = 64;           // pages per score work-group
constexpr int kIdxStages = 4;                // LDS ring stages per wave
constexpr int kIdxStage = 32 * kIdxKeyRow + 256;  // keys of a half page + its page's scales
constexpr int kIdxDmaPerStage = 5;           // load instructions per stage

// chunk swizzle of key row r inside a stage (8 chunks of 16 bytes per row)
__device__ __forceinline__ constexpr int idx_swz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }


__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  // exact: every E4M3 value is a BF16 value (unit scale)
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  u32x4 v;
  v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, false));
  v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, true));
  v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, false));
  v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, true));
  return __builtin_bit_cast(bf16x8, v);
}

// order-preserving image of a float: larger score -> larger key; -0 == +0;
// NaN below everything
__device__ __forceinline__ uint32_t score_key(float x) {
  if (x != x) return 0u;
  uint32_t u = __float_as_uint(x);
  if (x == 0.f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kHistBins = 2048;            // first and second digit: 11 bits

__global__ __launch_bounds__(256, 2) void indexer_score_kernel(IndexerArgs a) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31;   // position inside a 32-position group (B column)
  const int hl = lane >> 5;    // lane half
  int64_t T = sload(a.seq_lens + b);
  if (T > a.score_stride) T = a.score_stride;
  if (T > (int64_t)a.bt_stride * 64) T = (int64_t)a.bt_stride * 64;
  const int64_t p0 = (int64_t)blockIdx.x * kIdxChunkPages;
  if (T <= 0 || p0 * 64 >= T) return;
  // fused pick: first-digit histogram of this work-group's scores in LDS
  __shared__ uint32_t hist_l[kHistBins];
  const bool do_hist = a.hist != nullptr && T > a.topk;  // work-group uniform
  if (do_hist) {
    for (int i = threadIdx.x; i < kHistBins; i += 256) hist_l[i] = 0u;
    __syncthreads();
  }

  // A operand: query rows 32 mb + col, dims 64 hl + 8 kb .. +7
  const __bf16* qb = (const __bf16*)a.q + (int64_t)b * kIdxHeads * kIdxDim;
  bf16x8 qa[2][8];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) qa[mb][kb] = *(const bf16x8*)(qb + (32 * mb + col) * kIdxDim + 64 * hl + 8 * kb);
  // weights of the heads this lane's accumulators hold: 32 mb + 8 (r / 4) + 4 hl + r % 4
  float wt[2][16];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) wt[mb][r] = a.w[(int64_t)b * kIdxHeads + 32 * mb + 8 * (r >> 2) + 4 * hl + (r & 3)];
  float wh[2][16];  // halved weights (see the ReLU below)
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) wh[mb][r] = 0.5f * wt[mb][r];

  float* out = a.scores + (int64_t)b * a.score_stride;
  const int32_t* bt = a.block_table + (int64_t)b * a.bt_stride;

  // Wave w takes the half pages w, w + 4, ... of the chunk (32 positions
  // each) through a ring of kIdxStages LDS stages of its own: the keys (4 KiB)
  // and the page's 64 scales are moved HBM -> LDS by the load unit, so the
  // next stages are in flight while the current one is contracted, and the
  // waits are explicit counts.  A stage holds key row r's 16-byte chunk c at
  // chunk c ^ idx_swz(r), so the operand reads (row = lane % 32, 64 bytes at
  // 64 (lane / 32)) hit distinct banks; the swizzle is folded into the HBM
  // address of each lane, and every load instruction still covers 8 whole
  // rows (1 KiB contiguous).  No other wave touches the ring: no barriers.
  __shared__ __attribute__((aligned(16))) char idx_ring[4 * kIdxStages * kIdxStage];
  LDS char* ring = (LDS char*)idx_ring + w * kIdxStages * kIdxStage;
  const uint32_t ring_addr = (uint32_t)(uintptr_t)ring;
  const int64_t last_t = (T - 1) / 32 - 2 * p0;  // last half page before the context end
  const int last_hp = (int)(last_t < 2 * kIdxChunkPages - 1 ? last_t : 2 * kIdxChunkPages - 1);
  auto page_of = [&](int hp, bool& ok) {
    const int32_t page = sload(bt + p0 + (hp >> 1));
    ok = page >= 0 && page < a.num_pages;
    return a.pool + (ok ? (int64_t)page * a.page_bytes : 0);
  };
  // half pages past the context end load the last one again (never read), so
  // every iteration issues the same number of loads
  auto issue = [&](int hp, int st) {
    hp = hp <= last_hp ? hp : last_hp;
    bool ok;
    const uint8_t* pg = page_of(hp, ok);
    const uint8_t* keys = pg + 32 * (hp & 1) * kIdxKeyRow;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 8 * i + (lane >> 3);
      dma16_nt(keys + row * kIdxKeyRow + 16 * ((lane & 7) ^ idx_swz(row)), ring_addr + st * kIdxStage + 1024 * i);
    }
    dma4(pg + a.scale_off + 4 * ((32 * (hp & 1) + lane) & 63), ring_addr + st * kIdxStage + 4096);
  };

  // a wave with no half page skips the loop but still meets the barrier of
  // the histogram flush
  const bool any = w <= last_hp;
  // the query block and weights first: the loop's waits count ring loads only
  wait_vmcnt<0>();
  if (any) {
#pragma unroll
    for (int d = 0; d < kIdxStages; ++d) issue(w + 4 * d, d);
  }
  int st = 0;
  for (int hp = w; hp <= last_hp; hp += 4) {
    // this stage's loads are done when at most the newer stages' are pending
    wait_vmcnt<kIdxDmaPerStage * (kIdxStages - 1)>();
    __builtin_amdgcn_sched_barrier(0);
    const LDS char* sg = ring + st * kIdxStage;
    i32x4 kr[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) kr[m] = *(const LDS i32x4*)(sg + col * kIdxKeyRow + 16 * ((4 * hl + m) ^ idx_swz(col)));
    const float sc = *(const LDS float*)(sg + 4096 + 4 * col);
    bool ok;
    (void)page_of(hp, ok);
    const int64_t pos = (p0 + (hp >> 1)) * 64 + 32 * (hp & 1) + col;
    f32x16 acc0 = f32x16{}, acc1 = f32x16{};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const bf16x8 kv = e4m3x8_to_bf16((uint32_t)kr[kb >> 1][2 * (kb & 1)], (uint32_t)kr[kb >> 1][2 * (kb & 1) + 1]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][kb], kv, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][kb], kv, acc1, 0, 0, 0);
    }
    // w ReLU(x) as (w / 2)(x + |x|): one add with an abs modifier and the
    // fma, where fmaxf(x, 0) costs two instructions (it quiets x first).  The
    // product is exactly w x for x > 0 (halving and doubling are exact) and
    // +0 otherwise, so the sum is the same to the bit.
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sum = fmaf(wh[0][r], acc0[r] + fabsf(acc0[r]), sum);
      sum = fmaf(wh[1][r], acc1[r] + fabsf(acc1[r]), sum);
    }
    sum += wave_partner(sum);  // the other 32 heads of this position
    // a position on a page id out of range scores -infinity (its loads went
    // to page 0 and are discarded)
    if (hl == 0 && pos < T) {
      const float v = ok ? sum * sc : -INFINITY;
      out[pos] = v;
      if (do_hist) atomicAdd(&hist_l[score_key(v) >> 21], 1u);
    }
    // refill the stage just read (its reads returned before the MFMAs above)
    __builtin_amdgcn_sched_barrier(0);
    issue(hp + 4 * kIdxStages, st);
    st = st + 1 == kIdxStages ? 0 : st + 1;
  }
  // no load may still be writing this work-group's LDS when it ends
  wait_vmcnt<0>();
  if (do_hist) {
    __syncthreads();
    uint32_t* g = a.hist + (int64_t)b * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += 256)
      if (hist_l[i] != 0u) atomicAdd(&g[i], hist_l[i]);
  }
}

// ---- top-k pick ----
// Workspace sections (uint32, per request b):
//   hist [b][2048]   first-digit histogram
//   ctrl [b][16]     0: candidates gathered, 1: first digit, 2: picks left
//                    after it, 3: threshold key, 4: equal keys to take
//   gt0  [b][C]      per chunk: keys whose first digit is above the threshold's
//   off  [b][C]      per chunk: output offset of its first pick
//   take [b][C]      per chunk: threshold-equal keys it contributes
//   ckey, cpos [b][stride]  keys and positions of the threshold digit's bin
// with C = ceil(stride / 4096) chunks.
constexpr int kChunk = 4096;               // positions per chunk work-group
constexpr int kCtrl = 16;
constexpr int kRefineThreads = 1024;
constexpr int kMaxChunks = 2048;           // rows up to 8,388,608 positions

struct TopkSpace {
  uint32_t *hist, *ctrl, *gt0, *off, *take, *ckey, *cpos;
  int64_t nchunks;
};

__device__ __host__ inline int64_t topk_chunks(int64_t stride) { return (stride + kChunk - 1) / kChunk; }

__device__ __forceinline__ TopkSpace topk_space(const TopkArgs& a) {
  TopkSpace w;
  w.nchunks = topk_chunks(a.score_stride);
  uint32_t* p = a.hist;
  w.hist = p;
  p += (int64_t)a.batch * kHistBins;
  w.ctrl = p;
  p += (int64_t)a.batch * kCtrl;
  w.gt0 = p;
  p += (int64_t)a.batch * w.nchunks;
  w.off = p;
  p += (int64_t)a.batch * w.nchunks;
  w.take = p;
  p += (int64_t)a.batch * w.nchunks;
  w.ckey = p;
  p += (int64_t)a.batch * a.score_stride;
  w.cpos = p;
  return w;
}


__device__ __forceinline__ int64_t sel_len(const TopkArgs& a, int b) {
  int64_t T = sload(a.seq_lens + b);
  if (T < 0) T = 0;
  if (T > a.score_stride) T = a.score_stride;
  if (T > a.len_cap) T = a.len_cap;
  return T;
}

// exclusive prefix sum over a work-group of NT threads in thread order;
// `total` gets the sum over all threads.  Every thread must call it.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wave_tot, uint32_t& total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wave_tot[wv] = x;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t t = wave_tot[i];
    off += i < wv ? t : 0u;
    tot += t;
  }
  __syncthreads();  // wave_tot is reused by the next scan
  total = tot;
  return off + x - v;
}

// Given a histogram of `nbins` bins and kleft >= 1 keys still to pick from
// it, find the bin holding the kleft-th largest: returns the bin, and in
// *s_above how many keys lie in higher bins.  Threads take bins from the top.
template <int NT>
__device__ __forceinline__ int find_digit(const uint32_t* h, int nbins, uint32_t kleft, uint32_t* wave_tot,
                                          int* s_digit, uint32_t* s_above) {
  const int per = nbins / NT;
  const int t = threadIdx.x;
  uint32_t loc = 0;
  for (int e = 0; e < per; ++e) loc += h[nbins - 1 - (per * t + e)];
  uint32_t total;
  uint32_t above = block_excl_scan<NT>(loc, wave_tot, total);
  for (int e = 0; e < per; ++e) {
    const int bin = nbins - 1 - (per * t + e);
    const uint32_t c = h[bin];
    if (above < kleft && kleft <= above + c) {
      *s_digit = bin;
      *s_above = above;
    }
    above += c;
  }
  __syncthreads();
  return *s_digit;
}

__global__ __launch_bounds__(256) void topk_clear_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// 1. first digit (top 11 bits of the key) of every score, per request
__global__ __launch_bounds__(256) void topk_hist_kernel(TopkArgs a) {
  __shared__ uint32_t h[kHistBins];
  const int b = blockIdx.y;
  const int64_t T = sel_len(a, b);
  const int64_t i0 = (int64_t)blockIdx.x * kChunk;
  if (T <= a.k || i0 >= T) return;  // nothing to select in this request or chunk
  for (int i = threadIdx.x; i < kHistBins; i += 256) h[i] = 0u;
  __syncthreads();
  const float* s = a.scores + (int64_t)b * a.score_stride;
  const int64_t i1 = i0 + kChunk < T ? i0 + kChunk : T;
  for (int64_t i = i0 + threadIdx.x; i < i1; i += 256) atomicAdd(&h[score_key(s[i]) >> 21], 1u);
  __syncthreads();
  uint32_t* g = topk_space(a).hist + (int64_t)b * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += 256)
    if (h[i] != 0u) atomicAdd(&g[i], h[i]);
}

// four consecutive keys from position i (keys past n are 0 and flagged out)
__device__ __forceinline__ void keys4(const float* s, int64_t i, int64_t n, bool vec_ok, uint32_t (&key)[4]) {
  if (vec_ok && i + 3 < n) {
    const f32x4 v = *(const f32x4*)(s + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) key[e] = score_key(v[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) key[e] = i + e < n ? score_key(s[i + e]) : 0u;
  }
}

// 2. per chunk: the keys above the threshold's first digit are counted, the
// keys in its bin are gathered (with their positions) for the refinement
__global__ __launch_bounds__(256) void topk_gather_kernel(TopkArgs a) {
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t wave_tot[4];
  __shared__ int s_digit;
  __shared__ uint32_t s_above;
  const int b = blockIdx.y;
  const int64_t c = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t T = sel_len(a, b);
  const TopkSpace w = topk_space(a);
  if (T <= a.k) {
    // every visible position, then padding (one work-group per request)
    if (c == 0) {
      int32_t* out = a.idx_out + (int64_t)b * a.k;
      for (int64_t i = t; i < a.k; i += 256) out[i] = i < T ? (int32_t)i : -1;
    }
    return;
  }
  const int64_t i0 = c * kChunk;
  if (i0 >= T) return;
  const uint32_t* g = w.hist + (int64_t)b * kHistBins;
  for (int i = t; i < kHistBins; i += 256) h[i] = g[i];
  __syncthreads();
  const uint32_t d0 = (uint32_t)find_digit<256>(h, kHistBins, (uint32_t)a.k, wave_tot, &s_digit, &s_above);
  uint32_t* ctrl = w.ctrl + (int64_t)b * kCtrl;
  if (c == 0 && t == 0) {
    ctrl[1] = d0;
    ctrl[2] = (uint32_t)a.k - s_above;
  }
  const float* s = a.scores + (int64_t)b * a.score_stride;
  const bool vec_ok = (((uintptr_t)s) & 15) == 0;
  uint32_t* ckey = w.ckey + (int64_t)b * a.score_stride;
  uint32_t* cpos = w.cpos + (int64_t)b * a.score_stride;
  // this thread's 16 keys: four groups of four consecutive positions
  uint32_t key[kChunk / 1024][4];
#pragma unroll
  for (int sb = 0; sb < kChunk / 1024; ++sb) keys4(s, i0 + 1024 * sb + 4 * t, T, vec_ok, key[sb]);
  uint32_t ngt = 0, nin = 0;
#pragma unroll
  for (int sb = 0; sb < kChunk / 1024; ++sb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = i0 + 1024 * sb + 4 * t + e < T;
      ngt += (ok && (key[sb][e] >> 21) > d0) ? 1u : 0u;
      nin += (ok && (key[sb][e] >> 21) == d0) ? 1u : 0u;
    }
  // one counter update per work-group reserves the chunk's candidate slots
  uint32_t nin_tot;
  uint32_t slot = block_excl_scan<256>(nin, wave_tot, nin_tot);
  if (t == 0) s_above = nin_tot != 0u ? atomicAdd(&ctrl[0], nin_tot) : 0u;
  __syncthreads();
  slot += s_above;
  if (nin != 0u) {
#pragma unroll
    for (int sb = 0; sb < kChunk / 1024; ++sb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t i = i0 + 1024 * sb + 4 * t + e;
        if (i < T && (key[sb][e] >> 21) == d0) {
          ckey[slot] = key[sb][e];
          cpos[slot] = (uint32_t)i;
          ++slot;
        }
      }
  }
  uint32_t total;
  block_excl_scan<256>(ngt, wave_tot, total);
  if (t == 0) w.gt0[(int64_t)b * w.nchunks + c] = total;
}

// 3. per request: the two lower digits among the gathered keys give the
// threshold key; then each chunk's share of the output and its offset
__global__ __launch_bounds__(kRefineThreads) void topk_refine_kernel(TopkArgs a) {
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t cg[kMaxChunks], ce[kMaxChunks];
  __shared__ uint32_t wave_tot[kRefineThreads / 64];
  __shared__ int s_digit;
  __shared__ uint32_t s_above;
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t T = sel_len(a, b);
  if (T <= a.k) return;
  const TopkSpace w = topk_space(a);
  uint32_t* ctrl = w.ctrl + (int64_t)b * kCtrl;
  const uint32_t nc = ctrl[0];
  uint32_t prefix = ctrl[1] << 21;
  uint32_t kleft = ctrl[2];
  uint32_t mask = 0xFFE00000u;
  const uint32_t* ckey = w.ckey + (int64_t)b * a.score_stride;
  const uint32_t* cpos = w.cpos + (int64_t)b * a.score_stride;
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 10 : 0;
    const int nbins = pass == 0 ? 2048 : 1024;
    for (int i = t; i < nbins; i += kRefineThreads) h[i] = 0u;
    __syncthreads();
    for (uint32_t i = t; i < nc; i += kRefineThreads) {
      const uint32_t key = ckey[i];
      if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & (uint32_t)(nbins - 1)], 1u);
    }
    __syncthreads();
    prefix |= (uint32_t)find_digit<kRefineThreads>(h, nbins, kleft, wave_tot, &s_digit, &s_above) << shift;
    kleft -= s_above;
    mask |= (uint32_t)(nbins - 1) << shift;
    __syncthreads();
  }
  const uint32_t thr = prefix;
  // gathered keys above / equal to the threshold, per chunk
  const int64_t nch = (T + kChunk - 1) / kChunk;
  for (int64_t i = t; i < nch; i += kRefineThreads) {
    cg[i] = 0u;
    ce[i] = 0u;
  }
  __syncthreads();
  for (uint32_t i = t; i < nc; i += kRefineThreads) {
    const uint32_t key = ckey[i];
    const uint32_t ch = cpos[i] / kChunk;
    if (key > thr) atomicAdd(&cg[ch], 1u);
    else if (key == thr) atomicAdd(&ce[ch], 1u);
  }
  __syncthreads();
  // thread t owns chunks 2t, 2t + 1: the first `kleft` equal keys in
  // position order are taken, chunk by chunk
  uint32_t eqs[2], tot[2];
  uint32_t leq = 0;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int64_t ch = 2 * t + e;
    eqs[e] = ch < nch ? ce[ch] : 0u;
    leq += eqs[e];
  }
  uint32_t unused;
  uint32_t eq_before = block_excl_scan<kRefineThreads>(leq, wave_tot, unused);
  uint32_t take[2];
  uint32_t ltot = 0;
  const uint32_t* gt0 = w.gt0 + (int64_t)b * w.nchunks;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int64_t ch = 2 * t + e;
    take[e] = eq_before >= kleft ? 0u : (kleft - eq_before < eqs[e] ? kleft - eq_before : eqs[e]);
    eq_before += eqs[e];
    tot[e] = ch < nch ? gt0[ch] + cg[ch] + take[e] : 0u;
    ltot += tot[e];
  }
  uint32_t off = block_excl_scan<kRefineThreads>(ltot, wave_tot, unused);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int64_t ch = 2 * t + e;
    if (ch < nch) {
      w.off[(int64_t)b * w.nchunks + ch] = off;
      w.take[(int64_t)b * w.nchunks + ch] = take[e];
    }
    off += tot[e];
  }
  if (t == 0) ctrl[3] = thr;
}

// 4. per chunk: picked positions (keys above the threshold, and the chunk's
// share of the equal ones, first by position) in increasing order
__global__ __launch_bounds__(256) void topk_write_kernel(TopkArgs a) {
  __shared__ uint32_t wave_tot[4];
  const int b = blockIdx.y;
  const int64_t c = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t T = sel_len(a, b);
  if (T <= a.k) return;
  const int64_t i0 = c * kChunk;
  if (i0 >= T) return;
  const TopkSpace w = topk_space(a);
  const uint32_t thr = w.ctrl[(int64_t)b * kCtrl + 3];
  const uint32_t base = w.off[(int64_t)b * w.nchunks + c];
  const uint32_t take = w.take[(int64_t)b * w.nchunks + c];
  const float* s = a.scores + (int64_t)b * a.score_stride;
  const bool vec_ok = (((uintptr_t)s) & 15) == 0;
  int32_t* out = a.idx_out + (int64_t)b * a.k;
  uint32_t gt_run = 0, eq_run = 0;
  for (int sb = 0; sb < kChunk / 1024; ++sb) {
    const int64_t i = i0 + 1024 * sb + 4 * t;
    uint32_t key[4];
    keys4(s, i, T, vec_ok, key);
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ngt += (i + e < T && key[e] > thr) ? 1u : 0u;
      neq += (i + e < T && key[e] == thr) ? 1u : 0u;
    }
    uint32_t total;
    const uint32_t ex = block_excl_scan<256>((ngt << 16) | neq, wave_tot, total);
    uint32_t gt_before = gt_run + (ex >> 16), eq_before = eq_run + (ex & 0xFFFFu);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (i + e >= T) break;
      if (key[e] > thr) {
        out[base + gt_before + (eq_before < take ? eq_before : take)] = (int32_t)(i + e);
        ++gt_before;
      } else if (key[e] == thr) {
        if (eq_before < take) out[base + gt_before + eq_before] = (int32_t)(i + e);
        ++eq_before;
      }
    }
    gt_run += total >> 16;
    eq_run += total & 0xFFFFu;
  }
}

}  // namespace

hipError_t launch_indexer_scores(const IndexerArgs& a, hipStream_t s) {
  const dim3 grid((a.bt_stride + kIdxChunkPages - 1) / kIdxChunkPages, a.batch);
  hipLaunchKernelGGL(indexer_score_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

int64_t topk_max_stride() { return (int64_t)kMaxChunks * kChunk; }

size_t topk_workspace_bytes(int32_t batch, int64_t score_stride) {
  const int64_t words = (int64_t)batch * (kHistBins + kCtrl + 3 * topk_chunks(score_stride) + 2 * score_stride);
  return (size_t)words * 4;
}

hipError_t launch_topk_select(const TopkArgs& a, hipStream_t s) {
  // clear the histograms and the control words (candidate counters)
  const int64_t n = (int64_t)a.batch * (kHistBins + kCtrl);
  hipLaunchKernelGGL(topk_clear_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.hist, n);
  const dim3 chunks((unsigned)topk_chunks(a.score_stride), a.batch);
  hipLaunchKernelGGL(topk_hist_kernel, chunks, dim3(256), 0, s, a);
  hipLaunchKernelGGL(topk_gather_kernel, chunks, dim3(256), 0, s, a);
  hipLaunchKernelGGL(topk_refine_kernel, dim3(a.batch), dim3(kRefineThreads), 0, s, a);
  hipLaunchKernelGGL(topk_write_kernel, chunks, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_indexer_topk(const IndexerArgs& a, const TopkArgs& t, hipStream_t s) {
  const int64_t n = (int64_t)t.batch * (kHistBins + kCtrl);
  hipLaunchKernelGGL(topk_clear_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, t.hist, n);
  const dim3 grid((a.bt_stride + kIdxChunkPages - 1) / kIdxChunkPages, a.batch);
  hipLaunchKernelGGL(indexer_score_kernel, grid, dim3(256), 0, s, a);
  const dim3 chunks((unsigned)topk_chunks(t.score_stride), t.batch);
  hipLaunchKernelGGL(topk_gather_kernel, chunks, dim3(256), 0, s, t);
  hipLaunchKernelGGL(topk_refine_kernel, dim3(t.batch), dim3(kRefineThreads), 0, s, t);
  hipLaunchKernelGGL(topk_write_kernel, chunks, dim3(256), 0, s, t);
  return hipGetLastError();
}

}  // namespace mla
