// Lightning indexer scores and top-k pick, gfx950.
//
// Score ("DeepSeek's KV Cache", section "The score that picks positions",
// Figure 9): I(s) = sum_j w_j ReLU(q_j . k_s) over 64 indexer heads of width
// 128, with the search key k_s stored as E4M3 values times one float32 scale
// per position (section "Calculating V3.2's KV cache").
//
// Per work-group: 16 pages (1,024 positions) of one request, 4 waves, each
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
// (11 + 11 + 10 bits from the top).  The first digit's histogram is built by
// many work-groups at once (a chip-wide pass with LDS histograms flushed by
// global atomics), so its crowded top bins do not serialise one CU's LDS
// atomics; one work-group per request then finds the digit holding the k-th
// largest score, refines the two lower digits over the positions that still
// match, and writes the picked positions in increasing order with a block
// prefix sum (equal scores: the lowest positions first).
#include "attn_common.h"

namespace mla {
namespace {

constexpr int kIdxHeads = 64;
constexpr int kIdxDim = 128;
constexpr int kIdxKeyRow = kIdxDim;          // bytes of one E4M3 key
constexpr int kIdxChunkPages = 16;           // pages per score work-group

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

  float* out = a.scores + (int64_t)b * a.score_stride;
  const int32_t* bt = a.block_table + (int64_t)b * a.bt_stride;

  // wave w takes the half pages w, w + 4, ... of the chunk (32 positions each)
  for (int hp = w; hp < 2 * kIdxChunkPages; hp += 4) {
    const int64_t p = p0 + (hp >> 1);
    const int64_t pos0 = p * 64 + 32 * (hp & 1);
    if (pos0 >= T) break;  // wave-uniform; later half pages are further out
    const int32_t page = sload(bt + p);
    const int64_t pos = pos0 + col;
    if (page < 0 || page >= a.num_pages) {
      if (hl == 0 && pos < T) out[pos] = -INFINITY;
      continue;
    }
    const uint8_t* pg = a.pool + (int64_t)page * a.page_bytes;
    const int slot = 32 * (hp & 1) + col;
    const i32x4* src = (const i32x4*)(pg + slot * kIdxKeyRow + 64 * hl);
    const i32x4 r0 = src[0], r1 = src[1], r2 = src[2], r3 = src[3];
    const float sc = *(const float*)(pg + a.scale_off + 4 * slot);
    const uint32_t raw[16] = {(uint32_t)r0[0], (uint32_t)r0[1], (uint32_t)r0[2], (uint32_t)r0[3],
                              (uint32_t)r1[0], (uint32_t)r1[1], (uint32_t)r1[2], (uint32_t)r1[3],
                              (uint32_t)r2[0], (uint32_t)r2[1], (uint32_t)r2[2], (uint32_t)r2[3],
                              (uint32_t)r3[0], (uint32_t)r3[1], (uint32_t)r3[2], (uint32_t)r3[3]};
    f32x16 acc0 = f32x16{}, acc1 = f32x16{};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const bf16x8 kv = e4m3x8_to_bf16(raw[2 * kb], raw[2 * kb + 1]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][kb], kv, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][kb], kv, acc1, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s = fmaf(wt[0][r], fmaxf(acc0[r], 0.f), s);
      s = fmaf(wt[1][r], fmaxf(acc1[r], 0.f), s);
    }
    s += wave_partner(s);  // the other 32 heads of this position
    if (hl == 0 && pos < T) out[pos] = s * sc;
  }
}

// ---- top-k pick ----
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kHistBins = 2048;            // first and second digit: 11 bits
constexpr int kHistChunk = 4096;           // scores per histogram work-group

// order-preserving image of a float: larger score -> larger key; -0 == +0;
// NaN below everything
__device__ __forceinline__ uint32_t score_key(float x) {
  if (x != x) return 0u;
  uint32_t u = __float_as_uint(x);
  if (x == 0.f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int64_t sel_len(const TopkArgs& a, int b) {
  int64_t T = sload(a.seq_lens + b);
  if (T < 0) T = 0;
  if (T > a.score_stride) T = a.score_stride;
  return T;
}

__global__ __launch_bounds__(256) void topk_clear_kernel(uint32_t* hist, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) hist[i] = 0u;
}

// first digit (top 11 bits of the key) of every score, per request
__global__ __launch_bounds__(256) void topk_hist_kernel(TopkArgs a) {
  __shared__ uint32_t h[kHistBins];
  const int b = blockIdx.y;
  const int64_t T = sel_len(a, b);
  const int64_t i0 = (int64_t)blockIdx.x * kHistChunk;
  if (T <= a.k || i0 >= T) return;  // nothing to select in this request or chunk
  for (int i = threadIdx.x; i < kHistBins; i += 256) h[i] = 0u;
  __syncthreads();
  const float* s = a.scores + (int64_t)b * a.score_stride;
  const int64_t i1 = i0 + kHistChunk < T ? i0 + kHistChunk : T;
  for (int64_t i = i0 + threadIdx.x; i < i1; i += 256) atomicAdd(&h[score_key(s[i]) >> 21], 1u);
  __syncthreads();
  uint32_t* g = a.hist + (int64_t)b * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += 256)
    if (h[i] != 0u) atomicAdd(&g[i], h[i]);
}

// exclusive prefix sum over the work-group in thread order; `total` gets the
// sum over all threads.  Every thread must call it.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wave_tot, uint32_t& total) {
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
  for (int i = 0; i < kSelWaves; ++i) {
    const uint32_t t = wave_tot[i];
    off += i < wv ? t : 0u;
    tot += t;
  }
  __syncthreads();  // wave_tot is reused by the next scan
  total = tot;
  return off + x - v;
}

// Given a histogram of `nbins` bins (LDS) and kleft >= 1 keys still to pick
// from it, find the bin holding the kleft-th largest: returns the bin and, in
// `above`, how many keys lie in higher bins.  Threads take bins from the top.
__device__ __forceinline__ int find_digit(const uint32_t* h, int nbins, uint32_t kleft, uint32_t* wave_tot,
                                          int* s_digit, uint32_t* s_above) {
  const int per = nbins / kSelThreads;  // 2 or 1
  const int t = threadIdx.x;
  uint32_t loc = 0;
  for (int e = 0; e < per; ++e) loc += h[nbins - 1 - (per * t + e)];
  uint32_t total;
  uint32_t above = block_excl_scan(loc, wave_tot, total);
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

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(TopkArgs a) {
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t wave_tot[kSelWaves];
  __shared__ int s_digit;
  __shared__ uint32_t s_above;
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t T = sel_len(a, b);
  const int k = a.k;
  int32_t* out = a.idx_out + (int64_t)b * k;
  const float* s = a.scores + (int64_t)b * a.score_stride;

  if (T <= k) {
    // every visible position, then padding
    for (int64_t i = t; i < k; i += kSelThreads) out[i] = i < T ? (int32_t)i : -1;
    return;
  }

  // digit 1 (bits 31..21): the chip-wide histogram
  const uint32_t* g = a.hist + (int64_t)b * kHistBins;
  for (int i = t; i < kHistBins; i += kSelThreads) h[i] = g[i];
  __syncthreads();
  uint32_t kleft = (uint32_t)k;
  uint32_t prefix = (uint32_t)find_digit(h, kHistBins, kleft, wave_tot, &s_digit, &s_above) << 21;
  kleft -= s_above;
  uint32_t mask = 0xFFE00000u;

  // digits 2 (bits 20..10) and 3 (bits 9..0) over the keys that still match
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 10 : 0;
    const int nbins = pass == 0 ? 2048 : 1024;
    for (int i = t; i < nbins; i += kSelThreads) h[i] = 0u;
    __syncthreads();
    for (int64_t i = t; i < T; i += kSelThreads) {
      const uint32_t key = score_key(s[i]);
      if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & (uint32_t)(nbins - 1)], 1u);
    }
    __syncthreads();
    prefix |= (uint32_t)find_digit(h, nbins, kleft, wave_tot, &s_digit, &s_above) << shift;
    kleft -= s_above;
    mask |= (uint32_t)(nbins - 1) << shift;
    __syncthreads();  // s_digit / s_above are rewritten by the next pass
  }

  // The k-th largest key is `prefix`; every larger key is picked, and the
  // first `kleft` equal ones by position.  Positions are visited in order and
  // each picked one lands at its rank among the picked: increasing order.
  const uint32_t thr = prefix;
  uint32_t gt_run = 0, eq_run = 0;
  for (int64_t base = 0; base < T; base += kSelThreads) {
    const int64_t i = base + t;
    const uint32_t key = i < T ? score_key(s[i]) : 0u;
    const bool gt = i < T && key > thr;
    const bool eq = i < T && key == thr;
    uint32_t total;
    const uint32_t ex = block_excl_scan((gt ? 0x10000u : 0u) | (eq ? 1u : 0u), wave_tot, total);
    const uint32_t gt_before = gt_run + (ex >> 16), eq_before = eq_run + (ex & 0xFFFFu);
    if (gt) out[gt_before + (eq_before < kleft ? eq_before : kleft)] = (int32_t)i;
    if (eq && eq_before < kleft) out[gt_before + eq_before] = (int32_t)i;
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

size_t topk_workspace_bytes(int32_t batch) { return (size_t)batch * kHistBins * 4; }

hipError_t launch_topk_select(const TopkArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.batch * kHistBins;
  hipLaunchKernelGGL(topk_clear_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.hist, n);
  const int64_t chunks = (a.score_stride + kHistChunk - 1) / kHistChunk;
  hipLaunchKernelGGL(topk_hist_kernel, dim3((unsigned)chunks, a.batch), dim3(256), 0, s, a);
  hipLaunchKernelGGL(topk_select_kernel, dim3(a.batch), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
