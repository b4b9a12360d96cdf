// Log-sum-exp merge of split partials.
//
// A partial over a disjoint set of positions S_s holds the softmax-normalised
// weighted latent o_s and lse_s = log sum_{j in S_s} exp(score_j).  Softmax
// over the union of the sets is then
//   o = sum_s exp(lse_s - LSE) o_s,   LSE = log sum_s exp(lse_s),
// an exact identity.  Which slots hold request b's partials follows from the
// same tile partition the attention kernel used (worker p writes slot p + b).
//
// One wave per (request, head) -- or, for small batches, one work-group per
// (request, head) with its partials split over the waves: each lane owns 8
// consecutive latent columns (one 16-byte load per partial for BF16 partials,
// two for FP32), so a head row of 512 values is one coalesced read per
// partial, and the loads of 8 partials are in flight together.  The merge weights are computed one
// partial per lane and read back with readlane.
#include "tile_space.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 8;  // partials whose loads are in flight together

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

// Wave-wide reductions without the LDS crossbar: butterflies inside each
// 16-lane row by DPP (swap neighbours, swap pairs, mirror 8, mirror 16), then
// the neighbouring row and the other half of the wave by the permlane swaps.
// Every lane ends with the result.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_partner(float v) {
  // value held by lane l ^ 16
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((__lane_id() & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float half_partner(float v) {
  // value held by lane l ^ 32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((__lane_id() < 32) ? r[1] : r[0]);
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm 1,0,3,2
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm 2,3,0,1
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(v));  // row_mirror
  v = fmaxf(v, row_partner(v));
  return fmaxf(v, half_partner(v));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  v += row_partner(v);
  return v + half_partner(v);
}

// 8 consecutive partial values starting at src, as FP32
template <typename PT>
__device__ __forceinline__ void load8(const PT* src, f32x4& lo, f32x4& hi) {
  if constexpr (sizeof(PT) == 2) {
    const bf16x8 v = *(const bf16x8*)src;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[e] = (float)v[e];
      hi[e] = (float)v[4 + e];
    }
  } else {
    lo = ((const f32x4*)src)[0];
    hi = ((const f32x4*)src)[1];
  }
}

// Merge plan of one (request b, head h): which workers hold partials of b and
// the normalised merge weights, one candidate partial per lane (64 per chunk).
struct MergePlan {
  int64_t p_first, W, P;
  int32_t np, nchunks;
  float mref, inv, tot;
  float lc[4];           // this lane's lse in chunks 0..3 (loaded once, together)
  const float* lse_col;  // slot s: lse_col[s * H]
  int H;
  bool some_empty;

  __device__ __forceinline__ void init(const CombineArgs& a, int32_t b, int h) {
    // units of the split space (each request: its lead, then its tiles)
    init(a, b, h, spans_below(a.seq_lens, a.batch, a.topk), spans_below(a.seq_lens, b, a.topk));
  }
  // the same, given W and the units below request b
  __device__ __forceinline__ void init(const CombineArgs& a, int32_t b, int h, int64_t W_, int64_t below) {
    const int32_t nt_b = a.topk > 0 ? tiles_of(a.topk) : tiles_dense(a.seq_lens[b]);
    int64_t pf, pl;
    slot_range(a, W_, below, nt_b, &pf, &pl);
    init_range(a, b, h, W_, pf, (int32_t)(pl - pf + 1));
  }
  // Workers [*pf, *pl] hold the partials of a request with nt_b tiles and
  // `below` units below it (an empty range, *pl = *pf - 1, for no tiles).
  __device__ __forceinline__ static void slot_range(const CombineArgs& a, int64_t W_, int64_t below, int32_t nt_b,
                                                    int64_t* pf, int64_t* pl) {
    const int64_t start = below + lead_of(a.topk);  // first tile of the request
    *pf = 0;
    *pl = -1;
    if (nt_b > 0) {
      *pf = worker_of(start, W_, a.num_workers, a.topk);
      *pl = worker_of(start + nt_b - 1, W_, a.num_workers, a.topk);
    }
  }
  // the same, given the first candidate worker and the candidate count
  __device__ __forceinline__ void init_range(const CombineArgs& a, int32_t b, int h, int64_t W_, int64_t pf,
                                             int32_t n) {
    W = W_;
    P = a.num_workers;
    H = a.H;
    p_first = pf;
    np = n;  // candidate partials (some workers may be empty)
    nchunks = (np + 63) / 64;
    lse_col = a.part_lse + (int64_t)b * a.H + h;
    // Workers are empty only when there are fewer units than workers; then
    // p * W < P * P and the test needs no 64-bit division.
    some_empty = W < P;
    // the first 256 candidates' lse in one burst of loads, kept in registers
#pragma unroll
    for (int c = 0; c < 4; ++c) lc[c] = c < nchunks ? lane_lse(c) : -INFINITY;
    float mx = fmaxf(fmaxf(lc[0], lc[1]), fmaxf(lc[2], lc[3]));
    for (int32_t c = 4; c < nchunks; ++c) mx = fmaxf(mx, lane_lse(c));
    mx = wave_max(mx);
    mref = (mx == -INFINITY) ? 0.f : mx;
    float t = 0.f;
    for (int32_t c = 0; c < nchunks; ++c) {
      const float l = chunk_lse(c);
      t += (l == -INFINITY) ? 0.f : expf(l - mref);
    }
    tot = wave_sum(t);
    inv = tot > 0.f ? 1.0f / tot : 0.f;
  }
  // lse of chunk c for this lane: from registers for the first four chunks
  __device__ __forceinline__ float chunk_lse(int32_t c) const {
    if (c < 4) return c == 0 ? lc[0] : c == 1 ? lc[1] : c == 2 ? lc[2] : lc[3];
    return lane_lse(c);
  }
  // lse of partial p_first + 64c + lane; an empty worker wrote nothing and
  // counts as lse = -inf
  __device__ __forceinline__ float lane_lse(int32_t c) const {
    const int64_t p = p_first + 64 * c + __lane_id();
    if (p >= p_first + np) return -INFINITY;
    if (some_empty) {
      const uint32_t pw = (uint32_t)p * (uint32_t)W, p32 = (uint32_t)P;
      if (pw / p32 == (pw + (uint32_t)W) / p32) return -INFINITY;
    }
    return lse_col[p * H];
  }
  __device__ __forceinline__ float lse() const { return tot > 0.f ? mref + logf(tot) : -INFINITY; }
};

// Weighted sum over the partials of columns d0 .. d0 + 7 (VEC) or column d0
// of row0 + p * row_stride.  Every lane must take part (the weights are read
// from other lanes with readlane).
// Only candidate partials j_lo <= j < j_hi (indices from p_first) are summed;
// the weights stay normalised over all of them, so sums over disjoint ranges
// add up to the merge.
template <typename PT, bool VEC>
__device__ __forceinline__ void merge_cols(const MergePlan& m, const PT* row0, int64_t row_stride, int d0,
                                           f32x4& acc0, f32x4& acc1, float& acc, int32_t j_lo = 0,
                                           int32_t j_hi = 0x7fffffff) {
  acc0 = f32x4{0.f, 0.f, 0.f, 0.f};
  acc1 = acc0;
  acc = 0.f;
  if (j_hi > m.np) j_hi = m.np;
  for (int32_t c = j_lo >> 6; 64 * c < j_hi; ++c) {
    const float l = m.chunk_lse(c);
    const float wl = (l == -INFINITY) ? 0.f : expf(l - m.mref) * m.inv;  // lane's weight
    const int32_t n = j_hi - 64 * c < 64 ? j_hi - 64 * c : 64;
    for (int32_t j = j_lo - 64 * c > 0 ? j_lo - 64 * c : 0; j < n; j += kUnroll) {
      // issue every load of the group first; slots past the end are
      // clamped to a valid slot and get weight 0 (selected away, so
      // whatever an empty worker's slot holds never reaches the sum)
      f32x4 v0[kUnroll], v1[kUnroll];
      float vs[kUnroll], wg[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int32_t jj = j + u < n ? j + u : n - 1;
        wg[u] = j + u < n ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), jj)) : 0.f;
        const int64_t p = m.p_first + 64 * c + jj;
        const PT* src = row0 + p * row_stride + d0;
        if (VEC) load8(src, v0[u], v1[u]);
        else vs[u] = (float)src[0];
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const float w = wg[u];
        if (VEC) {
          acc0 += w == 0.f ? f32x4{0.f, 0.f, 0.f, 0.f} : w * v0[u];
          acc1 += w == 0.f ? f32x4{0.f, 0.f, 0.f, 0.f} : w * v1[u];
        } else {
          acc += w == 0.f ? 0.f : w * vs[u];
        }
      }
    }
  }
}

// PT: partial element type (__bf16 or float); VEC: 8 columns per lane.
// SPLIT: one (request, head) per work-group, its partials split into 4
// contiguous ranges, one per wave, whose float32 sums are added in LDS (for
// small batches, where one wave per (request, head) would leave most of the
// chip idle and walk hundreds of partials serially).  Otherwise each wave
// owns one head.
template <typename PT, bool VEC, bool SPLIT>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  __shared__ float red[SPLIT ? kWaves * 512 : 1];
  const int32_t b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int h = SPLIT ? (int)blockIdx.x : (int)blockIdx.x * kWaves + wv;
  if (!SPLIT && h >= a.H) return;
  MergePlan m;
  m.init(a, b, h);
  const int64_t dst = ((int64_t)b * a.H + h) * a.D_C;
  const int64_t row_stride = (int64_t)a.H * a.D_C;  // elements between slots
  // worker p's row (slot p + b): row0 + p * row_stride
  const PT* row0 = (const PT*)a.part_o + ((int64_t)b * a.H + h) * a.D_C;
  const int32_t j_lo = SPLIT ? (int32_t)((int64_t)m.np * wv / kWaves) : 0;
  const int32_t j_hi = SPLIT ? (int32_t)((int64_t)m.np * (wv + 1) / kWaves) : 0x7fffffff;

  // lanes past the row end load a valid column and skip the store
  for (int dbase = 0; dbase < a.D_C; dbase += VEC ? 512 : 64) {
    const int dl = dbase + (VEC ? lane * 8 : lane);
    const bool act = dl < a.D_C;
    const int d0 = act ? dl : 0;
    f32x4 acc0, acc1;
    float acc;
    merge_cols<PT, VEC>(m, row0, row_stride, d0, acc0, acc1, acc, j_lo, j_hi);
    if (SPLIT) {
      // add the 4 waves' sums; wave 0 stores
      if (VEC) {
        *(f32x4*)(red + wv * 512 + 8 * lane) = acc0;
        *(f32x4*)(red + wv * 512 + 8 * lane + 4) = acc1;
      } else {
        red[wv * 512 + lane] = acc;
      }
      __syncthreads();
      if (wv == 0) {
        for (int g = 1; g < kWaves; ++g) {
          if (VEC) {
            acc0 += *(const f32x4*)(red + g * 512 + 8 * lane);
            acc1 += *(const f32x4*)(red + g * 512 + 8 * lane + 4);
          } else {
            acc += red[g * 512 + lane];
          }
        }
      }
      __syncthreads();  // red is reused by the next column block
      if (wv != 0) continue;
    }
    if (!act) continue;
    if (VEC) {
      if (a.out_bf16) {
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = (__bf16)acc0[e];
          o[4 + e] = (__bf16)acc1[e];
        }
        *(bf16x8*)((__bf16*)a.o_lat + dst + d0) = o;
      } else {
        f32x4* o = (f32x4*)((float*)a.o_lat + dst + d0);
        o[0] = acc0;
        o[1] = acc1;
      }
    } else {
      if (a.out_bf16) ((__bf16*)a.o_lat)[dst + d0] = (__bf16)acc;
      else ((float*)a.o_lat)[dst + d0] = acc;
    }
  }
  if (a.lse_out != nullptr && lane == 0 && (!SPLIT || wv == 0)) a.lse_out[(int64_t)b * a.H + h] = m.lse();
}

// merge_cols for BF16 rows of 512 columns, each lane 8 of them, for a plan
// whose request and head are the same in every lane: the row addresses are
// scalar, the loads of a group take 4 registers each until they are summed,
// and the sum runs in the same order as merge_cols, so the result is the same.
__device__ __forceinline__ void merge_rows_bf16(const MergePlan& m, const char* row0, int64_t row_bytes,
                                                f32x4& acc0, f32x4& acc1, int32_t j_lo, int32_t j_hi) {
  acc0 = f32x4{0.f, 0.f, 0.f, 0.f};
  acc1 = acc0;
  if (j_hi > m.np) j_hi = m.np;
  const uint32_t lane_off = 16u * __lane_id();
  for (int32_t c = j_lo >> 6; 64 * c < j_hi; ++c) {
    const float l = m.chunk_lse(c);
    const float wl = (l == -INFINITY) ? 0.f : expf(l - m.mref) * m.inv;  // lane's weight
    const int32_t n = j_hi - 64 * c < 64 ? j_hi - 64 * c : 64;
    for (int32_t j = j_lo - 64 * c > 0 ? j_lo - 64 * c : 0; j < n; j += kUnroll) {
      bf16x8 raw[kUnroll];
      float wg[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int32_t jj = j + u < n ? j + u : n - 1;
        wg[u] = j + u < n ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), jj)) : 0.f;
        const char* row = row0 + (m.p_first + 64 * c + jj) * row_bytes;
        raw[u] = *(const bf16x8*)(row + lane_off);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const float w = wg[u];
        f32x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = (float)raw[u][e];
          hi[e] = (float)raw[u][4 + e];
        }
        acc0 += w == 0.f ? f32x4{0.f, 0.f, 0.f, 0.f} : w * lo;
        acc1 += w == 0.f ? f32x4{0.f, 0.f, 0.f, 0.f} : w * hi;
      }
    }
  }
}

// ---- merge and value up-projection in one launch (V2 dims, BF16) ----
// Work-group (head h, 32 requests), 16 waves: each wave merges two requests'
// partials of head h into BF16 rows in LDS (the same arithmetic as
// combine_kernel, rounded to BF16 as o_lat would be).  With fewer than 16
// requests in the group, the 16 / n waves of a request split its partials
// into contiguous ranges and their float32 sums are added in LDS, so a lone
// long request (hundreds of partials) is merged by all 16 waves.  Each wave
// loads its slice of W_UV[h] (32 rows, a quarter of K) before merging, so
// those reads overlap the merge; then every wave multiplies its slice by the
// merged rows on MFMA 32x32x16, the four K quarters meet in LDS, and waves
// 0..3 store out^T[m][b] = sum_k W_UV[h][m][k] o[b][k] for 32 rows m each
// ("DeepSeek's KV Cache", Figure 6, form (2)).  The merged latent never goes
// to HBM.  16 waves of at most 128 registers (4 per SIMD) keep twice as many
// requests' loads in flight as 8 waves of 169.
constexpr int kCuThreads = 1024;
constexpr int kCuWaves = kCuThreads / 64;
constexpr int kCuReq = 32;                // MFMA N: requests per work-group at most
// requests per work-group: 16 up to 32 requests, so that 32 requests still
// make two work-groups per head and fill the chip (the MFMA columns of the
// missing requests are zero)
__host__ __device__ constexpr int cu_group(int batch) { return batch <= 32 ? 16 : kCuReq; }
constexpr int kCuRow = kLatent * 2 + 16;  // LDS row pitch in bytes (padded against bank conflicts)
constexpr int kDv = 128;

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;

__global__ __launch_bounds__(kCuThreads) void combine_up_kernel(CombineUpArgs u) {
  __shared__ __attribute__((aligned(16))) char olds[kCuReq * kCuRow];
  // per-wave float32 sums: the merge of small groups, then the up-projection's K quarters
  __shared__ __attribute__((aligned(16))) float red[kCuWaves * 1024];
  __shared__ int64_t below_s[kCuReq + 1];  // units below each request of the group; [kCuReq] = total
  // first candidate worker and candidate count of each request of the group
  __shared__ int32_t pfirst_s[kCuReq], np_s[kCuReq];
  __shared__ int32_t tiles_s[kCuReq];  // tiles of each request of the group
  const CombineArgs& a = u.c;
  const int h = blockIdx.x;
  const int grp = cu_group(a.batch);
  const int32_t b0 = blockIdx.y * grp;
  const int32_t nb = a.batch - b0 < grp ? a.batch - b0 : grp;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row_bytes = (int64_t)kHeads * kLatent * 2;

  // This wave's share of the up-projection: rows 32 (wv % 4) .. +31 of
  // W_UV[h], latent columns 128 (wv / 4) .. +127.  Loaded first, so the
  // weight reads overlap the merge.
  constexpr int kKB = kLatent / 16 / (kCuWaves / 4);  // K-blocks per wave
  const int rb = wv & 3, kq = wv >> 2;
  bf16x8 wreg[kKB];
  {
    const __bf16* wp = (const __bf16*)u.w_uv + ((int64_t)h * kDv + 32 * rb + (lane & 31)) * kLatent +
                       16 * kKB * kq + 8 * (lane >> 5);
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) wreg[kb] = *(const bf16x8*)(wp + 16 * kb);
  }

  if (wv == 0) {
    // exclusive prefix of the request spans, once for the whole group
    int64_t off = 0;
    for (int32_t base = 0; base < a.batch; base += 64) {
      const int32_t r = base + lane;
      const int32_t nt = r < a.batch ? (a.topk > 0 ? tiles_of(a.topk) : tiles_dense(a.seq_lens[r])) : 0;
      const int64_t sp = span_of(nt, a.topk);
      if (r >= b0 && r < b0 + kCuReq) tiles_s[r - b0] = nt;
      int64_t incl = sp;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int64_t up = __shfl_up(incl, d);
        if (lane >= d) incl += up;
      }
      if (r >= b0 && r < b0 + kCuReq) below_s[r - b0] = off + incl - sp;
      off += __shfl(incl, 63);
    }
    if (lane == 0) below_s[kCuReq] = off;
    // each request's slot range, one request per lane, once for all waves
    if (lane < kCuReq && b0 + lane < a.batch) {
      int64_t pf, pl;
      MergePlan::slot_range(a, off, below_s[lane], tiles_s[lane], &pf, &pl);
      pfirst_s[lane] = (int32_t)pf;
      np_s[lane] = (int32_t)(pl - pf + 1);
    }
  }
  __syncthreads();

  const int G = nb >= kCuWaves ? 1 : kCuWaves / nb;  // waves per request
  if (G > 1) {
    // wave wv: request wv / G, partial range part wv % G of G
    const int bl = wv / G, g = wv % G;
    f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
    if (bl < nb) {  // wave-uniform
      const int32_t b = b0 + bl;
      MergePlan m;
      m.init_range(a, b, h, uniform_i64(below_s[kCuReq]), __builtin_amdgcn_readfirstlane(pfirst_s[bl]),
                   __builtin_amdgcn_readfirstlane(np_s[bl]));
      const char* row0 = (const char*)a.part_o + ((int64_t)b * kHeads + h) * kLatent * 2;
      const int32_t j_lo = (int32_t)((int64_t)m.np * g / G), j_hi = (int32_t)((int64_t)m.np * (g + 1) / G);
      merge_rows_bf16(m, row0, row_bytes, acc0, acc1, j_lo, j_hi);
      if (g == 0 && a.lse_out != nullptr && lane == 0) a.lse_out[(int64_t)b * kHeads + h] = m.lse();
    }
    *(f32x4*)(red + wv * kLatent + 8 * lane) = acc0;
    *(f32x4*)(red + wv * kLatent + 8 * lane + 4) = acc1;
    __syncthreads();
    for (int r = wv; r < kCuReq; r += kCuWaves) {
      f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
      if (r < nb) {
        for (int gg = 0; gg < G; ++gg) {
          s0 += *(const f32x4*)(red + (r * G + gg) * kLatent + 8 * lane);
          s1 += *(const f32x4*)(red + (r * G + gg) * kLatent + 8 * lane + 4);
        }
      }
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = (__bf16)s0[e];
        o[4 + e] = (__bf16)s1[e];
      }
      *(bf16x8*)(olds + r * kCuRow + 16 * lane) = o;
    }
  }
  for (int bl = wv; G == 1 && bl < kCuReq; bl += kCuWaves) {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)0.f;
    if (bl < nb) {  // wave-uniform
      const int32_t b = b0 + bl;
      MergePlan m;
      m.init_range(a, b, h, uniform_i64(below_s[kCuReq]), __builtin_amdgcn_readfirstlane(pfirst_s[bl]),
                   __builtin_amdgcn_readfirstlane(np_s[bl]));
      const char* row0 = (const char*)a.part_o + ((int64_t)b * kHeads + h) * kLatent * 2;
      f32x4 acc0, acc1;
      merge_rows_bf16(m, row0, row_bytes, acc0, acc1, 0, 0x7fffffff);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = (__bf16)acc0[e];
        o[4 + e] = (__bf16)acc1[e];
      }
      if (a.lse_out != nullptr && lane == 0) a.lse_out[(int64_t)b * kHeads + h] = m.lse();
    }
    *(bf16x8*)(olds + bl * kCuRow + 16 * lane) = o;
  }
  __syncthreads();

  // A: W_UV[h] rows 32 rb + (lane % 32), 8 columns per lane per K-block;
  // B: merged row (lane % 32), the same 8 columns; this wave's K quarter
  const char* op = olds + (lane & 31) * kCuRow + 16 * (lane >> 5) + 32 * kKB * kq;
  f32x16 acc = f32x16{};
#pragma unroll
  for (int kb = 0; kb < kKB; ++kb) {
    const bf16x8 bv = *(const bf16x8*)(op + 32 * kb);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wreg[kb], bv, acc, 0, 0, 0);
  }
  // the four K quarters of each row block meet in LDS
#pragma unroll
  for (int r = 0; r < 16; ++r) red[wv * 1024 + r * 64 + lane] = acc[r];
  __syncthreads();
  if (wv < kDv / 32) {
#pragma unroll
    for (int q = 1; q < kCuWaves / 4; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] += red[(rb + 4 * q) * 1024 + r * 64 + lane];
    // lane holds rows m = 32 rb + 8 g + 4 (lane / 32) + e of request lane % 32:
    // staged in LDS as one 256-byte row of outputs per request (over olds,
    // whose reads all finished before the last barrier), 16-byte chunks
    // XOR-swizzled by the request
    const int bl = lane & 31;
    char* row = olds + bl * (kDv * 2);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[4 * g + e];
      *(bf16x4*)(row + 16 * ((4 * rb + g) ^ (bl & 15)) + 8 * (lane >> 5)) = v;
    }
  }
  __syncthreads();
  // each request's 256 output bytes leave as 16 lanes x 16 bytes
  if (threadIdx.x < kCuReq * 16) {
    const int r = threadIdx.x >> 4, ch = threadIdx.x & 15;
    if (r < nb)
      *(i32x4*)((char*)u.out + ((int64_t)(b0 + r) * kHeads + h) * kDv * 2 + 16 * ch) =
          *(const i32x4*)(olds + r * (kDv * 2) + 16 * (ch ^ (r & 15)));
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  // few (request, head) rows: split each one's partials over a work-group
  const bool split = (int64_t)a.batch * a.H < 4096;
  const dim3 grid(split ? a.H : (a.H + kWaves - 1) / kWaves, a.batch);
#define MLA_COMBINE(PT, VEC)                                                                      \
  do {                                                                                            \
    if (split) hipLaunchKernelGGL((combine_kernel<PT, VEC, true>), grid, dim3(kThreads), 0, s, a); \
    else hipLaunchKernelGGL((combine_kernel<PT, VEC, false>), grid, dim3(kThreads), 0, s, a);      \
  } while (0)
  if (a.part_bf16) {
    if (a.D_C % 8 == 0) MLA_COMBINE(__bf16, true);
    else MLA_COMBINE(__bf16, false);
  } else {
    if (a.D_C % 8 == 0) MLA_COMBINE(float, true);
    else MLA_COMBINE(float, false);
  }
#undef MLA_COMBINE
  return hipGetLastError();
}

hipError_t launch_combine_up(const CombineUpArgs& u, hipStream_t s) {
  // V2 dims, BF16 partials and output (checked by the caller)
  const int grp = cu_group(u.c.batch);
  const dim3 grid(kHeads, (u.c.batch + grp - 1) / grp);
  hipLaunchKernelGGL(combine_up_kernel, grid, dim3(kCuThreads), 0, s, u);
  return hipGetLastError();
}

}  // namespace mla
