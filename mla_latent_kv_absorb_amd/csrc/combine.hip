// Log-sum-exp merge of split partials.
//
// A partial over a disjoint set of positions S_s holds the softmax-normalised
// weighted latent o_s and lse_s = log sum_{j in S_s} exp(score_j).  Softmax
// over the union of the sets is then
//   o = sum_s exp(lse_s - LSE) o_s,   LSE = log sum_s exp(lse_s),
// an exact identity.  Which slots hold request b's partials follows from the
// same tile partition the attention kernel used (worker p writes slot p + b).
//
// One wave per (request, head): each lane owns 8 consecutive latent columns
// (one 16-byte load per partial for BF16 partials, two for FP32), so a head
// row of 512 values is one coalesced read per partial, and the loads of 8
// partials are in flight together.  The merge weights are computed one
// partial per lane and read back with readlane.
#include "tile_space.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 8;  // partials whose loads are in flight together

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
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

// PT: partial element type (__bf16 or float); VEC: 8 columns per lane.
template <typename PT, bool VEC>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  const int32_t b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.x * kWaves + (threadIdx.x >> 6);

  // units of the split space (each request: its lead, then its tiles)
  const int64_t W = spans_below(a.seq_lens, a.batch, a.topk);
  const int64_t start = spans_below(a.seq_lens, b, a.topk) + kLeadTiles;  // first tile of request b
  const int32_t nt_b = a.topk > 0 ? tiles_of(a.topk) : tiles_dense(a.seq_lens[b]);
  if (h >= a.H) return;
  const int64_t P = a.num_workers;
  int64_t p_first = 0, p_last = -1;
  if (nt_b > 0) {
    p_first = worker_of(start, W, P);
    p_last = worker_of(start + nt_b - 1, W, P);
  }
  const int32_t np = (int32_t)(p_last - p_first + 1);  // candidate partials (some workers may be empty)
  const float* lse_col = a.part_lse + (int64_t)b * a.H + h;  // slot s: lse_col[s * H]

  // Merge weights.  Lane i looks after partial p_first + 64c + i of chunk c;
  // an empty worker wrote nothing and counts as lse = -inf.
  // Workers are empty only when there are fewer tiles than workers; then
  // p * W < P * P and the test needs no 64-bit division.
  const bool some_empty = W < P;
  auto lane_lse = [&](int32_t c) -> float {
    const int64_t p = p_first + 64 * c + lane;
    if (p > p_last) return -INFINITY;
    if (some_empty) {
      const uint32_t pw = (uint32_t)p * (uint32_t)W, p32 = (uint32_t)P;
      if (pw / p32 == (pw + (uint32_t)W) / p32) return -INFINITY;
    }
    return lse_col[p * a.H];
  };
  const int32_t nchunks = (np + 63) / 64;
  float mx = -INFINITY;
  for (int32_t c = 0; c < nchunks; ++c) mx = fmaxf(mx, lane_lse(c));
  mx = wave_max(mx);
  const float mref = (mx == -INFINITY) ? 0.f : mx;
  float tot = 0.f;
  for (int32_t c = 0; c < nchunks; ++c) {
    const float l = lane_lse(c);
    tot += (l == -INFINITY) ? 0.f : expf(l - mref);
  }
  tot = wave_sum(tot);
  const float inv = tot > 0.f ? 1.0f / tot : 0.f;
  const int64_t dst = ((int64_t)b * a.H + h) * a.D_C;
  const int64_t row_stride = (int64_t)a.H * a.D_C;  // elements between slots
  const PT* row0 = (const PT*)a.part_o + ((int64_t)b * a.H + h) * a.D_C;  // worker p's row (slot p + b): row0 + p * row_stride

  // Every lane runs every iteration (the weights are read from other lanes
  // with readlane, so no lane may sit out); lanes past the row end load a
  // valid column and skip the store.
  for (int dbase = 0; dbase < a.D_C; dbase += VEC ? 512 : 64) {
    const int dl = dbase + (VEC ? lane * 8 : lane);
    const bool act = dl < a.D_C;
    const int d0 = act ? dl : 0;
    f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
    float acc = 0.f;
    for (int32_t c = 0; c < nchunks; ++c) {
      const float l = lane_lse(c);
      const float wl = (l == -INFINITY) ? 0.f : expf(l - mref) * inv;  // lane's weight
      const int32_t n = np - 64 * c < 64 ? np - 64 * c : 64;
      for (int32_t j = 0; j < n; j += kUnroll) {
        // issue every load of the group first; slots past the end are
        // clamped to a valid slot and get weight 0 (selected away, so
        // whatever an empty worker's slot holds never reaches the sum)
        f32x4 v0[kUnroll], v1[kUnroll];
        float vs[kUnroll], wg[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int32_t jj = j + u < n ? j + u : n - 1;
          wg[u] = j + u < n ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), jj)) : 0.f;
          const int64_t p = p_first + 64 * c + jj;  // its slot is p + b
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
  if (a.lse_out != nullptr && lane == 0)
    a.lse_out[(int64_t)b * a.H + h] = tot > 0.f ? mref + logf(tot) : -INFINITY;
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  const dim3 grid((a.H + kWaves - 1) / kWaves, a.batch);
  if (a.part_bf16) {
    if (a.D_C % 8 == 0) hipLaunchKernelGGL((combine_kernel<__bf16, true>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<__bf16, false>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (a.D_C % 8 == 0) hipLaunchKernelGGL((combine_kernel<float, true>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<float, false>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace mla
