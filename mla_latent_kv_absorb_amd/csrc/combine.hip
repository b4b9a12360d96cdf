// Log-sum-exp merge of split partials.
//
// A partial over a disjoint set of positions S_s holds the softmax-normalised
// weighted latent o_s and lse_s = log sum_{j in S_s} exp(score_j).  Softmax
// over the union of the sets is then
//   o = sum_s exp(lse_s - LSE) o_s,   LSE = log sum_s exp(lse_s),
// an exact identity.  Which slots hold request b's partials follows from the
// same tile partition the attention kernel used (worker p writes slot p + b).
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kHeadsPerBlock = 8;

__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  const int32_t b = blockIdx.y;
  const int tid = threadIdx.x;
  const int h = blockIdx.x * kHeadsPerBlock + tid / 32;
  const int sub = tid & 31;

  // tile range of request b in the concatenated tile space
  int64_t W = 0, start = 0;
  int32_t nt_b = 0;
  for (int32_t r = 0; r < a.batch; ++r) {
    int32_t nt;
    if (a.topk > 0) nt = tiles_of(a.topk);
    else {
      const int32_t T = a.seq_lens[r];
      nt = T > 0 ? tiles_of(T) : 0;
    }
    if (r == b) { start = W; nt_b = nt; }
    W += nt;
  }
  if (h >= a.H) return;
  const int64_t P = a.num_workers;
  int64_t p_first = 0, p_last = -1;
  if (nt_b > 0) {
    p_first = worker_of(start, W, P);
    p_last = worker_of(start + nt_b - 1, W, P);
  }
  // weights
  float mx = -INFINITY;
  for (int64_t p = p_first; p <= p_last; ++p) {
    if (worker_lo(p, W, P) == worker_lo(p + 1, W, P)) continue;  // empty worker
    mx = fmaxf(mx, a.part_lse[(p + b) * a.H + h]);
  }
  const float mref = (mx == -INFINITY) ? 0.f : mx;
  float tot = 0.f;
  for (int64_t p = p_first; p <= p_last; ++p) {
    if (worker_lo(p, W, P) == worker_lo(p + 1, W, P)) continue;
    tot += expf(a.part_lse[(p + b) * a.H + h] - mref);
  }
  const float inv = tot > 0.f ? 1.0f / tot : 0.f;
  for (int d0 = sub * 4; d0 < a.D_C; d0 += 128) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int64_t p = p_first; p <= p_last; ++p) {
      if (worker_lo(p, W, P) == worker_lo(p + 1, W, P)) continue;
      const int64_t slot = p + b;
      const float wgt = expf(a.part_lse[slot * a.H + h] - mref) * inv;
      const float* src = a.part_o + (slot * a.H + h) * a.D_C + d0;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (d0 + e < a.D_C) acc[e] = fmaf(wgt, src[e], acc[e]);
    }
    const int64_t dst = ((int64_t)b * a.H + h) * a.D_C + d0;
    if (a.out_bf16) {
      __bf16* o = (__bf16*)a.o_lat + dst;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (d0 + e < a.D_C) o[e] = (__bf16)acc[e];
    } else {
      float* o = (float*)a.o_lat + dst;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (d0 + e < a.D_C) o[e] = acc[e];
    }
  }
  if (a.lse_out != nullptr && sub == 0)
    a.lse_out[(int64_t)b * a.H + h] = tot > 0.f ? mref + logf(tot) : -INFINITY;
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  const dim3 grid((a.H + kHeadsPerBlock - 1) / kHeadsPerBlock, a.batch);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
