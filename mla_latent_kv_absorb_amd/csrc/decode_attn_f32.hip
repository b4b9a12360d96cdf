// Generic float32 latent attention for small dimensions.
//
// Same computation and the same split partition as the MFMA kernel (scores
// against the cached latent plus the rotary part, online softmax, weighted
// latent), written with plain fp32 arithmetic and everything staged in LDS, so
// any head count / latent / rope width that fits in LDS works.  It serves the
// float32 cache configuration, where exact fp32 arithmetic is wanted.
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;

template <bool TOPK, bool DIRECT>
__global__ __launch_bounds__(kThreads) void decode_f32_kernel(DecodeArgs a) {
  extern __shared__ float sm[];
  const int H = a.H, DC = a.D_C, DR = a.D_R;
  const F32Layout lay(H, DC, DR);
  float* sq = sm + lay.q;
  float* sqr = sm + lay.qr;
  float* sc = sm + lay.c;
  float* sr = sm + lay.r;
  float* ss = sm + lay.s;
  float* so = sm + lay.o;
  float* smx = sm + lay.m;
  float* sl = sm + lay.l;
  float* sal = sm + lay.al;
  int* sval = (int*)(sm + lay.valid);
  const int tid = threadIdx.x;

  auto ntiles = [&](int32_t b) -> int32_t {
    if (TOPK) return tiles_of(a.topk);
    const int32_t T = a.seq_lens[b];
    return T > 0 ? tiles_of(T) : 0;
  };

  int32_t cb, ct = 0;
  int64_t cv, n;
  const int64_t worker = blockIdx.x;
  const int32_t lead = lead_of(TOPK ? a.topk : 0);
  if (DIRECT) {
    cb = blockIdx.x;
    cv = lead;  // straight to tile 0
    n = ntiles(cb);
  } else {
    // n units of the split space from offset cv of request cb's span (the
    // request's lead, then its tiles)
    int64_t W = 0;
    for (int32_t b = 0; b < a.batch; ++b) W += span_of(ntiles(b), TOPK ? a.topk : 0);
    const int64_t g0 = worker_lo(worker, W, a.num_workers, TOPK ? a.topk : 0);
    const int64_t g1 = worker_lo(worker + 1, W, a.num_workers, TOPK ? a.topk : 0);
    n = g1 - g0;
    if (n <= 0) return;
    int64_t acc = 0;
    int32_t b = 0;
    while (acc + span_of(ntiles(b), TOPK ? a.topk : 0) <= g0) {
      acc += span_of(ntiles(b), TOPK ? a.topk : 0);
      ++b;
    }
    cb = b;
    cv = g0 - acc;
  }
  if (n == 0) {
    if (DIRECT) {
      float* o = (float*)a.o_lat + (int64_t)cb * H * DC;
      for (int e = tid; e < H * DC; e += kThreads) o[e] = 0.f;
      if (a.lse_out != nullptr)
        for (int h = tid; h < H; h += kThreads) a.lse_out[(int64_t)cb * H + h] = -INFINITY;
    }
    return;
  }

  const float* qlat = (const float*)a.q_lat;
  const float* qrope = (const float*)a.q_rope;
  int64_t i = 0;
  while (i < n) {
    if (cb >= a.batch) break;  // unreachable when the tile accounting is consistent
    if (cv < lead) {  // the lead of request cb carries no work
      const int64_t skip = lead - cv < n - i ? lead - cv : n - i;
      i += skip;
      cv += skip;
      if (i >= n) break;
    }
    ct = (int32_t)(cv - lead);
    const int64_t left = ntiles(cb) - ct;
    const int64_t seg = left < n - i ? left : n - i;
    if (seg <= 0) break;
    const int32_t T = a.seq_lens[cb];
    __syncthreads();
    for (int e = tid; e < H * DC; e += kThreads) {
      sq[e] = qlat[(int64_t)cb * H * DC + e];
      so[e] = 0.f;
    }
    for (int e = tid; e < H * DR; e += kThreads) sqr[e] = qrope[(int64_t)cb * H * DR + e];
    for (int h = tid; h < H; h += kThreads) {
      smx[h] = -INFINITY;
      sl[h] = 0.f;
    }
    for (int64_t j = 0; j < seg; ++j, ++i, ++ct) {
      __syncthreads();
      // rows of this tile
      for (int r = tid; r < kTile; r += kThreads) {
        const int lp = ct * kTile + r;
        int32_t pos;
        if (TOPK) pos = lp < a.topk ? a.topk_idx[(int64_t)cb * a.topk + lp] : -1;
        else pos = lp < T ? lp : -1;
        bool v = pos >= 0 && pos < T && (pos >> 6) < a.bt_stride;
        int32_t page = v ? a.block_table[(int64_t)cb * a.bt_stride + (pos >> 6)] : -1;
        v = v && page >= 0 && page < a.num_pages;
        sval[r] = v ? (int)(((int64_t)page << 6) | (pos & 63)) : -1;
      }
      __syncthreads();
      for (int e = tid; e < kTile * DC; e += kThreads) {
        const int r = e / DC, d = e - r * DC;
        const int code = sval[r];
        float x = 0.f;
        if (code >= 0) {
          const uint8_t* pg = a.pool + (int64_t)(code >> 6) * a.page_bytes;
          x = ((const float*)pg)[(code & 63) * DC + d];
        }
        sc[e] = x;
      }
      for (int e = tid; e < kTile * DR; e += kThreads) {
        const int r = e / DR, d = e - r * DR;
        const int code = sval[r];
        float x = 0.f;
        if (code >= 0) {
          const uint8_t* pg = a.pool + (int64_t)(code >> 6) * a.page_bytes + a.rope_off;
          x = ((const float*)pg)[(code & 63) * DR + d];
        }
        sr[e] = x;
      }
      __syncthreads();
      // scores
      for (int e = tid; e < H * kTile; e += kThreads) {
        const int h = e / kTile, r = e - h * kTile;
        float s = -INFINITY;
        if (sval[r] >= 0) {
          float acc = 0.f;
          for (int d = 0; d < DC; ++d) acc = fmaf(sq[h * DC + d], sc[r * DC + d], acc);
          for (int d = 0; d < DR; ++d) acc = fmaf(sqr[h * DR + d], sr[r * DR + d], acc);
          s = acc * a.scale;
        }
        ss[e] = s;
      }
      __syncthreads();
      // online softmax per head
      for (int h = tid; h < H; h += kThreads) {
        float mt = -INFINITY;
        for (int r = 0; r < kTile; ++r) mt = fmaxf(mt, ss[h * kTile + r]);
        const float mo = smx[h];
        const float mn = fmaxf(mo, mt);
        const float alpha = (mo == -INFINITY) ? 0.f : expf(mo - mn);
        float sum = 0.f;
        for (int r = 0; r < kTile; ++r) {
          const float s = ss[h * kTile + r];
          const float p = (s == -INFINITY) ? 0.f : expf(s - mn);
          ss[h * kTile + r] = p;
          sum += p;
        }
        sl[h] = sl[h] * alpha + sum;
        smx[h] = mn;
        sal[h] = alpha;
      }
      __syncthreads();
      // weighted latent
      for (int e = tid; e < H * DC; e += kThreads) {
        const int h = e / DC, d = e - h * DC;
        float acc = so[e] * sal[h];
        for (int r = 0; r < kTile; ++r) acc = fmaf(ss[h * kTile + r], sc[r * DC + d], acc);
        so[e] = acc;
      }
    }
    __syncthreads();
    // write
    const int32_t b = cb;
    for (int e = tid; e < H * DC; e += kThreads) {
      const int h = e / DC;
      const float l = sl[h];
      const float v = l > 0.f ? so[e] / l : 0.f;
      if (DIRECT) ((float*)a.o_lat)[(int64_t)b * H * DC + e] = v;
      else ((float*)a.part_o)[((worker + b) * H) * DC + e] = v;
    }
    for (int h = tid; h < H; h += kThreads) {
      const float l = sl[h];
      const float lse = l > 0.f ? smx[h] + logf(l) : -INFINITY;
      if (DIRECT) { if (a.lse_out != nullptr) a.lse_out[(int64_t)b * H + h] = lse; }
      else a.part_lse[(worker + b) * H + h] = lse;
    }
    ++cb;
    cv = 0;
    while (cb < a.batch && ntiles(cb) == 0) ++cb;
  }
}

}  // namespace

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s) {
  const bool topk = a.topk_idx != nullptr;
  const bool direct = a.num_workers == 0;
  const dim3 grid(direct ? a.batch : a.num_workers);
  const size_t lds = decode_f32_lds_bytes(a.H, a.D_C, a.D_R);
  if (topk) {
    if (direct) hipLaunchKernelGGL((decode_f32_kernel<true, true>), grid, dim3(kThreads), lds, s, a);
    else hipLaunchKernelGGL((decode_f32_kernel<true, false>), grid, dim3(kThreads), lds, s, a);
  } else {
    if (direct) hipLaunchKernelGGL((decode_f32_kernel<false, true>), grid, dim3(kThreads), lds, s, a);
    else hipLaunchKernelGGL((decode_f32_kernel<false, false>), grid, dim3(kThreads), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace mla
