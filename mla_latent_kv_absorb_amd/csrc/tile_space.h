// Device helpers over the concatenated tile space of all requests (the
// split partition of mla_internal.h).  Included by kernel translation units
// only.
#pragma once

#include "mla_internal.h"

namespace mla {

// ---- the concatenated tile space of all requests (see worker_lo) ----
// Computed by the whole wave, 64 requests per load, so the per-request
// lengths are read in parallel rather than one dependent scalar load after
// another.  Every lane must be active; results are wave-uniform.
__device__ inline int32_t tiles_dense(int32_t T) { return T > 0 ? tiles_of(T) : 0; }

// Wave-uniform copy of a value every lane holds (keeps it in scalar registers).
__device__ inline int64_t uniform_i64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ inline int64_t wave_sum_i64(int64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return uniform_i64(v);
}

// Worker index of work-group b of P.  Work-groups are dispatched round-robin
// over the 8 XCDs (work-group b runs on XCD b % 8), each with its own L2.
// Consecutive workers share requests (their queries and page-table rows), so
// they are given to work-groups of one XCD: worker (b % 8) * (P / 8) + b / 8.
__device__ inline int64_t xcd_worker(uint32_t b, uint32_t P) {
  constexpr uint32_t kXcds = 8;
  if (P % kXcds != 0) return b;
  return (int64_t)(b % kXcds) * (P / kXcds) + b / kXcds;
}

// Units of the split space (span_of) taken by requests [0, upto).
__device__ inline int64_t spans_below(const int32_t* seq_lens, int32_t upto, int32_t topk) {
  if (topk > 0) return (int64_t)upto * span_of(tiles_of(topk), topk);
  const int lane = __lane_id();
  int64_t sum = 0;
  for (int32_t base = 0; base < upto; base += 64) {
    const int32_t r = base + lane;
    sum += r < upto ? span_of(tiles_dense(seq_lens[r]), 0) : 0;
  }
  return wave_sum_i64(sum);
}

// Request whose span holds unit g of the split space (0 <= g < total) and
// the unit's offset inside that span (below the lead: the lead; else tile
// offset + lead).
__device__ inline void locate_span(const int32_t* seq_lens, int32_t batch, int32_t topk, int64_t g,
                                   int32_t* b, int32_t* t) {
  if (topk > 0) {
    const int64_t sp = span_of(tiles_of(topk), topk);
    *b = (int32_t)(g / sp);
    *t = (int32_t)(g % sp);
    return;
  }
  const int lane = __lane_id();
  int64_t off = 0;
  for (int32_t base = 0; base < batch; base += 64) {
    const int32_t r = base + lane;
    const int64_t sp = r < batch ? span_of(tiles_dense(seq_lens[r]), 0) : 0;
    int64_t incl = sp;  // inclusive scan over the lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t up = __shfl_up(incl, d);
      if (lane >= d) incl += up;
    }
    incl += off;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(incl > g);
    if (hit != 0) {
      const int l = __builtin_ctzll(hit);
      const int64_t end = __shfl(incl, l), len = __shfl(sp, l);
      *b = base + l;
      *t = __builtin_amdgcn_readfirstlane((int32_t)(g - (end - len)));
      return;
    }
    off = uniform_i64(__shfl(incl, 63));
  }
  *b = batch;  // g beyond the last span
  *t = 0;
}

// A worker's place in the split space: W (the space's units), its range
// [g0, g1), and the request b and offset t of unit g0 (as locate_span; b is
// the batch size when the range is empty at the end).  For a batch that fits
// the wave's lanes, one load of the context lengths and one scan give both W
// and the place (spans_below then locate_span would read them twice, one
// dependent round trip after the other); index lists need no load at all.
struct WorkerSpan {
  int64_t W, g0, g1;
  int32_t b, t;
};
__device__ inline WorkerSpan locate_worker(const int32_t* seq_lens, int32_t batch, int32_t topk, int64_t p,
                                           int64_t P) {
  WorkerSpan s;
  if (topk > 0) {
    const int64_t sp = span_of(tiles_of(topk), topk);
    s.W = (int64_t)batch * sp;
    s.g0 = worker_lo(p, s.W, P, topk);
    s.g1 = worker_lo(p + 1, s.W, P, topk);
    // g0 / sp without a 64-bit division
    int64_t q = (int64_t)((double)s.g0 / (double)sp);
    while (q > 0 && q * sp > s.g0) --q;
    while ((q + 1) * sp <= s.g0) ++q;
    s.b = (int32_t)q;
    s.t = (int32_t)(s.g0 - q * sp);
    return s;
  }
  if (batch > 64) {
    s.W = spans_below(seq_lens, batch, 0);
    s.g0 = worker_lo(p, s.W, P, 0);
    s.g1 = worker_lo(p + 1, s.W, P, 0);
    s.b = batch;
    s.t = 0;
    if (s.g1 > s.g0) locate_span(seq_lens, batch, 0, s.g0, &s.b, &s.t);
    return s;
  }
  const int lane = __lane_id();
  const int64_t sp = lane < batch ? span_of(tiles_dense(seq_lens[lane]), 0) : 0;
  int64_t incl = sp;  // inclusive scan over the lanes
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t up = __shfl_up(incl, d);
    if (lane >= d) incl += up;
  }
  s.W = uniform_i64(__shfl(incl, 63));
  s.g0 = worker_lo(p, s.W, P, 0);
  s.g1 = worker_lo(p + 1, s.W, P, 0);
  const uint64_t hit = __builtin_amdgcn_ballot_w64(incl > s.g0);
  s.b = batch;
  s.t = 0;
  if (hit != 0) {
    const int l = __builtin_ctzll(hit);
    const int64_t end = __shfl(incl, l), len = __shfl(sp, l);
    s.b = l;
    s.t = __builtin_amdgcn_readfirstlane((int32_t)(s.g0 - (end - len)));
  }
  return s;
}

}  // namespace mla
