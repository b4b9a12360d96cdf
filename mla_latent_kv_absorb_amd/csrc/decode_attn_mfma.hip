// Weight-absorbed MLA decode attention over a paged latent cache, gfx950.
//
// Per work-group: 4 waves, each owning 32 of the 128 heads.  For every tile
// of 32 cached positions the work-group streams the latent rows (512 wide)
// and rotary-key rows (64 wide) from HBM straight into LDS and each wave
//   * scores its heads against the tile with MFMA 32x32x16 (bf16 in, fp32
//     accumulate): S^T[pos][head] = C[pos] . q_lat[head] + k_rope[pos] .
//     q_rope[head] -- the absorbed score of "DeepSeek's KV Cache", Figure 5
//     form (2), plus the unabsorbed rotary part (section "Why the positional
//     part is kept separate");
//   * runs an online softmax per head (each lane owns one head);
//   * accumulates the weighted latent U^T[latent][head] += C^T P^T on MFMA
//     (Figure 6 form (2), first step).  The S^T accumulator registers are the
//     B operand of this product as they are; the positions inside the MFMA K
//     dimension are permuted to match, and the C^T operand comes from
//     transposing LDS reads (ds_read_b64_tr_b16).
// Each latent row is read from HBM once and serves as both key and value
// (same page, section "Looking at reads": one item counted once for both
// roles).
//
// Loads use global_load_lds_dwordx4 (HBM -> LDS without registers) through a
// 4-stage ring (5 for FP8) with explicit vmcnt waits; the rows are stored with
// an XOR swizzle of their 16-byte chunks so the MFMA operand reads are free of
// bank conflicts.  Page ids and index lists are read with scalar loads so
// they never wait behind the LDS-bound vector loads.
//
// This kernel serves BF16 caches with an index list and FP8 caches with one
// float32 scale per 128 latent channels of a position ("DeepSeek's KV Cache",
// section "Calculating V3.2's KV cache"); FP8 caches with one scale per
// position have their own kernel (decode_attn_fp8.hip).  For the group-scaled
// FP8 cache a conversion pass turns the tile into BF16 in LDS: each value
// times its group's scale is rounded once to BF16, and the scores and the
// weighted latent then run exactly as for a BF16 cache.
//
// Sparse selection ("DeepSeek's KV Cache", Figure 10): with an index list the
// tile rows are the listed positions, gathered one row per load; entries that
// are -1, out of range or on an invalid page are masked.
#include "attn_common.h"

namespace mla {
namespace {

// FP8: E4M3 latent; GS: with one scale per 128 latent channels of a position
// (4 per position) instead of one per position.
template <bool FP8, bool GS>
struct Cfg {
  static constexpr int NS = FP8 ? 5 : 4;                       // ring stages
  static constexpr int C_STAGE = FP8 ? kTile * kC8Row : kTile * kCRow;
  static constexpr int R_STAGE = kTile * kRRow;
  static constexpr int SCALES = GS ? kLatent / 128 : 1;        // scales per position
  static constexpr int SC_STAGE = FP8 ? kTile * 4 * SCALES : 0;
  static constexpr int STAGE = C_STAGE + R_STAGE + SC_STAGE;
  static constexpr int CONV_OFF = NS * STAGE;                  // BF16 copy of an FP8 tile
  static constexpr int CONV = FP8 ? kTile * kCRow : 0;
  static constexpr int LIST_OFF = CONV_OFF + CONV;             // page ids / row codes of a chunk
  static constexpr int LIST = 2048;                            // entries (int32)
  static constexpr int MASK_OFF = LIST_OFF + LIST * 4;
  // FP8: the rotary queries of the segment's request live in LDS
  // ([head][64] BF16, rows swizzled) instead of 16 registers per lane
  static constexpr bool QR_LDS = FP8;
  static constexpr int QR_OFF = MASK_OFF + 32;
  static constexpr int LDS_BYTES = QR_LDS ? QR_OFF + kHeads * kRRow : MASK_OFF + NS * 4;
  static constexpr int DMA_PER_WAVE = FP8 ? 6 : 9;             // loads per wave per tile
};

// Tiles of one request processed between two pipeline drains: bounded by the
// LDS list (2048 page ids cover 4096 dense tiles; 2048 index entries cover 64
// gathered tiles).
template <bool TOPK>
__device__ __forceinline__ constexpr int chunk_tiles() { return TOPK ? 2048 / kTile : 4000; }

template <int NS, int DPW>
__device__ __forceinline__ void wait_tiles(int64_t ahead) {
  // wait until at most `ahead` newer tiles of this wave are still in flight
  if (ahead >= NS - 2) { wait_vmcnt<DPW * (NS - 2)>(); return; }
  if constexpr (NS - 2 > 4) { if (ahead == 4) { wait_vmcnt<DPW * 4>(); return; } }
  if constexpr (NS - 2 > 3) { if (ahead == 3) { wait_vmcnt<DPW * 3>(); return; } }
  if constexpr (NS - 2 > 2) { if (ahead == 2) { wait_vmcnt<DPW * 2>(); return; } }
  if constexpr (NS - 2 > 1) { if (ahead == 1) { wait_vmcnt<DPW * 1>(); return; } }
  wait_vmcnt<0>();
}

template <bool FP8, bool GS, bool TOPK>
struct Loader {
  const DecodeArgs& a;
  uint32_t smem_base;
  int lane, w;

  __device__ __forceinline__ int32_t ntiles(int32_t b) const {
    if (TOPK) return tiles_of(a.topk);
    int32_t T = sload(a.seq_lens + b);
    return T > 0 ? tiles_of(T) : 0;
  }

  // Fill the LDS list for tiles [tc0, tc0 + len) of request b (all threads;
  // the caller synchronises).  Dense: page id of each page the tiles touch,
  // -1 when outside the table or the pool.  Gathered: per listed position the
  // row code page * 64 + slot, -1 for padding, out-of-range or invalid pages.
  __device__ __forceinline__ void fill_list(int32_t b, int32_t tc0, int32_t len, int32_t T, LDS int32_t* list,
                                            int tid) const {
    if (!TOPK) {
      const int32_t p0 = tc0 >> 1;
      const int32_t np = ((tc0 + len - 1) >> 1) - p0 + 1;
      for (int k = tid; k < np; k += 256) {
        const int32_t p = p0 + k;
        int32_t page = p < a.bt_stride ? a.block_table[(int64_t)b * a.bt_stride + p] : -1;
        list[k] = (page >= 0 && page < a.num_pages) ? page : -1;
      }
    } else {
      fill_index_codes(a, b, tc0, len, T, list, tid);
    }
  }

  // Issue this wave's share of tile t (chunk starts at tc0) into stage st.
  __device__ __forceinline__ void issue(int st, int32_t t, int32_t tc0, int32_t T, const LDS int32_t* list,
                                        char* smem) const {
    using C = Cfg<FP8, GS>;
    const uint32_t sb = smem_base + st * C::STAGE;
    const uint8_t* pool = a.pool;
    uint32_t bits = 0;
    if (!TOPK) {
      const int32_t page = __builtin_amdgcn_readfirstlane(list[(t >> 1) - (tc0 >> 1)]);
      const bool pv = page >= 0;
      const uint8_t* pg = pool + (pv ? (int64_t)page * a.page_bytes : 0);
      const int slot0 = (t & 1) * kTile + 8 * w;  // first row of this wave in the page
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int pos = t * kTile + 8 * w + k;
        if (pv && pos < T) bits |= 1u << k;
      }
      if (FP8) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          dma16_nt(pg + (int64_t)(slot0 + 2 * q) * kC8Row + 16 * lane, sb + (8 * w + 2 * q) * kC8Row);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          dma16_nt(pg + (int64_t)(slot0 + k) * kCRow + 16 * (lane ^ swz(8 * w + k)), sb + (8 * w + k) * kCRow);
      }
      const int rr = lane >> 3, rc = lane & 7;
      dma16_nt(pg + a.rope_off + (int64_t)(slot0 + rr) * kRRow + 16 * (rc ^ swz_r(8 * w + rr)),
            sb + C::C_STAGE + 8 * w * kRRow);
      if (FP8) {
        // this wave's 8 positions' scales: 32 B, or 128 B with group scales
        if (GS) {
          if (lane < 8) dma16_nt(pg + a.scale_off + (int64_t)(slot0 + lane) * 16, sb + C::C_STAGE + C::R_STAGE + 128 * w);
        } else {
          if (lane < 8) dma4(pg + a.scale_off + (int64_t)(slot0 + lane) * 4, sb + C::C_STAGE + C::R_STAGE + 32 * w);
        }
      }
    } else {
      // gathered rows: this wave's 8 row codes
      const LDS int32_t* lc = list + (t - tc0) * kTile + 8 * w;
      const i32x4 c0 = *(const LDS i32x4*)lc;
      const i32x4 c1 = *(const LDS i32x4*)(lc + 4);
      int32_t code[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        code[k] = __builtin_amdgcn_readfirstlane(c0[k]);
        code[k + 4] = __builtin_amdgcn_readfirstlane(c1[k]);
      }
      const uint8_t* pgk[8];
      int slk[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const bool v = code[k] >= 0;
        pgk[k] = pool + (v ? (int64_t)(code[k] >> 6) * a.page_bytes : 0);
        slk[k] = v ? (code[k] & 63) : 0;
        if (v) bits |= 1u << k;
      }
      constexpr int CR = FP8 ? kC8Row : kCRow;
      if (FP8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint8_t* src = (lane < 32) ? pgk[2 * q] + slk[2 * q] * CR : pgk[2 * q + 1] + slk[2 * q + 1] * CR;
          dma16_nt(src + 16 * (lane & 31), sb + (8 * w + 2 * q) * kC8Row);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          dma16_nt(pgk[k] + slk[k] * CR + 16 * (lane ^ swz(8 * w + k)), sb + (8 * w + k) * kCRow);
      }
      const int rr = lane >> 3, rc = lane & 7;
      const uint8_t* rp = pgk[0];
      int rs = slk[0];
#pragma unroll
      for (int k = 1; k < 8; ++k) {
        rp = (rr == k) ? pgk[k] : rp;
        rs = (rr == k) ? slk[k] : rs;
      }
      dma16_nt(rp + a.rope_off + rs * kRRow + 16 * (rc ^ swz_r(8 * w + rr)), sb + C::C_STAGE + 8 * w * kRRow);
      if (FP8) {
        if (lane < 8) {
          const uint8_t* sp = pgk[0];
          int ss = slk[0];
#pragma unroll
          for (int k = 1; k < 8; ++k) {
            sp = (lane == k) ? pgk[k] : sp;
            ss = (lane == k) ? slk[k] : ss;
          }
          if (GS) dma16_nt(sp + a.scale_off + ss * 16, sb + C::C_STAGE + C::R_STAGE + 128 * w);
          else dma4(sp + a.scale_off + ss * 4, sb + C::C_STAGE + C::R_STAGE + 32 * w);
        }
      }
    }
    if (lane == 0) smem[C::MASK_OFF + st * 4 + w] = (char)bits;
  }
};

template <bool FP8, bool GS, bool TOPK, bool DIRECT>
__global__ __launch_bounds__(kThreads, 1) void decode_mfma_kernel(DecodeArgs a) {
  static_assert(FP8 == GS, "FP8 caches served here carry group scales");
  using C = Cfg<FP8, GS>;
  constexpr int NS = C::NS;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
  LDS char* L = (LDS char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5;
  const float scale_log2 = a.scale * kLog2e;

  Loader<FP8, GS, TOPK> ld{a, (uint32_t)(uintptr_t)smem, lane, w};

  // ---- this work-group's share: n units of the split space from offset v0
  // of request b0's span (a span is the request's lead, then its tiles) ----
  int32_t b0, v0;
  int64_t n;
  const int64_t worker = DIRECT ? (int64_t)blockIdx.x : xcd_worker(blockIdx.x, gridDim.x);
  const int32_t lead = lead_of(TOPK ? a.topk : 0);
  if (DIRECT) {
    b0 = blockIdx.x;
    v0 = lead;  // straight to tile 0
    n = ld.ntiles(b0);
  } else {
    const WorkerSpan ws = locate_worker(a.seq_lens, a.batch, TOPK ? a.topk : 0, worker, a.num_workers);
    n = ws.g1 - ws.g0;
    if (n <= 0) return;
    b0 = ws.b;
    v0 = ws.t;
  }

  // ---- per-lane LDS offsets (relative to a tile) ----
  const OperandOffsets off(lane);
  const int (&s_off)[8] = off.s_off;
  const int (&r_off)[4] = off.r_off;
  const int (&tr_off)[2][4] = off.tr_off;
  const int row = lane & 31;
  const int head = 32 * w + row;

  // Weighted-latent accumulators: 32 heads x 512 latent columns per wave,
  // 16 MFMA blocks (the whole accumulator register file).
  f32x16 O[16];
  bf16x8 q[32];
  bf16x8 qr[4];

  int32_t cb = b0;      // current request
  int64_t cv = v0;      // offset of the next unit inside request cb's span
  LDS int32_t* list = (LDS int32_t*)(L + C::LIST_OFF);

  if (n == 0) {  // only in direct mode: a request with no position
    if (DIRECT) {
      __bf16* o = (__bf16*)a.o_lat + ((int64_t)b0 * kHeads + head) * kLatent + 4 * hi;
      for (int d = 0; d < kLatent; d += 8) *(uint64_t*)(o + d) = 0;
      if (a.lse_out != nullptr && hi == 0) a.lse_out[(int64_t)b0 * kHeads + head] = -INFINITY;
    }
    return;
  }

  int64_t i = 0;  // units of this work-group consumed so far
  while (i < n) {
    // ---- one segment: tiles [ct, ct + seg_len) of request cb ----
    if (cb >= a.batch) break;  // unreachable when the tile accounting is consistent
    if (cv < lead) {  // the lead of request cb carries no work
      const int64_t skip = lead - cv < n - i ? lead - cv : n - i;
      i += skip;
      cv += skip;
      if (i >= n) break;
    }
    const int32_t ct = (int32_t)(cv - lead);
    const int32_t nt_cb = ld.ntiles(cb);
    const int64_t left_in_req = nt_cb - ct;
    const int32_t seg_len = (int32_t)(left_in_req < n - i ? left_in_req : n - i);
    if (seg_len <= 0) break;
    const int32_t T = sload(a.seq_lens + cb);

#pragma unroll
    for (int mb = 0; mb < 16; ++mb) O[mb] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    for (int32_t tc0 = ct; tc0 < ct + seg_len; tc0 += chunk_tiles<TOPK>()) {
      const int32_t clen = min(chunk_tiles<TOPK>(), ct + seg_len - tc0);
      // Drain (earlier output stores count on vmcnt too), then stage this
      // chunk's page ids / row codes in LDS and, at a segment start, fetch the
      // request's queries -- all before tiles go in flight again.
      wait_vmcnt<0>();
      __syncthreads();
      ld.fill_list(cb, tc0, clen, T, list, tid);
      if (tc0 == ct) {
        const __bf16* ql = (const __bf16*)a.q_lat + ((int64_t)cb * kHeads + head) * kLatent + 8 * hi;
        const __bf16* qp = (const __bf16*)a.q_rope + ((int64_t)cb * kHeads + head) * kRope + 8 * hi;
#pragma unroll
        for (int kb = 0; kb < 32; ++kb) q[kb] = *(const bf16x8*)(ql + 16 * kb);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) qr[kb] = *(const bf16x8*)(qp + 16 * kb);
        if (C::QR_LDS) {
          // chunk 2 kb + hi of this lane's head, swizzled like the rotary keys
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            *(LDS bf16x8*)(L + C::QR_OFF + head * kRRow + 16 * ((2 * kb + hi) ^ swz_r(head))) = qr[kb];
        }
      }
      __syncthreads();  // the row list is complete
      // the first tiles go in flight while the queries are still loading
      const int32_t pro = clen < NS - 1 ? clen : NS - 1;
      for (int32_t k = 0; k < pro; ++k) ld.issue(k, tc0 + k, tc0, T, list, smem);
      if (tc0 == ct) {
        // take the queries here, once per segment, so the wait for them is
        // placed before the tile loop and not inside it
#pragma unroll
        for (int kb = 0; kb < 32; ++kb) asm volatile("" ::"v"(q[kb]));
        if (!C::QR_LDS) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) asm volatile("" ::"v"(qr[kb]));
        }
      }

      for (int32_t j = 0; j < clen; ++j) {
        const int st = j % NS;
        wait_tiles<NS, C::DMA_PER_WAVE>(clen - 1 - j);
        __syncthreads();
        if (j + NS - 1 < clen) ld.issue((j + NS - 1) % NS, tc0 + j + NS - 1, tc0, T, list, smem);
        const uint32_t mask = *(const LDS uint32_t*)(L + C::MASK_OFF + st * 4);

        LDS char* Ct;   // BF16 latent tile (swizzled)
        LDS char* Rt = L + st * C::STAGE + C::C_STAGE;
        if (FP8) {
          // E4M3 -> BF16 into the conversion buffer (exact: every E4M3 value
          // is a BF16 value); masked rows become zeros.  Each wave converts
          // the 8 rows its own loads brought in: lane l takes bytes 8l .. 8l+7
          // of a row (one 512-byte read across the wave) and writes their
          // BF16 values as 16-byte chunk l of the swizzled row (one 1 KiB
          // write), so neither side has bank conflicts.
          Ct = L + C::CONV_OFF;
          const LDS char* src = L + st * C::STAGE + 8 * w * kC8Row + 8 * lane;
          const LDS float* scl = (const LDS float*)(L + st * C::STAGE + C::C_STAGE + C::R_STAGE);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int r = 8 * w + k;
            const i32x2 raw = *(const LDS i32x2*)(src + k * kC8Row);
            // E4M3 pairs -> exact float32 pairs; each value times its group's
            // scale (lane l covers channels 8l .. 8l + 7: group l / 16 of 128)
            // is rounded once to BF16.
            const f32x2 v[4] = {__builtin_amdgcn_cvt_pk_f32_fp8(raw[0], false),
                                __builtin_amdgcn_cvt_pk_f32_fp8(raw[0], true),
                                __builtin_amdgcn_cvt_pk_f32_fp8(raw[1], false),
                                __builtin_amdgcn_cvt_pk_f32_fp8(raw[1], true)};
            i32x4 outv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float sc = scl[C::SCALES * r + (lane >> 4)];
              const bf16x2 b = bf16x2{(__bf16)(v[e][0] * sc), (__bf16)(v[e][1] * sc)};
              outv[e] = __builtin_bit_cast(int, b);
            }
            if (!((mask >> r) & 1)) outv = i32x4{0, 0, 0, 0};
            *(LDS i32x4*)(Ct + r * kCRow + 16 * (lane ^ swz(r))) = outv;
          }
          __syncthreads();
        } else {
          Ct = L + st * C::STAGE;
          if (mask != 0xFFFFFFFFu) {
            // masked rows may hold anything; zero them so 0-probability x row stays 0
            const int r = tid >> 3, qq = tid & 7;
            if (!((mask >> r) & 1)) {
              LDS char* dst = Ct + r * kCRow + 128 * qq;
#pragma unroll
              for (int v = 0; v < 8; ++v) *(LDS i32x4*)(dst + 16 * v) = i32x4{0, 0, 0, 0};
            }
            __syncthreads();
          }
        }

        // ---- scores S^T[pos][head] ----
        // 32 latent K-blocks then 4 rotary K-blocks, one accumulator chain.
        // Operands are read SD blocks ahead into a register ring; scheduling
        // fences keep the order "MFMA k, then the read for k + SD" so the LDS
        // latency hides behind the MFMAs.
        auto rq_operand = [&](int v) -> bf16x8 {
          if (C::QR_LDS) return *(const LDS bf16x8*)(L + C::QR_OFF + head * kRRow + 16 * ((2 * v + hi) ^ swz_r(head)));
          return qr[v];
        };
        f32x16 sacc = f32x16{};
        {
          constexpr int SD = 4;
          auto s_operand = [&](int k) -> bf16x8 {
            if (k < 32) return *(const LDS bf16x8*)(Ct + s_off[k & 7] + 256 * (k >> 3));
            return *(const LDS bf16x8*)(Rt + r_off[k - 32]);
          };
          bf16x8 ring[SD];
#pragma unroll
          for (int k = 0; k < SD; ++k) ring[k] = s_operand(k);
          __builtin_amdgcn_sched_barrier(0);
          bf16x8 rq[4];
#pragma unroll
          for (int k = 0; k < 36; ++k) {
            if (k == 28) {
#pragma unroll
              for (int v = 0; v < 4; ++v) rq[v] = rq_operand(v);
            }
            const bf16x8 bq = k < 32 ? q[k] : rq[k - 32];
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[k % SD], bq, sacc, 0, 0, 0);
            if (k + SD < 36) ring[k % SD] = s_operand(k + SD);
            __builtin_amdgcn_sched_barrier(0);
          }
        }

        // ---- online softmax; lane owns head `head`, 16 of the 32 positions ----
        // Position of accumulator r: 8*(r/4) + 4*hi + r%4.  Work in log2
        // units: exp2(score * scale * log2(e) - m).  The row maximum is taken
        // on raw scores and scaled once (the scale is positive).
        float s[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = sacc[r];
        if (mask != 0xFFFFFFFFu) {  // ragged or gathered tile: masked positions
          const uint32_t mlane = mask >> (4 * hi);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[r] = ((mlane >> (8 * (r >> 2) + (r & 3))) & 1u) ? s[r] : -INFINITY;
        }
        float mloc = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
        mloc = fmaxf(mloc, fmaxf(fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11])),
                                 fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15]))));
        mloc = fmaxf(mloc, wave_partner(mloc)) * scale_log2;
        const float m_new = fmaxf(m_run, mloc);
        // Rescale lazily: keep the old reference maximum unless the new one
        // exceeds it by more than 16 (log2 units), so probabilities stay
        // <= 2^16, far inside the range of BF16 and of the float32 sums.  A
        // head whose maximum is still -inf has only zeros in the accumulator
        // (all its probabilities so far were 0): the first tile of a segment
        // never needs the accumulator pass.
        const bool need = m_new > m_run + 16.0f;
        {
          const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
          const bool held = m_run != -INFINITY;
          m_run = need ? m_new : m_run;
          l_run *= alpha;
          if (__builtin_amdgcn_ballot_w64(need && held) != 0) {
#pragma unroll
            for (int mb = 0; mb < 16; ++mb)
#pragma unroll
              for (int r = 0; r < 16; ++r) O[mb][r] = scale_acc(O[mb][r], alpha);
          }
        }
        const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
        float lsum = 0.f;
        bf16x8 P[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, neg_m));
          lsum += p;
          P[r >> 3][r & 7] = (__bf16)p;
        }
        l_run += lsum;

        // ---- weighted latent U^T[latent][head] += C^T P^T ----
        // 16 column blocks x 2 position halves; each operand is two transposing
        // LDS reads, prefetched PD operands ahead.
        {
          constexpr int PD = 3;
          auto pv_operand = [&](int j) -> bf16x8 {
            const int mb = j >> 1, kb2 = j & 1;
            const LDS char* p1 = Ct + tr_off[0][mb & 3] + 256 * (mb >> 2) + 16 * kCRow * kb2;
            const LDS char* p2 = Ct + tr_off[1][mb & 3] + 256 * (mb >> 2) + 16 * kCRow * kb2;
            s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)p1);
            s16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)p2);
            typedef __attribute__((ext_vector_type(8))) short s16x8;
            return __builtin_bit_cast(bf16x8, (s16x8)__builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
          };
          bf16x8 ring[PD];
#pragma unroll
          for (int j = 0; j < PD; ++j) ring[j] = pv_operand(j);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < 32; ++j) {
            O[j >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[j % PD], P[j & 1], O[j >> 1], 0, 0, 0);
            if (j + PD < 32) ring[j % PD] = pv_operand(j + PD);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
    i += seg_len;

    // ---- end of the segment: normalise and write ----
    {
      const float l_tot = l_run + wave_partner(l_run);
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
      const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
      // BF16 rows of this wave's 32 heads (the final o_lat, or the partial:
      // partials of the MFMA kernels are BF16), staged through LDS so that
      // every global store writes one contiguous 1 KiB row
      const int64_t slot = worker + cb;
      __bf16* rows = DIRECT ? (__bf16*)a.o_lat + (int64_t)cb * kHeads * kLatent
                            : (__bf16*)a.part_o + slot * kHeads * kLatent;
      store_rows_staged(L, rows + (int64_t)32 * w * kLatent, O, inv, w, [&]() {
        if (DIRECT) {
          if (a.lse_out != nullptr && hi == 0) a.lse_out[(int64_t)cb * kHeads + head] = lse;
        } else {
          if (hi == 0) a.part_lse[slot * kHeads + head] = lse;
        }
      });
    }
    // next request with tiles
    ++cb;
    cv = 0;
    while (cb < a.batch && ld.ntiles(cb) == 0) ++cb;
  }
  // Only stores can be in flight here (every tile load was waited for);
  // the wave may end with them outstanding.
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, CacheKind kind, hipStream_t s) {
  const bool topk = a.topk_idx != nullptr;
  const bool direct = a.num_workers == 0;
  const dim3 grid(direct ? a.batch : a.num_workers);
  const dim3 block(kThreads);
#define MLA_LAUNCH(F, G)                                                                                 \
  do {                                                                                                   \
    if (topk) {                                                                                          \
      if (direct) hipLaunchKernelGGL((decode_mfma_kernel<F, G, true, true>), grid, block, 0, s, a);     \
      else hipLaunchKernelGGL((decode_mfma_kernel<F, G, true, false>), grid, block, 0, s, a);           \
    } else {                                                                                             \
      if (direct) hipLaunchKernelGGL((decode_mfma_kernel<F, G, false, true>), grid, block, 0, s, a);    \
      else hipLaunchKernelGGL((decode_mfma_kernel<F, G, false, false>), grid, block, 0, s, a);          \
    }                                                                                                    \
  } while (0)
  switch (kind) {
    case CacheKind::kFp8Token: return launch_decode_fp8(a, s);
    case CacheKind::kFp8Group128: MLA_LAUNCH(true, true); break;
    default: MLA_LAUNCH(false, false); break;
  }
#undef MLA_LAUNCH
  return hipGetLastError();
}

}  // namespace mla
