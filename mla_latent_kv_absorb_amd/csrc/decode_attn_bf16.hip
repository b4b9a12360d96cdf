// Weight-absorbed MLA decode attention, BF16 latent cache, all positions
// visible (no index list), gfx950.
//
// Same work split and arithmetic as the general attention kernel (4 waves per
// work-group, each owning 32 of the 128 heads; scores S^T[pos][head] =
// C . q_lat + K_rope . q_rope on MFMA 32x32x16; online softmax with one head
// per lane; weighted latent U^T += C^T P^T on MFMA; "DeepSeek's KV Cache",
// Figures 5 and 6, form (2)), but the tile loop is software-pipelined so the
// softmax never stalls the matrix cores:
//
//   iteration j:  wait for tile j, barrier, start the load of tile j + 2
//                 (if the segment has it)
//                 scores of tile j                        (36 MFMAs)
//                 weighted latent of tile j - 1           (32 MFMAs)
//                   with the softmax of tile j interleaved between them
//                 rescale the accumulator if a running maximum jumped
//
// The softmax of tile j needs only the scores of tile j, and the weighted
// latent of tile j - 1 needs only the probabilities of tile j - 1, so the two
// are independent and the VALU work runs in the shadow of the MFMAs.  The 68
// MFMAs of an iteration read their LDS operands through one register ring
// that runs three MFMAs ahead across the switch from scores to weighted
// latent, and the rotary query blocks are fetched the same distance ahead, so
// no MFMA waits on a fresh LDS read.  The stage ring holds 4 tiles: j - 1
// (being consumed), j (being scored), j + 1 and j + 2 (in flight).
//
// Loads: each wave moves 8 latent rows (1 KiB each) and 8 rotary rows of a
// tile with global_load_lds_dwordx4 in its scalar-base form: one 64-bit page
// address per tile, per-lane 32-bit offsets fixed for the whole launch (the
// XOR swizzle of the LDS rows is folded into them), and M0 as the LDS
// destination.  Page ids come from the block table through scalar loads one
// tile ahead.  Positions past the context end or on an invalid page are still
// loaded from a valid page (so every wave issues the same loads per tile),
// then zeroed in LDS and masked out of the softmax.  No tile is loaded past a
// segment's end: the last two iterations wait for everything in flight.
#include <type_traits>

#include "attn_common.h"

namespace mla {
namespace {

constexpr int kNS = 4;                          // ring stages
constexpr int kCStage = kTile * kCRow;          // 32 KiB latent rows
constexpr int kStage = kCStage + kTile * kRRow;  // + 4 KiB rotary rows
constexpr int kDmaPerWave = 9;                  // 8 latent rows + 1 rotary block per wave and tile
constexpr int kQrOff = kNS * kStage;            // rotary queries of the request, [head][64] bf16
constexpr int kLdsBytes = kQrOff + kHeads * kRRow;  // 160 KiB

struct TileLoader {
  const uint8_t* pool;
  int64_t page_bytes, rope_off, num_pages;
  const int32_t* bt;  // block-table row of the current request
  int32_t bt_stride;
  uint32_t lds_base;  // LDS address of stage 0
  int w;
  uint32_t lane16;    // 16 * lane
  uint32_t voff_r;    // per-lane byte offset inside this wave's 8 rotary rows

  __device__ __forceinline__ void init(int lane) {
    lane16 = 16 * lane;
    const int rr = lane >> 3, rc = lane & 7;
    voff_r = rr * kRRow + 16 * (rc ^ swz_r(8 * w + rr));
  }

  // page id of logical page p of the current request, or -1
  __device__ __forceinline__ int32_t page_of(int32_t p) const { return checked(p, raw(p)); }
  // The same in two steps, so the load can be issued an iteration before its
  // value is needed: raw() loads (from a clamped column), checked() validates.
  __device__ __forceinline__ int32_t raw(int32_t p) const { return sload(bt + (p < bt_stride ? p : bt_stride - 1)); }
  __device__ __forceinline__ int32_t checked(int32_t p, int32_t pg) const {
    return (p < bt_stride && pg >= 0 && pg < num_pages) ? pg : -1;
  }

  // This wave's share of tile t (page id `page`, -1 = invalid or no tile)
  // into stage st, as kDmaPerWave single loads that the caller spreads over
  // its MFMAs (all loads of a work-group issued at once would queue in the
  // address unit and stall the issuing waves).  An invalid page is replaced
  // by page 0: its rows are zeroed after they land.
  struct Tile {
    const uint8_t* c_base;
    const uint8_t* r_base;
    uint32_t sb;
  };
  __device__ __forceinline__ Tile tile(int st, int32_t t, int32_t page) const {
    const int64_t pg = page >= 0 ? page : 0;
    const int slot0 = (t & 1) * kTile + 8 * w;
    return Tile{pool + pg * page_bytes + (int64_t)slot0 * kCRow,
                pool + pg * page_bytes + rope_off + (int64_t)slot0 * kRRow, lds_base + st * kStage};
  }
  __device__ __forceinline__ void issue_one(const Tile& tl, int k) const {
    if (k < 8)  // latent row 8w + k: lane l fetches chunk l ^ swz(row), so LDS chunk l holds it
      dma16s(lane16 ^ (16 * swz(8 * w + k)), tl.c_base + k * kCRow, tl.sb + (8 * w + k) * kCRow);
    else
      dma16s(voff_r, tl.r_base, tl.sb + kCStage + 8 * w * kRRow);
  }
  __device__ __forceinline__ void issue(int st, int32_t t, int32_t page) const {
    const Tile tl = tile(st, t, page);
#pragma unroll
    for (int k = 0; k < kDmaPerWave; ++k) issue_one(tl, k);
  }
};

template <bool DIRECT>
__global__ __launch_bounds__(kThreads, 1) void decode_bf16_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  LDS char* L = (LDS char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5;
  const int row = lane & 31;
  const int head = 32 * w + row;
  const float scale_log2 = a.scale * kLog2e;

  // ---- this work-group's share: n units of the split space from offset v0
  // of request b0's span (a span is the request's lead, then its tiles) ----
  int32_t b0, v0;
  int64_t n;
  const int64_t worker = DIRECT ? (int64_t)blockIdx.x : xcd_worker(blockIdx.x, gridDim.x);
  auto ntiles = [&](int32_t b) -> int32_t {
    const int32_t T = sload(a.seq_lens + b);
    return T > 0 ? tiles_of(T) : 0;
  };
  if (DIRECT) {
    b0 = blockIdx.x;
    v0 = kLeadTiles;  // no lead: straight to tile 0
    n = ntiles(b0);
  } else {
    const int64_t W = spans_below(a.seq_lens, a.batch, 0);
    const int64_t g0 = worker_lo(worker, W, a.num_workers);
    const int64_t g1 = worker_lo(worker + 1, W, a.num_workers);
    n = g1 - g0;
    if (n <= 0) return;
    locate_span(a.seq_lens, a.batch, 0, g0, &b0, &v0);
  }

  if (n == 0) {  // direct mode, a request with no position
    if (DIRECT) {
      __bf16* o = (__bf16*)a.o_lat + ((int64_t)b0 * kHeads + head) * kLatent + 4 * hi;
      for (int d = 0; d < kLatent; d += 8) *(uint64_t*)(o + d) = 0;
      if (a.lse_out != nullptr && hi == 0) a.lse_out[(int64_t)b0 * kHeads + head] = -INFINITY;
    }
    return;
  }

  const OperandOffsets off(lane);
  TileLoader ld;
  ld.pool = a.pool;
  ld.page_bytes = a.page_bytes;
  ld.rope_off = a.rope_off;
  ld.num_pages = a.num_pages;
  ld.bt_stride = a.bt_stride;
  ld.lds_base = (uint32_t)(uintptr_t)smem;
  ld.w = w;
  ld.init(lane);

  f32x16 O[16];
  bf16x8 q[32];

  // ---- the MFMA stream of one iteration ----
  // Operand i < 36: score K-block i of the tile in stage `sst` (latent blocks,
  // then rotary blocks); operand i >= 36: transposed latent block i - 36 of
  // the tile in stage `pst` for the weighted latent.  One ring of loads runs
  // three MFMAs ahead across both halves, so the matrix cores never wait for
  // the first operand of a phase.
  auto s_operand = [&](const LDS char* Ct, int k) -> bf16x8 {
    if (k < 32) return *(const LDS bf16x8*)(Ct + off.s_off[k & 7] + 256 * (k >> 3));
    return *(const LDS bf16x8*)(Ct + kCStage + off.r_off[k - 32]);
  };
  // step j: column block mb = j % 16, position half kb2 = j / 16, so that
  // consecutive MFMAs accumulate into different blocks
  auto pv_operand = [&](const LDS char* Ct, int j) -> bf16x8 {
    const int mb = j & 15, kb2 = j >> 4;
    const LDS char* p1 = Ct + off.tr_off[0][mb & 3] + 256 * (mb >> 2) + 16 * kCRow * kb2;
    const LDS char* p2 = Ct + off.tr_off[1][mb & 3] + 256 * (mb >> 2) + 16 * kCRow * kb2;
    s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)p1);
    s16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)p2);
    typedef __attribute__((ext_vector_type(8))) short s16x8;
    return __builtin_bit_cast(bf16x8, (s16x8)__builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // rotary query block v of this lane's head (rows swizzled as the rotary keys)
  auto rq_operand = [&](int v) -> bf16x8 {
    return *(const LDS bf16x8*)(L + kQrOff + head * kRRow + 16 * ((2 * v + hi) ^ swz_r(head)));
  };
  // HAS_S: scores of the tile in sst (36 MFMAs) before the weighted latent of
  // the tile in pst (32 MFMAs); without it only the weighted latent.
  // after_s(k) runs after score MFMA k, piece(k) after weighted MFMA k + 1;
  // the scores land in s before the first piece.
  auto stream = [&](auto has_s, int sst, int pst, const bf16x8& P0, const bf16x8& P1, f32x16& s, auto&& after_s,
                    auto&& piece) __attribute__((always_inline)) {
    constexpr bool HAS_S = decltype(has_s)::value;
    constexpr int I0 = HAS_S ? 0 : 36;
    constexpr int D = 3;
    const LDS char* Cs = L + sst * kStage;
    const LDS char* Cp = L + pst * kStage;
    auto operand = [&](int i) -> bf16x8 { return i < 36 ? s_operand(Cs, i) : pv_operand(Cp, i - 36); };
    bf16x8 ring[D];
    bf16x8 rq[D];
    f32x16 sacc;
#pragma unroll
    for (int i = I0; i < I0 + D; ++i) ring[i % D] = operand(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = I0; i < 36; ++i) {
      const bf16x8 bq = i < 32 ? q[i & 31] : rq[(i + 3 * D - 32) % D];
      if (i == 0) sacc = mfma_sv0(ring[i % D], bq);
      else mfma_sv(sacc, ring[i % D], bq);
      ring[i % D] = operand(i + D);
      // rotary query blocks, D MFMAs ahead of their use
      if (i >= 32 - D && i < 36 - D) rq[(i + D - 32) % D] = rq_operand(i + D - 32);
      after_s(i);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (HAS_S) {
      // the last score MFMA's result is read by VALU instructions: cover the
      // MFMA-write -> VALU-read distance (at most 19 wait states)
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(sacc));
      s = sacc;
    }
#pragma unroll
    for (int i = 36; i < 68; ++i) {
      const int j = i - 36;
      O[j & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % D], (j >> 4) ? P1 : P0, O[j & 15], 0, 0, 0);
      if (i + D < 68) ring[i % D] = operand(i + D);
      if (i > 36) piece(i - 37);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  int32_t cb = b0;
  int64_t cv = v0;   // offset of the next unit inside request cb's span
  int64_t done = 0;  // units consumed
  while (done < n) {
    // ---- one segment: tiles [ct, ct + seg) of request cb ----
    if (cb >= a.batch) break;  // unreachable when the tile accounting is consistent
    if (cv < kLeadTiles) {  // the lead of request cb carries no work
      const int64_t skip = kLeadTiles - cv < n - done ? kLeadTiles - cv : n - done;
      done += skip;
      cv += skip;
      if (done >= n) break;
    }
    const int32_t ct = (int32_t)(cv - kLeadTiles);
    const int32_t nt_cb = ntiles(cb);
    const int64_t left = nt_cb - ct;
    const int32_t seg = (int32_t)(left < n - done ? left : n - done);
    if (seg <= 0) break;
    const int32_t T = sload(a.seq_lens + cb);
    ld.bt = a.block_table + (int64_t)cb * a.bt_stride;

    // Stages are free once every wave has finished the previous segment;
    // earlier stores and loads count on vmcnt too, so drain first.
    wait_vmcnt<0>();
    __syncthreads();
    // Page ids are fetched one tile ahead of the load that needs them.  No
    // tile is loaded past the segment end, so nothing is left in flight when
    // the segment's result is written.  The page ids of the first two tiles
    // go out first; while they are in flight the queries are requested (the
    // latent queries into registers, the rotary queries straight into LDS),
    // then the two tiles; all of it lands before the loop, in one round trip
    // after the page ids.
    const int32_t raw_a = ld.raw(ct >> 1);                                  // tile ct
    const int32_t raw_b = ld.raw(seg > 1 ? (ct + 1) >> 1 : 0);             // tile ct + 1
    {
      const __bf16* ql = (const __bf16*)a.q_lat + ((int64_t)cb * kHeads + head) * kLatent + 8 * hi;
#pragma unroll
      for (int kb = 0; kb < 32; ++kb) q[kb] = *(const bf16x8*)(ql + 16 * kb);
      // rotary queries: rows 32 w + 8 p .. + 7 per load, lane l bringing the
      // chunk that LDS position l % 8 of its row holds (rows swizzled like
      // the rotary keys)
      const __bf16* qp = (const __bf16*)a.q_rope + (int64_t)cb * kHeads * kRope;
#pragma unroll
      for (int pass = 0; pass < 4; ++pass) {
        const int hh = 32 * w + 8 * pass + (lane >> 3);
        const int c = (lane & 7) ^ swz_r(hh);
        dma16(qp + hh * kRope + 8 * c, ld.lds_base + kQrOff + (32 * w + 8 * pass) * kRRow);
      }
    }
    const int32_t pg_a = ld.checked(ct >> 1, raw_a);
    const int32_t pg_b = seg > 1 ? ld.checked((ct + 1) >> 1, raw_b) : -1;
    ld.issue(0, ct, pg_a);
    if (seg > 1) ld.issue(1, ct + 1, pg_b);
    // page of tile ct + 2: loaded now, checked when its load is issued
    int32_t pg_next_p = seg > 2 ? (ct + 2) >> 1 : INT32_MAX;
    int32_t pg_next_raw = ld.raw(seg > 2 ? pg_next_p : 0);
    // validity of the tiles in flight, by stage: tile ct + j has stage j % 4
    bool valid_j = pg_a >= 0, valid_j1 = pg_b >= 0;
    {
      // The weighted latent of "tile -1" reads stage 3 with zero
      // probabilities; zero its latent rows so stale or uninitialised LDS
      // cannot turn 0 x NaN into NaN.  Ordered before the first read by the
      // barrier of iteration 0.
      LDS char* dst = L + 3 * kStage + (tid >> 3) * kCRow + 128 * (tid & 7);
#pragma unroll
      for (int v = 0; v < 8; ++v) *(LDS i32x4*)(dst + 16 * v) = i32x4{0, 0, 0, 0};
    }
    wait_vmcnt<0>();  // queries and the first two tiles
    // take the latent queries here, so the waits for them sit before the
    // tile loop (all satisfied) and not inside it
#pragma unroll
    for (int kb = 0; kb < 32; ++kb) asm volatile("" ::"v"(q[kb]));


#pragma unroll
    for (int mb = 0; mb < 16; ++mb) O[mb] = f32x16{};
    float m_run = -INFINITY;  // running maximum of this lane's head (log2 units)
    float l_run = 0.f;        // this lane's share of the running sum
    bf16x8 Pp0, Pp1;          // probabilities of the previous tile
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      Pp0[r] = (__bf16)0.f;
      Pp1[r] = (__bf16)0.f;
    }

    for (int32_t j = 0; j < seg; ++j) {
      const int32_t t = ct + j;
      // tile j landed (tile j + 1, if the segment has it, may still be in
      // flight)
      if (j + 1 < seg) wait_vmcnt<kDmaPerWave>();
      else wait_vmcnt<0>();
      __syncthreads();
      // stage (j + 2) % 4 held tile j - 2, consumed in the previous
      // iteration; tile j + 2 is loaded into it during the scores below
      const int32_t pg_next = ld.checked(pg_next_p, pg_next_raw);
      const bool valid_j2 = pg_next >= 0;
      const TileLoader::Tile next_tile = ld.tile((j + 2) & 3, t + 2, pg_next);
      const bool has_next = j + 2 < seg;
      pg_next_p = j + 3 < seg ? (t + 3) >> 1 : INT32_MAX;
      pg_next_raw = ld.raw(j + 3 < seg ? pg_next_p : 0);
      // rows of tile j that are visible
      const int32_t nvis = valid_j ? (T - t * kTile < kTile ? T - t * kTile : kTile) : 0;
      const bool full = nvis == kTile;
      if (!full) {
        // zero the invisible rows (they hold page-0 or past-the-end data,
        // which a zero probability must not turn into NaN)
        LDS char* Ct = L + (j & 3) * kStage;
        const int r = tid >> 3, qq = tid & 7;
        if (r >= nvis) {
          LDS char* dst = Ct + r * kCRow + 128 * qq;
#pragma unroll
          for (int v = 0; v < 8; ++v) *(LDS i32x4*)(dst + 16 * v) = i32x4{0, 0, 0, 0};
        }
        __syncthreads();
      }
      valid_j = valid_j1;
      valid_j1 = valid_j2;

      // ---- softmax of tile j, in pieces, inside the weighted latent of tile j - 1 ----
      f32x16 s;  // scores, then probabilities, of tile j
      float mt = -INFINITY, m_use = m_run, neg_m = 0.f, lsum = 0.f;
      bool need = false;
      bf16x8 Pc0, Pc1;
      auto piece = [&](int k) {
        // Each step ends with an empty asm that takes its result: code motion
        // cannot then sink the VALU work past the MFMAs that hide it.
        if (k == 0) {
          if (!full) {
            // position of accumulator r: 8 * (r / 4) + 4 * hi + r % 4
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int pos = 8 * (r >> 2) + 4 * hi + (r & 3);
              s[r] = pos < nvis ? s[r] : -INFINITY;
            }
          }
          mt = max3_raw(max3_raw(s[0], s[1], s[2]), max3_raw(s[3], s[4], s[5]), max_raw(s[6], s[7]));
          asm volatile("" : "+v"(mt));
        } else if (k == 1) {
          mt = max3_raw(max3_raw(mt, s[8], s[9]), max3_raw(s[10], s[11], s[12]), max3_raw(s[13], s[14], s[15]));
          asm volatile("" : "+v"(mt));
        } else if (k == 2) {
          mt = max_raw(mt, wave_partner(mt)) * scale_log2;
          asm volatile("" : "+v"(mt));
        } else if (k == 3) {
          // Lazy rescale: keep the reference maximum unless the tile's
          // maximum exceeds it by more than 8 (log2 units), so probabilities
          // stay <= 256 and the accumulator is rescaled rarely.
          const float m_new = max_raw(m_run, mt);
          need = m_new > m_run + 8.0f;
          m_use = need ? m_new : m_run;
          neg_m = (m_use == -INFINITY) ? 0.f : -m_use;
          asm volatile("" : "+v"(neg_m), "+v"(m_use));
        } else if (k >= 4 && k < 20) {
          const int r = k - 4;
          s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, neg_m));
          asm volatile("" : "+v"(s[r]));
        } else if (k >= 20 && k < 28) {
          const int r = 2 * (k - 20);
          lsum += s[r] + s[r + 1];
          if (r < 8) {
            Pc0[r] = (__bf16)s[r];
            Pc0[r + 1] = (__bf16)s[r + 1];
          } else {
            Pc1[r - 8] = (__bf16)s[r];
            Pc1[r - 7] = (__bf16)s[r + 1];
          }
          asm volatile("" : "+v"(lsum));
          if (k == 23) asm volatile("" : "+v"(Pc0));
          if (k == 27) asm volatile("" : "+v"(Pc1));
        }
      };
      stream(std::true_type{}, j & 3, (j + 3) & 3, Pp0, Pp1, s,
             [&](int k) {
               if (has_next && (k & 3) == 0 && (k >> 2) < kDmaPerWave) ld.issue_one(next_tile, k >> 2);
             },
             piece);

      // rescale what the accumulator holds (tiles up to j - 1) to the new reference
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.0f;
        l_run *= alpha;
#pragma unroll
        for (int mb = 0; mb < 16; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) O[mb][r] = scale_acc(O[mb][r], alpha);
      }
      m_run = m_use;
      l_run += lsum;
      Pp0 = Pc0;
      Pp1 = Pc1;
    }
    {
      // weighted latent of the last tile
      f32x16 s_unused;
      stream(std::false_type{}, 0, (seg + 3) & 3, Pp0, Pp1, s_unused, [](int) {}, [](int) {});
    }
    done += seg;

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
      store_rows_staged(L, rows + (int64_t)32 * w * kLatent, O, inv, w);
      if (DIRECT) {
        if (a.lse_out != nullptr && hi == 0) a.lse_out[(int64_t)cb * kHeads + head] = lse;
      } else {
        if (hi == 0) a.part_lse[slot * kHeads + head] = lse;
      }
    }
    // next request with tiles
    ++cb;
    cv = 0;
    while (cb < a.batch && ntiles(cb) == 0) ++cb;
  }
  // Only stores can be in flight here (every tile load was waited for);
  // the wave may end with them outstanding.
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
  const bool direct = a.num_workers == 0;
  const dim3 grid(direct ? a.batch : a.num_workers);
  if (direct) hipLaunchKernelGGL(decode_bf16_kernel<true>, grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(decode_bf16_kernel<false>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
