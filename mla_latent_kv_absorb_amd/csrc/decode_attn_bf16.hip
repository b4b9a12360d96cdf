// Weight-absorbed MLA decode attention, BF16 latent cache, all positions
// visible (no index list), gfx950.
//
// Scores as in the general attention kernel: each of the 4 waves owns 32 of
// the 128 heads, S^T[pos][head] = C . q_lat + K_rope . q_rope on MFMA
// 32x32x16 with the queries in registers, and an online softmax with one head
// per lane ("DeepSeek's KV Cache", Figures 5 and 6, form (2)).  The weighted
// latent is split the other way: wave w accumulates U^T[latent][head] for the
// latent columns 128 w .. 128 w + 127 and all 128 heads, and takes the
// probabilities of every head from LDS, where the owner of each head puts
// them.  A wave then reads only its quarter of a tile with transposing reads
// (each wave reading the whole tile transposed makes that phase wait on LDS),
// plus 8 KiB of probabilities with plain 16-byte reads.
//
//   iteration j:  wait for tile j, barrier, start the load of tile j + 2
//                 (if the segment has it)
//                 scores of tile j                        (36 MFMAs)
//                 rescale the accumulator if the running maximum of any head
//                 jumped at tile j - 1 (factors from the heads' owners)
//                 weighted latent of tile j - 1           (32 MFMAs)
//                   with the softmax of tile j interleaved between them; its
//                   probabilities and rescale factors go to LDS
//
// One barrier per iteration orders everything: what an owner writes for tile
// j (probabilities, rescale factors) is read in iteration j + 1, and the
// buffers alternate between even and odd tiles.
//
// LDS: 4 latent stages (tiles j - 1 .. j + 2), 3 rotary stages (j .. j + 2:
// the weighted latent needs no rotary rows), 2 probability buffers and 2
// rescale-factor buffers.
//
// Loads: each wave moves 8 latent rows (1 KiB each) and 8 rotary rows of a
// tile with global_load_lds_dwordx4 in its scalar-base form: one 64-bit page
// address per tile, per-lane 32-bit offsets (the XOR swizzle of the LDS rows
// is folded into them), and M0 as the LDS destination.  Page ids come from the
// block table through scalar loads one tile ahead.  Positions past the context
// end or on an invalid page are still loaded from a valid page (so every wave
// issues the same loads per tile), then zeroed in LDS and masked out of the
// softmax.  The last two iterations of a segment load page 0 into the free
// stages in place of the tiles past its end, so every iteration issues the
// same instructions; the segment's stores wait for them.
#include <type_traits>

#include "attn_common.h"

namespace mla {
namespace {

constexpr int kNS = 4;                           // latent stages
constexpr int kNR = 3;                           // rotary stages
constexpr int kLStage = kTile * kCRow;           // 32 KiB of latent rows
constexpr int kRStage = kTile * kRRow;           // 4 KiB of rotary rows
constexpr int kROff = kNS * kLStage;             // the rotary stages
constexpr int kPOff = kROff + kNR * kRStage;     // probabilities, 2 x [head][32] bf16
constexpr int kPBytes = kHeads * kTile * 2;      // 8 KiB
constexpr int kAOff = kPOff + 2 * kPBytes;       // rescale factors, 2 x [128] float
constexpr int kIOff = kAOff + 2 * kHeads * 4;    // 1 / row sum at a segment's end, [128] float
constexpr int kLdsBytes = kIOff + kHeads * 4;    // 157.5 KiB
constexpr int kDmaPerWave = 9;                   // 8 latent rows + 1 rotary block per wave and tile
constexpr int kQOff = 2 * kLStage;               // query staging at a segment's start (stages 2, 3)
constexpr int kD = 4;                            // score operands fetched ahead of their MFMA
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
static_assert(kSplitStage <= kPOff, "output staging must stay clear of the probability buffers");

struct TileLoader {
  const uint8_t* pool;
  int64_t page_bytes, rope_off, num_pages;
  const int32_t* bt;  // block-table row of the current request
  int32_t bt_stride;
  uint32_t lds_base;  // LDS address of the work-group's array
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
  // into latent stage ls and rotary stage rs, as kDmaPerWave single loads that
  // the caller spreads over its MFMAs (all loads of a work-group issued at
  // once would queue in the address unit and stall the issuing waves).  An
  // invalid page is replaced by page 0: its rows are zeroed after they land.
  struct Tile {
    const uint8_t* c_base;
    const uint8_t* r_base;
    uint32_t lsb, rsb;
  };
  __device__ __forceinline__ Tile tile(int ls, int rs, int32_t t, int32_t page) const {
    const int64_t pg = page >= 0 ? page : 0;
    const int slot0 = (t & 1) * kTile + 8 * w;
    return Tile{pool + pg * page_bytes + (int64_t)slot0 * kCRow,
                pool + pg * page_bytes + rope_off + (int64_t)slot0 * kRRow,
                lds_base + ls * kLStage, lds_base + kROff + rs * kRStage};
  }
  __device__ __forceinline__ void issue_one(const Tile& tl, int k) const {
    if (k < 8) {
      // latent row 8w + k: lane l fetches chunk l ^ swz(row), so LDS chunk l
      // holds it.  lane16 has no bit at or above 1 KiB, so one XOR both
      // applies the swizzle and adds the row offset k KiB; it is formed here
      // so no register per row stays live.
      const uint32_t x = 16 * swz(8 * w + k) + k * kCRow;
      uint32_t voff;
      asm volatile("v_xor_b32 %0, %1, %2" : "=v"(voff) : "s"(x), "v"(lane16));
      dma16s_nt(voff, tl.c_base, tl.lsb + (8 * w + k) * kCRow);
    } else {
      dma16s_nt(voff_r, tl.r_base, tl.rsb + 8 * w * kRRow);
    }
  }
  __device__ __forceinline__ void issue(const Tile& tl) const {
#pragma unroll
    for (int k = 0; k < kDmaPerWave; ++k) issue_one(tl, k);
  }
};

template <bool DIRECT>
__global__ __launch_bounds__(kThreads, 1) void decode_bf16_kernel(DecodeArgs a) {
  // the operand addresses below are a per-lane base XOR a swizzle constant:
  // stage bases must not touch the swizzled bits
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  LDS char* L = (LDS char*)smem;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5;
  const int row = lane & 31;
  const int head = 32 * w + row;  // the head this lane scores
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
    const WorkerSpan ws = locate_worker(a.seq_lens, a.batch, 0, worker, a.num_workers);
    n = ws.g1 - ws.g0;
    if (n <= 0) return;
    b0 = ws.b;
    v0 = ws.t;
  }

  if (n == 0) {  // direct mode, a request with no position
    if (DIRECT) {
      __bf16* o = (__bf16*)a.o_lat + ((int64_t)b0 * kHeads + head) * kLatent + 4 * hi;
      for (int d = 0; d < kLatent; d += 8) *(uint64_t*)(o + d) = 0;
      if (a.lse_out != nullptr && hi == 0) a.lse_out[(int64_t)b0 * kHeads + head] = -INFINITY;
    }
    return;
  }

  TileLoader ld;
  ld.pool = a.pool;
  ld.page_bytes = a.page_bytes;
  ld.rope_off = a.rope_off;
  ld.num_pages = a.num_pages;
  ld.bt_stride = a.bt_stride;
  ld.lds_base = lds0;
  ld.w = w;
  ld.init(lane);

  // ---- per-lane operand bases.  Each operand address is base ^ K + offset,
  // with K a compile-time swizzle constant that only touches bits the base
  // leaves to the swizzle (a 16-byte chunk index (2 v + hi) ^ s splits into
  // (v ^ (s >> 1)) and (hi ^ (s & 1))). ----
  uint32_t bs, br, bp, bt0, bt1;
  {
    const int sw = swz(row), sr = swz_r(row), ps = pswz(row);
    // score latent K-block k: row `row`, chunk (2 (k & 7) + hi) ^ swz(row) of column group k >> 3
    bs = row * kCRow + 16 * (hi ^ (sw & 1)) + 32 * (sw >> 1);
    // score rotary K-block v: chunk (2 v + hi) ^ swz_r(row)
    br = row * kRRow + 16 * (hi ^ (sr & 1)) + 32 * (sr >> 1);
    // probabilities of head 32 nb + row, position chunk 2 kb2 + hi
    bp = 64 * row + 16 * (hi ^ (ps & 1)) + 32 * (ps >> 1);
    // transposed latent of this wave's column block 4 w + mbl, rows
    // 16 kb2 + 8 h8 + tr_row: lane group (hh, ch), lane j16 in it
    const int j16 = lane & 15, g16 = lane >> 4, hh = g16 >> 1, ch = g16 & 1;
    const int tr_row = 4 * hh + (j16 >> 2);  // 0..7
    const int lo = 2 * ch + ((j16 & 3) >> 1);
    auto tb = [&](int r) {
      const int sz = swz(r);
      return (uint32_t)(r * kCRow + 8 * (j16 & 1) + 16 * (lo ^ (sz & 3)) + 64 * (sz >> 2) + 256 * w);
    };
    bt0 = tb(tr_row);
    bt1 = tb(tr_row + 8);
  }

  f32x16 O[16];  // O[4 mbl + nb]: U^T rows 32 (4 w + mbl) .., columns (heads) 32 nb ..
  bf16x8 q[32];  // latent queries of this lane's head
  bf16x8 qr[4];  // rotary queries of this lane's head

  // score K-block k < 32 (latent) of a tile whose eight latent read
  // addresses are sa (sa[v]: the lane's base ^ 32 v; the column group k / 8
  // goes in the offset field), or rotary block k - 32 at rb
  auto s_read = [&](const uint32_t (&sa)[8], uint32_t rb, auto kc) __attribute__((always_inline)) -> bf16x8 {
    constexpr int k = decltype(kc)::value;
    if constexpr (k < 32)
      return *(const LDS bf16x8*)((LDS char*)(uintptr_t)sa[k & 7] + 256 * (k >> 3));
    else
      return *(const LDS bf16x8*)(LDS char*)(uintptr_t)xor_here<32 * (k - 32)>(rb);
  };
  // transposed latent (A operand of the weighted latent): column block
  // 4 w + mbl, positions 16 kb2 .. 16 kb2 + 15 (st = 4 kb2 + mbl)
  auto a_read = [&](uint32_t t0, uint32_t t1, auto stc) __attribute__((always_inline)) -> bf16x8 {
    constexpr int st = decltype(stc)::value, mbl = st & 3, kb2 = st >> 2;
    const LDS char* p1 = (LDS char*)(uintptr_t)xor_here<64 * mbl>(t0) + 16 * kCRow * kb2;
    const LDS char* p2 = (LDS char*)(uintptr_t)xor_here<64 * mbl>(t1) + 16 * kCRow * kb2;
    s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)p1);
    s16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)p2);
    typedef __attribute__((ext_vector_type(8))) short s16x8;
    return __builtin_bit_cast(bf16x8, (s16x8)__builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // probabilities (B operand of the weighted latent): heads 32 nb .., position half kb2
  auto b_read = [&](uint32_t pb, int nb, auto kbc) __attribute__((always_inline)) -> bf16x8 {
    constexpr int kb2 = decltype(kbc)::value;
    return *(const LDS bf16x8*)((LDS char*)(uintptr_t)xor_here<32 * kb2>(pb) + 2048 * nb);
  };

  // ---- the MFMA stream of one iteration ----
  // HAS_S: the 36 score MFMAs of the tile at (sb, rb) first, then mid(), then
  // the 32 weighted-latent MFMAs of the tile at (t0, t1) with the
  // probabilities at pb.  Without HAS_S only mid() and the weighted latent.
  // after_s(k) runs after score MFMA k, piece(k) after weighted MFMA k + 1;
  // the scores land in s before mid().
  //
  // Score operands are fetched kD MFMAs ahead.  The weighted latent goes
  // column block by column block (st = 4 kb2 + mbl), each A operand serving
  // four MFMAs (one per head block nb); A operands alternate between two
  // registers, the four B operands of a position half sit in four.  The
  // first A operand and the B operands of half 0 are fetched in the place of
  // the last score operands.
  auto stream = [&](auto has_s, uint32_t sb, uint32_t rb, uint32_t t0, uint32_t t1, uint32_t pb, f32x16& s,
                    auto&& after_s, auto&& mid, auto&& piece) __attribute__((always_inline)) {
    constexpr bool HAS_S = decltype(has_s)::value;
    bf16x8 A[2], B[4];
    uint32_t ta0[4], ta1[4];  // transposed-read addresses of column block mbl (half 0; half 1 at +16 KiB)
    uint32_t pb1 = 0;         // probability read address of position half 1
    auto ar = [&](auto stc) __attribute__((always_inline)) -> bf16x8 {
      constexpr int st = decltype(stc)::value, mbl = st & 3, kb2 = st >> 2;
      if constexpr (kb2 == 0) {
        ta0[mbl] = xor_here<64 * mbl>(t0);
        ta1[mbl] = xor_here<64 * mbl>(t1);
      }
      s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)((LDS char*)(uintptr_t)ta0[mbl] + 16 * kCRow * kb2));
      s16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)((LDS char*)(uintptr_t)ta1[mbl] + 16 * kCRow * kb2));
      typedef __attribute__((ext_vector_type(8))) short s16x8;
      return __builtin_bit_cast(bf16x8, (s16x8)__builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // weighted-latent operands fetched before its first MFMA, in order of need
    auto pre = [&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i == 0) A[0] = ar(std::integral_constant<int, 0>{});
      else if constexpr (i <= 4) B[i - 1] = b_read(pb, i - 1, std::integral_constant<int, 0>{});
      else A[1] = ar(std::integral_constant<int, 1>{});
    };
    constexpr int kPre = 6;
    if constexpr (HAS_S) {
      bf16x8 ring[kD];
      f32x16 sacc;
      uint32_t sa[8];
      static_for<0, 8>([&](auto vc) { sa[decltype(vc)::value] = xor_here<32 * decltype(vc)::value>(sb); });
      static_for<0, kD>([&](auto ic) { ring[decltype(ic)::value] = s_read(sa, rb, ic); });
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, 36>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const bf16x8 bq = i < 32 ? q[i & 31] : qr[(i - 32) & 3];
        if constexpr (i == 0) sacc = mfma_sv0(ring[0], bq);
        else mfma_sv(sacc, ring[i % kD], bq);
        if constexpr (i + kD < 36) ring[i % kD] = s_read(sa, rb, std::integral_constant<int, i + kD>{});
        else if constexpr (i + kD - 36 < kPre) pre(std::integral_constant<int, i + kD - 36>{});
        after_s(i);
        __builtin_amdgcn_sched_barrier(0);
      });
      static_for<kD, kPre>([&](auto ic) { pre(ic); });
      // the last score MFMA's result is read by VALU instructions: cover the
      // MFMA-write -> VALU-read distance (at most 19 wait states)
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(sacc));
      s = sacc;
    } else {
      static_for<0, kPre>([&](auto ic) { pre(ic); });
    }
    mid();
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, 32>([&](auto jc) {
      constexpr int j = decltype(jc)::value, kb2 = j >> 4, mbl = (j >> 2) & 3, nb = j & 3;
      constexpr int st = 4 * kb2 + mbl;
      O[4 * mbl + nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[st & 1], B[nb], O[4 * mbl + nb], 0, 0, 0);
      // B operand (nb, 1) replaces (nb, 0) after its last use, then A operand
      // st + 2 replaces st after its last use (the B operand is needed first)
      if constexpr (j == 12) pb1 = xor_here<32>(pb);
      if constexpr (j >= 12 && j < 16) B[nb] = *(const LDS bf16x8*)((LDS char*)(uintptr_t)pb1 + 2048 * nb);
      if constexpr (nb == 3 && st + 2 < 8) A[st & 1] = ar(std::integral_constant<int, st + 2>{});
      if constexpr (j > 0) piece(j - 1);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // rescale factors of tile tt (written by the owners in its iteration)
  auto alpha_of = [&](int32_t tt) __attribute__((always_inline)) -> f32x4 { return *(const LDS f32x4*)(L + kAOff + (tt & 1) * 512 + 16 * row); };
  // rescale the accumulator by the factors of the previous tile, if any is not 1
  auto rescale = [&](const f32x4& al) __attribute__((always_inline)) {
    const bool mine = al[0] != 1.0f || al[1] != 1.0f || al[2] != 1.0f || al[3] != 1.0f;
    if (__builtin_amdgcn_ballot_w64(mine) != 0) {
#pragma unroll
      for (int b = 0; b < 16; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[b][r] = scale_acc(O[b][r], al[b & 3]);
    }
  };

  // Latent queries reach the registers through LDS, in two halves (latent
  // dims 0..255, then 256..511): a load straight into the operand layout
  // would touch 32 rows of 32 bytes per instruction, while each load here
  // moves two whole half rows.  Wave w stages its own 32 heads' half rows
  // ([head][512 bytes], chunks swizzled like the latent rows) at kQOff +
  // 16 KiB w, inside latent stages 2 and 3, which the first two tiles
  // leave free; only wave w reads them back, so no barrier is needed.
  // lanes 0..31 fetch head 32 w + 2 i, lanes 32..63 head 32 w + 2 i + 1,
  // lane chunk c the row's chunk c ^ swz(head); swz(2 i + 1) is swz(2 i)
  // with bit 2 set, so the per-lane offset is qd ^ 16 swz(2 i)
  const uint32_t qd = ((uint32_t)hi << 10) | ((16 * (lane & 31)) ^ (64 * hi));
  auto q_half = [&](int r, int32_t b) __attribute__((always_inline)) {
    const uint8_t* base = (const uint8_t*)a.q_lat + ((int64_t)b * kHeads + 32 * w) * kCRow + 512 * r;
    static_for<0, 16>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      dma16s(xor_here<16 * swz(2 * i)>(qd), base + 2 * i * kCRow, lds0 + kQOff + (32 * w + 2 * i) * 512);
    });
  };
  const uint32_t qb = lds0 + kQOff + (32 * w + row) * 512 + (bs - row * kCRow);
  auto q_take = [&](auto rc) __attribute__((always_inline)) {
    constexpr int r = decltype(rc)::value;
    uint32_t qa[8];
    static_for<0, 8>([&](auto vc) { qa[decltype(vc)::value] = xor_here<32 * decltype(vc)::value>(qb); });
    static_for<0, 16>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      q[16 * r + k] = *(const LDS bf16x8*)((LDS char*)(uintptr_t)qa[k & 7] + 256 * (k >> 3));
    });
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
    // Page ids are fetched one tile ahead of the load that needs them.  The
    // page ids of the first two tiles go out first, then the first half of
    // the latent queries (see q_half) and the rotary queries; the two tiles
    // follow as soon as their page ids are in.
    const int32_t raw_a = ld.raw(ct >> 1);                                  // tile ct
    const int32_t raw_b = ld.raw(seg > 1 ? (ct + 1) >> 1 : 0);             // tile ct + 1
    q_half(0, cb);
    {
      const __bf16* qp = (const __bf16*)a.q_rope + ((int64_t)cb * kHeads + head) * kRope + 8 * hi;
#pragma unroll
      for (int v = 0; v < 4; ++v) qr[v] = *(const bf16x8*)(qp + 16 * v);
    }
    const int32_t pg_a = ld.checked(ct >> 1, raw_a);
    const int32_t pg_b = seg > 1 ? ld.checked((ct + 1) >> 1, raw_b) : -1;
    ld.issue(ld.tile(0, 0, ct, pg_a));
    if (seg > 1) ld.issue(ld.tile(1, 1, ct + 1, pg_b));
    // the first query half has landed once at most the rotary queries and
    // the tile loads are in flight; its reads must be done before the second
    // half overwrites the area
    if (seg > 1) wait_vmcnt<4 + 2 * kDmaPerWave>();
    else wait_vmcnt<4 + kDmaPerWave>();
    q_take(std::integral_constant<int, 0>{});
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    q_half(1, cb);
    // page of tile ct + 2: loaded now, checked when its load is issued
    int32_t pg_next_p = seg > 2 ? (ct + 2) >> 1 : INT32_MAX;
    int32_t pg_next_raw = ld.raw(seg > 2 ? pg_next_p : 0);
    // validity of the tiles in flight: tile ct + j has latent stage j % 4
    // and rotary stage j % 3
    bool valid_j = pg_a >= 0, valid_j1 = pg_b >= 0;
    {
      // The weighted latent of "tile -1" reads latent stage 3 with the
      // probabilities of buffer 1: zero both (stage 3 below, once the query
      // rows staged there are read), so stale or uninitialised LDS cannot
      // turn 0 x NaN into NaN.  Ordered before the first read by the barrier
      // of iteration 0.
      LDS char* pz = L + kPOff + kPBytes + 32 * tid;
      *(LDS i32x4*)pz = i32x4{0, 0, 0, 0};
      *(LDS i32x4*)(pz + 16) = i32x4{0, 0, 0, 0};
    }
    wait_vmcnt<0>();  // queries and the first two tiles
    q_take(std::integral_constant<int, 1>{});
    // take the queries here, so the waits for them sit before the tile loop
    // (all satisfied) and not inside it
#pragma unroll
    for (int kb = 0; kb < 32; ++kb) asm volatile("" ::"v"(q[kb]));
#pragma unroll
    for (int v = 0; v < 4; ++v) asm volatile("" ::"v"(qr[v]));
    if (w >= 2) {
      // latent stage 3 held the query rows of waves 2 and 3: each zeroes its
      // own half, after its reads (one wave's LDS operations run in order)
      LDS char* z = L + 3 * kLStage + (w - 2) * (kLStage / 2) + 16 * lane;
#pragma unroll
      for (int v = 0; v < kLStage / 2 / 1024; ++v) *(LDS i32x4*)(z + 1024 * v) = i32x4{0, 0, 0, 0};
    }

#pragma unroll
    for (int b = 0; b < 16; ++b) O[b] = f32x16{};
    float m_run = -INFINITY;  // running maximum of this lane's head (log2 units)
    float l_run = 0.f;        // this lane's share of the running sum
    int rs = 0;               // rotary stage of tile j

    for (int32_t j = 0; j < seg; ++j) {
      const int32_t t = ct + j;
      // tile j landed (the loads of tile j + 1 may still be in flight)
      wait_vmcnt<kDmaPerWave>();
      __syncthreads();
      // stages (j + 2) % 4 and (j + 2) % 3 held tiles j - 2 and j - 1,
      // whose last reads were in the previous iteration; tile j + 2 is
      // loaded into them during the scores below
      const int rs2 = rs == 0 ? 2 : rs - 1;
      const int32_t pg_next = ld.checked(pg_next_p, pg_next_raw);
      const bool valid_j2 = pg_next >= 0;
      // Past the segment's end the same loads bring page 0 into the free
      // stages: every iteration issues the same instructions, with no branch
      // (the end of the segment waits for them before its stores).
      const TileLoader::Tile next_tile = ld.tile((j + 2) & 3, rs2, t + 2, pg_next);
      pg_next_p = j + 3 < seg ? (t + 3) >> 1 : INT32_MAX;
      pg_next_raw = ld.raw(j + 3 < seg ? pg_next_p : 0);
      // rescale factors of tile j - 1 (none before tile 0)
      const f32x4 al_prev = alpha_of(j + 1);
      // rows of tile j that are visible
      const int32_t nvis = valid_j ? (T - t * kTile < kTile ? T - t * kTile : kTile) : 0;
      const bool full = nvis == kTile;
      if (!full) {
        // zero the invisible latent rows (they hold page-0 or past-the-end
        // data, which a zero probability must not turn into NaN); their
        // scores are masked below, so the rotary rows may stay
        LDS char* Ct = L + (j & 3) * kLStage;
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
      float mt = -INFINITY, m_use = m_run, neg_m = 0.f, lsum = 0.f, alpha = 1.f;
      bool need = false;
      bf16x8 Pc0, Pc1;
      const uint32_t pw = lds0 + kPOff + (j & 1) * kPBytes + bp + 2048 * w;  // this lane's probability row
      auto piece = [&](int k) __attribute__((always_inline)) {
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
          // maximum exceeds it by more than 16 (log2 units): probabilities
          // stay <= 2^16, far inside the range of BF16 and of the float32
          // sums, and the accumulator (all 128 heads in every wave) is
          // rescaled rarely.
          const float m_new = max_raw(m_run, mt);
          need = m_new > m_run + 16.0f;
          m_use = need ? m_new : m_run;
          neg_m = (m_use == -INFINITY) ? 0.f : -m_use;
          asm volatile("" : "+v"(neg_m), "+v"(m_use));
        } else if (k == 4) {
          // factor that takes sums relative to m_run to m_use; every wave
          // applies it to its columns of this head before the next tile's
          // weighted latent
          alpha = need ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.0f;
          *(LDS float*)(L + kAOff + (j & 1) * 512 + 4 * head_slot(head)) = alpha;
        } else if (k >= 5 && k < 21) {
          const int r = k - 5;
          s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, neg_m));
          asm volatile("" : "+v"(s[r]));
        } else if (k >= 21 && k < 29) {
          const int r = 2 * (k - 21);
          lsum += s[r] + s[r + 1];
          if (r < 8) {
            Pc0[r] = (__bf16)s[r];
            Pc0[r + 1] = (__bf16)s[r + 1];
          } else {
            Pc1[r - 8] = (__bf16)s[r];
            Pc1[r - 7] = (__bf16)s[r + 1];
          }
          asm volatile("" : "+v"(lsum));
          if (k == 24) asm volatile("" : "+v"(Pc0));
          if (k == 28) asm volatile("" : "+v"(Pc1));
        } else if (k == 29) {
          *(LDS bf16x8*)(LDS char*)(uintptr_t)pw = Pc0;
        } else if (k == 30) {
          *(LDS bf16x8*)(LDS char*)(uintptr_t)xor_here<32>(pw) = Pc1;
        }
      };
      stream(std::true_type{}, lds0 + (j & 3) * kLStage + bs, lds0 + kROff + rs * kRStage + br,
             lds0 + ((j + 3) & 3) * kLStage + bt0, lds0 + ((j + 3) & 3) * kLStage + bt1,
             lds0 + kPOff + ((j + 1) & 1) * kPBytes + bp, s,
             [&](int k) {
               if ((k & 3) == 0 && (k >> 2) < kDmaPerWave) ld.issue_one(next_tile, k >> 2);
             },
             [&]() {
               // (through tile 0 the accumulator holds only the zero
               // weighted latent of "tile -1": nothing to rescale)
               if (j > 1) rescale(al_prev);
             },
             piece);

      m_run = m_use;
      l_run = l_run * alpha + lsum;
      rs = rs == 2 ? 0 : rs + 1;
    }
    {
      // weighted latent of the last tile, after its rescale; the barrier
      // makes every owner's probabilities and factors of that tile visible
      __syncthreads();
      const f32x4 al_last = alpha_of(seg - 1);
      f32x16 s_unused;
      stream(std::false_type{}, 0u, 0u, lds0 + ((seg + 3) & 3) * kLStage + bt0,
             lds0 + ((seg + 3) & 3) * kLStage + bt1, lds0 + kPOff + ((seg + 1) & 1) * kPBytes + bp, s_unused,
             [](int) {}, [&]() {
               if (seg > 1) rescale(al_last);
             },
             [](int) {});
    }
    done += seg;

    // ---- end of the segment: normalise and write ----
    {
      const float l_tot = l_run + wave_partner(l_run);
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
      const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
      *(LDS float*)(L + kIOff + 4 * head_slot(head)) = inv;
      // BF16 rows of all 128 heads (the final o_lat, or the partial:
      // partials of the MFMA kernels are BF16)
      const int64_t slot = worker + cb;
      __bf16* rows = DIRECT ? (__bf16*)a.o_lat + (int64_t)cb * kHeads * kLatent
                            : (__bf16*)a.part_o + slot * kHeads * kLatent;
      store_rows_split(L, kIOff, rows, O, w, [&]() {
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
