// Weight-absorbed MLA decode attention over an FP8 (E4M3) latent cache with
// one float32 scale per position, gfx950; all positions visible or an index
// list ("DeepSeek's KV Cache", section "Calculating V3.2's KV cache" for the
// cache item, Figure 10 for the selection).
//
// Same work split and arithmetic as the BF16 kernel (4 waves per work-group,
// each scoring 32 of the 128 heads: S^T[pos][head] = C . q_lat + K_rope .
// q_rope on MFMA 32x32x16, online softmax with one head per lane; weighted
// latent U^T += C^T P^T on MFMA, wave w taking latent columns 128 w .. + 127
// for all 128 heads, with the probabilities and rescale factors of every
// head passed through LDS; Figures 5 and 6, form (2)), and the same software
// pipeline: iteration j issues the scores of tile j and the weighted latent
// of tile j - 1 as one MFMA stream, with the softmax of tile j woven between
// the MFMAs.
//
// The latent rows stay FP8 in LDS and go from the load ring straight into the
// matrix cores: every MFMA operand is read as FP8 bytes -- 16-byte row reads
// for the scores (two K-blocks per read), 8-byte transposing reads
// (ds_read_b64_tr_b8: eight positions of one latent column) for the weighted
// latent, of this wave's column quarter only -- and widened to BF16 in
// registers (v_cvt_scalef32_pk_bf16_fp8 at scale 1, exact: every E4M3 value
// is a BF16 value).  There is no conversion
// pass, no conversion buffer and no barrier for one.  The position's scale is
// applied in float32: the latent part of each score is multiplied by it before
// the rotary part is added, and each probability that weights the row is
// multiplied by it before it is rounded to BF16 for the MFMA.
//
// LDS rows are 512 bytes; 16-byte chunk c of row r is stored at chunk
// c ^ fswz(r).  With the K dimension of the scores ordered so that lane
// (row, hi) reads chunk 2p + hi for K-blocks 2p and 2p + 1, and the positions
// of the weighted latent ordered as the score accumulator holds them, the row
// reads, the transposing reads and the DMA writes are all free of bank
// conflicts.
#include <type_traits>

#include "attn_common.h"

namespace mla {
namespace {

__device__ __forceinline__ constexpr int fswz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8); }

template <bool TOPK>
struct Fp8Cfg {
  static constexpr int NS = 5;                        // ring stages
  static constexpr int C_STAGE = kTile * kC8Row;      // 16 KiB FP8 latent rows
  static constexpr int R_STAGE = kTile * kRRow;       // 4 KiB BF16 rotary rows
  static constexpr int SC_STAGE = kTile * 4;          // 128 B scales
  // stages start on 256-byte boundaries: an operand address is then the
  // stage address plus a swizzled offset, formed by XOR on bits 5-7
  static constexpr int STAGE = (C_STAGE + R_STAGE + SC_STAGE + 255) / 256 * 256;
  static constexpr int MASK_OFF = NS * STAGE;         // one byte per wave and stage: visible rows
  static constexpr int QR_OFF = MASK_OFF + 32;        // rotary queries, [head][64] BF16, rows swizzled
  static constexpr int LIST_OFF = QR_OFF + kHeads * kRRow;
  static constexpr int LIST = TOPK ? 2048 : 0;        // row codes (page * 64 + slot) of a chunk
  // probabilities (times the row scales) of the tiles, 2 x [head][32] BF16
  static constexpr int P_OFF = (LIST_OFF + LIST * 4 + 255) / 256 * 256;
  static constexpr int P_BYTES = kHeads * kTile * 2;
  static constexpr int A_OFF = P_OFF + 2 * P_BYTES;   // rescale factors, 2 x [128] float
  static constexpr int I_OFF = A_OFF + 2 * kHeads * 4;  // 1 / row sum at a segment's end, [128] float
  static constexpr int LDS_BYTES = I_OFF + kHeads * 4;
  // the output rows are staged through the first kSplitStage bytes at a
  // segment's end, over the ring, the rotary queries, the list and the
  // probabilities (all free by then), never over the row sums
  static_assert(kSplitStage <= I_OFF, "output staging must stay clear of the row sums");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static constexpr int DPW = 6;                       // loads per wave and tile: 4 latent, rotary, scales
  static constexpr int CHUNK = TOPK ? LIST / kTile : 1 << 30;  // tiles between two pipeline drains
};

// Scores with the accumulator in ordinary registers (read by the softmax's
// VALU instructions; the accumulator registers hold the weighted latent).
// The A operand was just written by VALU conversions: two wait states first.
__device__ __forceinline__ f32x16 mfma_cv0(const bf16x8& a, const bf16x8& b) {
  f32x16 d;
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ void mfma_cv(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}

// Eight E4M3 codes (the bytes of lo, then hi) as their exact BF16 values.
__device__ __forceinline__ bf16x8 widen8(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Per-lane LDS offsets of the MFMA operands inside one tile.  The swizzle
// only moves address bits 5-7, so one base per operand kind serves every
// block: the block's offset is the base XOR a constant (plus a constant).
struct Fp8Offsets {
  int s_base;    // score operand pair p (K-blocks 2p, 2p + 1): (s_base ^ 32 (p % 8)) + 256 (p / 8)
  int r_off[4];  // rotary operand of K-block v (BF16 rows)
  int t_base;    // weighted-latent operand (column block mb, position half kb2):
                 // (t_base ^ 32 (mb % 8)) + 256 (mb / 8) + 16 * kC8Row * kb2

  __device__ __forceinline__ explicit Fp8Offsets(int lane) {
    const int r = lane & 31, hi = lane >> 5;
    // chunk (2p + hi) ^ fswz(r) = 2 (p ^ a) + b
    const int a = (r & 3) | ((r >> 1) & 4), b = hi ^ ((r >> 2) & 1);
    s_base = r * kC8Row + 32 * a + 16 * b;
#pragma unroll
    for (int v = 0; v < 4; ++v) r_off[v] = r * kRRow + 16 * ((2 * v + hi) ^ swz_r(r));
    // Transposing reads: in each group of 16 lanes, lane pair i names the row
    // that becomes element i of every lane's operand, and lane 2 i + e its
    // 8-byte half e of a 16-byte column group.  Element i of the operand of
    // lane (column, hi) must be position 8 (i / 4) + 4 hi + i % 4 (+ 16 kb2),
    // the position the score accumulator holds in register i (+ 8 kb2).
    const int g = lane >> 4, j = lane & 15, i = j >> 1, c = g & 1, h = g >> 1;
    const int prow = 8 * (i >> 2) + 4 * h + (i & 3);  // fswz(prow) = 2 i + h
    t_base = prow * kC8Row + 32 * i + 16 * (c ^ h) + 8 * (j & 1);
  }
};

template <bool TOPK>
struct Fp8Loader {
  using C = Fp8Cfg<TOPK>;
  const uint8_t* pool;
  int64_t page_bytes, rope_off, scale_off, num_pages;
  const int32_t* bt;  // block-table row of the current request
  int32_t bt_stride;
  uint32_t lds0;
  int w, lane;
  // Latent loads: this lane's 16 bytes of row 8 w + 2 q + hi go to LDS chunk
  // lane % 32 and come from chunk (lane % 32) ^ fswz(row).  Across q the
  // source chunk changes by a constant XOR (kChunkX[q]) and the row by 2 q.
  uint32_t chk_c;   // source chunk offset for q = 0
  uint32_t chk_r;   // rotary rows: source chunk offset of this lane's 16 bytes
  static constexpr uint32_t kChunkX[4] = {0, 64, 16, 80};

  __device__ __forceinline__ void init() {
    const int hi = lane >> 5;
    chk_c = 16 * ((lane & 31) ^ fswz(8 * w + hi));
    chk_r = 16 * ((lane & 7) ^ swz_r(8 * w + (lane >> 3)));
  }
  __device__ __forceinline__ uint32_t voff_c(int q) const {
    return (uint32_t)(8 * w + (lane >> 5)) * kC8Row + (chk_c ^ kChunkX[q]) + 2 * q * kC8Row;
  }
  __device__ __forceinline__ uint32_t voff_r() const { return (uint32_t)(8 * w + (lane >> 3)) * kRRow + chk_r; }
  __device__ __forceinline__ uint32_t voff_s() const { return (uint32_t)(8 * w + (lane & 7)) * 4; }

  __device__ __forceinline__ int32_t raw(int32_t p) const { return sload(bt + (p < bt_stride ? p : bt_stride - 1)); }
  __device__ __forceinline__ int32_t checked(int32_t p, int32_t pg) const {
    return (p < bt_stride && pg >= 0 && pg < num_pages) ? pg : -1;
  }

  // ---- dense: tile t of page `page` (-1: invalid, loaded from page 0 and masked) ----
  struct Dense {
    const uint8_t *c, *r, *s;
    uint32_t sb;
    uint32_t bits;  // visible rows of this wave
  };
  __device__ __forceinline__ Dense dense(int st, int32_t t, int32_t page, int32_t T) const {
    const int64_t pg = page >= 0 ? page : 0;
    const uint8_t* base = pool + pg * page_bytes;
    const int half = t & 1;
    uint32_t bits = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (page >= 0 && t * kTile + 8 * w + k < T) bits |= 1u << k;
    return Dense{base + half * kTile * kC8Row, base + rope_off + half * kTile * kRRow, base + scale_off + half * kTile * 4,
                 lds0 + st * C::STAGE, bits};
  }
  __device__ __forceinline__ void dense_one(const Dense& d, int k) const {
    if (k < 4) dma16s_nt(voff_c(k), d.c, d.sb + (8 * w + 2 * k) * kC8Row);
    else if (k == 4) dma16s_nt(voff_r(), d.r, d.sb + C::C_STAGE + 8 * w * kRRow);
    else if (lane < 8) dma4s(voff_s(), d.s, d.sb + C::C_STAGE + C::R_STAGE + 32 * w);
  }

  // ---- gathered: the rows of tile t are listed as codes page * 64 + slot (-1: masked) ----
  struct Gather {
    int32_t code_c[4], code_r, code_s;
    uint32_t sb;
  };
  // ln: the lane id (passed in, so a caller can hand over a fresh copy)
  __device__ __forceinline__ Gather gather(int st, const LDS int32_t* lc, int ln) const {
    // lc: the 32 codes of the tile; this wave loads rows 8 w .. 8 w + 7
    const int hi = ln >> 5;
    Gather g;
#pragma unroll
    for (int q = 0; q < 4; ++q) g.code_c[q] = lc[8 * w + 2 * q + hi];
    g.code_r = lc[8 * w + (ln >> 3)];
    g.code_s = lc[8 * w + (ln & 7)];
    g.sb = lds0 + st * C::STAGE;
    return g;
  }
  __device__ __forceinline__ const uint8_t* row_base(int32_t code) const {
    const int32_t c = code >= 0 ? code : 0;
    return pool + (int64_t)(c >> 6) * page_bytes;
  }
  __device__ __forceinline__ int slot_of(int32_t code) const { return code >= 0 ? (code & 63) : 0; }
  __device__ __forceinline__ void gather_one(const Gather& g, int k) const {
    if (k < 4) {
      dma16_nt(row_base(g.code_c[k]) + slot_of(g.code_c[k]) * kC8Row + (chk_c ^ kChunkX[k]), g.sb + (8 * w + 2 * k) * kC8Row);
    } else if (k == 4) {
      dma16_nt(row_base(g.code_r) + rope_off + slot_of(g.code_r) * kRRow + chk_r, g.sb + C::C_STAGE + 8 * w * kRRow);
    } else if (lane < 8) {
      dma4(row_base(g.code_s) + scale_off + slot_of(g.code_s) * 4, g.sb + C::C_STAGE + C::R_STAGE + 32 * w);
    }
  }
  __device__ __forceinline__ uint32_t gather_bits(const Gather& g) const {
    return (uint32_t)__builtin_amdgcn_ballot_w64(g.code_s >= 0) & 0xFFu;
  }
};

template <bool TOPK, bool DIRECT>
__global__ __launch_bounds__(kThreads, 1) void decode_fp8_kernel(DecodeArgs a) {
  using C = Fp8Cfg<TOPK>;
  constexpr int NS = C::NS;
  __shared__ __attribute__((aligned(256))) char smem[C::LDS_BYTES];
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
  const int32_t topk = TOPK ? a.topk : 0;
  const int32_t lead = lead_of(topk);
  auto ntiles = [&](int32_t b) -> int32_t {
    if (TOPK) return tiles_of(a.topk);
    const int32_t T = sload(a.seq_lens + b);
    return T > 0 ? tiles_of(T) : 0;
  };
  int32_t b0, v0;
  int64_t n;
  const int64_t worker = DIRECT ? (int64_t)blockIdx.x : xcd_worker(blockIdx.x, gridDim.x);
  if (DIRECT) {
    b0 = blockIdx.x;
    v0 = lead;
    n = ntiles(b0);
  } else {
    const WorkerSpan ws = locate_worker(a.seq_lens, a.batch, topk, worker, a.num_workers);
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

  const Fp8Offsets off(lane);
  // probabilities of head 32 nb + row, position chunk 2 kb2 + hi:
  // (bp ^ 32 kb2) + 2048 nb inside a probability buffer
  const int ps = pswz(row);
  const uint32_t bp = 64 * row + 16 * (hi ^ (ps & 1)) + 32 * (ps >> 1);
  // transposing reads of this wave's column block 4 w + mbl: (tq ^ 32 mbl)
  // + 16 rows * kb2 (off.t_base names block mb as t_base ^ 32 (mb % 8) plus
  // 256 (mb / 8); t_base has no bit 8)
  const uint32_t tq = ((uint32_t)off.t_base ^ (128u * (uint32_t)(w & 1))) | (256u * (uint32_t)(w >> 1));
  Fp8Loader<TOPK> ld;
  ld.pool = a.pool;
  ld.page_bytes = a.page_bytes;
  ld.rope_off = a.rope_off;
  ld.scale_off = a.scale_off;
  ld.num_pages = a.num_pages;
  ld.bt_stride = a.bt_stride;
  ld.lds0 = (uint32_t)(uintptr_t)smem;
  ld.w = w;
  ld.lane = lane;
  ld.init();
  LDS int32_t* list = (LDS int32_t*)(L + C::LIST_OFF);

  f32x16 O[16];
  // Latent query blocks: K-block 2 p + e of lane (head, hi) holds latent
  // columns 32 p + 16 hi + 8 e .. + 7, matching the FP8 row reads.
  bf16x8 q[32];

  // rotary query block v of this lane's head (rows swizzled as the rotary keys)
  auto rq_operand = [&](int v) -> bf16x8 {
    return *(const LDS bf16x8*)(L + C::QR_OFF + head * kRRow + 16 * ((2 * v + hi) ^ swz_r(head)));
  };
  // this lane's 16 positions' scales (rows 8 (r / 4) + 4 hi + r % 4); those
  // of masked rows were zeroed in LDS
  auto row_scales = [&](int st, float (&rsc)[16]) __attribute__((always_inline)) {
    const LDS float* scl = (const LDS float*)(L + st * C::STAGE + C::C_STAGE + C::R_STAGE);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x4 v = *(const LDS f32x4*)(scl + 8 * k + 4 * hi);
#pragma unroll
      for (int e = 0; e < 4; ++e) rsc[4 * k + e] = v[e];
    }
  };

  // ---- the MFMA stream of one iteration ----
  // HAS_S: the 32 latent score MFMAs of the tile in stage sst, then the 32
  // weighted-latent MFMAs of the tile in stage pst with the probabilities at
  // pb, with the rest of the tile-sst work between them: after weighted MFMA
  // 2 the latent scores are multiplied by the row scales, after MFMAs 3, 4, 6
  // and 7 the 4 rotary score MFMAs continue the same accumulator chain, and
  // from MFMA 10 on the softmax runs (piece(s) after weighted MFMA 10 + s).
  // Without HAS_S only the weighted latent.  after_s(k) runs after latent
  // score MFMA k, mid() before the first weighted MFMA.
  //
  // The weighted latent goes column block by column block (st = 4 kb2 +
  // mbl, block 4 w + mbl of this wave's quarter), each A operand serving four
  // MFMAs (one per head block nb): its raw FP8 read goes out two blocks
  // ahead and is widened one block ahead, in two alternating registers; the
  // four B operands of a position half sit in four.
  auto stream = [&](auto has_s, int sst, int pst, uint32_t pb, f32x16& S, float (&rsc)[16], auto&& after_s,
                    auto&& mid, auto&& piece) __attribute__((always_inline)) {
    constexpr bool HAS_S = decltype(has_s)::value;
    constexpr int DS = 3;  // score operand pairs in flight
    const uint32_t sb = ld.lds0 + sst * C::STAGE + off.s_base;
    const uint32_t pq = ld.lds0 + pst * C::STAGE + tq;
    auto pair_raw = [&](auto pc) -> i32x4 {
      constexpr int p = decltype(pc)::value;
      return *(const LDS i32x4*)((LDS char*)(uintptr_t)xor_here<32 * (p & 7)>(sb) + 256 * (p >> 3));
    };
    auto a_raw = [&](auto stc) __attribute__((always_inline)) -> i32x2 {
      constexpr int st = decltype(stc)::value, mbl = st & 3, kb2 = st >> 2;
      return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (LDS i32x2*)((LDS char*)(uintptr_t)xor_here<32 * mbl>(pq) + 16 * kC8Row * kb2));
    };
    auto b_read = [&](uint32_t pbk, int nb) __attribute__((always_inline)) -> bf16x8 {
      return *(const LDS bf16x8*)((LDS char*)(uintptr_t)pbk + 2048 * nb);
    };
    i32x2 araw[2];
    bf16x8 A[2], B[4];
    // weighted-latent operands read before its first MFMA: the raw A
    // operands of blocks 0 and 1, the B operands of position half 0
    auto pre = [&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i < 2) araw[i] = a_raw(std::integral_constant<int, i>{});
      else B[i - 2] = b_read(pb, i - 2);
    };
    constexpr int kPre = 6;
    bf16x8 ro[2], rq[2];
    if constexpr (HAS_S) {
      i32x4 sring[DS];
      static_for<0, DS>([&](auto pc) { sring[decltype(pc)::value] = pair_raw(pc); });
      __builtin_amdgcn_sched_barrier(0);
      // each operand is widened one MFMA ahead of its use, so the conversions
      // run while the previous MFMA executes
      bf16x8 cur = widen8((uint32_t)sring[0][0], (uint32_t)sring[0][1]);
      static_for<0, 16>([&](auto pc) {
        constexpr int p = decltype(pc)::value;
        if (p == 0) S = mfma_cv0(cur, q[0]);
        else mfma_cv(S, cur, q[2 * p]);
        cur = widen8((uint32_t)sring[p % DS][2], (uint32_t)sring[p % DS][3]);
        after_s(2 * p);
        __builtin_amdgcn_sched_barrier(0);
        mfma_cv(S, cur, q[2 * p + 1]);
        if constexpr (p + DS < 16) {
          sring[p % DS] = pair_raw(std::integral_constant<int, p + DS>{});
        } else {
          // the first weighted-latent operands, spread over the last DS pairs
          constexpr int i = p + DS - 16;
          static_for<i * kPre / DS, (i + 1) * kPre / DS>([&](auto xc) { pre(xc); });
        }
        if constexpr (p + 1 < 16) cur = widen8((uint32_t)sring[(p + 1) % DS][0], (uint32_t)sring[(p + 1) % DS][1]);
        after_s(2 * p + 1);
        __builtin_amdgcn_sched_barrier(0);
      });
    } else {
      static_for<0, kPre>([&](auto ic) { pre(ic); });
      __builtin_amdgcn_sched_barrier(0);
    }
    A[0] = widen8((uint32_t)araw[0][0], (uint32_t)araw[0][1]);
    mid();
    __builtin_amdgcn_sched_barrier(0);
    uint32_t pb1 = 0;  // probability read address of position half 1
    static_for<0, 32>([&](auto jc) {
      constexpr int jj = decltype(jc)::value, kb2 = jj >> 4, mbl = (jj >> 2) & 3, nb = jj & 3;
      constexpr int st = 4 * kb2 + mbl;
      O[4 * mbl + nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[st & 1], B[nb], O[4 * mbl + nb], 0, 0, 0);
      // block st + 2's raw read replaces st's (widened before this block);
      // block st + 1 is widened into the register block st - 1 used
      if constexpr (nb == 0 && st + 2 < 8) araw[st & 1] = a_raw(std::integral_constant<int, st + 2>{});
      if constexpr (nb == 1 && st + 1 < 8)
        A[(st + 1) & 1] = widen8((uint32_t)araw[(st + 1) & 1][0], (uint32_t)araw[(st + 1) & 1][1]);
      // B operand (nb, 1) replaces (nb, 0) after its last use
      if constexpr (jj == 12) pb1 = xor_here<32>(pb);
      if constexpr (jj >= 12 && jj < 16) B[nb] = b_read(pb1, nb);
      if constexpr (HAS_S) {
        // rotary operands: K-blocks 0, 1 read after weighted MFMA 0, K-blocks
        // 2, 3 after the rotary MFMAs that free their registers
        auto rot_read = [&](int v) {
          ro[v & 1] = *(const LDS bf16x8*)(L + sst * C::STAGE + C::C_STAGE + off.r_off[v]);
          rq[v & 1] = rq_operand(v);
        };
        if constexpr (jj == 0) {
          rot_read(0);
          rot_read(1);
          // the row scales for the latent scores (read here, not earlier, so
          // that they hold no registers while the score operands do)
          row_scales(sst, rsc);
        }
        if constexpr (jj == 1) {
          // two weighted MFMAs have run since the last latent score MFMA: its
          // result is readable (19 wait states at most; the nops make it certain)
          asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(S));
        }
        if constexpr (jj == 2) {
#pragma unroll
          for (int r = 0; r < 16; ++r) S[r] *= rsc[r];  // the latent part times the row's scale
        }
        if constexpr (jj == 3 || jj == 4 || jj == 6 || jj == 7) {
          constexpr int v = jj < 5 ? jj - 3 : jj - 4;
          mfma_cv(S, ro[v & 1], rq[v & 1]);  // + K_rope . q_rope
          if constexpr (v < 2) rot_read(v + 2);
        }
        if constexpr (jj == 9) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(S));
        if constexpr (jj >= 10) piece(jj - 10);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // rescale factors of tile tt of the chunk (written by the owners in its iteration)
  auto alpha_of = [&](int32_t tt) __attribute__((always_inline)) -> f32x4 {
    return *(const LDS f32x4*)(L + C::A_OFF + (tt & 1) * 512 + 16 * row);
  };
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

  int32_t cb = b0;
  int64_t cv = v0;   // offset of the next unit inside request cb's span
  int64_t done = 0;  // units consumed
  while (done < n) {
    // ---- one segment: tiles [ct, ct + seg) of request cb ----
    if (cb >= a.batch) break;  // unreachable when the tile accounting is consistent
    if (cv < lead) {  // the lead of request cb carries no work
      const int64_t skip = lead - cv < n - done ? lead - cv : n - done;
      done += skip;
      cv += skip;
      if (done >= n) break;
    }
    const int32_t ct = (int32_t)(cv - lead);
    const int32_t nt_cb = ntiles(cb);
    const int64_t left = nt_cb - ct;
    const int32_t seg = (int32_t)(left < n - done ? left : n - done);
    if (seg <= 0) break;
    const int32_t T = sload(a.seq_lens + cb);
    ld.bt = a.block_table + (int64_t)cb * a.bt_stride;

#pragma unroll
    for (int mb = 0; mb < 16; ++mb) O[mb] = f32x16{};
    float m_run = -INFINITY;  // running maximum of this lane's head (log2 units)
    float l_run = 0.f;        // this lane's share of the running sum

    // Stages are free once every wave has finished the previous segment;
    // earlier stores and loads count on vmcnt too, so drain first.  Then the
    // rotary queries (straight into LDS) and the index entries go out; the
    // latent queries follow once the row list is built.
    wait_vmcnt<0>();
    __syncthreads();
    {
      const __bf16* qp = (const __bf16*)a.q_rope + (int64_t)cb * kHeads * kRope;
#pragma unroll
      for (int pass = 0; pass < 4; ++pass) {
        const int hh = 32 * w + 8 * pass + (lane >> 3);
        const int c = (lane & 7) ^ swz_r(hh);
        dma16(qp + hh * kRope + 8 * c, ld.lds0 + C::QR_OFF + (32 * w + 8 * pass) * kRRow);
      }
    }

    for (int32_t tc0 = ct; tc0 < ct + seg; tc0 += C::CHUNK) {
      const int32_t clen = min(C::CHUNK, ct + seg - tc0);
      if (tc0 != ct) {  // a later chunk: the stages are free once every wave is done
        wait_vmcnt<0>();
        __syncthreads();
      }
      if (TOPK) fill_index_codes(a, cb, tc0, clen, T, list, tid);
      {
        // The weighted latent of "tile -1" reads the last stage with the
        // probabilities of buffer 1: zero both, so stale LDS cannot turn
        // 0 x NaN into NaN.
        LDS char* dst = L + (NS - 1) * C::STAGE + (tid >> 3) * kC8Row + 64 * (tid & 7);
#pragma unroll
        for (int v = 0; v < 4; ++v) *(LDS i32x4*)(dst + 16 * v) = i32x4{0, 0, 0, 0};
        LDS char* pz = L + C::P_OFF + C::P_BYTES + 32 * tid;
        *(LDS i32x4*)pz = i32x4{0, 0, 0, 0};
        *(LDS i32x4*)(pz + 16) = i32x4{0, 0, 0, 0};
      }
      __syncthreads();  // the row list and the zeroed stage are complete

      // pipeline fill: tiles tc0 .. tc0 + NS - 3.  The gathers take their
      // row-code addresses from a fresh copy of the lane id: a kept copy was
      // spilled and reloaded, and the compiler's wait for the reload, inside
      // this loop, waited (loads return in order) for the tiles issued in the
      // iterations before as well.
      const int32_t pro = clen < NS - 2 ? clen : NS - 2;
      int32_t pg_next_p = 0, pg_next_raw = 0;
      if (TOPK) {
        for (int32_t k = 0; k < pro; ++k) {
          const auto g = ld.gather(k, list + k * kTile, opaque(lane));
#pragma unroll
          for (int x = 0; x < C::DPW; ++x) ld.gather_one(g, x);
          const uint32_t bits = ld.gather_bits(g);
          if (lane == 0) L[C::MASK_OFF + 4 * k + w] = (char)bits;
        }
      } else {
        for (int32_t k = 0; k < pro; ++k) {
          const int32_t t = tc0 + k;
          const int32_t pg = ld.checked(t >> 1, ld.raw(t >> 1));
          const auto d = ld.dense(k, t, pg, T);
#pragma unroll
          for (int x = 0; x < C::DPW; ++x) ld.dense_one(d, x);
          if (lane == 0) L[C::MASK_OFF + 4 * k + w] = (char)d.bits;
        }
        pg_next_p = (tc0 + NS - 2) >> 1;
        pg_next_raw = ld.raw(NS - 2 < clen ? pg_next_p : 0);
      }
      if (tc0 == ct) {
        // the latent queries, behind the first tiles: the tiles do not wait
        // for them, and their latency overlaps that of the tiles
        const __bf16* ql = (const __bf16*)a.q_lat + ((int64_t)cb * kHeads + head) * kLatent + 16 * hi;
#pragma unroll
        for (int p = 0; p < 16; ++p) {
          q[2 * p] = *(const bf16x8*)(ql + 32 * p);
          q[2 * p + 1] = *(const bf16x8*)(ql + 32 * p + 8);
        }
      }
      // The queries and the first tiles: waited for here, every chunk, and
      // taken, so that no wait for them is left inside the tile loop.
      wait_vmcnt<0>();
#pragma unroll
      for (int kb = 0; kb < 32; ++kb) asm volatile("" ::"v"(q[kb]));

      for (int32_t j = 0; j < clen; ++j) {
        const int32_t t = tc0 + j;
        const int st = j % NS;
        // tile j landed: at most min(NS - 3, clen - 1 - j) newer tiles in flight
        const int32_t ahead = clen - 1 - j < NS - 3 ? clen - 1 - j : NS - 3;
        if (ahead >= 3) wait_vmcnt<C::DPW * 3>();
        else if (ahead == 2) wait_vmcnt<C::DPW * 2>();
        else if (ahead == 1) wait_vmcnt<C::DPW>();
        else wait_vmcnt<0>();
        __syncthreads();
        const uint32_t mask = __builtin_amdgcn_readfirstlane(*(const LDS uint32_t*)(L + C::MASK_OFF + 4 * st));
        if (mask != 0xFFFFFFFFu) {
          // zero the latent rows and the scales of masked positions (their
          // probability is 0, and the bytes may be anything)
          LDS char* Ct = L + st * C::STAGE;
          const int r = tid >> 3, qq = tid & 7;
          if (!((mask >> r) & 1)) {
            LDS char* dst = Ct + r * kC8Row + 64 * qq;
#pragma unroll
            for (int v = 0; v < 4; ++v) *(LDS i32x4*)(dst + 16 * v) = i32x4{0, 0, 0, 0};
            if (qq == 0) *(LDS float*)(Ct + C::C_STAGE + C::R_STAGE + 4 * r) = 0.f;
          }
          __syncthreads();
        }
        // tile j + NS - 2 goes into the stage of tile j - 2 (consumed)
        const bool has_next = j + NS - 2 < clen;
        const int nst = (j + NS - 2) % NS;
        typename Fp8Loader<TOPK>::Gather gnext;
        typename Fp8Loader<TOPK>::Dense dnext;
        if (TOPK) {
          gnext = ld.gather(nst, list + (has_next ? j + NS - 2 : 0) * kTile, lane);
        } else {
          const int32_t pg = ld.checked(pg_next_p, pg_next_raw);
          dnext = ld.dense(nst, t + NS - 2, pg, T);
          pg_next_p = (t + NS - 1) >> 1;
          pg_next_raw = ld.raw(j + NS - 1 < clen ? pg_next_p : 0);
        }

        // ---- softmax of tile j, in pieces, inside the weighted latent of tile j - 1 ----
        f32x16 S;
        float rsc[16];
        float mt = -INFINITY, m_use = m_run, neg_m = 0.f, lsum = 0.f, alpha = 1.f;
        bool need = false;
        bf16x8 Pc0, Pc1;
        // this lane's probability row of tile j (kb2 = 0 at pw, 1 at pw ^ 32)
        const uint32_t pw = ld.lds0 + C::P_OFF + (j & 1) * C::P_BYTES + bp + 2048 * w;
        // rescale factors of tile j - 1 (none before the chunk's first tile),
        // read near the end of the scores so that they hold registers briefly
        f32x4 al_prev;
        auto after_s = [&](int k) {
          if (k == 28) al_prev = alpha_of(j + 1);
          if (has_next && (k & 3) == 0 && (k >> 2) < C::DPW) {
            if (TOPK) ld.gather_one(gnext, k >> 2);
            else ld.dense_one(dnext, k >> 2);
          }
        };
        auto piece = [&](int k) {
          // Each step ends with an empty asm that takes its result: code motion
          // cannot then sink the VALU work past the MFMAs that hide it.
          if (k == 0 || k == 1) {
            // masked rows -inf (only in tiles that have any); running maximum
            // over the other 8
            if (mask != 0xFFFFFFFFu) {
              const uint32_t mlane = mask >> (4 * hi);
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const int r = 8 * k + e;
                S[r] = ((mlane >> (8 * (r >> 2) + (r & 3))) & 1u) ? S[r] : -INFINITY;
              }
            }
            const float m8 = max3_raw(max3_raw(S[8 * k], S[8 * k + 1], S[8 * k + 2]),
                                      max3_raw(S[8 * k + 3], S[8 * k + 4], S[8 * k + 5]), max_raw(S[8 * k + 6], S[8 * k + 7]));
            mt = k == 0 ? m8 : max_raw(mt, m8);
            asm volatile("" : "+v"(mt));
          } else if (k == 2) {
            mt = max_raw(mt, wave_partner(mt)) * scale_log2;
            asm volatile("" : "+v"(mt));
          } else if (k == 3) {
            // Lazy rescale: keep the reference maximum unless the tile's
            // maximum exceeds it by more than 16 (log2 units): probabilities
            // stay <= 2^16 (times a row scale), far inside the range of BF16
            // and of the float32 sums.
            const float m_new = max_raw(m_run, mt);
            need = m_new > m_run + 16.0f;
            m_use = need ? m_new : m_run;
            neg_m = (m_use == -INFINITY) ? 0.f : -m_use;
            asm volatile("" : "+v"(neg_m), "+v"(m_use));
          } else if (k >= 4 && k < 12) {
            const int r = 2 * (k - 4);
            S[r] = __builtin_amdgcn_exp2f(fmaf(S[r], scale_log2, neg_m));
            S[r + 1] = __builtin_amdgcn_exp2f(fmaf(S[r + 1], scale_log2, neg_m));
            asm volatile("" : "+v"(S[r]), "+v"(S[r + 1]));
            if (k == 8) {
              // the scales again, for the probability operands (read anew so
              // that they hold no registers in between)
              asm volatile("" ::: "memory");
              row_scales(st, rsc);
            }
          } else if (k >= 12 && k < 20) {
            // the weighted latent sums p times the dequantised row: the row's
            // scale goes into the probability operand
            const int r = 2 * (k - 12);
            lsum += S[r] + S[r + 1];
            const __bf16 p0 = (__bf16)(S[r] * rsc[r]), p1 = (__bf16)(S[r + 1] * rsc[r + 1]);
            if (r < 8) {
              Pc0[r] = p0;
              Pc0[r + 1] = p1;
            } else {
              Pc1[r - 8] = p0;
              Pc1[r - 7] = p1;
            }
            asm volatile("" : "+v"(lsum));
            if (k == 15) asm volatile("" : "+v"(Pc0));
            if (k == 19) asm volatile("" : "+v"(Pc1));
          } else if (k == 20) {
            // factor that takes sums relative to m_run to m_use; every wave
            // applies it to its columns of this head before the tile's
            // weighted latent.  A head whose maximum is still -inf has only
            // zeros there (all its probabilities so far were 0): factor 1, so
            // the first tile of a chunk costs no accumulator pass.
            alpha = (need && m_run != -INFINITY) ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.0f;
            *(LDS float*)(L + C::A_OFF + (j & 1) * 512 + 4 * head_slot(head)) = alpha;
            *(LDS bf16x8*)(LDS char*)(uintptr_t)pw = Pc0;
          } else if (k == 21) {
            *(LDS bf16x8*)(LDS char*)(uintptr_t)xor_here<32>(pw) = Pc1;
          }
        };
        stream(std::true_type{}, st, (j + NS - 1) % NS, ld.lds0 + C::P_OFF + ((j + 1) & 1) * C::P_BYTES + bp, S, rsc,
               after_s,
               [&]() {
                 if (j > 0) rescale(al_prev);
               },
               piece);
        if (TOPK && has_next) {
          const uint32_t bits = ld.gather_bits(gnext);
          if (lane == 0) L[C::MASK_OFF + 4 * nst + w] = (char)bits;
        } else if (!TOPK && has_next) {
          if (lane == 0) L[C::MASK_OFF + 4 * nst + w] = (char)dnext.bits;
        }

        m_run = m_use;
        l_run = l_run * alpha + lsum;
      }
      {
        // weighted latent of the chunk's last tile, after its rescale; the
        // barrier makes every owner's probabilities and factors visible
        __syncthreads();
        const f32x4 al_last = alpha_of(clen - 1);
        f32x16 S_unused;
        float rsc_unused[16];
        stream(std::false_type{}, 0, (clen + NS - 1) % NS, ld.lds0 + C::P_OFF + ((clen + 1) & 1) * C::P_BYTES + bp,
               S_unused, rsc_unused, [](int) {}, [&]() { rescale(al_last); }, [](int) {});
      }
    }
    done += seg;

    // ---- end of the segment: normalise and write ----
    {
      const float l_tot = l_run + wave_partner(l_run);
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
      const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
      const int64_t slot = worker + cb;
      __bf16* rows = DIRECT ? (__bf16*)a.o_lat + (int64_t)cb * kHeads * kLatent
                            : (__bf16*)a.part_o + slot * kHeads * kLatent;
      *(LDS float*)(L + C::I_OFF + 4 * head_slot(head)) = inv;
      store_rows_split(L, C::I_OFF, rows, O, w, [&]() {
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
  // Only stores can be in flight here (every tile load was waited for).
}

}  // namespace

hipError_t launch_decode_fp8(const DecodeArgs& a, hipStream_t s) {
  const bool topk = a.topk_idx != nullptr;
  const bool direct = a.num_workers == 0;
  const dim3 grid(direct ? a.batch : a.num_workers);
  const dim3 block(kThreads);
  if (topk) {
    if (direct) hipLaunchKernelGGL((decode_fp8_kernel<true, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((decode_fp8_kernel<true, false>), grid, block, 0, s, a);
  } else {
    if (direct) hipLaunchKernelGGL((decode_fp8_kernel<false, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((decode_fp8_kernel<false, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace mla
