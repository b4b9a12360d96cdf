// Device helpers shared by the attention kernels (gfx950).  Included by
// kernel translation units only.
#pragma once

#include <type_traits>

#include "mla_internal.h"
#include "tile_space.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) short s16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
#define LDS __attribute__((address_space(3)))

constexpr int kThreads = 256;

// f(integral_constant<int, i>) for i = B .. E - 1, unrolled at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}
constexpr int kCRow = kLatent * 2;  // bytes of one BF16 latent row (1024)
constexpr int kRRow = kRope * 2;    // bytes of one BF16 rotary row (128)
constexpr int kC8Row = kLatent;     // bytes of one FP8 latent row (512)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// LDS row swizzles (16-byte chunks).  Chunk c of latent row r is stored at
// chunk c ^ swz(r), of rotary row r at c ^ swz_r(r).  Chosen so that the three
// operand read patterns -- 16-byte row reads for the scores (16 consecutive
// rows per access phase), 8-byte transposing reads (4 rows x 64 bytes) and
// the rotary row reads -- touch distinct banks on a 64-bank LDS and on a
// 32-bank one.
__device__ __forceinline__ constexpr int swz(int r) {
  r &= 15;
  return (((r & 3) << 2) | ((r >> 2) & 3)) ^ (r & 2);
}
__device__ __forceinline__ constexpr int swz_r(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

// HBM -> LDS without registers: lane l's bytes land at lds_addr + size * l.
// lds_addr must be wave-uniform (it goes to M0).
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_addr) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}
// The same with a 64-bit scalar base and a per-lane 32-bit offset.
__device__ __forceinline__ void dma16s(uint32_t voff, const void* sbase, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
}
// Cache-stream forms: every line of the paged cache is read once per launch,
// so these loads are marked non-temporal (nt) and leave the lines that are
// reused (queries, block tables, index lists) in L2.
__device__ __forceinline__ void dma16_nt(const void* g, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}
__device__ __forceinline__ void dma16s_nt(uint32_t voff, const void* sbase, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
}
__device__ __forceinline__ void dma4s(uint32_t voff, const void* sbase, uint32_t lds_addr) {
  asm volatile("global_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x0F70);
}

// a ^ K (an LDS address and a swizzle constant), computed where it is used:
// the compiler can then neither keep one register per K alive across a tile
// loop nor merge two uses into one long-lived value
template <int K>
__device__ __forceinline__ uint32_t xor_here(uint32_t a) {
  if constexpr (K == 0) {
    return a;
  } else {
    uint32_t r;
    asm volatile("v_xor_b32 %0, %1, %2" : "=v"(r) : "i"(K), "v"(a));
    return r;
  }
}

// Maximum of two or three floats in one instruction.  fmaxf first quiets
// each input (one more instruction per operand); scores are finite or -inf,
// so nothing needs quieting.
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// A copy of v that the compiler cannot see through: what is derived from it
// is computed anew where it is used, not kept (or spilled and reloaded) from
// an earlier computation.
__device__ __forceinline__ int opaque(int v) {
  int r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
  return r;
}

__device__ __forceinline__ float wave_partner(float v) {
  // value held by lane (l ^ 32)
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((__lane_id() < 32) ? r[1] : r[0]);
}

// Normalised accumulator (times inv) of a wave's 32 heads (w: the wave) as
// BF16 rows [32][512] at dst, staged through LDS so that every global store
// writes one contiguous 1 KiB row instead of 32-byte pieces of 32 rows.  The
// staging area is the first 4 x 32 rows of 1,040 bytes of the work-group's
// LDS (the tile ring): every tile load must have landed and every wave must
// be done reading the ring, which the barrier here provides; the caller's
// next use of the ring synchronises again.
// before_flush(): as in store_rows_split, between the staging and the global
// stores.
template <typename F>
__device__ __forceinline__ void store_rows_staged(LDS char* L, __bf16* dst, const f32x16 (&O)[16], float inv, int w,
                                                  F&& before_flush) {
  wait_vmcnt<0>();
  __syncthreads();
  const int lane = __lane_id();
  const int hi = lane >> 5, row = lane & 31;
  constexpr int kPitch = kCRow + 16;  // padded rows: the row-wise writes spread over the banks
  LDS char* mine = L + w * 32 * kPitch;
  LDS char* rowL = mine + row * kPitch;
  // lane (row, hi) holds columns 32 mb + 8 g + 4 hi + e; the two lanes of a
  // row swap half of each group pair so each writes 16 contiguous bytes
#pragma unroll
  for (int mb = 0; mb < 16; ++mb)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int g0 = 2 * k, g1 = 2 * k + 1;
      uint32_t keep[2], send[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const bf16x2 k0 = {(__bf16)(O[mb][4 * g0 + 2 * e] * inv), (__bf16)(O[mb][4 * g0 + 2 * e + 1] * inv)};
        const bf16x2 k1 = {(__bf16)(O[mb][4 * g1 + 2 * e] * inv), (__bf16)(O[mb][4 * g1 + 2 * e + 1] * inv)};
        const uint32_t u0 = __builtin_bit_cast(uint32_t, k0), u1 = __builtin_bit_cast(uint32_t, k1);
        keep[e] = hi ? u1 : u0;
        send[e] = hi ? u0 : u1;
      }
      uint32_t recv[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) recv[e] = __float_as_uint(wave_partner(__uint_as_float(send[e])));
      const i32x4 v = hi ? i32x4{(int)recv[0], (int)recv[1], (int)keep[0], (int)keep[1]}
                         : i32x4{(int)keep[0], (int)keep[1], (int)recv[0], (int)recv[1]};
      *(LDS i32x4*)(rowL + 2 * (32 * mb + 8 * (hi ? g1 : g0))) = v;
    }
  // each wave reads back only its own rows: no barrier needed
  before_flush();
#pragma unroll
  for (int r = 0; r < 32; ++r)
    *(i32x4*)(dst + r * kLatent + 8 * lane) = *(const LDS i32x4*)(mine + r * kPitch + 16 * lane);
}

// ---- split-column weighted latent (wave w accumulates latent columns
// 128 w .. 128 w + 127 for all 128 heads; the heads' owners share their
// probabilities, rescale factors and row sums through LDS) ----

// Per-head values that every wave reads (rescale factors, 1 / row sums) are
// stored with head 32 nb + r at float 4 r + nb: lane r reads its four heads
// with one 16-byte read.
__device__ __forceinline__ constexpr int head_slot(int head) { return 4 * (head & 31) + (head >> 5); }

// Probability rows: chunk c (16 bytes) of head h is stored at chunk
// c ^ pswz(h), so that 16 consecutive heads of one chunk column touch
// distinct banks (64-bank and 32-bank LDS alike).
__device__ __forceinline__ constexpr int pswz(int h) { return ((h >> 1) & 3) ^ ((h >> 3) & 1); }

constexpr int kSplitPitch = kCRow + 16;                 // output staging rows (padded: spread over banks)
constexpr int kSplitStage = kHeads * kSplitPitch;       // bytes of the output staging

// Normalised accumulator of this wave's latent quarter for all 128 heads as
// BF16 rows [128][512] at dst.  The rows are assembled in LDS (the latent and
// rotary stages, free once every tile has landed and every wave is past its
// last read, which the first barrier provides), then every wave writes 32
// whole rows with 1 KiB stores.  The 1 / row sums come from the heads'
// owners through the float array at inv_off ([128], head_slot order),
// written before the call; the rows are assembled in the first kSplitStage
// bytes of the work-group's LDS.
// before_flush() runs after the rows are staged and before their global
// stores are issued: a store it makes (the log-sum-exps) goes out without
// waiting behind the row stores, as a wait for any value it reloads would.
template <typename F>
__device__ __forceinline__ void store_rows_split(LDS char* L, int inv_off, __bf16* dst, const f32x16 (&O)[16],
                                                 int w, F&& before_flush) {
  wait_vmcnt<0>();
  __syncthreads();
  const int lane = __lane_id();
  const int hi = lane >> 5, row = lane & 31;
  const f32x4 inv = *(const LDS f32x4*)(L + inv_off + 16 * row);
  // lane (row, hi) of block (mbl, nb) holds head 32 nb + row, latent columns
  // 32 (4 w + mbl) + 8 g + 4 hi + e; the two lanes of a head swap half of each
  // group pair so each writes 16 contiguous bytes
#pragma unroll
  for (int mbl = 0; mbl < 4; ++mbl)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const f32x16& o = O[4 * mbl + nb];
      LDS char* rowL = L + (32 * nb + row) * kSplitPitch + 2 * 32 * (4 * w + mbl);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int g0 = 2 * k, g1 = 2 * k + 1;
        uint32_t keep[2], send[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const bf16x2 k0 = {(__bf16)(o[4 * g0 + 2 * e] * inv[nb]), (__bf16)(o[4 * g0 + 2 * e + 1] * inv[nb])};
          const bf16x2 k1 = {(__bf16)(o[4 * g1 + 2 * e] * inv[nb]), (__bf16)(o[4 * g1 + 2 * e + 1] * inv[nb])};
          const uint32_t u0 = __builtin_bit_cast(uint32_t, k0), u1 = __builtin_bit_cast(uint32_t, k1);
          keep[e] = hi ? u1 : u0;
          send[e] = hi ? u0 : u1;
        }
        uint32_t recv[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) recv[e] = __float_as_uint(wave_partner(__uint_as_float(send[e])));
        const i32x4 v = hi ? i32x4{(int)recv[0], (int)recv[1], (int)keep[0], (int)keep[1]}
                           : i32x4{(int)keep[0], (int)keep[1], (int)recv[0], (int)recv[1]};
        *(LDS i32x4*)(rowL + 2 * 8 * (hi ? g1 : g0)) = v;
      }
    }
  __syncthreads();
  before_flush();
#pragma unroll
  for (int r = 0; r < 32; ++r)
    *(i32x4*)(dst + (32 * w + r) * kLatent + 8 * lane) = *(const LDS i32x4*)(L + (32 * w + r) * kSplitPitch + 16 * lane);
}

// x * alpha for an accumulator value, kept in its accumulator register.  The
// online-softmax rescale runs only when a head's running maximum grows by a
// large step; writing it this way keeps the register allocator from moving
// the whole accumulator file through ordinary registers around that branch.
// The trailing s_nop covers the accumulator-write -> MFMA-read distance.
__device__ __forceinline__ float scale_acc(float x, float alpha) {
  float t;
  asm volatile(
      "v_accvgpr_read_b32 %1, %0\n\t"
      "v_mul_f32 %1, %1, %2\n\t"
      "v_accvgpr_write_b32 %0, %1\n\t"
      "s_nop 2"
      : "+a"(x), "=&v"(t)
      : "v"(alpha));
  return x;
}

// Score MFMA with its accumulator in ordinary registers (the softmax reads the
// scores with VALU instructions, and the accumulator registers hold the
// weighted latent).  Back-to-back MFMAs that accumulate into the same
// registers need no wait states; the reader of the final value waits.  The
// operands must come from loads (the compiler waits for those), not from VALU
// instructions.
__device__ __forceinline__ f32x16 mfma_sv0(const bf16x8& a, const bf16x8& b) {
  f32x16 d;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ void mfma_sv(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}

// Uniform metadata reads go through the constant address space so they become
// scalar loads (lgkmcnt), never vector loads that would queue behind the
// in-flight LDS-bound loads on vmcnt.
__device__ __forceinline__ int32_t sload(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)(uintptr_t)p;
}

// Row codes of the listed positions of tiles [tc0, tc0 + len) of request b
// (all threads; the caller synchronises): page * 64 + slot per entry, -1 for
// padding, positions out of range and invalid pages.
__device__ __forceinline__ void fill_index_codes(const DecodeArgs& a, int32_t b, int32_t tc0, int32_t len, int32_t T,
                                                 LDS int32_t* list, int tid) {
  const int32_t n = len * kTile;
  for (int k = tid; k < n; k += kThreads) {
    const int32_t lp = tc0 * kTile + k;
    const int32_t idx = lp < a.topk ? a.topk_idx[(int64_t)b * a.topk + lp] : -1;
    bool v = idx >= 0 && idx < T && (idx >> 6) < a.bt_stride;
    const int32_t page = v ? a.block_table[(int64_t)b * a.bt_stride + (idx >> 6)] : -1;
    v = v && page >= 0 && page < a.num_pages;
    list[k] = v ? page * 64 + (idx & 63) : -1;
  }
}

// Per-lane LDS offsets of the MFMA operands inside one tile (relative to the
// tile's latent or rotary section).  The swizzles only touch the low 4 bits
// of a chunk index, so every operand address is one of a few per-lane bases
// plus a compile-time offset.
struct OperandOffsets {
  int s_off[8];      // latent operand of score K-block k: s_off[k & 7] + 256 * (k >> 3)
  int r_off[4];      // rotary operand of score K-block v
  int tr_off[2][4];  // transposed latent operand of column block mb, position half h8:
                     // tr_off[h8][mb & 3] + 256 * (mb >> 2) + 16 KiB * kb2

  __device__ __forceinline__ explicit OperandOffsets(int lane) {
    const int row = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int v = 0; v < 8; ++v) s_off[v] = row * kCRow + 16 * ((2 * v + hi) ^ swz(row));
#pragma unroll
    for (int v = 0; v < 4; ++v) r_off[v] = row * kRRow + 16 * ((2 * v + hi) ^ swz_r(row));
    const int j16 = lane & 15, g16 = lane >> 4, hh = g16 >> 1, ch = g16 & 1;
    const int tr_row = 4 * hh + (j16 >> 2);  // 0..7
    const int lo = 2 * ch + ((j16 & 3) >> 1);
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        tr_off[h8][e] = (tr_row + 8 * h8) * kCRow + 16 * ((4 * e + lo) ^ swz(tr_row + 8 * h8)) + (j16 & 1) * 8;
  }
};

}  // namespace
}  // namespace mla
