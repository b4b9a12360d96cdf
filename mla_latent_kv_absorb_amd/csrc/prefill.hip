// Prefill on the expanded path, gfx950.
//
// With many queries per request a key expanded once is shared by all of them
// ("DeepSeek's KV Cache", section on absorption after Figure 5, and Figure 5
// (1) / Figure 6 (1)), so prefill expands the cached latent per head once --
// K_nope[s][h] = W_UK[h]^T c_s and V[s][h] = W_UV[h] c_s -- and then runs
// causal attention with 192-wide keys (content + the shared rotary key) and
// 128-wide values.
//
// expand_kernel: an NT GEMM out[s][n] = sum_k C[s][k] W[n][k] over the 512
// latent channels, C gathered row by row from the cache pages, W one of the
// two weights viewed as [H * 128][512] (W_UV as stored; W_UK transposed once
// by transpose_w_uk_kernel).  Tiles of 128 positions x 128 features, K in
// chunks of 64 moved HBM -> LDS without registers (double buffered), four
// waves of 64 x 64 on MFMA 32x32x16.  FP8 caches ("DeepSeek's KV Cache",
// section "Calculating V3.2's KV cache": the latent is the E4M3 value times
// its scale): each chunk's codes come through registers and go to LDS as
// BF16.  With one scale per position the codes go as their exact BF16 values
// and each output row is multiplied by its position's scale in float32; with
// one scale per 128 channels each value times its group's scale is rounded
// once to BF16 (a 64-channel chunk lies in one group).
//
// prefill_attn_kernel: per work-group one head and 4 x 32 x QB queries (32 x QB
// per wave, one query per lane column of each column block).  Tiles of 32 positions (content key, rotary key,
// value) stream through a 4-stage LDS ring; S^T[pos][query] on MFMA, online
// softmax per query with the causal bound, O^T[v][query] += V^T P^T with V^T
// from transposing LDS reads -- the decode kernel's pattern with queries in
// place of heads.
#include "attn_common.h"
#include "side_calls.h"

namespace mla {
namespace {

// ---------------- expansion GEMM ----------------
constexpr int kGM = 128, kGN = 128, kGK = 64;
constexpr int kGRow = kGK * 2;          // bytes of one LDS row (one K chunk)
constexpr int kGTile = kGM * kGRow;     // 16 KiB per operand tile
constexpr int kGChunks = kLatent / kGK; // 8

__device__ __forceinline__ int gswz(int r) { return r & 7; }

// FMT: kExpandBf16, kExpandFp8Token (one scale per position), kExpandFp8Group
// (one scale per 128 latent channels)
template <int FMT>
__global__ __launch_bounds__(256) void expand_kernel(ExpandArgs a) {
  constexpr bool FP8 = FMT != kExpandBf16;
  __shared__ __attribute__((aligned(16))) char lds[2 * 2 * kGTile];
  __shared__ float srow[kGM];  // one scale per position: the tile rows' scales
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t m0 = (int64_t)blockIdx.y * kGM;
  const int64_t n0 = (int64_t)blockIdx.x * kGN;
  const int row = lane & 31, hi = lane >> 5;
  const uint32_t base = (uint32_t)(uintptr_t)lds;

  // this lane's share of a chunk's loads: 4 rows-of-8 per operand per wave
  const int rl = lane >> 3, cc = lane & 7;
  const uint8_t* asrc[4];
  const __bf16* bsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * (4 * w + i) + rl;  // tile row 0..127
    int64_t s = m0 + r;
    if (s >= a.T) s = a.T - 1;           // rows past the end load a valid row; never stored
    int32_t page = a.block_table[s >> 6];
    if (page < 0 || page >= a.num_pages) page = 0;  // out-of-range ids read page 0 (values unspecified)
    asrc[i] = a.pool + (int64_t)page * a.page_bytes + (s & 63) * kCRow + 16 * (cc ^ gswz(r));
    bsrc[i] = a.w + (n0 + r) * kLatent + 8 * (cc ^ gswz(r));
  }
  auto issue = [&](int buf, int kc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t dst = base + buf * 2 * kGTile + 8 * (4 * w + i) * kGRow;
      if (!FP8) dma16(asrc[i] + kc * kGRow, dst);
      dma16(bsrc[i] + kc * kGK, dst + kGTile);
    }
  };

  // FP8: thread t takes 32 codes (channels 32 (t % 2) .. + 31 of a chunk) of
  // tile row t / 2
  const int r8 = threadIdx.x >> 1, h8 = threadIdx.x & 1;
  const uint8_t* csrc = nullptr;
  const float* ssrc = nullptr;
  float row_scale = 1.0f;
  if (FP8) {
    int64_t s = m0 + r8;
    if (s >= a.T) s = a.T - 1;
    int32_t page = a.block_table[s >> 6];
    if (page < 0 || page >= a.num_pages) page = 0;
    const uint8_t* pg = a.pool + (int64_t)page * a.page_bytes;
    csrc = pg + (s & 63) * kC8Row + 32 * h8;
    ssrc = (const float*)(pg + a.scale_off) + (s & 63) * (FMT == kExpandFp8Group ? kLatent / 128 : 1);
    if (FMT == kExpandFp8Token) row_scale = *ssrc;  // to LDS with the first chunk's codes
  }
  struct Codes {
    i32x4 c0, c1;
    float sc;  // the chunk's group scale (one scale per 128 channels)
  };
  auto load_codes = [&](int kc) -> Codes {
    Codes c;
    c.c0 = *(const i32x4*)(csrc + kc * kGK);
    c.c1 = *(const i32x4*)(csrc + kc * kGK + 16);
    c.sc = FMT == kExpandFp8Group ? ssrc[kc >> 1] : 1.0f;
    return c;
  };
  // the chunk's codes as BF16 into the A tile of buffer buf (chunk 4 h8 + i
  // of row r8 holds channels 8 (4 h8 + i) .. + 7)
  auto put_codes = [&](int buf, const Codes& c) {
    LDS char* A = (LDS char*)lds + buf * 2 * kGTile + r8 * kGRow;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const i32x4& q = i < 2 ? c.c0 : c.c1;
      const int w0 = q[2 * (i & 1)], w1 = q[2 * (i & 1) + 1];
      bf16x8 v;
      if (FMT == kExpandFp8Token) {
        const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
        const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
        const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
        const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
        v = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
      } else {
        const f32x2 f[4] = {__builtin_amdgcn_cvt_pk_f32_fp8(w0, false), __builtin_amdgcn_cvt_pk_f32_fp8(w0, true),
                            __builtin_amdgcn_cvt_pk_f32_fp8(w1, false), __builtin_amdgcn_cvt_pk_f32_fp8(w1, true)};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = (__bf16)(f[e][0] * c.sc);
          v[2 * e + 1] = (__bf16)(f[e][1] * c.sc);
        }
      }
      *(LDS bf16x8*)(A + 16 * ((4 * h8 + i) ^ gswz(r8))) = v;
    }
  };

  const int wm = w >> 1, wn = w & 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  issue(0, 0);
  Codes cur;
  if (FP8) cur = load_codes(0);
  for (int kc = 0; kc < kGChunks; ++kc) {
    const int buf = kc & 1;
    if (FP8) {
      // the weight rows and the codes of chunk kc have landed (issued last,
      // nothing after them); the codes go to LDS, then chunk kc + 1 goes out
      wait_vmcnt<0>();
      put_codes(buf, cur);
      if (FMT == kExpandFp8Token && kc == 0 && h8 == 0) srow[r8] = row_scale;
      if (kc + 1 < kGChunks) {
        issue(buf ^ 1, kc + 1);
        cur = load_codes(kc + 1);
      }
    } else if (kc + 1 < kGChunks) {
      issue(buf ^ 1, kc + 1);
      wait_vmcnt<8>();  // chunk kc landed (chunk kc + 1 may be in flight)
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    const LDS char* A = (const LDS char*)lds + buf * 2 * kGTile;
    const LDS char* Bt = A + kGTile;
#pragma unroll
    for (int kb = 0; kb < kGK / 16; ++kb) {
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ra = 64 * wm + 32 * i + row, rb = 64 * wn + 32 * i + row;
        av[i] = *(const LDS bf16x8*)(A + ra * kGRow + 16 * ((2 * kb + hi) ^ gswz(ra)));
        bv[i] = *(const LDS bf16x8*)(Bt + rb * kGRow + 16 * ((2 * kb + hi) ^ gswz(rb)));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();  // the buffer is refilled two chunks later
  }

  // D[s][n]: lane holds column n = lane % 32 and rows 8 (r / 4) + 4 hi + r % 4.
  // The wave's 64 x 64 block goes through LDS (free after the last chunk) so
  // the global stores are whole 16-byte pieces of 128-byte row segments.
  constexpr int kOPitch = 64 * 2 + 16;  // padded row: the column-wise writes spread over the banks
  LDS char* ob = (LDS char*)lds + w * 64 * kOPitch;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int sr = 32 * i + 8 * (r >> 2) + 4 * hi + (r & 3);
        const float sc = FMT == kExpandFp8Token ? srow[64 * wm + sr] : 1.0f;
        *(LDS __bf16*)(ob + sr * kOPitch + 2 * (32 * j + row)) = (__bf16)(acc[i][j][r] * sc);
      }
  // each wave reads back only its own block: no barrier needed
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int sr = 8 * it + (lane >> 3), c = lane & 7;
    const int64_t s = m0 + 64 * wm + sr;
    const bf16x8 v = *(const LDS bf16x8*)(ob + sr * kOPitch + 16 * c);
    if (s < a.T) *(bf16x8*)(a.out + s * a.N + n0 + 64 * wn + 8 * c) = v;
  }

  // the shared rotary keys of the tile's positions (once, by the first column of tiles)
  if (a.k_rope != nullptr && blockIdx.x == 0) {
    for (int e = threadIdx.x; e < kGM * (kRope / 8); e += 256) {
      const int r = e / (kRope / 8), c = e % (kRope / 8);
      const int64_t s = m0 + r;
      if (s >= a.T) continue;
      int32_t page = a.block_table[s >> 6];
      if (page < 0 || page >= a.num_pages) page = 0;
      const bf16x8 v = *(const bf16x8*)(a.pool + (int64_t)page * a.page_bytes + a.rope_off + (s & 63) * kRRow + 16 * c);
      *(bf16x8*)(a.k_rope + s * kRope + 8 * c) = v;
    }
  }
}

// W_UK [H][512][128] -> [H][128][512] (done once per set of weights)
__global__ __launch_bounds__(256) void transpose_w_uk_kernel(const __bf16* in, __bf16* out, int H, int D_C, int D_N) {
  __shared__ __bf16 t[64][65];
  const int h = blockIdx.z;
  const int k0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int kk = e / 64, nn = e % 64;
    if (k0 + kk < D_C && n0 + nn < D_N) t[kk][nn] = in[((int64_t)h * D_C + k0 + kk) * D_N + n0 + nn];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int nn = e / 64, kk = e % 64;
    if (k0 + kk < D_C && n0 + nn < D_N) out[((int64_t)h * D_N + n0 + nn) * D_C + k0 + kk] = t[kk][nn];
  }
}

// ---------------- causal attention over the expanded keys ----------------
constexpr int kPDv = 128;              // value and content-key width
constexpr int kPRow = kPDv * 2;        // bytes of a content-key or value row (256)
constexpr int kPK = kTile * kPRow;     // 8 KiB
constexpr int kPR = kTile * kRRow;     // 4 KiB
constexpr int kPStage = 2 * kPK + kPR; // content key, value, rotary key
constexpr int kPNS = 4;

// QB: 32-query column blocks per wave.  Every K / V operand read from LDS
// feeds QB matrix products, so QB = 2 halves the LDS reads per product (at
// one wave per SIMD); QB = 1 keeps two work-groups per CU.
template <int QB>
__global__ __launch_bounds__(256, QB == 1 ? 2 : 1) void prefill_attn_kernel(PrefillArgs a) {
  constexpr int WQ = 32 * QB;          // queries per wave
  __shared__ __attribute__((aligned(16))) char smem[kPNS * kPStage];
  LDS char* L = (LDS char*)smem;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.x;
  const int64_t q0 = (int64_t)blockIdx.y * 4 * WQ;
  const int col = lane & 31, hi = lane >> 5;
  const float scale_log2 = a.scale * kLog2e;
  const int64_t H = a.H;

  // this lane's queries (one per column block) and their positions
  int64_t qc[QB], qpos[QB];
  bool qvalid[QB];
#pragma unroll
  for (int c = 0; c < QB; ++c) {
    const int64_t qi = q0 + WQ * w + 32 * c + col;
    qvalid[c] = qi < a.N;
    qc[c] = qvalid[c] ? qi : a.N - 1;
    qpos[c] = a.q_start + qc[c];  // sees 0 .. qpos
  }

  // B operands: query rows, content dims then rotary dims
  bf16x8 q[QB][12];
#pragma unroll
  for (int c = 0; c < QB; ++c) {
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) q[c][kb] = *(const bf16x8*)(a.qn + (qc[c] * H + h) * kPDv + 16 * kb + 8 * hi);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) q[c][8 + kb] = *(const bf16x8*)(a.qr + (qc[c] * H + h) * kRope + 16 * kb + 8 * hi);
  }

  // positions the work-group needs: up to its last query's position
  int64_t span = a.q_start + q0 + 4 * WQ;
  if (span > a.T) span = a.T;
  const int32_t nt = (int32_t)((span + kTile - 1) / kTile);

  // per-lane LDS offsets (content key / value rows: 16 chunks, swizzle swz;
  // rotary rows: 8 chunks, swizzle swz_r)
  int k_off[8], r_off[4], tr_off[2][4];
#pragma unroll
  for (int v = 0; v < 8; ++v) k_off[v] = col * kPRow + 16 * ((2 * v + hi) ^ swz(col));
#pragma unroll
  for (int v = 0; v < 4; ++v) r_off[v] = col * kRRow + 16 * ((2 * v + hi) ^ swz_r(col));
  {
    const int j16 = lane & 15, g16 = lane >> 4, hh = g16 >> 1, ch = g16 & 1;
    const int tr_row = 4 * hh + (j16 >> 2);
    const int lo = 2 * ch + ((j16 & 3) >> 1);
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        tr_off[h8][e] = (tr_row + 8 * h8) * kPRow + 16 * ((4 * e + lo) ^ swz(tr_row + 8 * h8)) + (j16 & 1) * 8;
  }

  // loads of tile t into stage st: this wave's rows 8w .. 8w + 7
  const uint32_t sbase = (uint32_t)(uintptr_t)smem;
  auto issue = [&](int st, int32_t t) {
    const uint32_t sb = sbase + st * kPStage;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 8 * w + 4 * i + (lane >> 4), c = lane & 15;
      int64_t s = (int64_t)t * kTile + r;
      if (s >= a.T) s = a.T - 1;  // past the end: a valid row, masked below
      const int64_t off = (s * H + h) * kPDv + 8 * (c ^ swz(r));
      dma16(a.kn + off, sb + (8 * w + 4 * i) * kPRow);
      dma16(a.v + off, sb + kPK + (8 * w + 4 * i) * kPRow);
    }
    {
      const int r = 8 * w + (lane >> 3), c = lane & 7;
      int64_t s = (int64_t)t * kTile + r;
      if (s >= a.T) s = a.T - 1;
      dma16(a.kr + s * kRope + 8 * (c ^ swz_r(r)), sb + 2 * kPK + 8 * w * kRRow);
    }
  };
  constexpr int kDmaPerTile = 5;

  f32x16 O[QB][4];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int c = 0; c < QB; ++c) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) O[c][mb] = f32x16{};
    m_run[c] = -INFINITY;
    l_run[c] = 0.f;
  }

  const int pro = nt < kPNS - 1 ? nt : kPNS - 1;
  for (int t = 0; t < pro; ++t) issue(t, t);
  for (int32_t t = 0; t < nt; ++t) {
    const int st = t % kPNS;
    // tile t landed: at most (tiles issued after it) loads of this wave pending
    const int ahead = (nt - 1 - t) < (kPNS - 2) ? (nt - 1 - t) : (kPNS - 2);
    if (ahead >= 2) wait_vmcnt<2 * kDmaPerTile>();
    else if (ahead == 1) wait_vmcnt<kDmaPerTile>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (t + kPNS - 1 < nt) issue((t + kPNS - 1) % kPNS, t + kPNS - 1);
    const LDS char* Kt = L + st * kPStage;
    const LDS char* Vt = Kt + kPK;
    const LDS char* Rt = Kt + 2 * kPK;

    // S^T[pos][query]: each key operand serves every column block
    f32x16 sacc[QB];
#pragma unroll
    for (int c = 0; c < QB; ++c) sacc[c] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < 12; ++kb) {
      const bf16x8 kv = kb < 8 ? *(const LDS bf16x8*)(Kt + k_off[kb]) : *(const LDS bf16x8*)(Rt + r_off[kb - 8]);
#pragma unroll
      for (int c = 0; c < QB; ++c) sacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, q[c][kb], sacc[c], 0, 0, 0);
    }
    bf16x8 P[QB][2];
#pragma unroll
    for (int c = 0; c < QB; ++c) {
      // causal bound and the context end; position of accumulator r:
      // t * 32 + 8 (r / 4) + 4 hi + r % 4
      float s[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t kp = (int64_t)t * kTile + 8 * (r >> 2) + 4 * hi + (r & 3);
        s[r] = (kp <= qpos[c] && kp < a.T) ? sacc[c][r] : -INFINITY;
      }
      float mloc = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mloc = fmaxf(mloc, s[r]);
      mloc = fmaxf(mloc, wave_partner(mloc)) * scale_log2;
      // lazy rescale: the reference maximum moves only when the tile's
      // maximum exceeds it by more than 8 (log2 units), so probabilities
      // stay <= 256 and the accumulator is rescaled rarely
      const float m_new = fmaxf(m_run[c], mloc);
      const bool need = m_new > m_run[c] + 8.0f;
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run[c] - m_new) : 1.0f;
        l_run[c] *= alpha;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) O[c][mb][r] *= alpha;
        m_run[c] = need ? m_new : m_run[c];
      }
      const float neg_m = (m_run[c] == -INFINITY) ? 0.f : -m_run[c];
      float lsum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, neg_m));
        lsum += p;
        P[c][r >> 3][r & 7] = (__bf16)p;
      }
      l_run[c] += lsum;
    }

    // O^T[v][query] += V^T[v][pos] P^T[pos][query]: each value operand
    // serves every column block
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const LDS char* p1 = Vt + tr_off[0][mb] + 16 * kPRow * kb2;
        const LDS char* p2 = Vt + tr_off[1][mb] + 16 * kPRow * kb2;
        s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)p1);
        s16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)p2);
        typedef __attribute__((ext_vector_type(8))) short s16x8;
        const bf16x8 vt = __builtin_bit_cast(bf16x8, (s16x8)__builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int c = 0; c < QB; ++c) O[c][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt, P[c][kb2], O[c][mb], 0, 0, 0);
      }
  }
  wait_vmcnt<0>();

  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
#pragma unroll
  for (int c = 0; c < QB; ++c) {
    const float l_tot = l_run[c] + wave_partner(l_run[c]);
    if (!qvalid[c]) continue;
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    __bf16* o = a.out + (qc[c] * H + h) * kPDv + 4 * hi;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(O[c][mb][4 * g + e] * inv);
        *(bf16x4*)(o + 32 * mb + 8 * g) = v;
      }
    if (a.lse != nullptr && hi == 0) a.lse[qc[c] * H + h] = l_tot > 0.f ? (m_run[c] + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_expand(const ExpandArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.N / kGN), (unsigned)((a.T + kGM - 1) / kGM));
  if (a.fmt == kExpandFp8Token) hipLaunchKernelGGL(expand_kernel<kExpandFp8Token>, grid, dim3(256), 0, s, a);
  else if (a.fmt == kExpandFp8Group) hipLaunchKernelGGL(expand_kernel<kExpandFp8Group>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(expand_kernel<kExpandBf16>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_transpose_w_uk(const void* w_uk, void* w_uk_t, int H, int D_C, int D_N, hipStream_t s) {
  const dim3 grid((D_N + 63) / 64, (D_C + 63) / 64, H);
  hipLaunchKernelGGL(transpose_w_uk_kernel, grid, dim3(256), 0, s, (const __bf16*)w_uk, (__bf16*)w_uk_t, H, D_C, D_N);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(const PrefillArgs& a, hipStream_t s) {
  // x = head: work-groups of one head share an XCD's L2 (launch order is
  // round-robin over the 8 XCDs and 128 heads is a multiple of 8)
  // QB = 2 (half the LDS reads per product, one work-group per CU) measured
  // 1.42 ms against 1.11 ms for QB = 1 on a 4,096-token prompt: the second
  // work-group per CU hides more latency than the saved LDS reads buy
  constexpr int QB = 1;
  const dim3 grid((unsigned)a.H, (unsigned)((a.N + 4 * 32 * QB - 1) / (4 * 32 * QB)));
  hipLaunchKernelGGL(prefill_attn_kernel<QB>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
