// Per-head batched products used on the query side and the output side:
//   y[b][h][m] = sum_k w[h][m][k] * x[b][h][k]
// absorb:  x = q_nope, w = W_UK ([H][D_C][D_N]), y = q_lat  (M = D_C, K = D_N)
// out-up:  x = o_lat,  w = W_UV ([H][D_V][D_C]), y = out    (M = D_V, K = D_C)
// ("DeepSeek's KV Cache", Figure 5 form (2) and Figure 6 form (2)).
//
// BF16: each wave computes Y^T[m][b] for 32 rows of w and 64 batch columns on
// MFMA 32x32x16 with both operands loaded straight from HBM in operand layout
// (the contraction dimension is contiguous in w and x, so every lane loads 16
// contiguous bytes).  At decode batch sizes the work is bounded by reading
// the weights once.
// F32: one thread per output element, fp32 FMA.
#include "mla_internal.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;

// Work-group: 4 waves, 64 batch columns (two 32-column accumulators per
// wave, so each weight row is read from HBM once per 64 requests).
//   KS = 1: the 4 waves take 4 consecutive 32-row blocks of w, full K.
//   KS = 4: the 4 waves take one 32-row block and a quarter of K each; the
//           partial sums meet in LDS.  Used for long K (the up-projection,
//           K = D_C) so the grid still has enough waves to cover the weights.
template <int KS>
__global__ __launch_bounds__(256) void head_gemm_bf16_kernel(HeadGemmArgs a) {
  constexpr int kMBlocks = 4 / KS;
  __shared__ float red[KS > 1 ? (KS - 1) * 32 * 64 : 1];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int m0 = (blockIdx.x * kMBlocks + (KS > 1 ? 0 : wv)) * 32;
  const int kpart = KS > 1 ? wv : 0;
  const int h = blockIdx.y;
  const int n0 = blockIdx.z * 64;
  const int kg = lane >> 5;
  const int klen = a.K / KS;
  const int kbeg = kpart * klen;
  const int colA = n0 + (lane & 31), colB = colA + 32;
  const bool vA = colA < a.batch, vB = colB < a.batch;
  if (KS == 1 && m0 >= a.M) return;
  const __bf16* wp = (const __bf16*)a.w + ((int64_t)h * a.M + m0 + (lane & 31)) * a.K + kbeg + 8 * kg;
  const __bf16* xa = (const __bf16*)a.x + ((int64_t)(vA ? colA : 0) * a.H + h) * a.K + kbeg + 8 * kg;
  const __bf16* xb = (const __bf16*)a.x + ((int64_t)(vB ? colB : 0) * a.H + h) * a.K + kbeg + 8 * kg;
  f32x16 accA = f32x16{}, accB = f32x16{};
  const int nk = klen / 16;
  int kk = 0;
  constexpr int U = 8;
  for (; kk + U <= nk; kk += U) {
    bf16x8 av[U], ba[U], bb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      av[u] = *(const bf16x8*)(wp + 16 * (kk + u));
      ba[u] = vA ? *(const bf16x8*)(xa + 16 * (kk + u)) : bf16x8{};
      bb[u] = vB ? *(const bf16x8*)(xb + 16 * (kk + u)) : bf16x8{};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      accA = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[u], ba[u], accA, 0, 0, 0);
      accB = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[u], bb[u], accB, 0, 0, 0);
    }
  }
  for (; kk < nk; ++kk) {
    const bf16x8 av = *(const bf16x8*)(wp + 16 * kk);
    const bf16x8 ba = vA ? *(const bf16x8*)(xa + 16 * kk) : bf16x8{};
    const bf16x8 bb = vB ? *(const bf16x8*)(xb + 16 * kk) : bf16x8{};
    accA = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, ba, accA, 0, 0, 0);
    accB = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bb, accB, 0, 0, 0);
  }
  if (KS > 1) {
    if (wv > 0) {
      float* r = red + (wv - 1) * 32 * 64 + lane;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        r[i * 64] = accA[i];
        r[(16 + i) * 64] = accB[i];
      }
    }
    __syncthreads();
    if (wv > 0) return;
#pragma unroll
    for (int w = 0; w < KS - 1; ++w) {
      const float* r = red + w * 32 * 64 + lane;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        accA[i] += r[i * 64];
        accB[i] += r[(16 + i) * 64];
      }
    }
  }
  // lane holds rows m0 + 8g + 4 kg + e (e = 0..3) of its column
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int col = half ? colB : colA;
    if (col >= a.batch) continue;
    const f32x16& acc = half ? accB : accA;
    __bf16* yp = (__bf16*)a.y + ((int64_t)col * a.H + h) * a.M + m0 + 4 * kg;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[4 * g + e];
      *(bf16x4*)(yp + 8 * g) = v;
    }
  }
}

// K = 128 (the absorb at V2 dims): the work-group's 128 x 128 block of w
// (32 KiB, contiguous in HBM) and its 64 x 128 block of x (16 KiB) are first
// copied to LDS with fully coalesced 16-byte loads, each row's 16-byte chunks
// XOR-swizzled by the row index so the operand reads below are free of bank
// conflicts; then every wave reads its MFMA operands from LDS.  Each weight
// byte is read from HBM once, in whole cache lines, and x once per
// work-group.  The results go back through LDS as well, so that each
// request's 256 output bytes leave in one 16-byte store per lane (storing
// straight from the accumulator layout scatters 8-byte pieces over 32
// requests per instruction, 1.4 us slower in a 7 us launch).
constexpr int kAbK = 128;
constexpr int kAbRow = kAbK * 2;  // bytes per row
__device__ __forceinline__ int ab_off(int row, int chunk) { return row * kAbRow + 16 * (chunk ^ (row & 15)); }

__global__ __launch_bounds__(256) void absorb_k128_kernel(HeadGemmArgs a) {
  __shared__ __attribute__((aligned(16))) char ws[128 * kAbRow];
  __shared__ __attribute__((aligned(16))) char xs[64 * kAbRow];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int h = blockIdx.y;
  const int mb = blockIdx.x * 128;  // first row of w
  const int n0 = blockIdx.z * 64;   // first batch column
  {
    const char* wsrc = (const char*)a.w + ((int64_t)h * a.M + mb) * kAbRow;
    i32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = *(const i32x4*)(wsrc + 16 * (t + 256 * i));
    i32x4 xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = t + 256 * i, col = n0 + (q >> 4);
      xv[i] = col < a.batch ? *(const i32x4*)((const char*)a.x + ((int64_t)col * a.H + h) * kAbRow + 16 * (q & 15))
                            : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = t + 256 * i;
      *(i32x4*)(ws + ab_off(q >> 4, q & 15)) = v[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = t + 256 * i;
      *(i32x4*)(xs + ab_off(q >> 4, q & 15)) = xv[i];
    }
  }
  __syncthreads();
  // wave wv: rows 32 wv .. +31 of the block; lane: row / column lane % 32,
  // K chunk 2 kk + lane / 32
  const int r = 32 * wv + (lane & 31), c = lane & 31, kg = lane >> 5;
  f32x16 accA = f32x16{}, accB = f32x16{};
#pragma unroll
  for (int kk = 0; kk < kAbK / 16; ++kk) {
    const bf16x8 av = *(const bf16x8*)(ws + ab_off(r, 2 * kk + kg));
    const bf16x8 ba = *(const bf16x8*)(xs + ab_off(c, 2 * kk + kg));
    const bf16x8 bb = *(const bf16x8*)(xs + ab_off(c + 32, 2 * kk + kg));
    accA = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, ba, accA, 0, 0, 0);
    accB = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bb, accB, 0, 0, 0);
  }
  // lane holds rows mb + 32 wv + 8g + 4 kg + e (e = 0..3) of its column:
  // staged as BF16 rows of 128 values per column in LDS (over ws, whose
  // reads all finished at the barrier), then stored 16 bytes per lane with
  // every column's 256 bytes contiguous
  __syncthreads();
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const f32x16& acc = half ? accB : accA;
    char* row = ws + (c + 32 * half) * kAbRow;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[4 * g + e];
      // values 32 wv + 8 g + 4 kg .. +3: chunk 4 wv + g, half kg of it
      *(bf16x4*)(row + 16 * ((4 * wv + g) ^ (c & 15)) + 8 * kg) = v;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = t + 256 * i, cl = q >> 4, ch = q & 15, col = n0 + cl;
    if (col < a.batch)
      *(i32x4*)((char*)a.y + (((int64_t)col * a.H + h) * a.M + mb) * 2 + 16 * ch) =
          *(const i32x4*)(ws + cl * kAbRow + 16 * (ch ^ (cl & 15)));
  }
}

__global__ __launch_bounds__(256) void head_gemm_f32_kernel(HeadGemmArgs a) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.batch * a.H * a.M;
  if (e >= total) return;
  const int m = (int)(e % a.M);
  const int h = (int)((e / a.M) % a.H);
  const int64_t b = e / ((int64_t)a.M * a.H);
  const float* w = (const float*)a.w + ((int64_t)h * a.M + m) * a.K;
  const float* x = (const float*)a.x + (b * a.H + h) * a.K;
  float acc = 0.f;
  for (int k = 0; k < a.K; ++k) acc = fmaf(w[k], x[k], acc);
  ((float*)a.y)[e] = acc;
}

}  // namespace

hipError_t launch_head_gemm_bf16(const HeadGemmArgs& a, hipStream_t s) {
  // requires M % 32 == 0 and K % 16 == 0 (checked by the caller)
  if (a.K == kAbK && a.M % 128 == 0) {
    const dim3 grid(a.M / 128, a.H, (a.batch + 63) / 64);
    hipLaunchKernelGGL(absorb_k128_kernel, grid, dim3(256), 0, s, a);
  } else if (a.K >= 256 && a.K % 64 == 0) {
    const dim3 grid(a.M / 32, a.H, (a.batch + 63) / 64);
    hipLaunchKernelGGL(head_gemm_bf16_kernel<4>, grid, dim3(256), 0, s, a);
  } else {
    const dim3 grid((a.M + 127) / 128, a.H, (a.batch + 63) / 64);
    hipLaunchKernelGGL(head_gemm_bf16_kernel<1>, grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_head_gemm_f32(const HeadGemmArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.batch * a.H * a.M;
  const dim3 grid((unsigned)((total + 255) / 256));
  hipLaunchKernelGGL(head_gemm_f32_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
