// Per-head batched products used on the query side and the output side:
//   y[b][h][m] = sum_k w[h][m][k] * x[b][h][k]
// absorb:  x = q_nope, w = W_UK ([H][D_C][D_N]), y = q_lat  (M = D_C, K = D_N)
// out-up:  x = o_lat,  w = W_UV ([H][D_V][D_C]), y = out    (M = D_V, K = D_C)
// ("DeepSeek's KV Cache", Figure 5 form (2) and Figure 6 form (2)).
//
// BF16: one wave per (32 rows of w, head, 32 batch columns) computes
// Y^T[m][b] on MFMA 32x32x16 with both operands loaded straight from HBM in
// operand layout (the contraction dimension is contiguous in w and x, so
// every lane loads 16 contiguous bytes).  At decode batch sizes the work is
// bounded by reading the weights once.
// F32: one thread per output element, fp32 FMA.
#include "mla_internal.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;

__global__ __launch_bounds__(64) void head_gemm_bf16_kernel(HeadGemmArgs a) {
  const int lane = threadIdx.x;
  const int m0 = blockIdx.x * 32;
  const int h = blockIdx.y;
  const int n0 = blockIdx.z * 32;
  const int kg = lane >> 5;
  const int col = n0 + (lane & 31);
  const bool colv = col < a.batch;
  const __bf16* wp = (const __bf16*)a.w + ((int64_t)h * a.M + m0 + (lane & 31)) * a.K + 8 * kg;
  const __bf16* xp = (const __bf16*)a.x + ((int64_t)(colv ? col : 0) * a.H + h) * a.K + 8 * kg;
  f32x16 acc = f32x16{};
  const int nk = a.K / 16;
  int kk = 0;
  for (; kk + 4 <= nk; kk += 4) {
    bf16x8 av[4], bv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      av[u] = *(const bf16x8*)(wp + 16 * (kk + u));
      bv[u] = colv ? *(const bf16x8*)(xp + 16 * (kk + u)) : bf16x8{};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[u], bv[u], acc, 0, 0, 0);
  }
  for (; kk < nk; ++kk) {
    bf16x8 av = *(const bf16x8*)(wp + 16 * kk);
    bf16x8 bv = colv ? *(const bf16x8*)(xp + 16 * kk) : bf16x8{};
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
  }
  if (!colv) return;
  __bf16* yp = (__bf16*)a.y + ((int64_t)col * a.H + h) * a.M + m0 + 4 * kg;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    bf16x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[4 * g + e];
    *(bf16x4*)(yp + 8 * g) = v;
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
  const dim3 grid(a.M / 32, a.H, (a.batch + 31) / 32);
  hipLaunchKernelGGL(head_gemm_bf16_kernel, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_head_gemm_f32(const HeadGemmArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.batch * a.H * a.M;
  const dim3 grid((unsigned)((total + 255) / 256));
  hipLaunchKernelGGL(head_gemm_f32_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
