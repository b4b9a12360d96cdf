// Append one decoded token per request to the paged latent cache, gfx950.
//
// The latent goes in unrotated and the shared rotary key with RoPE applied
// ("DeepSeek's KV Cache", section "MLA: the cache holds one latent", Figure 3);
// the FP8 formats keep the latent as E4M3 values with float32 scales (one per
// token, or one per 128 latent channels) and the rotary key in BF16 (section
// "Calculating V3.2's KV cache").  One wave per request: lanes take pairs of
// latent channels and pairs of rotary dims; the FP8 scale is a wave maximum
// (per token), or the maximum over each 128-channel group, which is the same
// pair index of every lane.
#include "attn_common.h"
#include "side_calls.h"

namespace mla {
namespace {

constexpr int kAppendWaves = 4;  // requests per work-group

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

template <int KIND>  // 0: F32 cache, 1: BF16 cache, 2: FP8 per token, 3: FP8 per 128 channels
__global__ __launch_bounds__(64 * kAppendWaves) void cache_append_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * kAppendWaves + (threadIdx.x >> 6);
  if (b >= a.batch) return;
  const int32_t pos = a.positions[b];
  if (pos < 0 || (int64_t)pos >= (int64_t)a.bt_stride * 64) return;
  if (a.rope_cos != nullptr && pos >= a.rope_rows) return;
  const int32_t page = a.block_table[(int64_t)b * a.bt_stride + pos / 64];
  if (page < 0 || page >= a.num_pages) return;
  const int slot = pos % 64;
  uint8_t* pg = a.pool + (int64_t)page * a.page_bytes;

  // ---- latent ----
  if (KIND == 0) {
    const float* c = (const float*)a.c_new + (int64_t)b * a.D_C;
    float* dst = (float*)pg + (int64_t)slot * a.D_C;
    for (int e = lane; e < a.D_C; e += 64) dst[e] = c[e];
  } else if (KIND == 1) {
    const uint16_t* c = (const uint16_t*)a.c_new + (int64_t)b * a.D_C;  // BF16 activations: stored as they are
    uint16_t* dst = (uint16_t*)pg + (int64_t)slot * a.D_C;
    for (int e = lane; e < a.D_C; e += 64) dst[e] = c[e];
  } else {
    // V2 dims: 512 channels; lane takes channels 2 lane + 128 j, +1 (j = 0..3),
    // so pair j of every lane lies in 128-channel group j
    const __bf16* c = (const __bf16*)a.c_new + (int64_t)b * kLatent;
    float v[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x2 p = *(const bf16x2*)(c + 128 * j + 2 * lane);
      v[j][0] = (float)p[0];
      v[j][1] = (float)p[1];
    }
    float scale[4];
    if (KIND == 2) {
      float m = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(v[j][0]), fabsf(v[j][1])));
      m = wave_max_f(m);
      const float s = m > 0.f ? m / 448.0f : 1.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) scale[j] = s;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float m = wave_max_f(fmaxf(fabsf(v[j][0]), fabsf(v[j][1])));
        scale[j] = m > 0.f ? m / 448.0f : 1.0f;
      }
    }
    uint8_t* dst = pg + (int64_t)slot * kC8Row;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // float32 quotient, clamped to the format's range, rounded to the
      // nearest E4M3 value (ties to even) by the conversion instruction
      const float q0 = fminf(fmaxf(v[j][0] / scale[j], -448.0f), 448.0f);
      const float q1 = fminf(fmaxf(v[j][1] / scale[j], -448.0f), 448.0f);
      const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
      *(uint16_t*)(dst + 128 * j + 2 * lane) = (uint16_t)(packed & 0xFFFF);
    }
    float* sc = (float*)(pg + a.scale_off);
    if (KIND == 2) {
      if (lane == 0) sc[slot] = scale[0];
    } else {
      if (lane < 4) sc[4 * slot + lane] = lane == 0 ? scale[0] : lane == 1 ? scale[1] : lane == 2 ? scale[2] : scale[3];
    }
  }

  // ---- rotary key: pairs (2i, 2i + 1) rotated by the position's angles ----
  for (int i = lane; 2 * i < a.D_R; i += 64) {
    float x, y;
    if (KIND == 0) {
      const float* k = (const float*)a.k_new + (int64_t)b * a.D_R;
      x = k[2 * i];
      y = k[2 * i + 1];
    } else {
      const bf16x2 p = *(const bf16x2*)((const __bf16*)a.k_new + (int64_t)b * a.D_R + 2 * i);
      x = (float)p[0];
      y = (float)p[1];
    }
    float ox = x, oy = y;
    if (a.rope_cos != nullptr) {
      const float cs = a.rope_cos[(int64_t)pos * (a.D_R / 2) + i];
      const float sn = a.rope_sin[(int64_t)pos * (a.D_R / 2) + i];
      ox = x * cs - y * sn;
      oy = x * sn + y * cs;
    }
    if (KIND == 0) {
      float* dst = (float*)(pg + a.rope_off) + (int64_t)slot * a.D_R;
      dst[2 * i] = ox;
      dst[2 * i + 1] = oy;
    } else {
      bf16x2* dst = (bf16x2*)((__bf16*)(pg + a.rope_off) + (int64_t)slot * a.D_R + 2 * i);
      *dst = bf16x2{(__bf16)ox, (__bf16)oy};
    }
  }
}

}  // namespace

hipError_t launch_cache_append(const AppendArgs& a, int kind, hipStream_t s) {
  const dim3 grid((a.batch + kAppendWaves - 1) / kAppendWaves), block(64 * kAppendWaves);
  switch (kind) {
    case 0: hipLaunchKernelGGL(cache_append_kernel<0>, grid, block, 0, s, a); break;
    case 1: hipLaunchKernelGGL(cache_append_kernel<1>, grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL(cache_append_kernel<2>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(cache_append_kernel<3>, grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace mla
