// Measurement helpers for the benchmark (libmla_bench.so; not part of the
// decode library and not called by it):
//
//   mlab_stream_read  a plain streaming read of a device buffer: every byte is
//                     loaded once with 16-byte loads and folded into one word
//                     per work-group, so the read cannot be dropped.  Its rate
//                     is the read ceiling the decode kernels are set beside.
//   mlab_clock_probe  each work-group records the shader-clock counter
//                     (s_memtime), the constant-rate real-time counter
//                     (s_memrealtime, 100 MHz) and where it runs (XCD and
//                     hardware id).  Two probes around a timed region give
//                     the mean shader clock over it, delta(memtime) /
//                     delta(realtime), from work-groups that ran on the same
//                     compute unit both times (the counters of different
//                     units are not aligned).
//   mlab_stamp        one wave writes the real-time counter to a slot: launched
//                     between two launches on a stream it marks the boundary
//                     between them, for per-launch times without events.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;  // 16-byte loads in flight per lane

// Work-group g reads the contiguous chunk [g * chunk, (g + 1) * chunk) of the
// buffer; the host makes `chunk` a multiple of 16 * kReadThreads * kReadUnroll.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* __restrict__ src, uint64_t chunk16,
                                                                   uint32_t* __restrict__ sink) {
  const u32x4* p = src + (uint64_t)blockIdx.x * chunk16;
  uint32_t acc = 0;
  for (uint64_t i = threadIdx.x; i < chunk16; i += kReadThreads * kReadUnroll) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * kReadThreads);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // one word per work-group; a lane writes only if its fold is the magic
  // value no real buffer produces by accident often enough to matter
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t* __restrict__ out) {
  const uint64_t t = __builtin_amdgcn_s_memtime();
  const uint64_t r = __builtin_amdgcn_s_memrealtime();
  // HW_REG_XCC_ID (hardware register 20), bits [3:0]: the XCD of this wave;
  // HW_REG_HW_ID (hardware register 4): CU, shader array and engine ids
  const uint32_t xcc = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xF;
  const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);
  if (threadIdx.x == 0) {
    out[blockIdx.x * 4 + 0] = t;
    out[blockIdx.x * 4 + 1] = r;
    out[blockIdx.x * 4 + 2] = xcc;
    out[blockIdx.x * 4 + 3] = hw;
  }
}

// One wave writes the real-time counter (100 MHz) to *slot.  Launched on the
// stream between two launches it time-stamps the boundary between them
// without the cache writeback and invalidate of an event.
__global__ __launch_bounds__(64) void stamp_kernel(uint64_t* __restrict__ slot) {
  const uint64_t r = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) *slot = r;
}

}  // namespace

extern "C" {

// *slot = the real-time counter when the stamp runs on `stream`.
int mlab_stamp(uint64_t* slot, void* stream) {
  if (!slot) return 1;
  hipLaunchKernelGGL(stamp_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, slot);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}


// Read `bytes` bytes of `src` (16-byte aligned) once.  `bytes` must be a
// multiple of 16 * 256 * 8 * num_groups; sink holds num_groups words (written
// only by chance).  Returns 0, or 1 on a bad argument, 3 on a failed launch.
int mlab_stream_read(const void* src, uint64_t bytes, int32_t num_groups, uint32_t* sink, void* stream) {
  if (!src || !sink || num_groups < 1 || ((uintptr_t)src & 15)) return 1;
  const uint64_t per = (uint64_t)16 * kReadThreads * kReadUnroll;
  if (bytes % (per * (uint64_t)num_groups)) return 1;
  const uint64_t chunk16 = bytes / 16 / (uint64_t)num_groups;
  hipLaunchKernelGGL(stream_read_kernel, dim3(num_groups), dim3(kReadThreads), 0, (hipStream_t)stream,
                     (const u32x4*)src, chunk16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

// out: num_groups * 4 uint64 words (memtime, realtime, xcc id, hardware id
// per group).
int mlab_clock_probe(uint64_t* out, int32_t num_groups, void* stream) {
  if (!out || num_groups < 1 || num_groups > 4096) return 1;
  hipLaunchKernelGGL(clock_probe_kernel, dim3(num_groups), dim3(64), 0, (hipStream_t)stream, out);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
