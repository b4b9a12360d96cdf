// mla_decode_noalloc: the split decode of mla_decode_attn and its merge in
// one call, with the split partials in a static device buffer owned by the
// library instead of a caller workspace, for callers that cannot allocate.
//
// The buffer is the file-scope array `scratch` below: every GPU the library
// runs on holds its own copy until the process ends.  In host code `scratch`
// names a host-side stand-in, not a device address, so the device address of
// each GPU's copy is looked up once per device (hipGetSymbolAddress, with that
// device current) and kept; kernels only ever receive that address.
#include <mutex>

#include "../../include/mla_absorb.h"
#include "host_checks.h"
#include "mla_internal.h"

using namespace mla_host;

namespace {

constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, null until looked up

// Device address of the current device's copy of `scratch`.
mla_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MLA_ERR_LAUNCH;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MLA_OK;
}

mla_status launch_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH; }

}  // namespace

extern "C" {

mla_status mla_decode_noalloc(const mla_config* cfg, const void* q_lat, const void* q_rope, const void* kv_pool,
                              int64_t num_pages, const int32_t* block_table, int32_t block_table_stride,
                              const int32_t* seq_lens, const int32_t* topk_idx, int32_t topk, int32_t batch,
                              const mla_plan* plan, void* o_lat, const void* w_uv, void* out, float* lse_out,
                              void* stream) {
  // Every check runs before the scratch is touched; the argument checks take
  // a stand-in workspace address (aligned, never dereferenced) and no size
  // limit, and the packed size of the partials is checked against the scratch.
  void* const stand_in = (void*)(uintptr_t)256;
  mla::DecodeArgs a;
  Path path;
  mla_status st = prepare_decode(cfg, q_lat, q_rope, kv_pool, num_pages, block_table, block_table_stride, seq_lens,
                                 topk_idx, topk, batch, plan, stand_in, SIZE_MAX, nullptr, nullptr, &a, &path);
  if (st != MLA_OK) return st;
  if ((o_lat == nullptr) == (out == nullptr)) return MLA_ERR_INVALID_ARG;  // exactly one output form
  mla::CombineArgs c{};
  mla::CombineUpArgs u{};
  if (o_lat != nullptr)
    st = prepare_combine(cfg, stand_in, SIZE_MAX, seq_lens, topk, batch, plan, o_lat, lse_out, &c);
  else
    st = prepare_combine_up(cfg, stand_in, SIZE_MAX, seq_lens, topk, batch, plan, w_uv, out, lse_out, &u);
  if (st != MLA_OK) return st;
  const int64_t slots = (int64_t)plan->num_workers + batch - 1;
  if (packed_partials_bytes(cfg, path, slots) > kScratchBytes) return MLA_ERR_SCRATCH;

  void* base = nullptr;
  st = scratch_of_current_device(&base);
  if (st != MLA_OK) return st;
  void* part_o;
  float* part_lse;
  partials_at(cfg, path, base, slots, true, &part_o, &part_lse);
  a.part_o = part_o;
  a.part_lse = part_lse;
  c.part_o = u.c.part_o = part_o;
  c.part_lse = u.c.part_lse = part_lse;

  // The merge reads only the partials this call's attention launch writes
  // (the two kernels derive the same worker ranges), so nothing in the
  // scratch needs clearing.
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (path == Path::kF32)
    e = mla::launch_decode_f32(a, s);
  else if (path == Path::kMfmaBf16 && topk_idx == nullptr)
    e = mla::launch_decode_bf16(a, s);
  else
    e = mla::launch_decode_mfma(a, cache_kind(path), s);
  if (e != hipSuccess) return MLA_ERR_LAUNCH;
  return launch_status(o_lat != nullptr ? mla::launch_combine(c, s) : mla::launch_combine_up(u, s));
}

}  // extern "C"
