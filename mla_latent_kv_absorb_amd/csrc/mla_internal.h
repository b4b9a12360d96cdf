// Internal declarations shared by the host API and the kernel translation
// units: the kernel launchers.  Their arguments and the split partition are
// in mla_args.h.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_args.h"

namespace mla {

hipError_t launch_decode_mfma(const DecodeArgs& a, CacheKind kind, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s);  // BF16 cache, dense
hipError_t launch_decode_fp8(const DecodeArgs& a, hipStream_t s);   // FP8 cache, one scale per position
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_combine_up(const CombineUpArgs& u, hipStream_t s);  // V2 dims, BF16
hipError_t launch_head_gemm_bf16(const HeadGemmArgs& a, hipStream_t s);
hipError_t launch_head_gemm_f32(const HeadGemmArgs& a, hipStream_t s);

}  // namespace mla
