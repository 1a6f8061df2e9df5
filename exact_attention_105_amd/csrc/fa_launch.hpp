// Internal launch entry points of the attention kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include "fa_device.hpp"

namespace fa {

// bf16 inputs, head dim 64 or 128.  Fills n_qtiles itself.
hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, hipStream_t stream);

// fp8 e4m3 inputs, head dim 128.  Fills n_qtiles itself.
hipError_t launch_fwd_fp8(const FwdParams& p, int d, bool causal, hipStream_t stream);

// Few query rows per head (Nq <= 16), bf16, head dim 128: grouped-query packed,
// keys split over the waves of a workgroup.
bool decode_applies(const FwdParams& p, int d, bool is_bf16);
hipError_t launch_fwd_decode(const FwdParams& p, bool causal, hipStream_t stream);

}  // namespace fa
