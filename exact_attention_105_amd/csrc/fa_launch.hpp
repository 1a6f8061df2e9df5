// Internal launch entry points of the attention kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include "fa_device.hpp"

namespace fa {

// Dynamic LDS, in bytes, to launch a kernel that declares `static_lds` bytes
// of LDS with, never touched by it: the value of the environment variable
// FA_TEST_EXTRA_LDS (decimal, read once per process; 0 when unset), cut so
// that static plus dynamic LDS stays within 128 KiB (the decode kernel's own
// static LDS; gfx950 allows 160 KiB per workgroup), and 0 for a kernel whose
// static LDS already keeps it to one workgroup per CU (the decode kernel).
// A test hook: it lowers the number of workgroups resident on each CU, so
// tests can check that results do not depend on occupancy.  Used by the
// prefill, decode and backward launches.
size_t test_extra_lds(size_t static_lds);

// bf16 inputs, head dim 64 or 128.  Fills n_qtiles itself.
hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, hipStream_t stream);

// fp8 e4m3 inputs, head dim 128.  Fills n_qtiles itself.
hipError_t launch_fwd_fp8(const FwdParams& p, int d, bool causal, hipStream_t stream);

// Few query rows per head (Nq <= 16), bf16, head dim 128: grouped-query packed,
// keys split over the waves of a workgroup.
bool decode_applies(const FwdParams& p, int d, bool is_bf16);
hipError_t launch_fwd_decode(const FwdParams& p, bool causal, hipStream_t stream);
// The decode kernel with the keys split over n_splits workgroups: partials go
// to ws (n_splits * B * Hq * Nq * (128 + 1) floats), then a merge kernel
// writes O and LSE.  n_splits == 1 is the direct path (ws unused).
hipError_t launch_fwd_decode_split(const FwdParams& p, bool causal, int n_splits, float* ws, hipStream_t stream);

// Random-sign Hadamard rotation + per-tensor E4M3 quantisation of [rows, d].
struct RotParams {
    const void* x;            // [rows, d] bf16 or fp32
    uint8_t* codes;           // [rows, d] E4M3 codes (written)
    float* scale;             // one float: amax / 448 (written)
    unsigned* work;           // one word of workspace (amax bit pattern)
    int64_t rows;
    uint32_t sign_bits[4];    // bit j set: feature j is negated before the transform
    int rotate;               // 0: quantise without rotating
};
hipError_t launch_rotate_quantize(const RotParams& p, bool x_is_f32, int d, hipStream_t stream);

}  // namespace fa
