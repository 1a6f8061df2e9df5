// Variable-length batches for the bf16 prefill kernel (fa_fwd_bf16.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"

namespace fa {

// Packed ("varlen") layout: q and o are [total_q, Hq, d], k and v are
// [total_k, Hkv, d], token-major; sequence s owns query tokens
// cu_q[s] .. cu_q[s+1]-1 and key tokens cu_k[s] .. cu_k[s+1]-1; lse is
// [Hq, total_q].  In FwdParams, B counts sequences, Nq is the largest query
// length (it sizes the grid) and Nk is unused.
struct VarlenParams {
    const int* cu_q;     // n_seqs + 1 offsets (device)
    const int* cu_k;     // n_seqs + 1 offsets (device)
    int total_q;
    int total_k;
};

hipError_t launch_fwd_bf16_varlen(const FwdParams& p, const VarlenParams& vp, int d, bool causal,
                                  hipStream_t stream);

}  // namespace fa
