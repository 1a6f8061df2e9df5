// Host/device interface of the attention backward kernels (fa_bwd.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct BwdParams {
    const void* q;       // [B, Hq, Nq, d] bf16
    const void* k;       // [B, Hkv, Nk, d] bf16
    const void* v;       // [B, Hkv, Nk, d] bf16
    const void* o;       // [B, Hq, Nq, d] bf16, the forward output
    const float* lse;    // [B, Hq, Nq], the forward log-sum-exp (natural log)
    const void* dout;    // [B, Hq, Nq, d] bf16, gradient of the output
    void* dq;            // [B, Hq, Nq, d] bf16
    void* dk;            // [B, Hkv, Nk, d] bf16
    void* dv;            // [B, Hkv, Nk, d] bf16
    float* ws;           // 2 * B * Hq * Nq floats: delta, then the log2-domain LSE
    int B, Hq, Hkv, Nq, Nk;
    int group;           // Hq / Hkv
    int causal_shift;    // Nk - Nq: key j visible to query i iff j <= i + causal_shift
    int n_qtiles;        // dQ kernel: query tiles per head
    int n_ktiles;        // dK/dV kernel: key tiles per key/value head
    int group_dkv;       // workgroup orders (bwd_order): 0 heads first, G > 0 each XCD's
    int group_dq;        // key/value heads G at a time
    float c;             // scale * log2(e), signed
    float scale;         // multiplies dQ and dK
    // Variable-length batches (packed [tokens, H, d] layouts): B counts
    // sequences, Nq / Nk are the largest lengths (they size the grids), the
    // workspace is [2][Hq][total_q] and lse is [Hq, total_q].
    const int* cu_q;     // n_seqs + 1 offsets (device), or null
    const int* cu_k;
    int total_q;
    int total_k;
    int compact_dkv;     // set by the launcher: 1 = the compact grid of varlen_slot for the
    int compact_dq;      // dK/dV (key tiles) or dQ (query tiles) kernel, 0 = the padded grid
};

hipError_t launch_bwd(const BwdParams& p, int d, bool causal, hipStream_t stream);
hipError_t launch_bwd_varlen(const BwdParams& p, int d, bool causal, hipStream_t stream);

}  // namespace fa
