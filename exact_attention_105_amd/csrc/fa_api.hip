// C ABI of the attention forward library: argument validation and dispatch.
// The contract of every entry point is documented in include/fa.h.
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>

#include "fa.h"
#include "fa_bwd.hpp"
#include "fa_launch.hpp"
#include "fa_varlen.hpp"

namespace {

constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

}  // namespace

namespace fa {

size_t test_extra_lds(size_t static_lds) {
    static const size_t want = [] {
        const char* v = getenv("FA_TEST_EXTRA_LDS");
        const long long x = v == nullptr ? 0 : atoll(v);
        return (size_t)(x < 0 ? 0 : x);
    }();
    constexpr size_t kLdsPerCu = 160 << 10;      // gfx950
    // total per workgroup while the hook is on: no more than the decode
    // kernel's own static LDS, well inside the 160 KiB limit
    constexpr size_t kCap = 128 << 10;
    // a kernel whose own LDS already limits it to one workgroup per CU is left alone
    if (want == 0 || 2 * static_lds > kLdsPerCu || static_lds >= kCap) return 0;
    const size_t room = kCap - static_lds;
    return want < room ? want : room;
}

}  // namespace fa

// Split-KV partials for fa_fwd_splitkv_noalloc: one copy per GPU, held until
// the process ends.  In host code `scratch` names a host-side stand-in, not
// the device array: host code only ever uses the address that
// hipGetSymbolAddress returns for the current device (scratch_on_device).
static __device__ __align__(256) float scratch[FA_SPLITKV_SCRATCH_FLOATS];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device with
// that device current; nullptr if the lookup fails.
float* scratch_on_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
        g_scratch_ptr[dev] = static_cast<float*>(ptr);
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" fa_status_t fa_fwd_validate(const void* q, const void* k, const void* v, const void* o,
                                       const float* lse, int B, int Hq, int Hkv, int Nq, int Nk,
                                       int d, int causal, float scale, fa_dtype_t dtype,
                                       const float* descale_qkv) {
    if (B < 0 || Hq < 1 || Hkv < 1 || Nq < 0 || Nk < 0 || d < 1) return FA_ERROR_INVALID_VALUE;
    if (Hq % Hkv != 0) return FA_ERROR_INVALID_VALUE;
    if (causal != 0 && causal != 1) return FA_ERROR_INVALID_VALUE;
    if (!isfinite(scale)) return FA_ERROR_INVALID_VALUE;
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP8_E4M3 && dtype != FA_DTYPE_F32)
        return FA_ERROR_INVALID_VALUE;
    if (dtype != FA_DTYPE_FP8_E4M3 && descale_qkv != nullptr) return FA_ERROR_INVALID_VALUE;
    if (dtype == FA_DTYPE_FP8_E4M3) {
        if (descale_qkv == nullptr) return FA_ERROR_INVALID_VALUE;
        for (int i = 0; i < 3; ++i)
            if (!isfinite(descale_qkv[i]) || !(descale_qkv[i] > 0.f)) return FA_ERROR_INVALID_VALUE;
    }
    const int64_t q_elems = (int64_t)B * Hq * Nq * d;
    const int64_t kv_elems = (int64_t)B * Hkv * Nk * d;
    if (q_elems > kMaxElems || kv_elems > kMaxElems) return FA_ERROR_INVALID_VALUE;
    const int64_t rows = (int64_t)B * Hq * Nq;
    if (rows > 0) {
        if (Nk == 0) return FA_ERROR_INVALID_VALUE;   // rows to compute but no key to attend to
        if (q == nullptr || o == nullptr) return FA_ERROR_INVALID_VALUE;
        if (!aligned(q, 16) || !aligned(o, 16)) return FA_ERROR_INVALID_VALUE;
        if (lse != nullptr && !aligned(lse, 4)) return FA_ERROR_INVALID_VALUE;
        if (kv_elems > 0) {
            if (k == nullptr || v == nullptr) return FA_ERROR_INVALID_VALUE;
            if (!aligned(k, 16) || !aligned(v, 16)) return FA_ERROR_INVALID_VALUE;
        }
    }
    if (dtype == FA_DTYPE_BF16 && d != 64 && d != 128) return FA_ERROR_NOT_SUPPORTED;
    if (dtype == FA_DTYPE_FP8_E4M3 && d != 128) return FA_ERROR_NOT_SUPPORTED;
    if (dtype == FA_DTYPE_F32) return FA_ERROR_NOT_SUPPORTED;   // no fp32 attention kernel
    return FA_SUCCESS;
}

extern "C" fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                              float scale, fa_dtype_t dtype, const float* descale_qkv,
                              hipStream_t stream) {
    const fa_status_t st = fa_fwd_validate(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale,
                                           dtype, descale_qkv);
    if (st != FA_SUCCESS) return st;
    if ((int64_t)B * Hq * Nq == 0) return FA_SUCCESS;

    fa::FwdParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Nq = Nq;
    p.Nk = Nk;
    p.group = Hq / Hkv;
    p.n_heads = B * Hq;
    p.causal_shift = Nk - Nq;
    // A negative scale is applied by flipping the sign bit of every Q
    // element on load (exact in both formats) and using |scale|.
    const float mag = fabsf(scale);
    const bool neg = scale < 0.f;
    if (dtype == FA_DTYPE_BF16) {
        p.c = mag * fa::kLog2e;
        p.o_scale = 1.f;
        p.q_sign = neg ? 0x80008000u : 0u;
    } else {
        p.c = mag * descale_qkv[0] * descale_qkv[1] * fa::kLog2e;
        p.o_scale = descale_qkv[2];
        p.q_sign = neg ? 0x80808080u : 0u;
    }

    // The kernels mask scores with -inf and rely on exp2(-inf * c) = 0, which
    // needs c > 0.  A zero (or underflowing) scale uses the smallest normal
    // float instead: every visible score times it rounds away against the
    // exponent reference, so the weights stay exactly uniform.
    p.c = fmaxf(p.c, FLT_MIN);

    hipError_t err;
    if (dtype == FA_DTYPE_BF16)
        err = fa::decode_applies(p, d, true) ? fa::launch_fwd_decode(p, causal != 0, stream)
                                             : fa::launch_fwd_bf16(p, d, causal != 0, stream);
    else
        err = fa::launch_fwd_fp8(p, d, causal != 0, stream);
    return err == hipSuccess ? FA_SUCCESS : FA_ERROR_LAUNCH_FAILURE;
}

extern "C" fa_status_t fa_rotate_quantize_validate(const void* x, fa_dtype_t x_dtype, long long rows,
                                                   int d, int rotate, const unsigned char* codes,
                                                   const float* scale, const float* work) {
    if (rows < 0 || d < 1) return FA_ERROR_INVALID_VALUE;
    if (rotate != 0 && rotate != 1) return FA_ERROR_INVALID_VALUE;
    if (x_dtype != FA_DTYPE_BF16 && x_dtype != FA_DTYPE_FP8_E4M3 && x_dtype != FA_DTYPE_F32)
        return FA_ERROR_INVALID_VALUE;
    if ((int64_t)rows * d > kMaxElems) return FA_ERROR_INVALID_VALUE;
    if (scale == nullptr || work == nullptr || !aligned(scale, 4) || !aligned(work, 4))
        return FA_ERROR_INVALID_VALUE;
    if (rows > 0) {
        if (x == nullptr || codes == nullptr) return FA_ERROR_INVALID_VALUE;
        if (!aligned(x, 16) || !aligned(codes, 16)) return FA_ERROR_INVALID_VALUE;
    }
    if (d != 64 && d != 128) return FA_ERROR_NOT_SUPPORTED;
    if (x_dtype == FA_DTYPE_FP8_E4M3) return FA_ERROR_NOT_SUPPORTED;
    return FA_SUCCESS;
}

extern "C" fa_status_t fa_rotate_quantize_e4m3(const void* x, fa_dtype_t x_dtype, long long rows, int d,
                                               int rotate, const unsigned int* sign_bits,
                                               unsigned char* codes, float* scale, float* work,
                                               hipStream_t stream) {
    const fa_status_t st = fa_rotate_quantize_validate(x, x_dtype, rows, d, rotate, codes, scale, work);
    if (st != FA_SUCCESS) return st;
    fa::RotParams p{};
    p.x = x;
    p.codes = codes;
    p.scale = scale;
    p.work = reinterpret_cast<unsigned*>(work);
    p.rows = rows;
    p.rotate = rotate;
    if (rotate && sign_bits != nullptr)
        for (int w = 0; w < d / 32; ++w) p.sign_bits[w] = sign_bits[w];
    const hipError_t err = fa::launch_rotate_quantize(p, x_dtype == FA_DTYPE_F32, d, stream);
    return err == hipSuccess ? FA_SUCCESS : FA_ERROR_LAUNCH_FAILURE;
}

extern "C" const char* fa_status_string(fa_status_t status) {
    switch (status) {
        case FA_SUCCESS: return "FA_SUCCESS: no error";
        case FA_ERROR_INVALID_VALUE: return "FA_ERROR_INVALID_VALUE: an argument is outside its documented range";
        case FA_ERROR_NOT_SUPPORTED: return "FA_ERROR_NOT_SUPPORTED: no kernel for this head dim / dtype combination";
        case FA_ERROR_LAUNCH_FAILURE: return "FA_ERROR_LAUNCH_FAILURE: the HIP runtime rejected the kernel launch";
    }
    return "unknown fa_status_t";
}

extern "C" int fa_version(void) { return 100; }

extern "C" fa_status_t fa_bwd_validate(const void* q, const void* k, const void* v, const void* o,
                                       const float* lse, const void* dout, const void* dq,
                                       const void* dk, const void* dv, const float* workspace, int B,
                                       int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                                       fa_dtype_t dtype) {
    if (B < 0 || Hq < 1 || Hkv < 1 || Nq < 0 || Nk < 0 || d < 1) return FA_ERROR_INVALID_VALUE;
    if (Hq % Hkv != 0) return FA_ERROR_INVALID_VALUE;
    if (causal != 0 && causal != 1) return FA_ERROR_INVALID_VALUE;
    if (!isfinite(scale)) return FA_ERROR_INVALID_VALUE;
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP8_E4M3 && dtype != FA_DTYPE_F32)
        return FA_ERROR_INVALID_VALUE;
    const int64_t q_elems = (int64_t)B * Hq * Nq * d;
    const int64_t kv_elems = (int64_t)B * Hkv * Nk * d;
    if (q_elems > kMaxElems || kv_elems > kMaxElems) return FA_ERROR_INVALID_VALUE;
    if (q_elems > 0) {
        if (Nk == 0) return FA_ERROR_INVALID_VALUE;   // rows to differentiate and no key, as in fa_fwd
        if (q == nullptr || o == nullptr || dout == nullptr || dq == nullptr || lse == nullptr ||
            workspace == nullptr)
            return FA_ERROR_INVALID_VALUE;
        if (!aligned(q, 16) || !aligned(o, 16) || !aligned(dout, 16) || !aligned(dq, 16) ||
            !aligned(lse, 4) || !aligned(workspace, 4))
            return FA_ERROR_INVALID_VALUE;
    }
    if (kv_elems > 0) {
        if (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr) return FA_ERROR_INVALID_VALUE;
        if (!aligned(k, 16) || !aligned(v, 16) || !aligned(dk, 16) || !aligned(dv, 16))
            return FA_ERROR_INVALID_VALUE;
    }
    if (dtype != FA_DTYPE_BF16) return FA_ERROR_NOT_SUPPORTED;   // backward is bf16 only
    if (d != 64 && d != 128) return FA_ERROR_NOT_SUPPORTED;
    return FA_SUCCESS;
}

extern "C" fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, void* dq, void* dk, void* dv, float* workspace, int B,
                              int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                              fa_dtype_t dtype, hipStream_t stream) {
    const fa_status_t st = fa_bwd_validate(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, Hq, Hkv, Nq,
                                           Nk, d, causal, scale, dtype);
    if (st != FA_SUCCESS) return st;
    if ((int64_t)B * Hq * Nq == 0 && (int64_t)B * Hkv * Nk == 0) return FA_SUCCESS;
    fa::BwdParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.dout = dout;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.ws = workspace;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Nq = Nq;
    p.Nk = Nk;
    p.group = Hq / Hkv;
    p.causal_shift = Nk - Nq;
    p.c = scale * fa::kLog2e;
    p.scale = scale;
    const hipError_t err = fa::launch_bwd(p, d, causal != 0, stream);
    return err == hipSuccess ? FA_SUCCESS : FA_ERROR_LAUNCH_FAILURE;
}

extern "C" fa_status_t fa_fwd_varlen_validate(const void* q, const void* k, const void* v, const void* o,
                                              const float* lse, const int* cu_seqlens_q,
                                              const int* cu_seqlens_k, int n_seqs, int max_seqlen_q,
                                              int total_q, int total_k, int Hq, int Hkv, int d, int causal,
                                              float scale, fa_dtype_t dtype) {
    if (n_seqs < 0 || max_seqlen_q < 0 || total_q < 0 || total_k < 0 || Hq < 1 || Hkv < 1 || d < 1)
        return FA_ERROR_INVALID_VALUE;
    if (Hq % Hkv != 0) return FA_ERROR_INVALID_VALUE;
    if (causal != 0 && causal != 1) return FA_ERROR_INVALID_VALUE;
    if (!isfinite(scale)) return FA_ERROR_INVALID_VALUE;
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP8_E4M3 && dtype != FA_DTYPE_F32)
        return FA_ERROR_INVALID_VALUE;
    const int64_t q_elems = (int64_t)total_q * Hq * d;
    const int64_t kv_elems = (int64_t)total_k * Hkv * d;
    if (q_elems > kMaxElems || kv_elems > kMaxElems) return FA_ERROR_INVALID_VALUE;
    // the grid covers max_seqlen_q rows of every sequence and query head
    if ((int64_t)((max_seqlen_q + 127) / 128) * n_seqs * Hq > 0x7FFFFFFFLL) return FA_ERROR_INVALID_VALUE;
    if (n_seqs > 0) {
        if (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr) return FA_ERROR_INVALID_VALUE;
        if (!aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4)) return FA_ERROR_INVALID_VALUE;
    }
    if (q_elems > 0) {
        if (q == nullptr || o == nullptr) return FA_ERROR_INVALID_VALUE;
        if (!aligned(q, 16) || !aligned(o, 16)) return FA_ERROR_INVALID_VALUE;
        if (lse != nullptr && !aligned(lse, 4)) return FA_ERROR_INVALID_VALUE;
    }
    if (kv_elems > 0) {
        if (k == nullptr || v == nullptr) return FA_ERROR_INVALID_VALUE;
        if (!aligned(k, 16) || !aligned(v, 16)) return FA_ERROR_INVALID_VALUE;
    }
    if (dtype != FA_DTYPE_BF16) return FA_ERROR_NOT_SUPPORTED;   // variable-length batches: bf16 only
    if (d != 64 && d != 128) return FA_ERROR_NOT_SUPPORTED;
    return FA_SUCCESS;
}

extern "C" fa_status_t fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                                     const int* cu_seqlens_q, const int* cu_seqlens_k, int n_seqs,
                                     int max_seqlen_q, int total_q, int total_k, int Hq, int Hkv, int d,
                                     int causal, float scale, fa_dtype_t dtype, hipStream_t stream) {
    const fa_status_t st = fa_fwd_varlen_validate(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, n_seqs,
                                                  max_seqlen_q, total_q, total_k, Hq, Hkv, d, causal, scale,
                                                  dtype);
    if (st != FA_SUCCESS) return st;
    if (n_seqs == 0 || max_seqlen_q == 0 || total_q == 0) return FA_SUCCESS;
    fa::FwdParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.B = n_seqs;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Nq = max_seqlen_q;            // sizes the grid; each workgroup reads its sequence's length
    p.Nk = 0;
    p.group = Hq / Hkv;
    p.n_heads = n_seqs * Hq;
    p.causal_shift = 0;
    const float mag = fabsf(scale);
    p.c = fmaxf(mag * fa::kLog2e, FLT_MIN);
    p.o_scale = 1.f;
    p.q_sign = scale < 0.f ? 0x80008000u : 0u;
    fa::VarlenParams vp{};
    vp.cu_q = cu_seqlens_q;
    vp.cu_k = cu_seqlens_k;
    vp.total_q = total_q;
    vp.total_k = total_k;
    const hipError_t err = fa::launch_fwd_bf16_varlen(p, vp, d, causal != 0, stream);
    return err == hipSuccess ? FA_SUCCESS : FA_ERROR_LAUNCH_FAILURE;
}

extern "C" fa_status_t fa_fwd_splitkv_validate(const void* q, const void* k, const void* v, const void* o,
                                               const float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                               int causal, float scale, fa_dtype_t dtype, int n_splits,
                                               const float* workspace) {
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP8_E4M3 && dtype != FA_DTYPE_F32)
        return FA_ERROR_INVALID_VALUE;
    // sizes, pointers and alignment as for fa_fwd
    if (fa_fwd_validate(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, FA_DTYPE_BF16, nullptr) ==
        FA_ERROR_INVALID_VALUE)
        return FA_ERROR_INVALID_VALUE;
    if (n_splits < 1 || n_splits > 256) return FA_ERROR_INVALID_VALUE;
    const int64_t rows = (int64_t)B * Hq * Nq;
    if (n_splits > 1 && rows > 0) {
        if (workspace == nullptr || !aligned(workspace, 16)) return FA_ERROR_INVALID_VALUE;
        if (rows * n_splits * (int64_t)(d + 1) > kMaxElems) return FA_ERROR_INVALID_VALUE;
    }
    if (dtype != FA_DTYPE_BF16) return FA_ERROR_NOT_SUPPORTED;   // split-KV decode: bf16 only
    if (d != 128 || Nq > 16) return FA_ERROR_NOT_SUPPORTED;      // decode shapes only
    return FA_SUCCESS;
}

extern "C" fa_status_t fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                      int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                                      fa_dtype_t dtype, int n_splits, float* workspace, hipStream_t stream) {
    const fa_status_t st = fa_fwd_splitkv_validate(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, dtype,
                                                   n_splits, workspace);
    if (st != FA_SUCCESS) return st;
    if ((int64_t)B * Hq * Nq == 0) return FA_SUCCESS;
    fa::FwdParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Nq = Nq;
    p.Nk = Nk;
    p.group = Hq / Hkv;
    p.n_heads = B * Hq;
    p.causal_shift = Nk - Nq;
    p.c = fmaxf(fabsf(scale) * fa::kLog2e, FLT_MIN);
    p.o_scale = 1.f;
    p.q_sign = scale < 0.f ? 0x80008000u : 0u;
    const hipError_t err = fa::launch_fwd_decode_split(p, causal != 0, n_splits, workspace, stream);
    return err == hipSuccess ? FA_SUCCESS : FA_ERROR_LAUNCH_FAILURE;
}

extern "C" fa_status_t fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                              int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                                              float scale, fa_dtype_t dtype, int n_splits, hipStream_t stream) {
    // Argument checks with a stand-in workspace pointer (aligned, non-null);
    // the real one is looked up only for a call that launches.
    static float stand_in[4] __attribute__((aligned(16)));
    fa_status_t st = fa_fwd_splitkv_validate(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, dtype,
                                             n_splits, stand_in);
    if (st != FA_SUCCESS) return st;
    const int64_t rows = (int64_t)B * Hq * Nq;
    if (n_splits > 1 && rows * n_splits * (int64_t)(d + 1) > (int64_t)FA_SPLITKV_SCRATCH_FLOATS)
        return FA_ERROR_INVALID_VALUE;
    if (rows == 0) return FA_SUCCESS;
    float* ws = nullptr;
    if (n_splits > 1) {
        ws = scratch_on_device();
        if (ws == nullptr) return FA_ERROR_LAUNCH_FAILURE;
    }
    // Every split writes its whole partial (O and LSE) before the merge reads
    // it, so nothing in the scratch has to start at zero.
    return fa_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, dtype, n_splits, ws, stream);
}

extern "C" fa_status_t fa_bwd_varlen_validate(const void* q, const void* k, const void* v, const void* o,
                                              const float* lse, const void* dout, const void* dq, const void* dk,
                                              const void* dv, const float* workspace, const int* cu_seqlens_q,
                                              const int* cu_seqlens_k, int n_seqs, int max_seqlen_q,
                                              int max_seqlen_k, int total_q, int total_k, int Hq, int Hkv, int d,
                                              int causal, float scale, fa_dtype_t dtype) {
    if (n_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0 || Hq < 1 || Hkv < 1 ||
        d < 1)
        return FA_ERROR_INVALID_VALUE;
    if (Hq % Hkv != 0) return FA_ERROR_INVALID_VALUE;
    if (causal != 0 && causal != 1) return FA_ERROR_INVALID_VALUE;
    if (!isfinite(scale)) return FA_ERROR_INVALID_VALUE;
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP8_E4M3 && dtype != FA_DTYPE_F32)
        return FA_ERROR_INVALID_VALUE;
    const int64_t q_elems = (int64_t)total_q * Hq * d;
    const int64_t kv_elems = (int64_t)total_k * Hkv * d;
    if (q_elems > kMaxElems || kv_elems > kMaxElems) return FA_ERROR_INVALID_VALUE;
    if ((int64_t)((max_seqlen_q + 127) / 128) * n_seqs * Hq > 0x7FFFFFFFLL ||
        (int64_t)((max_seqlen_k + 127) / 128) * n_seqs * Hkv > 0x7FFFFFFFLL)
        return FA_ERROR_INVALID_VALUE;
    if (n_seqs > 0) {
        if (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr) return FA_ERROR_INVALID_VALUE;
        if (!aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4)) return FA_ERROR_INVALID_VALUE;
    }
    if (q_elems > 0) {
        if (q == nullptr || o == nullptr || dout == nullptr || dq == nullptr || lse == nullptr ||
            workspace == nullptr)
            return FA_ERROR_INVALID_VALUE;
        if (!aligned(q, 16) || !aligned(o, 16) || !aligned(dout, 16) || !aligned(dq, 16) ||
            !aligned(lse, 4) || !aligned(workspace, 4))
            return FA_ERROR_INVALID_VALUE;
    }
    if (kv_elems > 0) {
        if (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr) return FA_ERROR_INVALID_VALUE;
        if (!aligned(k, 16) || !aligned(v, 16) || !aligned(dk, 16) || !aligned(dv, 16))
            return FA_ERROR_INVALID_VALUE;
    }
    if (dtype != FA_DTYPE_BF16) return FA_ERROR_NOT_SUPPORTED;
    if (d != 64 && d != 128) return FA_ERROR_NOT_SUPPORTED;
    return FA_SUCCESS;
}

extern "C" fa_status_t fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                     float* workspace, const int* cu_seqlens_q, const int* cu_seqlens_k,
                                     int n_seqs, int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                                     int Hq, int Hkv, int d, int causal, float scale, fa_dtype_t dtype,
                                     hipStream_t stream) {
    const fa_status_t st = fa_bwd_varlen_validate(q, k, v, o, lse, dout, dq, dk, dv, workspace, cu_seqlens_q,
                                                  cu_seqlens_k, n_seqs, max_seqlen_q, max_seqlen_k, total_q,
                                                  total_k, Hq, Hkv, d, causal, scale, dtype);
    if (st != FA_SUCCESS) return st;
    if (n_seqs == 0) return FA_SUCCESS;
    fa::BwdParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.dout = dout;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.ws = workspace;
    p.B = n_seqs;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Nq = max_seqlen_q;       // size the grids; each workgroup reads its sequence's lengths
    p.Nk = max_seqlen_k;
    p.group = Hq / Hkv;
    p.causal_shift = 0;
    p.c = scale * fa::kLog2e;
    p.scale = scale;
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.total_q = total_q;
    p.total_k = total_k;
    const hipError_t err = fa::launch_bwd_varlen(p, d, causal != 0, stream);
    return err == hipSuccess ? FA_SUCCESS : FA_ERROR_LAUNCH_FAILURE;
}

