// The d = 64 forward kernel's per-tile instruction mix without memory: how
// busy can the MFMA pipe get when every wave alternates a matrix phase with a
// softmax phase that depends on it?
//
// Each wave loops over "tiles" of 32 keys against its 32 query rows:
//   S^T     4 dependent v_mfma_f32_32x32x16_bf16 (K fragments and Q operands
//           held in registers: no LDS),
//   softmax 16 x (v_fma_f32, v_exp_f32), 15 v_add_f32 for the row sum, 8
//           v_cvt_pk_bf16_f32 to form P,
//   O^T     4 v_mfma_f32_32x32x16_bf16 into two accumulators, B = P.
// The same mix as the kernel (8 MFMAs, 16 exponentials, 39 other VALU
// instructions per tile and wave), the same dependencies, no barriers and no
// LDS.  Workgroups of 256 threads (one wave per SIMD), WPS per CU (1-4; the
// kernel fits four waves per SIMD).  With and
// without raised wave priority (s_setprio 1) around the MFMA blocks, as the
// kernel does.  Reported per SIMD: shader cycles per tile of one wave, and
// the MFMA pipe's busy fraction, 8 MFMAs x 32 cycles x waves / cycles.
//
// Two more orders of the d = 128 bf16 mix over 64-key tiles (two 32-key
// halves, 32 MFMAs per tile): "both first" issues both halves' S^T before
// either half's softmax (the prefill kernel's order); "halves interleaved"
// issues the second half's S^T MFMAs in one basic block with the first
// half's softmax, and the first half's O^T MFMAs with the second half's
// softmax (one MFMA, then seven VALU instructions, by sched_group_barrier),
// then the second half's O^T and the next tile's first S^T.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#define CHECK(x)                                                                          \
    do {                                                                                  \
        hipError_t e_ = (x);                                                              \
        if (e_ != hipSuccess) {                                                           \
            printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);         \
            exit(1);                                                                      \
        }                                                                                 \
    } while (0)

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int kTiles = 512;

struct Times {
    long long cyc0, cyc1, rt0, rt1;
};

__device__ __forceinline__ void stamp(Times* t, bool end) {
    const long long c = __builtin_readcyclecounter();
    const long long r = __builtin_amdgcn_s_memrealtime();
    if (end) { t->cyc1 = c; t->rt1 = r; }
    else { t->cyc0 = c; t->rt0 = r; }
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// D = 64 or 128: the bf16 tile of 32 keys (D / 16 S^T MFMAs, D / 16 O^T MFMAs
// into D / 32 accumulators).  D = 8 stands for the fp8 tile of 64 keys: two
// 32x32x64 fp8 MFMAs per 32-key half for S^T, the per-lane maximum of the 32
// raw scores (the kernel's threshold test), 32 exponentials, the row sum,
// 16 v_cvt_pk_fp8_f32, and four fp8 MFMAs for O^T.
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

// Softmax of one 32-key half: exponentials, row sum into l, P as two bf16 B operands.
__device__ __forceinline__ void softmax_half(f32x16& s, float c, float m, float& l, bf16x8& pa, bf16x8& pb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c, -m));
    float t8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t8[i] = s[2 * i] + s[2 * i + 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) t8[i] = t8[2 * i] + t8[2 * i + 1];
    l += (t8[0] + t8[1]) + (t8[2] + t8[3]);
    u32x4 p0, p1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        p0[e] = pack2(s[2 * e], s[2 * e + 1]);
        p1[e] = pack2(s[8 + 2 * e], s[8 + 2 * e + 1]);
    }
    pa = __builtin_bit_cast(bf16x8, p0);
    pb = __builtin_bit_cast(bf16x8, p1);
}

// 1: d = 128, 64-key tiles, both halves' S^T first; 2: halves interleaved.
template <int ORDER, bool PRIO>
__global__ __launch_bounds__(256, 3) void phases64_kernel(float* out, Times* times, float seed) {
    constexpr int KS = 8, DB = 4;
    bf16x8 kf[KS], qf[KS];
    for (int j = 0; j < KS; ++j)
        for (int i = 0; i < 8; ++i) {
            kf[j][i] = (__bf16)(seed * (threadIdx.x + i + j));
            qf[j][i] = (__bf16)(seed * (i + 1 + j));
        }
    f32x16 o[DB];
    for (int db = 0; db < DB; ++db) o[db] = f32x16{};
    float l = 0.f, m = 0.f;
    const float c = 0.18f;
    auto scores = [&](int h) {
        f32x16 s{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[(ks + h) % KS], qf[ks], s, 0, 0, 0);
        return s;
    };
    auto accumulate = [&](int h, bf16x8 pa, bf16x8 pb) {
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[(db + h) % KS], pa, o[db], 0, 0, 0);
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[(db + h + 1) % KS], pb, o[db], 0, 0, 0);
    };
    auto interleave8 = [] {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
        }
    };
    Times t;
    stamp(&t, false);
    f32x16 s0 = scores(0);
    for (int it = 0; it < kTiles; ++it) {
        bf16x8 p0a, p0b, p1a, p1b;
        if constexpr (ORDER == 1) {
            if (PRIO) __builtin_amdgcn_s_setprio(1);
            if (it > 0) s0 = scores(0);
            f32x16 s1 = scores(1);
            if (PRIO) __builtin_amdgcn_s_setprio(0);
            softmax_half(s0, c, m, l, p0a, p0b);
            softmax_half(s1, c, m, l, p1a, p1b);
            if (PRIO) __builtin_amdgcn_s_setprio(1);
            accumulate(0, p0a, p0b);
            accumulate(1, p1a, p1b);
            if (PRIO) __builtin_amdgcn_s_setprio(0);
        } else {
            __builtin_amdgcn_sched_barrier(0);
            f32x16 s1 = scores(1);
            softmax_half(s0, c, m, l, p0a, p0b);
            interleave8();
            __builtin_amdgcn_sched_barrier(0);
            accumulate(0, p0a, p0b);
            softmax_half(s1, c, m, l, p1a, p1b);
            interleave8();
            __builtin_amdgcn_sched_barrier(0);
            if (PRIO) __builtin_amdgcn_s_setprio(1);
            accumulate(1, p1a, p1b);
            s0 = scores(0);
            if (PRIO) __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_sched_barrier(0);
        }
        m += 1e-9f * l;                         // keeps the loop from being hoisted
    }
    stamp(&t, true);
    float r = l + m + s0[0];
    for (int db = 0; db < DB; ++db)
        for (int i = 0; i < 16; ++i) r += o[db][i];
    out[blockIdx.x * blockDim.x + threadIdx.x] = r;
    if ((threadIdx.x & 63) == 0) times[blockIdx.x * 4 + (threadIdx.x >> 6)] = t;
}

template <int D, bool PRIO>
__global__ __launch_bounds__(256, D == 64 ? 4 : 3) void phases_kernel(float* out, Times* times, float seed) {
    constexpr int KS = D == 8 ? 2 : D / 16;          // S^T MFMAs per 32 keys
    constexpr int DB = D == 8 ? 4 : D / 32;          // O^T accumulators
    // K (also standing in for V^T) and Q operands; their values do not matter
    bf16x8 kf[KS], qf[KS];
    i32x8 k8[2], q8[2];
    for (int j = 0; j < KS; ++j)
        for (int i = 0; i < 8; ++i) {
            kf[j][i] = (__bf16)(seed * (threadIdx.x + i + j));
            qf[j][i] = (__bf16)(seed * (i + 1 + j));
        }
    for (int j = 0; j < 2; ++j)
        for (int i = 0; i < 8; ++i) {
            k8[j][i] = (int)(0x38383838u + threadIdx.x + i + j);   // e4m3 codes near 1
            q8[j][i] = (int)(0x30303030u + i + j);
        }
    f32x16 o[DB];
    for (int db = 0; db < DB; ++db) o[db] = f32x16{};
    float l = 0.f, m = 0.f, thr = 1e30f;
    const float c = 0.18f;
    Times t;
    stamp(&t, false);
    for (int it = 0; it < kTiles; ++it) {
        if constexpr (D == 8) {
            f32x16 s[2];
            if (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                s[kh] = f32x16{};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    s[kh] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k8[ks], q8[ks], s[kh], 0, 0, 0, 0, 0, 0);
            }
            if (PRIO) __builtin_amdgcn_s_setprio(0);
            float mx = s[0][0];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kh][i]);
            if (__builtin_amdgcn_ballot_w64(mx > thr) != 0) thr = mx;      // never taken
            float sum = 0.f;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    s[kh][i] = __builtin_amdgcn_exp2f(fmaf(s[kh][i], c, -m));
                    sum += s[kh][i];
                }
            l += sum;
            i32x8 pb;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    int r = __builtin_amdgcn_cvt_pk_fp8_f32(s[kh][4 * q4], s[kh][4 * q4 + 1], 0, false);
                    pb[4 * kh + q4] = __builtin_amdgcn_cvt_pk_fp8_f32(s[kh][4 * q4 + 2], s[kh][4 * q4 + 3], r, true);
                }
            if (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int db = 0; db < 4; ++db)
                o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k8[db & 1], pb, o[db], 0, 0, 0, 0, 0, 0);
            if (PRIO) __builtin_amdgcn_s_setprio(0);
        } else {
            if (PRIO) __builtin_amdgcn_s_setprio(1);
            f32x16 s{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s, 0, 0, 0);
            if (PRIO) __builtin_amdgcn_s_setprio(0);
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c, -m));
            float t8[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) t8[i] = s[2 * i] + s[2 * i + 1];
#pragma unroll
            for (int i = 0; i < 4; ++i) t8[i] = t8[2 * i] + t8[2 * i + 1];
            l += (t8[0] + t8[1]) + (t8[2] + t8[3]);
            u32x4 p0, p1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p0[e] = pack2(s[2 * e], s[2 * e + 1]);
                p1[e] = pack2(s[8 + 2 * e], s[8 + 2 * e + 1]);
            }
            const bf16x8 pb0 = __builtin_bit_cast(bf16x8, p0), pb1 = __builtin_bit_cast(bf16x8, p1);
            if (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[db % KS], pb0, o[db], 0, 0, 0);
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[(db + 1) % KS], pb1, o[db], 0, 0, 0);
            if (PRIO) __builtin_amdgcn_s_setprio(0);
        }
        m += 1e-9f * l;                         // keeps the loop from being hoisted
    }
    stamp(&t, true);
    float r = l + m + thr;
    for (int db = 0; db < DB; ++db)
        for (int i = 0; i < 16; ++i) r += o[db][i];
    out[blockIdx.x * blockDim.x + threadIdx.x] = r;
    if ((threadIdx.x & 63) == 0) times[blockIdx.x * 4 + (threadIdx.x >> 6)] = t;
}

static Times h_times[256 * 8 * 4];

// MFMA pipe cycles per tile and wave: 32 per bf16 32x32x16, 64 per fp8 32x32x64.
// D = 1 and 2 select phases64_kernel's orders (32 MFMAs per 64-key tile).
template <int D>
static void run(int cus, float* out, Times* d_times, int max_wps, const char* name) {
    const double mfma_cycles = D == 8 ? 8 * 64.0 : D <= 2 ? 32 * 32.0 : 2 * (D / 16) * 32.0;
    for (int wps = 1; wps <= max_wps; ++wps)
        for (int prio = 0; prio < 2; ++prio) {
            const int nb = cus * wps;
            for (int rep = 0; rep < 2; ++rep) {
                if constexpr (D <= 2) {
                    if (prio) hipLaunchKernelGGL((phases64_kernel<D, true>), dim3(nb), dim3(256), 0, 0, out, d_times, 0.001f);
                    else hipLaunchKernelGGL((phases64_kernel<D, false>), dim3(nb), dim3(256), 0, 0, out, d_times, 0.001f);
                } else {
                    if (prio) hipLaunchKernelGGL((phases_kernel<D, true>), dim3(nb), dim3(256), 0, 0, out, d_times, 0.001f);
                    else hipLaunchKernelGGL((phases_kernel<D, false>), dim3(nb), dim3(256), 0, 0, out, d_times, 0.001f);
                }
                CHECK(hipDeviceSynchronize());
            }
            CHECK(hipMemcpy(h_times, d_times, (size_t)nb * 4 * sizeof(Times), hipMemcpyDeviceToHost));
            long long rt0 = h_times[0].rt0, rt1 = h_times[0].rt1;
            double clk = 0;
            for (int i = 0; i < nb * 4; ++i) {
                rt0 = h_times[i].rt0 < rt0 ? h_times[i].rt0 : rt0;
                rt1 = h_times[i].rt1 > rt1 ? h_times[i].rt1 : rt1;
                clk += (double)(h_times[i].cyc1 - h_times[i].cyc0) / (double)(h_times[i].rt1 - h_times[i].rt0);
            }
            clk /= nb * 4;
            const double per_tile = (double)(rt1 - rt0) * clk / kTiles;   // all wps waves of a SIMD each did kTiles
            printf("| %s | %d | %s | %7.1f | %.3f | %6.0f |\n", name, wps, prio ? "yes" : "no", per_tile / wps,
                   mfma_cycles * wps / per_tile, clk * 100.0);
        }
}

int main() {
    hipDeviceProp_t prop;
    CHECK(hipGetDeviceProperties(&prop, 0));
    const int cus = prop.multiProcessorCount;
    if (cus > 256) return 1;
    float* out;
    Times* d_times;
    CHECK(hipMalloc(&out, (size_t)cus * 8 * 256 * sizeof(float)));
    CHECK(hipMalloc(&d_times, sizeof(h_times)));
    printf("device %s, %d CUs; %d tiles per wave\n\n", prop.gcnArchName, cus, kTiles);
    printf("| tile | waves per SIMD | s_setprio around MFMAs | shader cycles per tile per wave | MFMA busy | clock MHz |\n|---|---|---|---|---|---|\n");
    run<64>(cus, out, d_times, 4, "bf16 d=64, 32 keys");
    run<128>(cus, out, d_times, 3, "bf16 d=128, 32 keys");
    run<1>(cus, out, d_times, 3, "bf16 d=128, 64 keys, both halves' S^T first");
    run<2>(cus, out, d_times, 3, "bf16 d=128, 64 keys, halves interleaved");
    run<8>(cus, out, d_times, 3, "fp8 d=128, 64 keys");
    CHECK(hipFree(out));
    CHECK(hipFree(d_times));
    return 0;
}
