// Does vector-ALU work of one wave hide under the matrix instructions of
// another wave on the same SIMD?  The attention kernels rely on it: a wave's
// softmax (v_fma_f32, v_exp_f32) is meant to run while co-resident waves keep
// the MFMA pipe busy.
//
// One 512-thread workgroup (eight waves) per CU; waves 0-3 and 4-7 take one
// role each (waves w and w + 4 share SIMD w % 4).  Roles: idle (the wave only
// reads the clock), MFMA (2048 v_mfma_f32_32x32x16_bf16 in four independent
// accumulator chains), FMA (32768 v_fma_f32 in 16 independent chains), EXP
// (8192 v_exp_f32 in 16 chains).  Each wave reads s_memtime and
// s_memrealtime around its loop; the report gives, for each group of four
// waves, the span of its loops in shader cycles (first start to last end),
// alone (the other group idle) and next to the other group.  A group whose
// span does not grow next to the other one overlapped it completely.
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
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

enum Role { kIdle = 0, kMfma = 1, kFma = 2, kExp = 3 };
constexpr int kMfmaOps = 2048, kFmaIters = 2048, kExpIters = 512;

struct Times {
    long long cyc0, cyc1, rt0, rt1;
};

__device__ __forceinline__ void stamp(Times* t, bool end) {
    const long long c = __builtin_readcyclecounter();
    const long long r = __builtin_amdgcn_s_memrealtime();
    if (end) { t->cyc1 = c; t->rt1 = r; }
    else { t->cyc0 = c; t->rt0 = r; }
}

template <int ROLE>
__device__ __forceinline__ float run(float seed, Times* t) {
    float s = 0.f;
    if constexpr (ROLE == kMfma) {
        bf16x8 a, b;
        for (int i = 0; i < 8; ++i) { a[i] = (__bf16)(seed * (threadIdx.x + i)); b[i] = (__bf16)(seed * (i + 1)); }
        f32x16 c0{}, c1{}, c2{}, c3{};
        stamp(t, false);
        for (int it = 0; it < kMfmaOps / 4; ++it) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
        }
        stamp(t, true);
        for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    } else if constexpr (ROLE == kFma || ROLE == kExp) {
        float a[16];
        for (int i = 0; i < 16; ++i) a[i] = ROLE == kFma ? seed * (threadIdx.x + i) : 0.5f + seed * i;
        stamp(t, false);
        for (int it = 0; it < (ROLE == kFma ? kFmaIters : kExpIters); ++it) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if constexpr (ROLE == kFma) a[i] = fmaf(a[i], 0.999f, 0.001f);
                else a[i] = __builtin_amdgcn_exp2f(-a[i]);   // stays in [1/2, 1]
            }
        }
        stamp(t, true);
        for (int i = 0; i < 16; ++i) s += a[i];
    } else {
        stamp(t, false);
        stamp(t, true);
    }
    return s;
}

template <int LO, int HI>
__global__ __launch_bounds__(512) void coexec_kernel(float* out, Times* times, float seed) {
    const int w = threadIdx.x >> 6;
    Times t;
    const float s = w < 4 ? run<LO>(seed, &t) : run<HI>(seed, &t);
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    if ((threadIdx.x & 63) == 0) times[blockIdx.x * 8 + w] = t;
}

static Times h_times[1024 * 8];

// Span of the loops of waves [w0, w0 + 4) of every workgroup, in shader cycles.
static double span(int nblocks, int w0, double* mhz) {
    long long rt0 = -1, rt1 = -1;
    double clk = 0;
    int n = 0;
    for (int b = 0; b < nblocks; ++b)
        for (int w = w0; w < w0 + 4; ++w) {
            const Times& t = h_times[b * 8 + w];
            rt0 = (rt0 < 0 || t.rt0 < rt0) ? t.rt0 : rt0;
            rt1 = (rt1 < 0 || t.rt1 > rt1) ? t.rt1 : rt1;
            if (t.rt1 > t.rt0) {
                clk += (double)(t.cyc1 - t.cyc0) / (double)(t.rt1 - t.rt0);
                ++n;
            }
        }
    clk = n ? clk / n : 0;
    *mhz = clk * 100.0;
    return (double)(rt1 - rt0) * clk;
}

static const char* kName[] = {"idle", "MFMA", "FMA", "EXP"};

template <int LO, int HI>
static void run_case(int cus, float* out, Times* d_times) {
    hipLaunchKernelGGL((coexec_kernel<LO, HI>), dim3(cus), dim3(512), 0, 0, out, d_times, 0.001f);   // warm-up
    CHECK(hipDeviceSynchronize());
    hipLaunchKernelGGL((coexec_kernel<LO, HI>), dim3(cus), dim3(512), 0, 0, out, d_times, 0.001f);
    CHECK(hipDeviceSynchronize());
    CHECK(hipMemcpy(h_times, d_times, (size_t)cus * 8 * sizeof(Times), hipMemcpyDeviceToHost));
    double m0, m1;
    const double s0 = LO == kIdle ? 0 : span(cus, 0, &m0);
    const double s1 = HI == kIdle ? 0 : span(cus, 4, &m1);
    printf("| %-4s + %-4s | %10.0f | %10.0f | %6.0f |\n", kName[LO], kName[HI], s0, s1,
           LO != kIdle ? m0 : m1);
}

int main() {
    hipDeviceProp_t prop;
    CHECK(hipGetDeviceProperties(&prop, 0));
    const int cus = prop.multiProcessorCount;
    if (cus > 1024) return 1;
    float* out;
    Times* d_times;
    CHECK(hipMalloc(&out, (size_t)cus * 512 * sizeof(float)));
    CHECK(hipMalloc(&d_times, (size_t)cus * 8 * sizeof(Times)));
    printf("device %s, %d CUs; per SIMD one wave of each group: %d MFMAs, %d FMAs or %d exponentials per wave\n\n",
           prop.gcnArchName, cus, kMfmaOps, 16 * kFmaIters, 16 * kExpIters);
    printf("| waves 0-3 + waves 4-7 | span of waves 0-3 (shader cycles) | span of waves 4-7 | clock MHz |\n|---|---|---|---|\n");
    run_case<kMfma, kIdle>(cus, out, d_times);
    run_case<kIdle, kFma>(cus, out, d_times);
    run_case<kIdle, kExp>(cus, out, d_times);
    run_case<kMfma, kFma>(cus, out, d_times);
    run_case<kMfma, kExp>(cus, out, d_times);
    run_case<kMfma, kMfma>(cus, out, d_times);
    CHECK(hipFree(out));
    CHECK(hipFree(d_times));
    return 0;
}
