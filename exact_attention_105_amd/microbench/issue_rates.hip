// Microbenchmarks of the gfx950 instruction rates that decide the softmax
// design of the attention kernels: how much vector-ALU issue time an
// exponential (v_exp_f32) costs next to a fused multiply-add, whether the two
// overlap, what a polynomial exponential on the FMA pipe costs instead, the
// LDS read bandwidth of the two operand reads the kernels use, and the
// 32x32x16 bf16 matrix instruction rate.
//
// Each case is one kernel of 256-thread workgroups (one wave per SIMD per
// workgroup), WPS workgroups per CU, every wave running the same unrolled
// loop of independent chains.  Per wave, s_memtime (shader clock) and
// s_memrealtime (100 MHz) are read at the start and the end of the loop; the
// report gives, per SIMD, the shader cycles per wave-instruction: the kernel's
// loop span in shader cycles divided by the instructions all waves of one
// SIMD issued.  With one wave per SIMD that is the issue cost of one wave;
// with more it is the throughput of the SIMD.
//
// The polynomial exponential (software exp2, page "FlashAttention 4",
// centron.de, section on software exponential functions): Cody-Waite range
// reduction x = n + f with n = rint(x), |f| <= 1/2, 2^f by a degree-3
// polynomial fitted here by least squares in relative error on Chebyshev
// nodes of [-1/2, 1/2] (max relative error 7.8e-5, printed by the host), and
// 2^n applied with v_ldexp_f32.
#include <hip/hip_runtime.h>
#include <math.h>
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
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

constexpr int NIT = 2048;
constexpr float kP0 = 0.99992895f, kP1 = 0.69327623f, kP2 = 0.24260405f, kP3 = 0.05508868f;

__device__ __forceinline__ float poly_exp2(float x) {
    const float n = __builtin_rintf(x);
    const float f = x - n;
    const float p = fmaf(fmaf(fmaf(kP3, f, kP2), f, kP1), f, kP0);
    return __builtin_ldexpf(p, (int)n);
}

struct Times {
    long long cyc0, cyc1, rt0, rt1;
};

__device__ __forceinline__ void stamp(Times* t, bool end) {
    const long long c = __builtin_readcyclecounter();
    const long long r = __builtin_amdgcn_s_memrealtime();
    if (end) { t->cyc1 = c; t->rt1 = r; }
    else { t->cyc0 = c; t->rt0 = r; }
}

// MODE 0: fma x16; 1: exp x16; 2: fma x16 + exp x16 interleaved; 3: polynomial exp2 x16
template <int MODE>
__global__ __launch_bounds__(256) void valu_kernel(float* out, Times* times, float seed) {
    float a[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = seed * (threadIdx.x + i);
    float b[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) b[i] = seed * (i + 1);
    Times t;
    stamp(&t, false);
    for (int it = 0; it < NIT; ++it) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if constexpr (MODE == 0 || MODE == 2) a[i] = fmaf(a[i], 0.999f, 0.001f);
            // b stays in [1/2, 1]: 2^-b of a value in [0, 1]
            if constexpr (MODE == 1 || MODE == 2) b[i] = __builtin_amdgcn_exp2f(-b[i]);
            if constexpr (MODE == 3) b[i] = poly_exp2(-b[i]);
        }
    }
    stamp(&t, true);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += a[i] + b[i];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (threadIdx.x % 64 == 0) times[blockIdx.x * 4 + threadIdx.x / 64] = t;
}

// LDS reads: 8 independent reads per iteration, conflict-free addresses.
template <int KIND>
__global__ __launch_bounds__(256) void lds_kernel(uint32_t* out, Times* times) {
    __shared__ __attribute__((aligned(16))) char smem[65536];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = tid * 16; i < 65536; i += 256 * 16) *reinterpret_cast<u32x4*>(smem + i) = u32x4{(uint32_t)i, 1u, 2u, 3u};
    __syncthreads();
    typedef __attribute__((address_space(3))) char lchar;
    const lchar* ls = (const lchar*)smem;
    u32x4 acc = {0, 0, 0, 0};
    Times t;
    stamp(&t, false);
    for (int it = 0; it < NIT; ++it) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if constexpr (KIND == 0) {
                const int off = ((w * 8 + r + it) & 63) * 1024 + lane * 16;          // < 64 KiB
                acc ^= *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(ls + off);
            } else {
                typedef __attribute__((address_space(3))) i16x4 li16x4;
                const int off = ((w * 8 + r + it) & 63) * 1024 + lane * 8;           // < 64 KiB
                const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((li16x4*)(ls + off));
                acc[0] ^= (uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
                acc[1] ^= (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
            }
        }
    }
    stamp(&t, true);
    out[blockIdx.x * blockDim.x + tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (lane == 0) times[blockIdx.x * 4 + w] = t;
}

// 32x32x16 bf16 MFMA, four independent accumulator chains.
__global__ __launch_bounds__(256) void mfma_kernel(float* out, Times* times) {
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) { a[i] = (__bf16)(0.001f * (threadIdx.x + i)); b[i] = (__bf16)(0.002f * (i + threadIdx.x)); }
    f32x16 c0{}, c1{}, c2{}, c3{};
    Times t;
    stamp(&t, false);
    for (int it = 0; it < NIT / 4; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    stamp(&t, true);
    float s = 0.f;
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (threadIdx.x % 64 == 0) times[blockIdx.x * 4 + threadIdx.x / 64] = t;
}

static Times h_times[256 * 8 * 4];

// Shader cycles per SIMD over the loop span of all waves (first start to last
// end, in real time, converted with the waves' own clock), and that clock.
static void span(int nwaves, double* cycles, double* mhz) {
    long long rt0 = h_times[0].rt0, rt1 = h_times[0].rt1;
    double clk = 0;
    for (int i = 0; i < nwaves; ++i) {
        rt0 = h_times[i].rt0 < rt0 ? h_times[i].rt0 : rt0;
        rt1 = h_times[i].rt1 > rt1 ? h_times[i].rt1 : rt1;
        clk += (double)(h_times[i].cyc1 - h_times[i].cyc0) / (double)(h_times[i].rt1 - h_times[i].rt0);
    }
    clk /= nwaves;                                  // shader cycles per 10 ns tick
    *mhz = clk * 100.0;
    *cycles = (double)(rt1 - rt0) * clk;
}

template <typename F>
static void run_case(const char* name, F launch, int nblocks, double instr_per_wave, int wps) {
    Times* d_times;
    CHECK(hipMalloc(&d_times, sizeof(h_times)));
    launch(d_times);                                // warm-up
    CHECK(hipDeviceSynchronize());
    launch(d_times);
    CHECK(hipDeviceSynchronize());
    const int nw = nblocks * 4;
    CHECK(hipMemcpy(h_times, d_times, nw * sizeof(Times), hipMemcpyDeviceToHost));
    CHECK(hipFree(d_times));
    double cycles, mhz;
    span(nw, &cycles, &mhz);
    printf("| %-44s | %d | %7.2f | %6.0f |\n", name, wps, cycles / (instr_per_wave * wps), mhz);
}

int main() {
    hipDeviceProp_t prop;
    CHECK(hipGetDeviceProperties(&prop, 0));
    const int cus = prop.multiProcessorCount;
    float* out;
    CHECK(hipMalloc(&out, 256 * 8 * 256 * sizeof(float)));
    // host-side accuracy of the polynomial exponential
    double worst = 0;
    for (int i = -200000; i <= 200000; ++i) {
        const double x = i * 1e-4;
        const double n = rint(x), f = x - n;
        const double p = fma(fma(fma((double)kP3, f, (double)kP2), f, (double)kP1), f, (double)kP0);
        const double r = fabs(ldexp(p, (int)n) / exp2(x) - 1.0);
        worst = r > worst ? r : worst;
    }
    printf("device %s, %d CUs; polynomial exp2 max relative error on [-20, 20]: %.2e\n\n", prop.gcnArchName, cus, worst);
    printf("| case | waves per SIMD | shader cycles per wave-op per SIMD | clock MHz |\n|---|---|---|---|\n");
    for (int wps : {1, 2, 4}) {
        const int nb = cus * wps;
        run_case("v_fma_f32 (16 chains)", [&](Times* t) { hipLaunchKernelGGL(valu_kernel<0>, dim3(nb), dim3(256), 0, 0, out, t, 0.001f); }, nb, 16.0 * NIT, wps);
        run_case("v_exp_f32 (16 chains)", [&](Times* t) { hipLaunchKernelGGL(valu_kernel<1>, dim3(nb), dim3(256), 0, 0, out, t, 0.001f); }, nb, 16.0 * NIT, wps);
        run_case("v_fma_f32 + v_exp_f32 interleaved (per pair)", [&](Times* t) { hipLaunchKernelGGL(valu_kernel<2>, dim3(nb), dim3(256), 0, 0, out, t, 0.001f); }, nb, 16.0 * NIT, wps);
        run_case("polynomial exp2 (per exponential)", [&](Times* t) { hipLaunchKernelGGL(valu_kernel<3>, dim3(nb), dim3(256), 0, 0, out, t, 0.001f); }, nb, 16.0 * NIT, wps);
        run_case("32x32x16 bf16 MFMA, 4 chains (per MFMA)", [&](Times* t) { hipLaunchKernelGGL(mfma_kernel, dim3(nb), dim3(256), 0, 0, out, t); }, nb, (double)NIT, wps);
        run_case("ds_read_b128 (per read)", [&](Times* t) { hipLaunchKernelGGL(lds_kernel<0>, dim3(nb), dim3(256), 0, 0, (uint32_t*)out, t); }, nb, 8.0 * NIT, wps);
        run_case("ds_read_b64_tr_b16 (per read)", [&](Times* t) { hipLaunchKernelGGL(lds_kernel<1>, dim3(nb), dim3(256), 0, 0, (uint32_t*)out, t); }, nb, 8.0 * NIT, wps);
    }
    printf("\nLDS bytes per read per wave: ds_read_b128 1024, ds_read_b64_tr_b16 512; a CU has 4 SIMDs.\n");
    CHECK(hipFree(out));
    return 0;
}
