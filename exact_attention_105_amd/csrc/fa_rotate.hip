// Incoherent processing before FP8 attention, gfx950: every row of a tensor is
// multiplied by M = D H / sqrt(d) (D = diag of random signs, H the d x d
// Sylvester-Hadamard matrix) and the result is quantised per tensor to OCP
// E4M3 (page "FlashAttention-3 (DE)", systems-analysis.ru, technical
// innovation 3: a random orthogonal transform of Q and K spreads outlier
// features over all coordinates before the FP8 quantisation and leaves
// Q K^T unchanged).
//
// The work is a stream over the tensor (HBM-bound), in three launches:
//   1. clear the amax word of the caller's workspace (one thread; a kernel,
//      not a memset, so the sequence can be captured into a graph);
//   2. rotate every row and fold max |y| into the amax word (atomic max on
//      the bit pattern: for non-negative floats it orders like the value);
//   3. rotate every row again, scale by 448 / amax and convert to E4M3
//      (round to nearest even, clamped to +-448); workgroup 0 writes the
//      per-tensor scale amax / 448.
// Recomputing the rotation costs a second read of the input and saves a
// rotated copy (a write and a read of a float per element).
//
// Layout: each wave owns whole rows; lane l holds elements E*l .. E*l+E-1 of a
// row (E = d / 64).  The fast Walsh-Hadamard transform runs in registers: the
// stride-1 butterfly stage inside a lane when E = 2, every wider stage as one
// cross-lane exchange (__shfl_xor) per element.  Each wave keeps four rows in
// flight to cover the memory latency.
#include <algorithm>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

constexpr int kRotRows = 4;           // rows per wave per iteration
constexpr int kRotBlock = 256;        // threads per workgroup

template <typename T, int E>
struct RowIO;

template <>
struct RowIO<float, 2> {              // d = 128, fp32: 8 bytes per lane
    __device__ static void load(const void* x, int64_t row, int lane, float (&v)[2]) {
        const f32x2 t = *reinterpret_cast<const f32x2*>(reinterpret_cast<const float*>(x) + row * 128 + 2 * lane);
        v[0] = t[0];
        v[1] = t[1];
    }
};
template <>
struct RowIO<float, 1> {              // d = 64, fp32
    __device__ static void load(const void* x, int64_t row, int lane, float (&v)[1]) {
        v[0] = reinterpret_cast<const float*>(x)[row * 64 + lane];
    }
};
template <>
struct RowIO<__bf16, 2> {             // d = 128, bf16: 4 bytes per lane
    __device__ static void load(const void* x, int64_t row, int lane, float (&v)[2]) {
        const uint32_t t = reinterpret_cast<const uint32_t*>(x)[row * 64 + lane];
        v[0] = __uint_as_float(t << 16);
        v[1] = __uint_as_float(t & 0xFFFF0000u);
    }
};
template <>
struct RowIO<__bf16, 1> {             // d = 64, bf16
    __device__ static void load(const void* x, int64_t row, int lane, float (&v)[1]) {
        const uint16_t t = reinterpret_cast<const uint16_t*>(x)[row * 64 + lane];
        v[0] = __uint_as_float((uint32_t)t << 16);
    }
};

// Rotate one row in place: signs (as XOR masks on the float bits), the
// butterflies of the fast Walsh-Hadamard transform in natural (Sylvester)
// order, then 1/sqrt(d).
template <int E>
__device__ __forceinline__ void rotate_row(float (&v)[E], const uint32_t (&flip)[E], int lane, float norm) {
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = __uint_as_float(__float_as_uint(v[e]) ^ flip[e]);
    if (E == 2) {
        const float a = v[0], b = v[E - 1];
        v[0] = a + b;
        v[E - 1] = a - b;
    }
    // stride h (in elements) pairs lane l with lane l ^ (h / E)
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float p = __shfl_xor(v[e], m, 64);
            v[e] = upper ? p - v[e] : v[e] + p;
        }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] *= norm;
}

__global__ void rot_clear(unsigned* work) { *work = 0u; }

template <typename T, int E>
__global__ __launch_bounds__(kRotBlock) void rot_amax(RotParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * kRotBlock + threadIdx.x) >> 6;
    const int64_t n_waves = ((int64_t)gridDim.x * kRotBlock) >> 6;
    uint32_t flip[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int j = E * lane + e;
        flip[e] = (p.rotate && ((p.sign_bits[j >> 5] >> (j & 31)) & 1)) ? 0x80000000u : 0u;
    }
    const float norm = E == 2 ? 0.08838834764831845f : 0.125f;   // 1 / sqrt(d)
    float amax = 0.f;
    for (int64_t r0 = wave * kRotRows; r0 < p.rows; r0 += n_waves * kRotRows) {
        float v[kRotRows][E];
#pragma unroll
        for (int k = 0; k < kRotRows; ++k)
            if (r0 + k < p.rows) RowIO<T, E>::load(p.x, r0 + k, lane, v[k]);
#pragma unroll
        for (int k = 0; k < kRotRows; ++k) {
            if (r0 + k >= p.rows) break;
            if (p.rotate) rotate_row<E>(v[k], flip, lane, norm);
#pragma unroll
            for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(v[k][e]));
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    if (lane == 0 && amax > 0.f) atomicMax(p.work, __float_as_uint(amax));
}

template <typename T, int E>
__global__ __launch_bounds__(kRotBlock) void rot_quant(RotParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * kRotBlock + threadIdx.x) >> 6;
    const int64_t n_waves = ((int64_t)gridDim.x * kRotBlock) >> 6;
    const float amax = __uint_as_float(*p.work);
    const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0) *p.scale = amax > 0.f ? amax / 448.0f : 1.0f;
    uint32_t flip[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int j = E * lane + e;
        flip[e] = (p.rotate && ((p.sign_bits[j >> 5] >> (j & 31)) & 1)) ? 0x80000000u : 0u;
    }
    const float norm = E == 2 ? 0.08838834764831845f : 0.125f;
    for (int64_t r0 = wave * kRotRows; r0 < p.rows; r0 += n_waves * kRotRows) {
        float v[kRotRows][E];
#pragma unroll
        for (int k = 0; k < kRotRows; ++k)
            if (r0 + k < p.rows) RowIO<T, E>::load(p.x, r0 + k, lane, v[k]);
#pragma unroll
        for (int k = 0; k < kRotRows; ++k) {
            if (r0 + k >= p.rows) break;
            if (p.rotate) rotate_row<E>(v[k], flip, lane, norm);
            float q[2];
#pragma unroll
            for (int e = 0; e < E; ++e) q[e] = fminf(fmaxf(v[k][e] * inv, -448.0f), 448.0f);
            if (E == 1) q[1] = 0.f;
            // v_cvt_pk_fp8_f32: two values to OCP E4M3, round to nearest even
            const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
            uint8_t* dst = p.codes + (r0 + k) * (64 * E) + E * lane;
            if (E == 2)
                *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(packed & 0xFFFF);
            else
                *dst = (uint8_t)(packed & 0xFF);
        }
    }
}

template <typename T, int E>
hipError_t launch_rot(const RotParams& p, hipStream_t stream) {
    RotParams pp = p;
    // enough waves to cover the chip several times over, at most one per kRotRows rows
    const int64_t waves_needed = (p.rows + kRotRows - 1) / kRotRows;
    const int64_t blocks = std::min<int64_t>(std::max<int64_t>((waves_needed + 3) / 4, 1), 4096);
    void* args[] = {&pp};
    void* cargs[] = {&pp.work};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&rot_clear), dim3(1), dim3(1), cargs, 0, stream);
    if (e != hipSuccess) return e;
    e = hipLaunchKernel(reinterpret_cast<const void*>(&rot_amax<T, E>), dim3((unsigned)blocks), dim3(kRotBlock),
                        args, 0, stream);
    if (e != hipSuccess) return e;
    return hipLaunchKernel(reinterpret_cast<const void*>(&rot_quant<T, E>), dim3((unsigned)blocks),
                           dim3(kRotBlock), args, 0, stream);
}

}  // namespace

hipError_t launch_rotate_quantize(const RotParams& p, bool x_is_f32, int d, hipStream_t stream) {
    if (d == 128) return x_is_f32 ? launch_rot<float, 2>(p, stream) : launch_rot<__bf16, 2>(p, stream);
    if (d == 64) return x_is_f32 ? launch_rot<float, 1>(p, stream) : launch_rot<__bf16, 1>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa
