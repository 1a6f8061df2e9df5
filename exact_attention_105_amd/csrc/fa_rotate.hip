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
// Layout: lane l of a wave holds 16 contiguous elements of one row -- elements
// 16*(l % L) .. 16*(l % L)+15 of row l / L of a chunk of R = 1024 / d rows
// (L = d / 16 lanes per row; a chunk is 1024 contiguous elements, 64 B (fp32)
// or 32 B (bf16) per lane).  The fast Walsh-Hadamard transform runs in
// registers: the strides 1..8 inside a lane (one add or subtract per element),
// the strides 16*m (m < L) as an exchange with lane l ^ m, which is a DPP lane
// permutation within 8 lanes (no LDS traffic).  1/sqrt(d) is folded into the
// maximum and into the quantisation multiplier.  Each wave keeps kRotChunks
// chunks in flight to cover the memory latency.
#include <algorithm>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

#ifndef FA_ROT_CHUNKS
#define FA_ROT_CHUNKS 2                   // chunks per wave per iteration
#endif
#ifndef FA_ROT_MAX_BLOCKS
#define FA_ROT_MAX_BLOCKS 1024            // 4 workgroups (16 waves) per CU
#endif
constexpr int kRotChunks = FA_ROT_CHUNKS;
constexpr int kRotBlock = 256;            // threads per workgroup
constexpr int kEl = 16;                   // elements per lane
constexpr int kChunk = 64 * kEl;          // elements per chunk

__device__ __forceinline__ void load_lane(const float* src, float (&v)[kEl]) {
#pragma unroll
    for (int i = 0; i < kEl / 4; ++i) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(src + 4 * i);
#pragma unroll
        for (int k = 0; k < 4; ++k) v[4 * i + k] = t[k];
    }
}
__device__ __forceinline__ void load_lane(const __bf16* src, float (&v)[kEl]) {
#pragma unroll
    for (int i = 0; i < kEl / 8; ++i) {
        const u32x4 t = *reinterpret_cast<const u32x4*>(src + 8 * i);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t w = t[k];
            v[8 * i + 2 * k] = __uint_as_float(w << 16);
            v[8 * i + 2 * k + 1] = __uint_as_float(w & 0xFFFF0000u);
        }
    }
}

// The value v holds in lane l ^ M (M = 1, 2, 4), as DPP permutations:
// quad_perm [1,0,3,2] is l ^ 1, quad_perm [2,3,0,1] is l ^ 2, and l ^ 4 is
// row_half_mirror (l ^ 7 within 8 lanes) after quad_perm [3,2,1,0] (l ^ 3).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
    static_assert(M == 1 || M == 2 || M == 4, "exchange within 8 lanes");
    if constexpr (M == 1) return dpp<0xB1>(v);
    else if constexpr (M == 2) return dpp<0x4E>(v);
    else return dpp<0x141>(dpp<0x1B>(v));
}

template <int M, int L>
__device__ __forceinline__ void cross_stage(float (&v)[kEl], int lane) {
    if constexpr (M < L) {
        // lower lane: v + partner; upper lane: partner - v
        const uint32_t neg = (lane & M) ? 0x80000000u : 0u;
#pragma unroll
        for (int e = 0; e < kEl; ++e) {
            const float q = lane_xor<M>(v[e]);
            v[e] = q + __uint_as_float(__float_as_uint(v[e]) ^ neg);
        }
        cross_stage<2 * M, L>(v, lane);
    }
}

// x D H for the lane's part of a row (no 1/sqrt(d)): signs as XOR masks on
// the float bits, then the butterflies of the fast Walsh-Hadamard transform
// in natural (Sylvester) order.  Every lane of the wave must call it.
template <int L>
__device__ __forceinline__ void rotate_row(float (&v)[kEl], const uint32_t (&flip)[kEl], int lane) {
#pragma unroll
    for (int e = 0; e < kEl; ++e) v[e] = __uint_as_float(__float_as_uint(v[e]) ^ flip[e]);
#pragma unroll
    for (int h = 1; h < kEl; h <<= 1)
#pragma unroll
        for (int e = 0; e < kEl; ++e)
            if ((e & h) == 0) {
                const float a = v[e], b = v[e + h];
                v[e] = a + b;
                v[e + h] = a - b;
            }
    cross_stage<1, L>(v, lane);
}

template <typename T, int D>
struct Lane {
    static constexpr int L = D / kEl, R = kChunk / D;
    int lane, sub;
    uint32_t flip[kEl];
    __device__ explicit Lane(const RotParams& p) : lane(threadIdx.x & 63), sub((threadIdx.x & 63) / L) {
#pragma unroll
        for (int e = 0; e < kEl; ++e) {
            const int j = kEl * (lane % L) + e;
            flip[e] = (p.rotate && ((p.sign_bits[j >> 5] >> (j & 31)) & 1)) ? 0x80000000u : 0u;
        }
    }
    // load chunk c (rows past the end read as zeros)
    __device__ void chunk(const RotParams& p, int64_t c, float (&v)[kEl]) const {
        if (c * R + sub < p.rows) {
            load_lane(reinterpret_cast<const T*>(p.x) + c * kChunk + kEl * lane, v);
        } else {
#pragma unroll
            for (int e = 0; e < kEl; ++e) v[e] = 0.f;
        }
    }
};

__global__ void rot_clear(unsigned* work) { *work = 0u; }

template <typename T, int D>
__global__ __launch_bounds__(kRotBlock) void rot_amax(RotParams p) {
    using Ln = Lane<T, D>;
    constexpr int L = Ln::L, R = Ln::R;
    const Ln ln(p);
    const int64_t wave = ((int64_t)blockIdx.x * kRotBlock + threadIdx.x) >> 6;
    const int64_t n_waves = ((int64_t)gridDim.x * kRotBlock) >> 6;
    const int64_t n_chunks = (p.rows + R - 1) / R;
    float amax = 0.f;                              // of x D H, before 1/sqrt(d)
    for (int64_t c0 = wave * kRotChunks; c0 < n_chunks; c0 += n_waves * kRotChunks) {
        float v[kRotChunks][kEl];
#pragma unroll
        for (int k = 0; k < kRotChunks; ++k)
            if (c0 + k < n_chunks) ln.chunk(p, c0 + k, v[k]);
#pragma unroll
        for (int k = 0; k < kRotChunks; ++k) {
            if (c0 + k >= n_chunks) break;                 // wave-uniform
            if (p.rotate) rotate_row<L>(v[k], ln.flip, ln.lane);
#pragma unroll
            for (int e = 0; e < kEl; ++e) amax = fmaxf(amax, fabsf(v[k][e]));
        }
    }
    // fl(norm * y) is monotonic in y, so scaling the maximum equals the
    // maximum of the scaled values
    if (p.rotate) amax *= D == 128 ? 0.08838834764831845f : 0.125f;
    // wave, then workgroup, then one device-scope atomic per workgroup: all
    // atomics hit one address and the device serialises them, so their number
    // (not the bytes) sets the kernel's time when every wave issues one.  The
    // stored maximum only grows, so a workgroup whose maximum does not exceed
    // a value already read from it skips the atomic.
    __shared__ float wave_max[kRotBlock / 64];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    if (ln.lane == 0) wave_max[threadIdx.x >> 6] = amax;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 1; w < kRotBlock / 64; ++w) amax = fmaxf(amax, wave_max[w]);
        const unsigned seen = __hip_atomic_load(p.work, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__float_as_uint(amax) > seen) atomicMax(p.work, __float_as_uint(amax));
    }
}

template <typename T, int D>
__global__ __launch_bounds__(kRotBlock) void rot_quant(RotParams p) {
    using Ln = Lane<T, D>;
    constexpr int L = Ln::L, R = Ln::R;
    const Ln ln(p);
    const int64_t wave = ((int64_t)blockIdx.x * kRotBlock + threadIdx.x) >> 6;
    const int64_t n_waves = ((int64_t)gridDim.x * kRotBlock) >> 6;
    const int64_t n_chunks = (p.rows + R - 1) / R;
    const float amax = __uint_as_float(*p.work);
    if (blockIdx.x == 0 && threadIdx.x == 0) *p.scale = amax > 0.f ? amax / 448.0f : 1.0f;
    // one multiplier per element: 1/sqrt(d) (when rotating) times 448 / amax
    const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
    const float mul = p.rotate ? inv * (D == 128 ? 0.08838834764831845f : 0.125f) : inv;
    for (int64_t c0 = wave * kRotChunks; c0 < n_chunks; c0 += n_waves * kRotChunks) {
        float v[kRotChunks][kEl];
#pragma unroll
        for (int k = 0; k < kRotChunks; ++k)
            if (c0 + k < n_chunks) ln.chunk(p, c0 + k, v[k]);
#pragma unroll
        for (int k = 0; k < kRotChunks; ++k) {
            if (c0 + k >= n_chunks) break;                 // wave-uniform
            if (p.rotate) rotate_row<L>(v[k], ln.flip, ln.lane);
            // v_cvt_pk_fp8_f32 converts two floats to OCP E4M3 (round to
            // nearest even) into the low or high half of a word
            u32x4 packed;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                float q[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) q[i] = fminf(fmaxf(v[k][4 * w + i] * mul, -448.0f), 448.0f);
                int word = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
                word = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], word, true);
                packed[w] = (uint32_t)word;
            }
            if ((c0 + k) * R + ln.sub < p.rows)
                *reinterpret_cast<u32x4*>(p.codes + (c0 + k) * kChunk + kEl * ln.lane) = packed;
        }
    }
}

template <typename T, int D>
hipError_t launch_rot(const RotParams& p, hipStream_t stream) {
    RotParams pp = p;
    constexpr int R = Lane<T, D>::R;
    // at most one wave per kRotChunks chunks, at most FA_ROT_MAX_BLOCKS workgroups
    const int64_t n_chunks = (p.rows + R - 1) / R;
    const int64_t waves_needed = (n_chunks + kRotChunks - 1) / kRotChunks;
    const int64_t blocks = std::min<int64_t>(std::max<int64_t>((waves_needed + 3) / 4, 1), FA_ROT_MAX_BLOCKS);
    void* args[] = {&pp};
    void* cargs[] = {&pp.work};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&rot_clear), dim3(1), dim3(1), cargs, 0, stream);
    if (e != hipSuccess) return e;
    e = hipLaunchKernel(reinterpret_cast<const void*>(&rot_amax<T, D>), dim3((unsigned)blocks), dim3(kRotBlock),
                        args, 0, stream);
    if (e != hipSuccess) return e;
    return hipLaunchKernel(reinterpret_cast<const void*>(&rot_quant<T, D>), dim3((unsigned)blocks),
                           dim3(kRotBlock), args, 0, stream);
}

}  // namespace

hipError_t launch_rotate_quantize(const RotParams& p, bool x_is_f32, int d, hipStream_t stream) {
    if (d == 128) return x_is_f32 ? launch_rot<float, 128>(p, stream) : launch_rot<__bf16, 128>(p, stream);
    if (d == 64) return x_is_f32 ? launch_rot<float, 64>(p, stream) : launch_rot<__bf16, 64>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa
