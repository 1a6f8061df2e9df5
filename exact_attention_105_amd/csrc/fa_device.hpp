// Device-side building blocks of the attention forward kernels (gfx950 / CDNA4).
//
// Wave64 throughout.  The matrix products use the gfx950 MFMA instructions
//   v_mfma_f32_32x32x16_bf16      (bf16 in, fp32 accumulate)
//   v_mfma_f32_32x32x64_f8f6f4    (fp8 e4m3 in, fp32 accumulate)
// whose 32x32 fp32 result is spread over the wave as: lane l holds column
// n = l % 32 and rows 8*(i/4) + 4*(l/32) + (i%4) for its 16 accumulator
// registers i = 0..15.  Both kernels put the query index on the column (n)
// side, so every lane owns exactly one query row and the row statistics of
// the online softmax live in that lane (and its partner lane l ^ 32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_index.hpp"

namespace fa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;


__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp8 e4m3 x e4m3 (format code 0 for both operands), 32 bytes per lane per operand.
__device__ __forceinline__ f32x16 mfma_fp8_32x32x64(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Value of `x` combined over the lane pair (l, l ^ 32) with v_permlane32_swap.
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum and sum of the 16 accumulator values of one lane, as shallow trees
// (max3 steps / pairwise adds) instead of 15-long dependency chains.
__device__ __forceinline__ float max16(const f32x16& s) {
    const float a = fmaxf(fmaxf(s[0], s[1]), s[2]);
    const float b = fmaxf(fmaxf(s[3], s[4]), s[5]);
    const float c = fmaxf(fmaxf(s[6], s[7]), s[8]);
    const float d = fmaxf(fmaxf(s[9], s[10]), s[11]);
    const float e = fmaxf(fmaxf(s[12], s[13]), s[14]);
    return fmaxf(fmaxf(fmaxf(a, b), c), fmaxf(fmaxf(d, e), s[15]));
}

__device__ __forceinline__ float sum16(const f32x16& s) {
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = s[2 * i] + s[2 * i + 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = t[2 * i] + t[2 * i + 1];
    return (t[0] + t[1]) + (t[2] + t[3]);
}

// Two fp32 values to packed bf16 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// 16-byte global load / store through plain vector pointers.
__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ void lds_store16(char* base, uint32_t off, u32x4 v) {
    *reinterpret_cast<u32x4*>(base + off) = v;
}
__device__ __forceinline__ void lds_store8(char* base, uint32_t off, u32x2 v) {
    *reinterpret_cast<u32x2*>(base + off) = v;
}
__device__ __forceinline__ u32x4 lds_load16(const char* base, uint32_t off) {
    return *reinterpret_cast<const u32x4*>(base + off);
}


typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

// One wave-wide 16-byte-per-lane copy global -> LDS: lane i's 16 bytes come
// from gbase + voff (voff per lane) and land at lds + 16*i (lds wave-uniform,
// through M0).  Issued as inline asm so the compiler does not order later LDS
// reads behind it; completion is awaited explicitly (vmcnt) before the
// barrier that publishes a tile.  M0 is listed as clobbered; clang warns about
// clobbering a reserved register, so correctness rests on the compiler keeping
// no value of its own in M0 across these copies.  tests/test_m0_isa.py checks
// that on the generated assembly of every kernel that uses dma16 (clang's
// __builtin_amdgcn_global_load_lds, which manages M0 itself, makes the
// compiler wait for the copies in flight before the V^T reads: 9-15 % slower).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const char* gbase, uint32_t voff, uint32_t lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);   // keeps the operand scalar
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(m0), "v"(voff), "s"(gbase) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ i16x4 lds_tr16(const lds_char* p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
}

__device__ __forceinline__ bf16x8 lds_b128(const lds_char* p) {
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(p);
}

// vmcnt(n) with the other counters left alone (gfx9 encoding)
#define FA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | 0x0F70)

// Instruction order inside one MFMA phase (a scheduling region between two
// sched_barriers): the LDS operand reads of the first PF MFMAs (RPM reads per
// MFMA) first, then each MFMA followed by the reads of the MFMA PF places
// later, then the last PF MFMAs -- so that each MFMA finds its operand read
// PF MFMAs earlier instead of waiting on the read just before it.
template <int NMFMA, int RPM, int PF>
__device__ __forceinline__ void order_reads_ahead() {
    if constexpr (PF > 0) {
        constexpr int P = PF < NMFMA ? PF : NMFMA;
        __builtin_amdgcn_sched_group_barrier(0x100, P * RPM, 0);
#pragma unroll
        for (int i = 0; i < NMFMA - P; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, P, 0);
    }
}

// 8 bytes per lane through the 8-bit transposing LDS read: within each group
// of 16 lanes, lane i receives byte i%8 of the 8 bytes read by lanes
// i/8 + 2r, r = 0..7 (in that order).
__device__ __forceinline__ u32x2 lds_tr8(const lds_char* p) {
    typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
    const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p);
    return u32x2{(uint32_t)r[0], (uint32_t)r[1]};
}

__device__ __forceinline__ u32x4 lds_u128(const lds_char* p) {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p);
}

}  // namespace fa
