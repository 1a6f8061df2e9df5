// Fused exact-attention forward pass, FP8 (OCP E4M3) inputs, head dim 128, gfx950.
//
// Low-precision attention (page "FlashAttention-3 (DE)", systems-analysis.ru,
// section on low precision: FP8 doubles the matrix throughput at the cost of
// dynamic range).  The structure follows the bf16 kernel (fa_fwd_bf16.hip):
// 128 query rows per workgroup, 64-key K/V tiles in double-buffered LDS, the
// query index on the MFMA column side so each lane owns one query row, and
// the online softmax in registers.  Differences:
//   * both products use v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3 -> fp32);
//   * the per-tensor scales are folded in: the exponent constant is
//     |scale| * sq * sk * log2(e), and the normalised output is multiplied
//     by sv;
//   * P is quantised to e4m3 for the second product after multiplying by
//     2^8 (added to the exp2 argument), so probabilities down to 2^-14 stay
//     in e4m3's normal range; the row sum uses the unquantised fp32 values
//     in the same 2^8 units, and the log-sum-exp removes the offset again.
// One 32x32x64 product covers a 64-key tile, so each lane feeds 32 keys of P:
// the 16 scores it holds of each 32-key half, in register order.  V^T rows
// in LDS hold those keys at positions 32*(l/32) + slot, which maps 4-key
// units as pu = 8*(ku & 1) + 4*(ku >> 3) + ((ku >> 1) & 3).
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

struct Fp8Cfg {
    static constexpr int D = 128;
    static constexpr int NW = 4;
    static constexpr int BM = 32 * NW;
    static constexpr int BN = 64;
    static constexpr int KROW = D;              // bytes of one K row
    static constexpr int VROW = BN;             // bytes of one V^T row
    static constexpr int K_BYTES = BN * D;
    static constexpr int V_BYTES = BN * D;
    static constexpr int STAGE = K_BYTES + V_BYTES;
    static constexpr int LDS = 2 * STAGE;
    static constexpr int CU = D / 16;           // 16-byte units per K row
    static constexpr int K_UNITS = BN * CU / 256;
};

// Four fp32 values to four e4m3 bytes (round to nearest even, OCP e4m3 on gfx950).
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return (uint32_t)r;
}

template <bool CAUSAL>
__global__ __launch_bounds__(256) void fa_fwd_fp8_kernel(FwdParams p) {
    using C = Fp8Cfg;
    constexpr int D = C::D;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int n = lane & 31;
    const int g = lane >> 5;

    const int head_x = blockIdx.x % p.n_heads;
    const int t_ord = blockIdx.x / p.n_heads;
    const int qt = CAUSAL ? (p.n_qtiles - 1 - t_ord) : t_ord;
    int b, hq, hkv;
    head_of(p, head_x, b, hq, hkv);
    const int q0 = qt * C::BM;
    const int qrow = q0 + w * 32 + n;

    const char* Qh = reinterpret_cast<const char*>(p.q) + ((int64_t)(b * p.Hq + hq) * p.Nq) * D;
    const char* Kh = reinterpret_cast<const char*>(p.k) + ((int64_t)(b * p.Hkv + hkv) * p.Nk) * D;
    const char* Vh = reinterpret_cast<const char*>(p.v) + ((int64_t)(b * p.Hkv + hkv) * p.Nk) * D;

    int kend = p.Nk;
    if (CAUSAL) kend = min(kend, max(q0 + C::BM + p.causal_shift, 0));
    const int n_tiles = (kend + C::BN - 1) / C::BN;

    // Q as B operands: k-step ks covers d = 64*ks + 32*g + [0, 32).
    i32x8 qf[2];
    if (qrow < p.Nq) {
        const char* src = Qh + (int64_t)qrow * D;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            u32x4 lo = ldg16(src + 64 * ks + 32 * g);
            u32x4 hi = ldg16(src + 64 * ks + 32 * g + 16);
            lo ^= p.q_sign;
            hi ^= p.q_sign;
            qf[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                           (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
    } else {
        qf[0] = i32x8{};
        qf[1] = i32x8{};
    }

    u32x4 kreg[C::K_UNITS];
    u32x2 vreg[4];
    const int vku = tid & 15;     // 4-key unit of the V block this thread moves
    const int vc = tid >> 4;      // 8-wide d chunk

    auto load_tile = [&](int j) {
        const int key0 = j * C::BN;
#pragma unroll
        for (int r = 0; r < C::K_UNITS; ++r) {
            const int u = tid + 256 * r;
            const int row = u / C::CU, cu = u % C::CU;
            const int key = key0 + row;
            kreg[r] = key < p.Nk ? ldg16(Kh + (int64_t)key * D + cu * 16) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = key0 + 4 * vku + r;
            vreg[r] = key < p.Nk ? *reinterpret_cast<const u32x2*>(Vh + (int64_t)key * D + vc * 8)
                                 : u32x2{0, 0};
        }
    };

    auto store_tile = [&](int stage) {
        char* kb = smem + stage * C::STAGE;
        char* vb = kb + C::K_BYTES;
#pragma unroll
        for (int r = 0; r < C::K_UNITS; ++r) {
            const int u = tid + 256 * r;
            const int row = u / C::CU, cu = u % C::CU;
            lds_store16(kb, row * C::KROW + ((cu ^ (row & 7)) << 4), kreg[r]);
        }
        // 4 keys x 8 bytes -> 8 rows of V^T x 4 keys (byte transpose with v_perm)
        const int pu = 8 * (vku & 1) + 4 * (vku >> 3) + ((vku >> 1) & 3);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const uint32_t A = vreg[0][half], Bv = vreg[1][half], Cv = vreg[2][half], Dv = vreg[3][half];
            const uint32_t ab_lo = __builtin_amdgcn_perm(Bv, A, 0x05010400u);
            const uint32_t ab_hi = __builtin_amdgcn_perm(Bv, A, 0x07030602u);
            const uint32_t cd_lo = __builtin_amdgcn_perm(Dv, Cv, 0x05010400u);
            const uint32_t cd_hi = __builtin_amdgcn_perm(Dv, Cv, 0x07030602u);
            const uint32_t out[4] = {__builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u),
                                     __builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u),
                                     __builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u),
                                     __builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u)};
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) {
                const int d = vc * 8 + half * 4 + t4;
                const int unit = (pu >> 2) ^ ((d >> 1) & 3);
                *reinterpret_cast<uint32_t*>(vb + d * C::VROW + (unit << 4) + ((pu & 3) << 2)) = out[t4];
            }
        }
    };

    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x16{};
    float m = -INFINITY;
    float l = 0.f;

    if (n_tiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int j = 0; j < n_tiles; ++j) {
        const int stage = j & 1;
        if (j + 1 < n_tiles) load_tile(j + 1);
        const char* kb = smem + stage * C::STAGE;
        const char* vb = kb + C::K_BYTES;

        f32x16 s[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            s[h] = f32x16{};
            const int row = 32 * h + n;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int u0 = 4 * ks + 2 * g;
                const u32x4 lo = lds_load16(kb, row * C::KROW + ((u0 ^ (row & 7)) << 4));
                const u32x4 hi = lds_load16(kb, row * C::KROW + (((u0 + 1) ^ (row & 7)) << 4));
                const i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                s[h] = mfma_fp8_32x32x64(a, qf[ks], s[h]);
            }
        }

        const int key0 = j * C::BN;
        const bool need_mask = (key0 + C::BN > p.Nk) || (CAUSAL && key0 + C::BN - 1 > q0 + p.causal_shift);
        const int lim = CAUSAL ? min(qrow + p.causal_shift, p.Nk - 1) : p.Nk - 1;
        if (need_mask) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = key0 + 32 * h + 8 * (i >> 2) + 4 * g + (i & 3);
                    if (key > lim) s[h][i] = -INFINITY;
                }
        }

        float mx = -INFINITY;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[h][i]);
        mx = pair_max(mx);
        const float m_new = fmaxf(m, mx);
        const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
        const float mc = m_ref * p.c;
        const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m * p.c - mc);
        m = m_new;

        // probabilities times 2^8
        const float off = 8.f - mc;
        float rs = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float e = fast_exp2(fmaf(s[h][i], p.c, off));
                if (need_mask) {
                    const int key = key0 + 32 * h + 8 * (i >> 2) + 4 * g + (i & 3);
                    if (key > lim) e = 0.f;
                }
                s[h][i] = e;
                rs += e;
            }
        l = l * alpha + rs;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] *= alpha;

        i32x8 pb;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                pb[4 * h + q4] = (int)pack_fp8x4(s[h][4 * q4], s[h][4 * q4 + 1], s[h][4 * q4 + 2], s[h][4 * q4 + 3]);

#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const int d = 32 * db + n;
            const int sw = (d >> 1) & 3;
            const u32x4 lo = lds_load16(vb, d * C::VROW + (((2 * g) ^ sw) << 4));
            const u32x4 hi = lds_load16(vb, d * C::VROW + (((2 * g + 1) ^ sw) << 4));
            const i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                             (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            o[db] = mfma_fp8_32x32x64(a, pb, o[db]);
        }

        if (j + 1 < n_tiles) store_tile(stage ^ 1);
        __syncthreads();
    }

    const float lt = pair_sum(l);
    if (qrow < p.Nq) {
        const float inv = lt > 0.f ? p.o_scale / lt : 0.f;
        char* Orow = reinterpret_cast<char*>(p.o) + (((int64_t)(b * p.Hq + hq) * p.Nq + qrow) * D) * 2;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d = 32 * db + 8 * i4 + 4 * g;
                u32x2 val;
                val[0] = pack_bf16x2(o[db][4 * i4 + 0] * inv, o[db][4 * i4 + 1] * inv);
                val[1] = pack_bf16x2(o[db][4 * i4 + 2] * inv, o[db][4 * i4 + 3] * inv);
                *reinterpret_cast<u32x2*>(Orow + d * 2) = val;
            }
        if (p.lse != nullptr && g == 0) {
            const float v = lt > 0.f ? (m * p.c + __builtin_amdgcn_logf(lt) - 8.f) * kLn2 : -INFINITY;
            p.lse[(int64_t)(b * p.Hq + hq) * p.Nq + qrow] = v;
        }
    }
}

template <bool CAUSAL>
static hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
    FwdParams pp = p;
    pp.n_qtiles = (p.Nq + Fp8Cfg::BM - 1) / Fp8Cfg::BM;
    const long long grid = (long long)pp.n_qtiles * pp.n_heads;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    void* args[] = {&pp};
    return hipLaunchKernel(reinterpret_cast<const void*>(&fa_fwd_fp8_kernel<CAUSAL>),
                           dim3((unsigned)grid), dim3(256), args, 0, stream);
}

hipError_t launch_fwd_fp8(const FwdParams& p, int d, bool causal, hipStream_t stream) {
    if (d != 128) return hipErrorInvalidValue;
    return causal ? launch_one<true>(p, stream) : launch_one<false>(p, stream);
}

}  // namespace fa
