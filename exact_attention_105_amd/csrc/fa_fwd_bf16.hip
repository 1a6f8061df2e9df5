// Fused exact-attention forward pass, bfloat16 inputs, head dim 64 or 128, gfx950.
//
// One workgroup owns BM = 128 query rows of one (batch, query head) and
// streams the key/value rows of that head's key/value head through LDS in
// tiles of BN = 64 keys ("FlashAttention (DE)", systems-analysis.info,
// section "Tiling und blockweise Verarbeitung").  Each of the four waves owns
// 32 query rows and keeps, per row, a running maximum and a running sum of
// exponentials (same page, section "Online-Softmax-Berechnung"); scores,
// mask, softmax and the product with V never leave the chip (same page,
// section "Zusammenfassen von Operationen in einem CUDA-Kernel").  Only O and
// the per-row log-sum-exp are written.
//
// Matrix layout choices (gfx950 MFMA 32x32x16 bf16, see fa_device.hpp):
//   S^T = K Q^T : A = K tile rows from LDS, B = Q rows held in registers for
//                 the whole key loop; lane l ends up with the 32 scores of
//                 query l%32 against 16 keys of each 32-key block.
//   O^T += V^T P^T : A = V^T from LDS, B = P straight from the score
//                 registers (converted to bf16), so P never touches LDS.
// V is therefore stored transposed in LDS ([d][key]); the keys inside each
// group of 16 are permuted (4-key units 0,2,1,3) so that the 8 keys a lane
// feeds to one MFMA are contiguous and read with one 16-byte LDS load.
// K and V^T rows are XOR-swizzled in 16-byte units to keep LDS reads and
// writes free of bank conflicts.
//
// Tiles are double-buffered: the global loads of tile j+1 are issued before
// the arithmetic on tile j and written to the other LDS buffer after it, so
// one barrier per tile suffices.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

template <int D>
struct Bf16Cfg {
    static constexpr int NW = 4;                 // waves per workgroup
    static constexpr int BM = 32 * NW;           // query rows per workgroup
    static constexpr int BN = 64;                // keys per K/V tile
    static constexpr int KROW = D * 2;           // bytes of one K row in LDS
    static constexpr int VROW = BN * 2;          // bytes of one V^T row in LDS
    static constexpr int K_BYTES = BN * D * 2;
    static constexpr int V_BYTES = BN * D * 2;
    static constexpr int STAGE = K_BYTES + V_BYTES;
    static constexpr int LDS = 2 * STAGE;
    static constexpr int KS = D / 16;            // MFMA steps over d for S
    static constexpr int DB = D / 32;            // 32-wide blocks of d in O
    static constexpr int CU = D / 8;             // 16-byte units per K row
    static constexpr int K_UNITS = BN * CU / 256;  // K units loaded per thread
    static constexpr int V_THREADS = (BN / 4) * (D / 8);  // threads holding a 4-key x 8-d block of V
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fa_fwd_bf16_kernel(FwdParams p) {
    using C = Bf16Cfg<D>;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int n = lane & 31;     // query column owned by this lane
    const int g = lane >> 5;     // which half of the 32x32 block's rows

    // Workgroup -> (head, query tile).  Consecutive workgroup ids walk the
    // heads first, so all heads progress through their query tiles together;
    // causal problems take the most expensive (last) query tiles first.
    const int head_x = blockIdx.x % p.n_heads;
    const int t_ord = blockIdx.x / p.n_heads;
    const int qt = CAUSAL ? (p.n_qtiles - 1 - t_ord) : t_ord;
    int b, hq, hkv;
    head_of(p, head_x, b, hq, hkv);
    const int q0 = qt * C::BM;
    const int qrow = q0 + w * 32 + n;

    const char* Qh = reinterpret_cast<const char*>(p.q) + ((int64_t)(b * p.Hq + hq) * p.Nq) * D * 2;
    const char* Kh = reinterpret_cast<const char*>(p.k) + ((int64_t)(b * p.Hkv + hkv) * p.Nk) * D * 2;
    const char* Vh = reinterpret_cast<const char*>(p.v) + ((int64_t)(b * p.Hkv + hkv) * p.Nk) * D * 2;

    // Keys this workgroup needs: all of them, or (causal) up to the last
    // visible key of its last row; key tiles beyond are skipped entirely.
    int kend = p.Nk;
    if (CAUSAL) kend = min(kend, max(q0 + C::BM + p.causal_shift, 0));
    const int n_tiles = (kend + C::BN - 1) / C::BN;

    // Q rows of this lane as MFMA B operands, resident for the whole loop.
    bf16x8 qf[C::KS];
    if (qrow < p.Nq) {
        const char* src = Qh + (int64_t)qrow * D * 2;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            u32x4 x = ldg16(src + (2 * ks + g) * 16);
            x ^= p.q_sign;
            qf[ks] = __builtin_bit_cast(bf16x8, x);
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }

    u32x4 kreg[C::K_UNITS];
    u32x4 vreg[4];
    const int vku = tid & 15;          // 4-key unit of the V block this thread moves
    const int vc = tid >> 4;           // 8-wide d chunk of that block

    auto load_tile = [&](int j) {
        const int key0 = j * C::BN;
#pragma unroll
        for (int r = 0; r < C::K_UNITS; ++r) {
            const int u = tid + 256 * r;
            const int row = u / C::CU, cu = u % C::CU;
            const int key = key0 + row;
            kreg[r] = key < p.Nk ? ldg16(Kh + ((int64_t)key * D + cu * 8) * 2) : u32x4{0, 0, 0, 0};
        }
        if (tid < C::V_THREADS) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = key0 + 4 * vku + r;
                vreg[r] = key < p.Nk ? ldg16(Vh + ((int64_t)key * D + vc * 8) * 2) : u32x4{0, 0, 0, 0};
            }
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
        if (tid < C::V_THREADS) {
            // position unit of this 4-key unit inside V^T rows: bits of the
            // unit index within its 16-key group are swapped (0,2,1,3)
            const int ku = vku & 3;
            const int pu = 4 * (vku >> 2) + (((ku & 1) << 1) | (ku >> 1));
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int d = vc * 8 + t;
                const int q = t >> 1;
                const uint32_t a0 = vreg[0][q], a1 = vreg[1][q], a2 = vreg[2][q], a3 = vreg[3][q];
                u32x2 val;
                if ((t & 1) == 0) {
                    val[0] = (a0 & 0xFFFFu) | (a1 << 16);
                    val[1] = (a2 & 0xFFFFu) | (a3 << 16);
                } else {
                    val[0] = (a0 >> 16) | (a1 & 0xFFFF0000u);
                    val[1] = (a2 >> 16) | (a3 & 0xFFFF0000u);
                }
                lds_store8(vb, d * C::VROW + ((((pu >> 1) ^ (d & 7))) << 4) + ((pu & 1) << 3), val);
            }
        }
    };

    f32x16 o[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) o[db] = f32x16{};
    float m = -INFINITY;   // running max of the raw (sign-adjusted) scores of query qrow
    float l = 0.f;         // this lane's part of the running sum of exponentials

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

        // S^T for 2 x 32 keys against this wave's 32 queries
        f32x16 s[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            s[h] = f32x16{};
            const int row = 32 * h + n;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const int cu = 2 * ks + g;
                const bf16x8 a = __builtin_bit_cast(bf16x8, lds_load16(kb, row * C::KROW + ((cu ^ (row & 7)) << 4)));
                s[h] = mfma_bf16_32x32x16(a, qf[ks], s[h]);
            }
        }

        // Mask: keys past Nk and, for causal problems, keys after the
        // query's diagonal.  Only tiles that straddle either edge pay for it.
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

        // Online softmax update for this tile.
        float mx = -INFINITY;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[h][i]);
        mx = pair_max(mx);
        const float m_new = fmaxf(m, mx);
        const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;   // no visible key yet
        const float mc = m_ref * p.c;
        const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m * p.c - mc);
        m = m_new;

        float rs = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float e = fast_exp2(fmaf(s[h][i], p.c, -mc));
                if (need_mask) {
                    const int key = key0 + 32 * h + 8 * (i >> 2) + 4 * g + (i & 3);
                    if (key > lim) e = 0.f;
                }
                s[h][i] = e;
                rs += e;
            }
        l = l * alpha + rs;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) o[db] *= alpha;

        // O^T += V^T P^T over 4 steps of 16 keys
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int h = st >> 1, i0 = 8 * (st & 1);
            u32x4 pk;
            pk[0] = pack_bf16x2(s[h][i0 + 0], s[h][i0 + 1]);
            pk[1] = pack_bf16x2(s[h][i0 + 2], s[h][i0 + 3]);
            pk[2] = pack_bf16x2(s[h][i0 + 4], s[h][i0 + 5]);
            pk[3] = pack_bf16x2(s[h][i0 + 6], s[h][i0 + 7]);
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pk);
            const int unit = 2 * st + g;
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
                const int d = 32 * db + n;
                const bf16x8 a = __builtin_bit_cast(bf16x8, lds_load16(vb, d * C::VROW + ((unit ^ (d & 7)) << 4)));
                o[db] = mfma_bf16_32x32x16(a, pb, o[db]);
            }
        }

        if (j + 1 < n_tiles) store_tile(stage ^ 1);
        __syncthreads();
    }

    // Epilogue: normalise once, write O (bf16) and the log-sum-exp.
    const float lt = pair_sum(l);
    if (qrow < p.Nq) {
        const float inv = lt > 0.f ? p.o_scale / lt : 0.f;
        char* Orow = reinterpret_cast<char*>(p.o) + (((int64_t)(b * p.Hq + hq) * p.Nq + qrow) * D) * 2;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d = 32 * db + 8 * i4 + 4 * g;
                u32x2 val;
                val[0] = pack_bf16x2(o[db][4 * i4 + 0] * inv, o[db][4 * i4 + 1] * inv);
                val[1] = pack_bf16x2(o[db][4 * i4 + 2] * inv, o[db][4 * i4 + 3] * inv);
                *reinterpret_cast<u32x2*>(Orow + d * 2) = val;
            }
        if (p.lse != nullptr && g == 0) {
            const float v = lt > 0.f ? (m * p.c + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
            p.lse[(int64_t)(b * p.Hq + hq) * p.Nq + qrow] = v;
        }
    }
}

template <int D, bool CAUSAL>
static hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
    using C = Bf16Cfg<D>;
    FwdParams pp = p;
    pp.n_qtiles = (p.Nq + C::BM - 1) / C::BM;
    const long long grid = (long long)pp.n_qtiles * pp.n_heads;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    void* args[] = {&pp};
    return hipLaunchKernel(reinterpret_cast<const void*>(&fa_fwd_bf16_kernel<D, CAUSAL>),
                           dim3((unsigned)grid), dim3(256), args, 0, stream);
}

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, hipStream_t stream) {
    if (d == 64) return causal ? launch_one<64, true>(p, stream) : launch_one<64, false>(p, stream);
    if (d == 128) return causal ? launch_one<128, true>(p, stream) : launch_one<128, false>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa
