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
// Matrix layout (gfx950 MFMA 32x32x16 bf16, see fa_device.hpp):
//   S^T = K Q^T    : A = K rows from LDS (ds_read_b128), B = Q rows held in
//                    registers for the whole key loop.  Lane l ends up with
//                    the scores of query l%32 against 16 of every 32 keys.
//   O^T += V^T P^T : A = V^T built from row-major V in LDS with the gfx950
//                    transposing read ds_read_b64_tr_b16 (16 lanes read a
//                    4-key x 16-d block; each lane receives one d column of
//                    4 keys), B = P straight from the score registers.
// So P never touches LDS and V is never transposed in memory.
//
// K/V staging: the global loads go straight into LDS (global_load_lds_dwordx4,
// 1 KiB per wave instruction, no staging registers).  LDS rows are XOR
// swizzled in 16-byte units -- by the row index for K, so the 32 rows a
// ds_read_b128 touches hit distinct banks, and by 2*(row%4) for V, so the
// four rows one transposing read touches do -- and the swizzle is realised
// by choosing which global 16 bytes each lane fetches.  Two LDS stages: the
// loads of tile j+1 are issued right after the barrier that publishes tile
// j and land while tile j is computed.
//
// Online softmax with a lazily updated reference: the exponent reference of
// a row only moves when its running maximum exceeds the reference by more
// than kRescaleLog2 (in log2 units); until then the exponentials are at most
// 2^kRescaleLog2 and no rescale of O and l is needed.  The result is the
// same softmax (the reference cancels between numerator and denominator)
// with far fewer rescales (the idea of page "FlashAttention 4", centron.de,
// section on smarter online-softmax rescaling; the threshold is this
// library's choice).  A wave skips the O rescale when none of its rows moved.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

constexpr float kRescaleLog2 = 8.0f;

template <int D>
struct Bf16Cfg {
    static constexpr int NW = 4;                 // waves per workgroup
    static constexpr int BM = 32 * NW;           // query rows per workgroup
    static constexpr int BN = 64;                // keys per K/V tile
    static constexpr int ROW = D * 2;            // bytes of one K or V row in LDS
    static constexpr int UPR = D / 8;            // 16-byte units per row
    static constexpr int TILE = BN * ROW;        // bytes of one K (or V) tile
    static constexpr int STAGE = 2 * TILE;       // K tile + V tile
    static constexpr int LDS = 2 * STAGE;
    static constexpr int CHUNKS = TILE / 1024;   // 1 KiB wave loads per tile and tensor
    static constexpr int CPW = CHUNKS / NW;      // ... per wave
    static constexpr int RPC = 1024 / ROW;       // rows per 1 KiB chunk
    static constexpr int KS = D / 16;            // MFMA steps over d for S
    static constexpr int DB = D / 32;            // 32-wide blocks of d in O
    static_assert(CHUNKS % NW == 0, "tile must split evenly over the waves");
    static_assert(BM * ROW <= STAGE, "O staging must fit in one stage");
};

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) short4 lds_short4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

// One wave-wide 16-byte-per-lane copy global -> LDS: lane i's 16 bytes land at
// ldst + 16*i (ldst is wave-uniform and goes to M0).  Issued as inline asm so
// the compiler does not order later LDS reads behind it; completion is
// awaited explicitly (vmcnt(0)) before the barrier that publishes a tile.
// M0 is listed as clobbered; clang warns about clobbering a reserved register,
// but no other code in these kernels keeps a value in M0 (checked in the ISA).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* gsrc, lds_char* ldst) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)ldst);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(m0), "v"(gsrc) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ i16x4 lds_tr16(const lds_char* p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fa_fwd_bf16_kernel(FwdParams p) {
    using C = Bf16Cfg<D>;
    __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS];
    lds_char* smem = (lds_char*)smem_raw;

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

    const char* Qh = reinterpret_cast<const char*>(p.q) + ((int64_t)(b * p.Hq + hq) * p.Nq) * C::ROW;
    const char* Kh = reinterpret_cast<const char*>(p.k) + ((int64_t)(b * p.Hkv + hkv) * p.Nk) * C::ROW;
    const char* Vh = reinterpret_cast<const char*>(p.v) + ((int64_t)(b * p.Hkv + hkv) * p.Nk) * C::ROW;

    // Keys this workgroup needs: all of them, or (causal) up to the last
    // visible key of its last row; key tiles beyond are skipped entirely.
    int kend = p.Nk;
    if (CAUSAL) kend = min(kend, max(q0 + C::BM + p.causal_shift, 0));
    const int n_tiles = (kend + C::BN - 1) / C::BN;

    // Q rows of this lane as MFMA B operands, resident for the whole loop.
    bf16x8 qf[C::KS];
    if (qrow < p.Nq) {
        const char* src = Qh + (int64_t)qrow * C::ROW;
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

    // This lane's part of each 1 KiB chunk: row-in-chunk and stored unit.
    const int c_row = lane / C::UPR;
    const int c_su = lane % C::UPR;

    // Issue the global->LDS copies of key tile j into `stage`.  Rows past Nk
    // are clamped to the last key (their scores are masked and their P is 0).
    auto issue_tile = [&](int j, int stage) {
        lds_char* kdst = smem + stage * C::STAGE;
        lds_char* vdst = kdst + C::TILE;
        const int key0 = j * C::BN;
#pragma unroll
        for (int t = 0; t < C::CPW; ++t) {
            const int c = w * C::CPW + t;
            const int row = c * C::RPC + c_row;
            const int key = min(key0 + row, p.Nk - 1);
            const int ku = c_su ^ (row & 7);                 // K: unit swizzled by row
            const int vu = c_su ^ (2 * (row & 3));           // V: unit swizzled by 2*(row%4)
            dma16(Kh + (int64_t)key * C::ROW + ku * 16, kdst + c * 1024);
            dma16(Vh + (int64_t)key * C::ROW + vu * 16, vdst + c * 1024);
        }
    };

    f32x16 o[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) o[db] = f32x16{};
    float mref = -INFINITY;  // exponent reference of this row, in log2 units (scaled scores)
    float l = 0.f;           // this lane's part of the sum of exponentials (relative to mref)

    // Per-lane constant parts of the transposing V reads: lane (n, g) sources
    // key row 4*g + (n%16)/4 (+8, +16*st) at d = 16*(n/16) + 4*(n%4) (+32*db).
    const int tr_row = 4 * g + ((n & 15) >> 2);
    const int tr_d = 16 * (n >> 4) + 4 * (n & 3);

    if (n_tiles > 0) issue_tile(0, 0);

    for (int j = 0; j < n_tiles; ++j) {
        const int stage = j & 1;
        __builtin_amdgcn_s_waitcnt(0x0F70);             // vmcnt(0): this wave's copies of tile j landed
        __syncthreads();                                 // ... and every other wave's
        if (j + 1 < n_tiles) issue_tile(j + 1, stage ^ 1);
        const lds_char* kb = smem + stage * C::STAGE;
        const lds_char* vb = kb + C::TILE;

        // S^T for 2 x 32 keys against this wave's 32 queries
        f32x16 s[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            s[h] = f32x16{};
            const int row = 32 * h + n;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const int cu = 2 * ks + g;
                const bf16x8 a = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
                    kb + row * C::ROW + ((cu ^ (row & 7)) << 4));
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

        // Online softmax with a lazily moved reference.
        float mx = -INFINITY;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[h][i]);
        mx = pair_max(mx) * p.c;                         // tile max in log2 units (-inf if none visible)
        const bool move = mx > mref + kRescaleLog2;      // false while nothing is visible
        if (__builtin_amdgcn_ballot_w64(move) != 0) {    // some row of this wave moves its reference
            const float mnew = move ? mx : mref;
            const float alpha = move ? ((mref == -INFINITY) ? 0.f : fast_exp2(mref - mnew)) : 1.f;
            mref = mnew;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < C::DB; ++db) o[db] *= alpha;
        }
        const float mb = (mref == -INFINITY) ? 0.f : mref;

        float rs = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float e = fast_exp2(fmaf(s[h][i], p.c, -mb));
                if (need_mask) {
                    const int key = key0 + 32 * h + 8 * (i >> 2) + 4 * g + (i & 3);
                    if (key > lim) e = 0.f;
                }
                s[h][i] = e;
                rs += e;
            }
        l += rs;

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
            const int r0 = 16 * st + tr_row;               // key rows r0 (slots 0-3) and r0 + 8 (slots 4-7)
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
                const int d = 32 * db + tr_d;
                const int u = d >> 3, half = (d & 7) * 2;
                const i16x4 lo = lds_tr16(vb + r0 * C::ROW + ((u ^ (2 * (r0 & 3))) << 4) + half);
                const i16x4 hi = lds_tr16(vb + (r0 + 8) * C::ROW + ((u ^ (2 * ((r0 + 8) & 3))) << 4) + half);
                const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                o[db] = mfma_bf16_32x32x16(a, pb, o[db]);
            }
        }
    }

    // Epilogue: normalise once, stage O as bf16 in LDS (the stage no longer
    // read), then write whole rows with 16-byte coalesced stores.
    const float lt = pair_sum(l);
    const float inv = lt > 0.f ? p.o_scale / lt : 0.f;
    __syncthreads();
    lds_char* ost = smem + (n_tiles & 1) * C::STAGE;
    {
        const int row = w * 32 + n;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int u = 4 * db + i4;               // 16-byte unit of d = 32*db + 8*i4 + 4*g
                u32x2 val;
                val[0] = pack_bf16x2(o[db][4 * i4 + 0] * inv, o[db][4 * i4 + 1] * inv);
                val[1] = pack_bf16x2(o[db][4 * i4 + 2] * inv, o[db][4 * i4 + 3] * inv);
                *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
                    ost + row * C::ROW + ((u ^ (row & 7)) << 4) + 8 * g) = val;
            }
    }
    if (p.lse != nullptr && g == 0 && qrow < p.Nq) {
        const float v = lt > 0.f ? (mref + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
        p.lse[(int64_t)(b * p.Hq + hq) * p.Nq + qrow] = v;
    }
    __syncthreads();
    char* Oh = reinterpret_cast<char*>(p.o) + ((int64_t)(b * p.Hq + hq) * p.Nq) * C::ROW;
#pragma unroll
    for (int it = 0; it < 32 * C::UPR / 64; ++it) {
        const int f = it * 64 + lane;
        const int row = w * 32 + f / C::UPR;
        const int su = f % C::UPR;
        const int grow = q0 + row;
        if (grow < p.Nq) {
            const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                ost + row * C::ROW + su * 16);
            *reinterpret_cast<u32x4*>(Oh + (int64_t)grow * C::ROW + ((su ^ (row & 7)) << 4)) = v;
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
