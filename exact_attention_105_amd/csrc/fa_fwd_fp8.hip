// Fused exact-attention forward pass, FP8 (OCP E4M3) inputs, head dim 128, gfx950.
//
// Low-precision attention (page "FlashAttention-3 (DE)", systems-analysis.ru,
// section on low precision: FP8 doubles the matrix throughput at the cost of
// dynamic range).  The structure follows the bf16 kernel (fa_fwd_bf16.hip):
// BM = 128 query rows per workgroup (32 per wave, up to three workgroups per CU),
// 64-key K/V tiles copied straight into double-buffered LDS, the query index
// on the MFMA column side so each lane owns one query row, and the online
// softmax with a lazily moved reference in registers.  Differences:
//   * both products use v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3 -> fp32); one
//     S^T product covers 64 d and one O^T product covers the whole 64-key tile;
//   * the per-tensor scales are folded in: the exponent constant is
//     |scale| * sq * sk * log2(e), and the normalised output is multiplied by sv;
//   * P is quantised to e4m3 for the second product.  The exponentials carry
//     a 2^kP8Offset factor and the reference moves as soon as the running max
//     exceeds it by more than 2^kP8Slack, so P stays below 2^(offset+slack) =
//     256 < 448 (e4m3's largest value) and probabilities down to ~2^-12 of the
//     reference stay in e4m3's normal range.  The row sums use the
//     unquantised fp32 values in the same units; the log-sum-exp removes the
//     offset again;
//   * V^T comes from row-major V through the 8-bit transposing LDS read
//     ds_read_b64_tr_b8 (16 lanes read 8 key rows x 16 bytes; each lane
//     receives one d column of 8 keys); four reads give a lane the 32 keys of
//     its P operand, in the order the scores sit in its registers.
// LDS swizzles (16-byte units, 128-byte rows): K by (row/2) mod 8, so the 16
// rows one ds_read_b128 touches hit distinct banks; V by
// 2*((row/2 mod 2) + 2*(row/8 mod 2)), which separates the 8 rows one
// transposing read touches.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

#ifndef FA_FP8_PF_S
#define FA_FP8_PF_S 3        // K read pairs kept ahead of the S^T MFMAs (0: the compiler's order)
#endif
#ifndef FA_FP8_PF_V
#define FA_FP8_PF_V 2        // V^T read quads kept ahead of the O^T MFMAs
#endif

constexpr float kP8Offset = 6.0f;   // log2 of the factor carried by the exponentials
constexpr float kP8Slack = 2.0f;    // log2 growth of the max tolerated before rescaling
// Reference of a row that has seen no visible key: finite, so the first move
// gives alpha = exp2(kNoRef8 - m) = 0 and an unmoved row exp2(0) = 1.
constexpr float kNoRef8 = -1.0e30f;

struct Fp8Cfg {
    static constexpr int D = 128;
    static constexpr int NW = 4;
    static constexpr int BM = 32 * NW;
    static constexpr int BN = 64;
    static constexpr int ROW = D;               // bytes of one K or V row
    static constexpr int UPR = D / 16;          // 16-byte units per row (8)
    static constexpr int TILE = BN * ROW;       // 8 KiB
    static constexpr int STAGE = 2 * TILE;
    static constexpr int NSTAGE = 2;
    static constexpr int OROW = D * 2;          // bytes of one bf16 O row
    static constexpr int LDS = NSTAGE * STAGE > BM * OROW ? NSTAGE * STAGE : BM * OROW;
    static constexpr int CHUNKS = TILE / 1024;  // 8
    static constexpr int CPW = CHUNKS / NW;     // 2
    static constexpr int RPC = 1024 / ROW;      // 8 rows per chunk
    static constexpr int DB = D / 32;           // 32-wide blocks of d in O
    static_assert(CHUNKS % NW == 0, "tile must split evenly over the waves");
};

__device__ __forceinline__ int k8_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int v8_swz(int row) { return 2 * (((row >> 1) & 1) | (((row >> 3) & 1) << 1)); }

// Four fp32 values to four e4m3 bytes (round to nearest even, OCP e4m3 on gfx950).
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return (uint32_t)r;
}

template <bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fa_fwd_fp8_kernel(FwdParams p) {
    using C = Fp8Cfg;
    constexpr int D = C::D;
    __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS];
    lds_char* smem = (lds_char*)smem_raw;
    const uint32_t smem_u32 = (uint32_t)(uintptr_t)smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31;
    const int g = lane >> 5;

    // Workgroup -> (head, query tile), XCD-aware (tile_of in fa_device.hpp).
    int b, hq, hkv, qt;
    tile_of<CAUSAL>(p, blockIdx.x, b, hq, hkv, qt);
    const int q0 = qt * C::BM;
    const int wq0 = q0 + w * 32;
    const int qrow = wq0 + n;

    const char* Qh = reinterpret_cast<const char*>(p.q) + ((int64_t)(b * p.Hq + hq) * p.Nq) * D;
    const char* Kh = reinterpret_cast<const char*>(p.k) + ((int64_t)(b * p.Hkv + hkv) * p.Nk) * D;
    const char* Vh = reinterpret_cast<const char*>(p.v) + ((int64_t)(b * p.Hkv + hkv) * p.Nk) * D;

    // (readfirstlane keeps these uniform bounds, and the loop control built
    // on them, in scalar registers)
    const int kend = key_end(q0, C::BM, p.Nk, p.causal_shift, CAUSAL);
    const int n_tiles = __builtin_amdgcn_readfirstlane((kend + C::BN - 1) / C::BN);
    const int wkend = __builtin_amdgcn_readfirstlane(key_end(wq0, 32, p.Nk, p.causal_shift, CAUSAL));

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

    // Loop-invariant per-lane offsets.
    const int c_row = lane / C::UPR;
    const int c_su = lane % C::UPR;
    uint32_t dk_off[C::CPW], dv_off[C::CPW];
#pragma unroll
    for (int t = 0; t < C::CPW; ++t) {
        const int row = (w * C::CPW + t) * C::RPC + c_row;
        dk_off[t] = row * C::ROW + ((c_su ^ k8_swz(row)) << 4);
        dv_off[t] = row * C::ROW + ((c_su ^ v8_swz(row)) << 4);
    }
    // K reads: row 32*kh + n, units 4*ks + 2*g + e (e = 0, 1); kh adds 32 rows.
    uint32_t k_off[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 2; ++e) k_off[ks][e] = n * C::ROW + (((4 * ks + 2 * g + e) ^ k8_swz(n)) << 4);
    // V^T reads: read q (0..3) gives P slots 8q..8q+7 = keys 16q + 8*(r/4) + 4g + r%4,
    // r = 0..7; this lane sources r = (n%16)/2 at d = 32*db + 16*(n/16) + 8*(n%2).
    uint32_t v_off[C::DB];
    {
        const int r = (n & 15) >> 1;
        const int vrow = 8 * (r >> 2) + 4 * g + (r & 3);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
            const int unit = 2 * db + (n >> 4);
            v_off[db] = vrow * C::ROW + ((unit ^ v8_swz(vrow)) << 4) + 8 * (n & 1);
        }
    }

    auto issue_tile = [&](int j, int stage) {
        const uint32_t kdst = smem_u32 + stage * C::STAGE + w * C::CPW * 1024;
        const uint32_t vdst = kdst + C::TILE;
        const int key0 = j * C::BN;
        const char* kb = Kh + (int64_t)key0 * C::ROW;
        const char* vb = Vh + (int64_t)key0 * C::ROW;
        if (key0 + C::BN <= p.Nk) {
#pragma unroll
            for (int t = 0; t < C::CPW; ++t) {
                dma16(kb, dk_off[t], kdst + t * 1024);
                dma16(vb, dv_off[t], vdst + t * 1024);
            }
        } else {
#pragma unroll
            for (int t = 0; t < C::CPW; ++t) {
                const int row = (w * C::CPW + t) * C::RPC + c_row;
                const int rc = copy_src_row(row, key0, p.Nk);
                dma16(kb, rc * C::ROW + ((c_su ^ k8_swz(row)) << 4), kdst + t * 1024);
                dma16(vb, rc * C::ROW + ((c_su ^ v8_swz(row)) << 4), vdst + t * 1024);
            }
        }
    };

    f32x16 o[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) o[db] = f32x16{};
    float mref = kNoRef8;     // exponent reference of this row, log2 units
    float thr = -INFINITY;    // raw score above which the reference must move
    float l = 0.f;            // this lane's part of the row sum, times 2^kP8Offset

    if (n_tiles > 0) issue_tile(0, 0);

    // One key tile.  Templated on the LDS stage so that every LDS address is a
    // loop-invariant per-lane register plus an immediate (+1.7 % over a
    // runtime stage, bit-identical); the barrier carries no memory fence, the
    // copies being awaited with vmcnt.
    const float inv_c = 1.0f / p.c;
    auto tile = [&](auto stage_c, int j) {
        constexpr int stage = decltype(stage_c)::value;
        FA_WAIT_VMCNT(0);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

        const int key0 = j * C::BN;
        if (key0 >= wkend) {
            if (j + 1 < n_tiles) issue_tile(j + 1, stage ^ 1);
            return;
        }
        const lds_char* kb = smem + stage * C::STAGE;
        const lds_char* vb = kb + C::TILE;

        // MFMA blocks run at raised wave priority, so a co-resident wave in
        // its softmax phase issues its VALU work around them.
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        f32x16 s[2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            s[kh] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const u32x4 lo = lds_u128(kb + k_off[ks][0] + kh * 32 * C::ROW);
                const u32x4 hi = lds_u128(kb + k_off[ks][1] + kh * 32 * C::ROW);
                const i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                s[kh] = mfma_fp8_32x32x64(a, qf[ks], s[kh]);
            }
        }
        order_reads_ahead<4, 2, FA_FP8_PF_S>();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        // the next tile's copies go out in the wait before the scores can be read
        if (j + 1 < n_tiles) issue_tile(j + 1, stage ^ 1);

        const bool need_mask = (key0 + C::BN > p.Nk) || (CAUSAL && key0 + C::BN - 1 > wq0 + p.causal_shift);
        if (need_mask) {
            const int lim = (CAUSAL ? min(qrow + p.causal_shift, p.Nk - 1) : p.Nk - 1) - key0 - 4 * g;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * kh + 8 * (i >> 2) + (i & 3) > lim) s[kh][i] = -INFINITY;
        }

        // Each lane compares the maximum of its own raw scores with the
        // threshold; only when some lane passes it does the wave form the row
        // maxima and move references.
        const float lm = fmaxf(max16(s[0]), max16(s[1]));
        if (__builtin_amdgcn_ballot_w64(lm > thr) != 0) {
            const float mx = pair_max(lm) * p.c;
            const bool move = mx > mref + kP8Slack;
            const float mnew = move ? mx : mref;
            const float alpha = fast_exp2(mref - mnew);   // 0 at the first move, 1 if unmoved
            mref = mnew;
            thr = (mnew + kP8Slack) * inv_c;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < C::DB; ++db) o[db] *= alpha;
        }
        const float off = kP8Offset - mref;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kh][i] = fast_exp2(fmaf(s[kh][i], p.c, off));
        l += sum16(s[0]) + sum16(s[1]);

        i32x8 pb;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                pb[4 * kh + q4] = (int)pack_fp8x4(s[kh][4 * q4], s[kh][4 * q4 + 1], s[kh][4 * q4 + 2], s[kh][4 * q4 + 3]);

        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
            i32x8 a;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x2 t = lds_tr8(vb + v_off[db] + 16 * q * C::ROW);
                a[2 * q] = (int)t[0];
                a[2 * q + 1] = (int)t[1];
            }
            o[db] = mfma_fp8_32x32x64(a, pb, o[db]);
        }
        order_reads_ahead<C::DB, 4, FA_FP8_PF_V>();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
    };
    for (int j = 0; j < n_tiles; j += 2) {
        tile(std::integral_constant<int, 0>{}, j);
        if (j + 1 < n_tiles) tile(std::integral_constant<int, 1>{}, j + 1);
    }

    // Epilogue: normalise, stage O as bf16 in LDS, coalesced 16-byte stores.
    const float lt = pair_sum(l);
    const float inv = lt > 0.f ? p.o_scale / lt : 0.f;
    __syncthreads();
    {
        const int row = w * 32 + n;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int u = 4 * db + i4;
                u32x2 val;
                val[0] = pack_bf16x2(o[db][4 * i4 + 0] * inv, o[db][4 * i4 + 1] * inv);
                val[1] = pack_bf16x2(o[db][4 * i4 + 2] * inv, o[db][4 * i4 + 3] * inv);
                *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
                    smem + row * C::OROW + ((u ^ (row & 15)) << 4) + 8 * g) = val;
            }
    }
    if (p.lse != nullptr && g == 0 && qrow < p.Nq) {
        const float v = lt > 0.f ? (mref + __builtin_amdgcn_logf(lt) - kP8Offset) * kLn2 : -INFINITY;
        p.lse[(int64_t)(b * p.Hq + hq) * p.Nq + qrow] = v;
    }
    __syncthreads();
    char* Oh = reinterpret_cast<char*>(p.o) + ((int64_t)(b * p.Hq + hq) * p.Nq) * C::OROW;
#pragma unroll
    for (int it = 0; it < 32 * 16 / 64; ++it) {
        const int f = it * 64 + lane;
        const int row = w * 32 + f / 16;
        const int su = f % 16;
        const int grow = q0 + row;
        if (grow < p.Nq) {
            const u32x4 v = lds_u128(smem + row * C::OROW + su * 16);
            *reinterpret_cast<u32x4*>(Oh + (int64_t)grow * C::OROW + ((su ^ (row & 15)) << 4)) = v;
        }
    }
}

template <bool CAUSAL>
static hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
    FwdParams pp = p;
    pp.n_qtiles = (p.Nq + Fp8Cfg::BM - 1) / Fp8Cfg::BM;
    pp.kv_group = stream_group((long long)p.B * p.Nk * p.Hkv * 128 * 2);
    const long long grid = (long long)pp.n_qtiles * pp.n_heads;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    void* args[] = {&pp};
    const void* kernel = reinterpret_cast<const void*>(&fa_fwd_fp8_kernel<CAUSAL>);
    return hipLaunchKernel(kernel, dim3((unsigned)grid), dim3(256), args, test_extra_lds(Fp8Cfg::LDS), stream);
}

hipError_t launch_fwd_fp8(const FwdParams& p, int d, bool causal, hipStream_t stream) {
    if (d != 128) return hipErrorInvalidValue;
    return causal ? launch_one<true>(p, stream) : launch_one<false>(p, stream);
}

}  // namespace fa
