// Fused exact-attention forward pass, bfloat16 inputs, head dim 64 or 128, gfx950.
//
// One workgroup owns BM = 128 query rows of one (batch, query head) and
// streams the key/value rows of that head's key/value head through LDS in
// tiles of BN = 32 keys ("FlashAttention (DE)", systems-analysis.info,
// section "Tiling und blockweise Verarbeitung").  Each of the four waves owns
// 32 query rows and keeps, per row, a running maximum and a running sum of
// exponentials (same page, section "Online-Softmax-Berechnung"); scores,
// mask, softmax and the product with V never leave the chip (same page,
// section "Zusammenfassen von Operationen in einem CUDA-Kernel").  Only O and
// the per-row log-sum-exp are written.
//
// Matrix layout (gfx950 MFMA 32x32x16 bf16, see fa_device.hpp), per wave and
// per 32-query block qb of its rows:
//   S^T = K Q^T    : A = K rows from LDS (ds_read_b128), B = Q rows held in
//                    registers for the whole key loop.  Lane l ends up with
//                    the scores of query l%32 against 16 of every 32 keys.
//   O^T += V^T P^T : A = V^T built from row-major V in LDS with the gfx950
//                    transposing read ds_read_b64_tr_b16 (16 lanes read a
//                    4-key x 16-d block; each lane receives one d column of
//                    4 keys), B = P straight from the score registers.
// Three workgroups (twelve waves) share a CU at d = 128 (FA_BF16_OCC), so
// one wave's softmax overlaps the others' MFMAs on each SIMD; the MFMA
// blocks run at raised wave priority so that a wave reaching its matrix work
// issues it first.  Short 32-key tiles make the waves alternate between MFMA
// and VALU phases often, which measured faster than 64-key tiles at the same
// occupancy (FA_BF16_BN); deeper LDS pipelines (FA_BF16_NSTAGE) did not help.
// 64 rows per wave (FA_BF16_RW128 / FA_BF16_RW64 = 64) would feed every K
// and V^T fragment read from LDS to two MFMAs, but needs the accumulators in
// AGPRs and runs one workgroup per CU; measured slower.
//
// Within each MFMA phase the LDS operand reads are ordered to run PF_S (K)
// or PF_V (V^T pairs) MFMAs ahead of their products (order_reads_ahead in
// fa_device.hpp): left to itself the scheduler keeps one read in flight, and
// every MFMA waits on the read just before it.
//
// K/V staging: the global loads go straight into LDS (global_load_lds_dwordx4,
// 1 KiB per wave instruction, no staging registers), NSTAGE tiles deep, with
// one barrier per tile.  LDS
// rows are XOR swizzled in 16-byte units so that the rows one ds_read_b128
// cycle (K) or one transposing-read cycle (V) touches hit distinct banks
// (Bf16Cfg::kswz / vswz) -- and the swizzle is realised by choosing which
// global 16 bytes each lane fetches.
// All per-lane LDS and global offsets are loop invariant; a tile only adds
// scalar bases.
//
// Online softmax with a lazily updated reference: the exponent reference of
// a row only moves when its running maximum exceeds the reference by more
// than kRescaleLog2 (in log2 units), and the wave only looks at the row
// maxima when some lane's sum of exponentials against the current reference
// passes kSumLimit; until then no rescale of O and l is needed and no row
// maximum is formed.  The result is the same softmax (the reference cancels
// between numerator and denominator) with far fewer rescales (the idea of
// page "FlashAttention 4", centron.de, section on smarter online-softmax
// rescaling; the thresholds are this library's choice).  A wave skips the O
// rescale when none of its rows moved.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_launch.hpp"
#include "fa_varlen.hpp"

namespace fa {

constexpr float kRescaleLog2 = 8.0f;
// A lane whose 16 exponentials sum past this sends its wave to the reference
// move; a sum above it implies some exponential above 2^kRescaleLog2.
constexpr float kSumLimit = 4096.0f;      // 2^(kRescaleLog2 + 4)
// Reference of a row that has seen no visible key: finite, so the first move
// gives alpha = exp2(kNoRef - m) = 0 and an unmoved row exp2(0) = 1 without
// special cases; any visible score moves it.
constexpr float kNoRef = -1.0e30f;

#ifndef FA_BF16_BN
#define FA_BF16_BN 32
#endif
#ifndef FA_BF16_NSTAGE
#define FA_BF16_NSTAGE 2
#endif
#ifndef FA_BF16_OCC
#define FA_BF16_OCC 3
#endif
// LDS operand reads kept in flight ahead of the MFMAs of the S^T and O^T
// phases at d = 128 (0: the compiler's order, which keeps one in flight).
#ifndef FA_BF16_PF_S
#define FA_BF16_PF_S 3
#endif
#ifndef FA_BF16_PF_V
#define FA_BF16_PF_V 3
#endif
#ifndef FA_BF16_RW128
#define FA_BF16_RW128 32     // query rows per wave at d = 128 (32 or 64)
#endif
#ifndef FA_BF16_RW64
#define FA_BF16_RW64 32      // query rows per wave at d = 64 (32 or 64)
#endif

// Wait until at most `ahead` tiles' worth of this wave's LDS copies (PER
// instructions each) are outstanding, ahead in 0..MAXA.
template <int PER, int MAXA>
__device__ __forceinline__ void wait_tiles(int ahead) {
    if (MAXA >= 2 && ahead >= 2) FA_WAIT_VMCNT(2 * PER);
    else if (MAXA >= 1 && ahead >= 1) FA_WAIT_VMCNT(PER);
    else FA_WAIT_VMCNT(0);
}

// Workgroup barrier without a memory fence (the copies are awaited with
// explicit vmcnt waits); the asm keeps the compiler from moving LDS accesses
// across it, and lgkmcnt(0) retires this wave's LDS reads of the stage the
// next copies will overwrite.
__device__ __forceinline__ void wg_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int D>
struct Bf16Cfg {
    static constexpr int NW = 4;                 // waves per workgroup
    static constexpr int RW = D == 128 ? FA_BF16_RW128 : FA_BF16_RW64;  // query rows per wave
    static constexpr int NQB = RW / 32;          // 32-row query blocks per wave
    static constexpr int BM = RW * NW;           // query rows per workgroup
    static constexpr int BN = FA_BF16_BN;        // keys per K/V tile
    static constexpr int KH = BN / 32;           // 32-key halves per tile
    static constexpr int NSTAGE = FA_BF16_NSTAGE; // K/V tiles resident in LDS
    static constexpr int OCC = RW == 32 ? FA_BF16_OCC : 1; // workgroups per CU
    static constexpr int ROW = D * 2;            // bytes of one K or V row in LDS
    static constexpr int UPR = D / 8;            // 16-byte units per row
    static constexpr int TILE = BN * ROW;        // bytes of one K (or V) tile
    static constexpr int STAGE = 2 * TILE;       // K tile + V tile
    static constexpr int LDS = NSTAGE * STAGE > BM * ROW ? NSTAGE * STAGE : BM * ROW;
    static constexpr int CHUNKS = TILE / 1024;   // 1 KiB wave loads per tile and tensor
    static constexpr int CPW = CHUNKS / NW;      // ... per wave
    static constexpr int RPC = 1024 / ROW;       // rows per 1 KiB chunk
    static constexpr int KS = D / 16;            // MFMA steps over d for S
    static constexpr int PF_S = D == 128 ? FA_BF16_PF_S : 0;   // K reads ahead of the S^T MFMAs
    static constexpr int PF_V = D == 128 ? FA_BF16_PF_V : 0;   // V^T read pairs ahead of the O^T MFMAs
    static constexpr int DB = D / 32;            // 32-wide blocks of d in O
    // LDS swizzles, in 16-byte units (LDS: 64 banks of 4 bytes, 256 B per cycle).
    // K: the 16 rows one ds_read_b128 cycle touches must cover all 16 units:
    //   256-byte rows (d=128) by row mod 16; 128-byte rows (d=64, two rows per
    //   bank sweep) by (row/2) mod 8.
    // V: the 4 rows x 64 bytes one transposing-read cycle touches must cover
    //   all 16 units: XOR bits 2-3 of the unit with row mod 4 (d=128), or bit 2
    //   with (row/2) mod 2 (d=64).
    __device__ static constexpr int kswz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
    __device__ static constexpr int vswz(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }
    static_assert(CHUNKS % NW == 0, "tile must split evenly over the waves");
    static_assert(RW == 32 || RW == 64, "32 or 64 query rows per wave");
    static_assert(NSTAGE >= 2 && NSTAGE <= 4, "2 to 4 LDS stages");
};

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(256, Bf16Cfg<D>::OCC) void fa_fwd_bf16_kernel(FwdParams pin, VarlenParams vp) {
    using C = Bf16Cfg<D>;
    __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS];
    lds_char* smem = (lds_char*)smem_raw;
    const uint32_t smem_u32 = (uint32_t)(uintptr_t)smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31;     // query column owned by this lane (in each 32-row block)
    const int g = lane >> 5;     // which half of the 32x32 block's rows

    // Workgroup -> (head, query tile), XCD-aware (tile_of in fa_device.hpp);
    // for a variable-length batch, b is the sequence.
    FwdParams p = pin;
    int b, hq, hkv, qt;
    if (VARLEN && vp.compact) {
        // compact grid: slot k of query head x (heads innermost), see varlen_slot
        const int k = blockIdx.x / p.Hq;
        const int x = blockIdx.x - k * p.Hq;
        hkv = x % p.Hkv;
        hq = hkv * p.group + x / p.Hkv;
        if (!varlen_slot<true>(vp.cu_q, vp.total_q, p.B, p.n_qtiles, C::BM, k, b, qt)) return;
        b = __builtin_amdgcn_readfirstlane(b);
        qt = __builtin_amdgcn_readfirstlane(qt);
    } else {
        tile_of<CAUSAL>(p, blockIdx.x, b, hq, hkv, qt);
    }
    const int q0 = qt * C::BM;
    const int wq0 = q0 + w * C::RW;              // first row of this wave

    // Bytes between consecutive rows of one head: rows are contiguous in the
    // [B, H, N, d] layout and H*d elements apart in the packed one.
    const int64_t QSTR = VARLEN ? (int64_t)p.Hq * C::ROW : C::ROW;
    const int64_t KVSTR = VARLEN ? (int64_t)p.Hkv * C::ROW : C::ROW;
    int64_t q_tok0 = 0, k_tok0 = 0;              // first token of the sequence (packed layout)
    if constexpr (VARLEN) {
        // The sequence's bounds, clamped so malformed offsets cannot move any
        // access outside the tensors; query tiles past its length exit here,
        // before any barrier.
        const int qa = min(max(vp.cu_q[b], 0), vp.total_q);
        const int qe = min(max(vp.cu_q[b + 1], qa), vp.total_q);
        const int ka = min(max(vp.cu_k[b], 0), vp.total_k);
        const int ke = min(max(vp.cu_k[b + 1], ka), vp.total_k);
        p.Nq = __builtin_amdgcn_readfirstlane(qe - qa);
        p.Nk = __builtin_amdgcn_readfirstlane(ke - ka);
        p.causal_shift = p.Nk - p.Nq;
        q_tok0 = __builtin_amdgcn_readfirstlane(qa);
        k_tok0 = __builtin_amdgcn_readfirstlane(ka);
        if (q0 >= p.Nq) return;
    }
    const int64_t qhead = VARLEN ? q_tok0 * QSTR + (int64_t)hq * C::ROW : ((int64_t)(b * p.Hq + hq) * p.Nq) * C::ROW;
    const int64_t kvhead = VARLEN ? k_tok0 * KVSTR + (int64_t)hkv * C::ROW : ((int64_t)(b * p.Hkv + hkv) * p.Nk) * C::ROW;
    const char* Qh = reinterpret_cast<const char*>(p.q) + qhead;
    const char* Kh = reinterpret_cast<const char*>(p.k) + kvhead;
    const char* Vh = reinterpret_cast<const char*>(p.v) + kvhead;

    // Keys this workgroup needs: all of them, or (causal) up to the last
    // visible key of its last row; key tiles beyond are skipped entirely.
    // (The bounds are workgroup- or wave-uniform; readfirstlane keeps them,
    // and the loop control built on them, in scalar registers -- the integer
    // division behind the head mapping is computed on the vector ALU.)
    const int kend = key_end(q0, C::BM, p.Nk, p.causal_shift, CAUSAL);
    const int n_tiles = __builtin_amdgcn_readfirstlane((kend + C::BN - 1) / C::BN);
    // Keys this wave needs (its other tiles only take part in the copies).
    const int wkend = __builtin_amdgcn_readfirstlane(key_end(wq0, C::RW, p.Nk, p.causal_shift, CAUSAL));

    // Q rows of this lane as MFMA B operands, resident for the whole loop.
    bf16x8 qf[C::NQB][C::KS];
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
        const int qrow = wq0 + 32 * qb + n;
        if (qrow < p.Nq) {
            const char* src = Qh + (int64_t)qrow * QSTR;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                u32x4 x = ldg16(src + (2 * ks + g) * 16);
                x ^= p.q_sign;
                qf[qb][ks] = __builtin_bit_cast(bf16x8, x);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) qf[qb][ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
        }
    }

    // Loop-invariant per-lane offsets.
    // copies: chunk c = w*CPW + t covers tile rows c*RPC .. +RPC-1
    const int c_row = lane / C::UPR;
    const int c_su = lane % C::UPR;
    uint32_t dk_off[C::CPW], dv_off[C::CPW];
#pragma unroll
    for (int t = 0; t < C::CPW; ++t) {
        const int row = (w * C::CPW + t) * C::RPC + c_row;
        dk_off[t] = row * (uint32_t)KVSTR + ((c_su ^ C::kswz(row)) << 4);
        dv_off[t] = row * (uint32_t)KVSTR + ((c_su ^ C::vswz(row)) << 4);
    }
    // K reads: row 32*kh + n, unit 2*ks + g, swizzled by row (kh adds 32 rows)
    uint32_t k_off[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) k_off[ks] = n * C::ROW + (((2 * ks + g) ^ C::kswz(n)) << 4);
    // V^T reads: lane (n, g) sources key row 4*g + (n%16)/4 (+8, +16*st) at
    // d = 32*db + 16*(n/16) + 4*(n%4); one base per d-block (the row steps
    // keep row mod 4 and are immediates).
    uint32_t v_off[C::DB];
    {
        const int tr_row = 4 * g + ((n & 15) >> 2);
        const int tr_d = 16 * (n >> 4) + 4 * (n & 3);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
            const int d = 32 * db + tr_d;
            v_off[db] = tr_row * C::ROW + (((d >> 3) ^ C::vswz(tr_row)) << 4) + (d & 7) * 2;
        }
    }

    // Issue the copies of key tile j into `stage`.  Full tiles use the
    // precomputed offsets; the last, partial tile clamps rows to the last key
    // (their scores are masked and their P is 0).
    auto issue_tile = [&](int j, int stage) {
        const uint32_t kdst = smem_u32 + stage * C::STAGE + w * C::CPW * 1024;
        const uint32_t vdst = kdst + C::TILE;
        const int key0 = j * C::BN;
        const char* kb = Kh + (int64_t)key0 * KVSTR;
        const char* vb = Vh + (int64_t)key0 * KVSTR;
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
                dma16(kb, rc * (uint32_t)KVSTR + ((c_su ^ C::kswz(row)) << 4), kdst + t * 1024);
                dma16(vb, rc * (uint32_t)KVSTR + ((c_su ^ C::vswz(row)) << 4), vdst + t * 1024);
            }
        }
    };

    f32x16 o[C::NQB][C::DB];
    float mref[C::NQB];      // exponent reference per row, log2 units
    float l[C::NQB];         // this lane's part of the row sums
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db) o[qb][db] = f32x16{};
        mref[qb] = kNoRef;
        l[qb] = 0.f;
    }

    // One key tile: wait for its copies, start the next tile's copies, then
    // compute.  Templated on the LDS stage so every LDS address below is a
    // loop-invariant per-lane register plus an immediate offset.
    auto tile = [&](auto stage_c, int j) {
        constexpr int STG = decltype(stage_c)::value;
        // this wave's copies of tile j landed (those of the next tiles may
        // still be in flight), then every other wave's
        wait_tiles<2 * C::CPW, C::NSTAGE - 2>(min(C::NSTAGE - 2, n_tiles - 1 - j));
        wg_barrier();

        const int key0 = j * C::BN;
        if (key0 >= wkend) {                    // every key of this tile is hidden from this wave
            if (j + C::NSTAGE - 1 < n_tiles) issue_tile(j + C::NSTAGE - 1, (STG + C::NSTAGE - 1) % C::NSTAGE);
            return;
        }
        const lds_char* kb = smem + STG * C::STAGE;
        const lds_char* vb = kb + C::TILE;
        const bool need_mask = (key0 + C::BN > p.Nk) || (CAUSAL && key0 + C::BN - 1 > wq0 + p.causal_shift);

        // S^T of one 32-key half for one 32-row query block, from the K tile
        // in LDS (also used to recompute scores in the rare reference move).
        auto scores = [&](int kh, int qb) {
            f32x16 acc{};
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks)
                acc = mfma_bf16_32x32x16(lds_b128(kb + k_off[ks] + kh * 32 * C::ROW), qf[qb][ks], acc);
            return acc;
        };
        // Mask keys past Nk and, for causal problems, keys after each query's
        // diagonal.  Only tiles that straddle either edge pay.
        auto mask = [&](int kh, int qb, f32x16& sv) {
            const int qrow = wq0 + 32 * qb + n;
            const int lim = (CAUSAL ? min(qrow + p.causal_shift, p.Nk - 1) : p.Nk - 1) - key0 - 32 * kh - 4 * g;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (8 * (i >> 2) + (i & 3) > lim) sv[i] = -INFINITY;
        };

        // S^T of every 32-key half of the tile first (64-key tiles: the MFMA
        // pipe works through the second half while the first half's softmax
        // runs on the VALU).
        f32x16 s[C::KH][C::NQB];
        // MFMA blocks run at raised wave priority, so a co-resident wave in
        // its softmax phase issues its VALU work around them.
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kh = 0; kh < C::KH; ++kh) {
#pragma unroll
            for (int qb = 0; qb < C::NQB; ++qb) s[kh][qb] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const bf16x8 a = lds_b128(kb + k_off[ks] + kh * 32 * C::ROW);
#pragma unroll
                for (int qb = 0; qb < C::NQB; ++qb) s[kh][qb] = mfma_bf16_32x32x16(a, qf[qb][ks], s[kh][qb]);
            }
        }
        if constexpr (C::KH == 1 && C::NQB == 1) order_reads_ahead<C::KS, 1, C::PF_S>();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        // The next tile's copies go out after the score MFMAs, in the wait
        // before their results can be read.
        if (j + C::NSTAGE - 1 < n_tiles) issue_tile(j + C::NSTAGE - 1, (STG + C::NSTAGE - 1) % C::NSTAGE);

        // Per half: mask, online softmax, O^T += V^T P^T.  The reference
        // decision is made per half, so the halves are two steps of the same
        // recurrence.
#pragma unroll
        for (int kh = 0; kh < C::KH; ++kh) {
            if (need_mask) {
#pragma unroll
                for (int qb = 0; qb < C::NQB; ++qb) mask(kh, qb, s[kh][qb]);
            }

            bf16x8 pb[C::NQB][2];
#pragma unroll
            for (int qb = 0; qb < C::NQB; ++qb) {
                f32x16& sv = s[kh][qb];
                // Exponentials against the current reference first.  Only when
                // some lane's sum of its 16 exceeds kSumLimit does the wave
                // recompute these scores, form the row maxima and move
                // references -- rare after the first tile, which has no
                // reference yet and takes that path directly.  Every accepted
                // exponential is therefore at most kSumLimit, and a row whose
                // sum passed it has a score above its reference by more than
                // kRescaleLog2, so it moves and its new exponentials are at
                // most 1.
                bool slow = j == 0;
                float ls = 0.f;
                if (!slow) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) sv[i] = fast_exp2(fmaf(sv[i], p.c, -mref[qb]));
                    ls = sum16(sv);
                    if (__builtin_amdgcn_ballot_w64(!(ls <= kSumLimit)) != 0) {
                        sv = scores(kh, qb);
                        if (need_mask) mask(kh, qb, sv);
                        slow = true;
                    }
                }
                if (slow) {
                    const float mx = pair_max(max16(sv)) * p.c;     // row max of the half, log2 units
                    const bool move = mx > mref[qb] + kRescaleLog2;
                    const float mnew = move ? mx : mref[qb];
                    const float alpha = fast_exp2(mref[qb] - mnew);  // 0 at the first move, 1 if unmoved
                    mref[qb] = mnew;
                    l[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < C::DB; ++db) o[qb][db] *= alpha;
#pragma unroll
                    for (int i = 0; i < 16; ++i) sv[i] = fast_exp2(fmaf(sv[i], p.c, -mref[qb]));
                    ls = sum16(sv);
                }
                l[qb] += ls;
#pragma unroll
                for (int h8 = 0; h8 < 2; ++h8) {
                    u32x4 pk;
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) pk[e2] = pack_bf16x2(sv[8 * h8 + 2 * e2], sv[8 * h8 + 2 * e2 + 1]);
                    pb[qb][h8] = __builtin_bit_cast(bf16x8, pk);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int h8 = 0; h8 < 2; ++h8) {
                const int st = 2 * kh + h8;                      // 16-key step within the tile
#pragma unroll
                for (int db = 0; db < C::DB; ++db) {
                    const lds_char* vp = vb + v_off[db] + 16 * st * C::ROW;
                    const i16x4 lo = lds_tr16(vp);
                    const i16x4 hi = lds_tr16(vp + 8 * C::ROW);
                    const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                    for (int qb = 0; qb < C::NQB; ++qb) o[qb][db] = mfma_bf16_32x32x16(a, pb[qb][h8], o[qb][db]);
                }
            }
            if constexpr (C::NQB == 1) order_reads_ahead<2 * C::DB, 2, C::PF_V>();
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
        }
    };

#pragma unroll
    for (int t = 0; t < C::NSTAGE - 1; ++t)
        if (t < n_tiles) issue_tile(t, t);
    for (int j = 0; j < n_tiles; j += C::NSTAGE) {
        tile(std::integral_constant<int, 0>{}, j);
        if (j + 1 < n_tiles) tile(std::integral_constant<int, 1 % C::NSTAGE>{}, j + 1);
        if (C::NSTAGE > 2 && j + 2 < n_tiles) tile(std::integral_constant<int, 2 % C::NSTAGE>{}, j + 2);
        if (C::NSTAGE > 3 && j + 3 < n_tiles) tile(std::integral_constant<int, 3 % C::NSTAGE>{}, j + 3);
    }

    // Epilogue: normalise once, stage O as bf16 in LDS, then write whole rows
    // with 16-byte coalesced stores.
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
        const float lt = pair_sum(l[qb]);
        const float inv = lt > 0.f ? p.o_scale / lt : 0.f;
        const int row = w * C::RW + 32 * qb + n;          // row within the workgroup tile
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int u = 4 * db + i4;                // 16-byte unit of d = 32*db + 8*i4 + 4*g
                u32x2 val;
                val[0] = pack_bf16x2(o[qb][db][4 * i4 + 0] * inv, o[qb][db][4 * i4 + 1] * inv);
                val[1] = pack_bf16x2(o[qb][db][4 * i4 + 2] * inv, o[qb][db][4 * i4 + 3] * inv);
                *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
                    smem + row * C::ROW + ((u ^ C::kswz(row)) << 4) + 8 * g) = val;
            }
        const int qrow = wq0 + 32 * qb + n;
        if (p.lse != nullptr && g == 0 && qrow < p.Nq) {
            const float v = lt > 0.f ? (mref[qb] + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
            const int64_t li = VARLEN ? (int64_t)hq * vp.total_q + q_tok0 + qrow : (int64_t)(b * p.Hq + hq) * p.Nq + qrow;
            p.lse[li] = v;
        }
    }
    __syncthreads();
    char* Oh = reinterpret_cast<char*>(p.o) + qhead;
#pragma unroll
    for (int it = 0; it < C::RW * C::UPR / 64; ++it) {
        const int f = it * 64 + lane;
        const int row = w * C::RW + f / C::UPR;
        const int su = f % C::UPR;
        const int grow = q0 + row;
        if (grow < p.Nq) {
            const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                smem + row * C::ROW + su * 16);
            *reinterpret_cast<u32x4*>(Oh + (int64_t)grow * QSTR + ((su ^ C::kswz(row)) << 4)) = v;
        }
    }
}

template <int D, bool CAUSAL, bool VARLEN>
static hipError_t launch_one(const FwdParams& p, const VarlenParams& vp, hipStream_t stream) {
    using C = Bf16Cfg<D>;
    FwdParams pp = p;
    VarlenParams vv = vp;
    pp.n_qtiles = (p.Nq + C::BM - 1) / C::BM;
    const long long kv_rows = VARLEN ? (long long)vp.total_k : (long long)p.B * p.Nk;
    pp.kv_group = stream_group(kv_rows * p.Hkv * D * 2 * 2);
    vv.compact = VARLEN && varlen_compact(vp.total_q, p.B, pp.n_qtiles, C::BM) ? 1 : 0;
    const long long grid = vv.compact ? varlen_slots(vp.total_q, p.B, pp.n_qtiles, C::BM) * p.Hq
                                      : (long long)pp.n_qtiles * pp.n_heads;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    void* args[] = {&pp, &vv};
    const void* kernel = reinterpret_cast<const void*>(&fa_fwd_bf16_kernel<D, CAUSAL, VARLEN>);
    return hipLaunchKernel(kernel, dim3((unsigned)grid), dim3(256), args, test_extra_lds(C::LDS), stream);
}

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, hipStream_t stream) {
    const VarlenParams none{};
    if (d == 64) return causal ? launch_one<64, true, false>(p, none, stream) : launch_one<64, false, false>(p, none, stream);
    if (d == 128) return causal ? launch_one<128, true, false>(p, none, stream) : launch_one<128, false, false>(p, none, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_fwd_bf16_varlen(const FwdParams& p, const VarlenParams& vp, int d, bool causal,
                                  hipStream_t stream) {
    if (d == 64) return causal ? launch_one<64, true, true>(p, vp, stream) : launch_one<64, false, true>(p, vp, stream);
    if (d == 128) return causal ? launch_one<128, true, true>(p, vp, stream) : launch_one<128, false, true>(p, vp, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa
