// Backward pass of exact attention, bfloat16, head dim 64 or 128, gfx950.
//
// The backward pass recomputes the attention probabilities from the stored
// per-row log-sum-exp instead of keeping P (page "Flash Attention",
// 21medien.de, key techniques, recomputation).  With S = scale Q K^T + mask,
// P = exp(S - LSE) row by row, and the upstream gradient dO:
//   dV = P^T dO,   dP = dO V^T,   dS = P o (dP - D) with D_i = <dO_i, O_i>,
//   dQ = scale dS K,   dK = scale dS^T Q
// (D_i equals sum_j P_ij dP_ij, the row term of the softmax Jacobian).
//
// Three kernels on the caller's stream:
//   1. fa_bwd_prep_kernel: D_i and the base-2 LSE per query row into the
//      caller's workspace (a row that saw no key gets +inf, so its P is 0);
//   2. dK and dV: a workgroup owns a block of keys of one key/value head and
//      streams the Q and dO rows of every query head of its group through
//      LDS; dK and dV accumulate in registers, so grouped-query sums need no
//      atomics and the result is deterministic.  d = 64: fa_bwd_dkv_kernel,
//      128 keys, one wave per 32 keys; d = 128: fa_bwd_dkv_pair_kernel, 64
//      keys, a pair of waves per 32 keys (one computes P and dV, the other
//      dS and dK);
//   3. dQ: one workgroup owns 128 query rows (32 per wave) and streams
//      32-key tiles of K and V, like the forward kernel (fa_bwd_dq_kernel;
//      at d = 128 fa_bwd_dq_pipe_kernel, which issues the next tile's score
//      products during the current tile's softmax).
// Splitting dQ from dK/dV computes S and dP twice (7 products instead of 5)
// but needs neither a float workspace for dQ nor atomics.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16; lane l holds column l % 32 and rows
// 8*(i/4) + 4*(l/32) + (i%4) of the 32x32 result, see fa_device.hpp):
//   dQ kernel, per wave and 32-key tile:
//     S^T = K Q^T, dP^T = V dO^T  (A: K / V rows from LDS, B: Q / dO rows in
//                                   registers; lane = query)
//     dQ^T += K^T dS^T            (A: K^T through ds_read_b64_tr_b16, B: dS
//                                   from the score registers)
//   dK/dV kernel, per wave and 32-query tile:
//     S = Q K^T, dP = dO V^T      (A: Q / dO rows from LDS, B: K / V rows in
//                                   registers; lane = key)
//     dV^T += dO^T P, dK^T += Q^T dS   (A: transposing LDS reads of dO / Q)
// Tiles are copied straight into LDS (global_load_lds_dwordx4), two stages
// (three in the pipelined dQ kernel), XOR-swizzled in 16-byte units so that
// both the ds_read_b128 row reads and the transposing reads are conflict-free
// (BwdCfg::swz).
#include <algorithm>
#include <type_traits>

#include "fa_bwd.hpp"
#include "fa_device.hpp"
#include "fa_launch.hpp"
#include "fa_varlen.hpp"


namespace fa {

namespace {

template <int D>
struct BwdCfg {
    static constexpr int NW = 4;                  // waves per workgroup
    static constexpr int ROWS = 128;              // query rows (dQ) or keys (dK/dV) per workgroup
    static constexpr int T = 32;                  // keys per streamed tile (dQ kernel)
    static constexpr int ROW = D * 2;             // bytes per row
    static constexpr int UPR = D / 8;             // 16-byte units per row
    static constexpr int KS = D / 16;             // MFMA steps over d
    static constexpr int DB = D / 32;             // 32-wide blocks of d
    static constexpr int TILE = T * ROW;          // bytes of one streamed tile of one tensor
    static constexpr int STAGE = 2 * TILE;        // two tensors per stage
    static constexpr int TILES = 2 * STAGE;       // two stages
    static constexpr int OUT = ROWS * ROW;        // epilogue staging of 128 output rows
    static constexpr int LDS = TILES > OUT ? TILES : OUT;                       // dQ kernel
    static constexpr int RPC = 1024 / ROW;        // rows per 1 KiB copy
    // 16-byte-unit XOR swizzle of LDS rows.  The tiles are read both as rows
    // (ds_read_b128: 16 lanes per cycle on 16 consecutive rows) and
    // transposed (ds_read_b64_tr_b16: 32 lanes per cycle on 4 rows, 4 units
    // each), and the swizzle keeps both patterns on distinct banks:
    //   256-byte rows: bits 2-3 = row mod 4 move the 4 rows of a transposed
    //     read to different 64-byte bank groups, bits 0-1 = (row / 4) mod 4
    //     complete a permutation of 16 consecutive rows;
    //   128-byte rows (two share a bank sweep): bit 2 = (row / 2) mod 2,
    //     bits 0-1 = (row / 4) mod 4, a permutation of the 8 rows of one
    //     parity in 16.
    // (row mod 16 alone, the plain row swizzle, put the 4 rows of a
    // transposed read into one bank group: a 4-way conflict.)  It is
    // unchanged by a step of 16 rows.
    __device__ static constexpr int swz(int row) {
        return D == 128 ? 4 * (row & 3) + ((row >> 2) & 3) : 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
    }
};

// LDS operand reads kept in flight ahead of the MFMAs of the score phases
// (S, dP) and of the accumulation phases (dV, dK, dQ); 0: the compiler's order.
#ifndef FA_BWD_PF_S
#define FA_BWD_PF_S 4
#endif
#ifndef FA_BWD_PF_V
#define FA_BWD_PF_V 3
#endif
#ifndef FA_BWD_DQ_PIPE
#define FA_BWD_DQ_PIPE 1     // d = 128: dQ with the key loop software-pipelined
#endif

// dK/dV kernel in one wave per key (the d = 64 path): NH = 2 32-row query
// halves per streamed tile give the MFMA pipe the second half's S and dP
// products while the first half's exponentials run.
template <int D>
struct KvCfg {
    using C = BwdCfg<D>;
    static constexpr int NH = 2;
    static constexpr int OCC = 2;                 // workgroups per CU
    static constexpr int TQ = 32 * NH;            // query rows per streamed tile
    static constexpr int QSTAGE = 2 * TQ * D * 2; // Q tile + dO tile
    static constexpr int QTILES = 2 * QSTAGE;     // two stages
    static constexpr int SCRATCH = 8 * TQ * C::NW;   // per wave: 2 * TQ floats of row statistics
    static constexpr int LDS = QTILES + SCRATCH > C::OUT ? QTILES + SCRATCH : C::OUT;
};

// Workgroup barrier without a memory fence; the tile copies are awaited with
// vmcnt before it.  lgkmcnt(0) retires this wave's LDS reads of the stage the
// next copies overwrite.
__device__ __forceinline__ void bwd_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Copy rows r0 .. r0+NR-1 of two tensors of D-element rows `stride` bytes
// apart (same layout, rows past N - 1 clamped to the last row) into an LDS
// stage: tensor a at dst, tensor b at dst + NR rows.  Every wave copies its
// share of the 1 KiB pieces of each.
template <int D, int NR>
__device__ __forceinline__ void copy_pair(const char* a, const char* b, int r0, int N, uint32_t dst,
                                          int w, int lane, int64_t stride) {
    using C = BwdCfg<D>;
    constexpr int BYTES = NR * C::ROW;
    constexpr int PW = BYTES / 1024 / C::NW;      // pieces per wave and tensor
    static_assert(PW >= 1, "a tile must give every wave a copy");
    const int c_row = lane / C::UPR, c_su = lane % C::UPR;
    const char* abase = a + (int64_t)r0 * stride;
    const char* bbase = b + (int64_t)r0 * stride;
#pragma unroll
    for (int t = 0; t < PW; ++t) {
        const int piece = w * PW + t;
        const int row = piece * C::RPC + c_row;
        const uint32_t off = copy_src_row(row, r0, N) * (uint32_t)stride + ((c_su ^ C::swz(row)) << 4);
        dma16(abase, off, dst + piece * 1024);
        dma16(bbase, off, dst + BYTES + piece * 1024);
    }
}

// Per-lane LDS offsets of a 32-row tile.
template <int D>
struct TileOffsets {
    using C = BwdCfg<D>;
    uint32_t b[C::KS];        // ds_read_b128 of row n, units 2*ks + g (MFMA A operand)
    uint32_t lo[C::DB];       // transposing reads: row 4g + (n%16)/4 ...
    uint32_t hi[C::DB];       // ... and 8 rows further; +16 rows per 16-row step
    __device__ TileOffsets(int n, int g) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) b[ks] = n * C::ROW + (((2 * ks + g) ^ C::swz(n)) << 4);
        const int tr_row = 4 * g + ((n & 15) >> 2);
        const int tr_d = 16 * (n >> 4) + 4 * (n & 3);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
            const int d = 32 * db + tr_d;
            lo[db] = tr_row * C::ROW + (((d >> 3) ^ C::swz(tr_row)) << 4) + (d & 7) * 2;
            hi[db] = (tr_row + 8) * C::ROW + (((d >> 3) ^ C::swz(tr_row + 8)) << 4) + (d & 7) * 2;
        }
    }
};

// A operand of X^T (d-block db, 16-row step st) from a row-major tile in LDS.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const lds_char* tile, const TileOffsets<D>& off, int db, int st) {
    using C = BwdCfg<D>;
    const i16x4 lo = lds_tr16(tile + off.lo[db] + 16 * st * C::ROW);
    const i16x4 hi = lds_tr16(tile + off.hi[db] + 16 * st * C::ROW);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// The 16 accumulator values of a lane as two bf16 B operands (16-row steps).
__device__ __forceinline__ void pack_b(const f32x16& v, bf16x8 (&out)[2]) {
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8) {
        u32x4 pk;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) pk[e2] = pack_bf16x2(v[8 * h8 + 2 * e2], v[8 * h8 + 2 * e2 + 1]);
        out[h8] = __builtin_bit_cast(bf16x8, pk);
    }
}

// Row `row` of a bf16 tensor with rows `stride` bytes apart as B operands
// (zeros past the end).
template <int D>
__device__ __forceinline__ void load_b_rows(const char* base, int row, int N, int g, bf16x8 (&f)[D / 16],
                                            int64_t stride) {
    using C = BwdCfg<D>;
    if (row < N) {
        const char* src = base + (int64_t)row * stride;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) f[ks] = __builtin_bit_cast(bf16x8, ldg16(src + (2 * ks + g) * 16));
    } else {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) f[ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }
}

// Scale 128 rows of fp32 accumulators (X^T blocks per wave: lane = row
// 32*w + n, d = 32*db + 8*i4 + 4*g + r), convert to bf16, stage them in LDS
// and write whole rows (`stride` bytes apart) to dst with 16-byte coalesced
// stores.
template <int D>
__device__ __forceinline__ void store_rows(lds_char* smem, const f32x16 (&acc)[D / 32], float mul, char* dst,
                                           int r0, int N, int w, int n, int g, int lane, int64_t stride) {
    using C = BwdCfg<D>;
    __syncthreads();
    const int row = w * 32 + n;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int u = 4 * db + i4;
            u32x2 val;
            val[0] = pack_bf16x2(acc[db][4 * i4 + 0] * mul, acc[db][4 * i4 + 1] * mul);
            val[1] = pack_bf16x2(acc[db][4 * i4 + 2] * mul, acc[db][4 * i4 + 3] * mul);
            *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
                smem + row * C::ROW + ((u ^ C::swz(row)) << 4) + 8 * g) = val;
        }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 32 * C::UPR / 64; ++it) {
        const int f = it * 64 + lane;
        const int r = w * 32 + f / C::UPR;
        const int su = f % C::UPR;
        const int grow = r0 + r;
        if (grow < N) {
            const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(smem + r * C::ROW + su * 16);
            *reinterpret_cast<u32x4*>(dst + (int64_t)grow * stride + ((su ^ C::swz(r)) << 4)) = v;
        }
    }
}

// Variable-length batches: the query and key token ranges of sequence s,
// clamped to the tensors, so malformed offsets cannot move an access out of
// bounds.  Sets p.Nq, p.Nk and the causal shift to the sequence's own.
__device__ __forceinline__ void seq_bounds(BwdParams& p, int s, int64_t& q_tok0, int64_t& k_tok0) {
    const int qa = min(max(p.cu_q[s], 0), p.total_q);
    const int qe = min(max(p.cu_q[s + 1], qa), p.total_q);
    const int ka = min(max(p.cu_k[s], 0), p.total_k);
    const int ke = min(max(p.cu_k[s + 1], ka), p.total_k);
    p.Nq = __builtin_amdgcn_readfirstlane(qe - qa);
    p.Nk = __builtin_amdgcn_readfirstlane(ke - ka);
    p.causal_shift = p.Nk - p.Nq;
    q_tok0 = __builtin_amdgcn_readfirstlane(qa);
    k_tok0 = __builtin_amdgcn_readfirstlane(ka);
}

// ---------------------------------------------------------------- 1. D and base-2 LSE

// Rows are taken in memory order; in the packed layout row r is token r / Hq
// of head r % Hq, whose workspace and lse index is head * total_q + token.
template <int D, bool VARLEN>
__global__ __launch_bounds__(256) void fa_bwd_prep_kernel(BwdParams p) {
    constexpr int LPR = D / 8;          // lanes per row, 16 bytes each
    constexpr int RPW = 64 / LPR;       // rows per wave per step
    const int64_t R = VARLEN ? (int64_t)p.total_q * p.Hq : (int64_t)p.B * p.Hq * p.Nq;
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
    const int64_t n_waves = ((int64_t)gridDim.x * 256) >> 6;
    const int sub = lane / LPR, part = lane % LPR;
    for (int64_t r0 = wave * RPW; r0 < R; r0 += n_waves * RPW) {
        const int64_t r = r0 + sub;
        float acc = 0.f;
        if (r < R) {
            const u32x4 a = ldg16(reinterpret_cast<const char*>(p.dout) + r * (D * 2) + part * 16);
            const u32x4 o = ldg16(reinterpret_cast<const char*>(p.o) + r * (D * 2) + part * 16);
#pragma unroll
            for (int k = 0; k < 4; ++k) acc += bf16_lo(a[k]) * bf16_lo(o[k]) + bf16_hi(a[k]) * bf16_hi(o[k]);
        }
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m, 64);
        if (part == 0 && r < R) {
            int64_t wi = r;
            if constexpr (VARLEN) {
                const int64_t t = r / p.Hq;
                wi = (r - t * p.Hq) * p.total_q + t;
            }
            p.ws[wi] = acc;
            const float l = p.lse[wi];
            p.ws[R + wi] = l == -INFINITY ? INFINITY : l * kLog2e;
        }
    }
}

// ---------------------------------------------------------------- 2. dK and dV

// The query tiles a dK/dV workgroup streams, in order: for each query head
// hkv*group + gi of the group, query tiles qt0 .. qt0 + nqt - 1.  The walk
// keeps the tile index within the head and the head's first row (bytes into
// q / dO, index into the workspace) and advances them by one tile per call
// of next(), instead of dividing the tile counter by nqt each time.
struct QueryWalk {
    int iq = 0;               // query tile qt0 + iq of the current head
    int nqt;
    int64_t qbase, wrow0;     // the current head's first row: bytes into q / dO, workspace index
    int64_t head_bytes, head_rows;
    __device__ QueryWalk(const BwdParams& p, int b, int hkv, int64_t q_tok0, int nqt_, bool varlen, int row_bytes)
        : nqt(nqt_) {
        const int h = hkv * p.group;
        const int64_t qstr = varlen ? (int64_t)p.Hq * row_bytes : row_bytes;
        qbase = varlen ? q_tok0 * qstr + (int64_t)h * row_bytes : (int64_t)(b * p.Hq + h) * p.Nq * row_bytes;
        wrow0 = varlen ? (int64_t)h * p.total_q + q_tok0 : (int64_t)(b * p.Hq + h) * p.Nq;
        head_bytes = varlen ? (int64_t)row_bytes : (int64_t)p.Nq * row_bytes;
        head_rows = varlen ? (int64_t)p.total_q : (int64_t)p.Nq;
    }
    __device__ void next() {
        if (++iq == nqt) {
            iq = 0;
            qbase += head_bytes;
            wrow0 += head_rows;
        }
    }
};

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(256, KvCfg<D>::OCC) void fa_bwd_dkv_kernel(BwdParams pin) {
    BwdParams p = pin;
    using C = BwdCfg<D>;
    using K = KvCfg<D>;
    constexpr int NH = K::NH, TQ = K::TQ;
    __shared__ __attribute__((aligned(1024))) char smem_raw[K::LDS];
    lds_char* smem = (lds_char*)smem_raw;
    const uint32_t smem_u32 = (uint32_t)(uintptr_t)smem;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31;
    const int g = lane >> 5;

    // workgroup -> (batch, key/value head, key tile); the key tiles with the
    // most visible queries (the first ones, for causal problems) come first
    int b, hkv, kt;
    if (VARLEN && p.compact_dkv) {
        // compact grid: slot k of key/value head hkv, key tiles from 0 up (varlen_slot)
        const int k = blockIdx.x / p.Hkv;
        hkv = blockIdx.x - k * p.Hkv;
        if (!varlen_slot<false>(p.cu_k, p.total_k, p.B, p.n_ktiles, C::ROWS, k, b, kt)) return;
        b = __builtin_amdgcn_readfirstlane(b);
        kt = __builtin_amdgcn_readfirstlane(kt);
    } else {
        int kvflat, unused;
        bwd_order(blockIdx.x, p.B * p.Hkv, 1, p.n_ktiles, p.group_dkv, kvflat, unused, kt);
        b = kvflat / p.Hkv;
        hkv = kvflat - b * p.Hkv;
    }
    const int k0 = kt * C::ROWS;
    const int wk0 = k0 + 32 * w;
    const int key = wk0 + n;

    // bytes between consecutive rows of one head (packed layout: H*d elements)
    const int64_t QSTR = VARLEN ? (int64_t)p.Hq * C::ROW : C::ROW;
    const int64_t KVSTR = VARLEN ? (int64_t)p.Hkv * C::ROW : C::ROW;
    int64_t q_tok0 = 0, k_tok0 = 0;
    if constexpr (VARLEN) {
        seq_bounds(p, b, q_tok0, k_tok0);
        if (k0 >= p.Nk) return;                  // past this sequence's keys: nothing to write
    }
    const int64_t kvbase = VARLEN ? k_tok0 * KVSTR + (int64_t)hkv * C::ROW
                                  : (int64_t)(b * p.Hkv + hkv) * p.Nk * C::ROW;
    bf16x8 kf[C::KS], vf[C::KS];
    load_b_rows<D>(reinterpret_cast<const char*>(p.k) + kvbase, key, p.Nk, g, kf, KVSTR);
    load_b_rows<D>(reinterpret_cast<const char*>(p.v) + kvbase, key, p.Nk, g, vf, KVSTR);

    // query tiles to visit, per query head of the group
    const int qs = CAUSAL ? max(0, k0 - p.causal_shift) : 0;       // first query that sees key k0
    const int qt0 = qs / TQ;
    const int nqt = qs < p.Nq ? (p.Nq + TQ - 1) / TQ - qt0 : 0;
    const int n_it = __builtin_amdgcn_readfirstlane(nqt * p.group);
    const int wqs = __builtin_amdgcn_readfirstlane(CAUSAL ? max(0, wk0 - p.causal_shift) : 0);
    const int64_t R = VARLEN ? (int64_t)p.Hq * p.total_q : (int64_t)p.B * p.Hq * p.Nq;

    const TileOffsets<D> off(n, g);
    float* scratch = reinterpret_cast<float*>(smem_raw + K::QTILES + w * 8 * TQ);

    f32x16 dk[C::DB], dv[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
        dk[db] = f32x16{};
        dv[db] = f32x16{};
    }

    // Tile `it` = (query head hkv*group + it / nqt, query tile qt0 + it % nqt).
    // Its copies go to LDS; the row statistics of its TQ rows to `pre`
    // (pre[h]: lanes 0-31 the base-2 LSE of row 32h + n, lanes 32-63 its D).
    float pre[NH];
    QueryWalk qw(p, b, hkv, q_tok0, nqt, VARLEN, C::ROW);
    auto issue = [&](int stage) {
        const int qt = qt0 + qw.iq;
        copy_pair<D, TQ>(reinterpret_cast<const char*>(p.q) + qw.qbase,
                         reinterpret_cast<const char*>(p.dout) + qw.qbase, qt * TQ, p.Nq,
                         smem_u32 + stage * K::QSTAGE, w, lane, QSTR);
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
            const int r = min(qt * TQ + 32 * hh + n, p.Nq - 1);
            pre[hh] = p.ws[(g ? 0 : R) + qw.wrow0 + r];
        }
        qw.next();
    };
    int cur_q = 0;                               // the computed tile is query tile qt0 + cur_q

    auto tile = [&](auto stage_c, int it) {
        constexpr int STG = decltype(stage_c)::value;
        FA_WAIT_VMCNT(0);
        bwd_barrier();
        // scratch: [0, TQ) base-2 LSE, [TQ, 2 TQ) D of the tile's rows
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) scratch[(g ? TQ : 0) + 32 * hh + n] = pre[hh];
        const int q0 = (qt0 + cur_q) * TQ;
        if (++cur_q == nqt) cur_q = 0;
        // no key of this wave is visible to these rows
        if (q0 + TQ - 1 < wqs) {
            if (it + 1 < n_it) issue(STG ^ 1);
            return;
        }
        const lds_char* qb = smem + STG * K::QSTAGE;
        const lds_char* ob = qb + TQ * C::ROW;
        // S and dP of every half first: the MFMA pipe works through the later
        // halves while the first half's exponentials run on the VALU
        f32x16 s[NH], dp[NH];
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
            s[hh] = f32x16{};
            dp[hh] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                s[hh] = mfma_bf16_32x32x16(lds_b128(qb + 32 * hh * C::ROW + off.b[ks]), kf[ks], s[hh]);
                dp[hh] = mfma_bf16_32x32x16(lds_b128(ob + 32 * hh * C::ROW + off.b[ks]), vf[ks], dp[hh]);
            }
        }
        order_reads_ahead<NH * C::KS * 2, 1, FA_BWD_PF_S>();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        if (it + 1 < n_it) issue(STG ^ 1);

#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
            const int q0h = q0 + 32 * hh;
            // row statistics of the 16 query rows this lane holds
            float l2[16], dl[16];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(scratch + 32 * hh + 8 * a + 4 * g);
                const f32x4 y = *reinterpret_cast<const f32x4*>(scratch + TQ + 32 * hh + 8 * a + 4 * g);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    l2[4 * a + r] = x[r];
                    dl[4 * a + r] = y[r];
                }
            }
            const bool need_mask = (q0h + 32 > p.Nq) || (CAUSAL && wk0 + 31 > q0h + p.causal_shift);
            f32x16 pv, ds;
#pragma unroll
            for (int i = 0; i < 16; ++i) pv[i] = fast_exp2(fmaf(s[hh][i], p.c, -l2[i]));
            if (need_mask) {
                // element i holds query row q0h + 4g + idx(i): rows past Nq, and
                // (causal) rows before the first one this lane's key is visible to
                const int hi = p.Nq - q0h - 4 * g;
                const int lo = CAUSAL ? key - p.causal_shift - q0h - 4 * g : 0;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int idx = 8 * (i >> 2) + (i & 3);
                    pv[i] = (idx >= hi || idx < lo) ? 0.f : pv[i];
                }
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) ds[i] = pv[i] * (dp[hh][i] - dl[i]);
            bf16x8 pp[2], pd[2];
            pack_b(pv, pp);
            pack_b(ds, pd);
            const lds_char* qbh = qb + 32 * hh * C::ROW;
            const lds_char* obh = ob + 32 * hh * C::ROW;
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int db = 0; db < C::DB; ++db) {
                    dv[db] = mfma_bf16_32x32x16(tr_operand<D>(obh, off, db, st), pp[st], dv[db]);
                    dk[db] = mfma_bf16_32x32x16(tr_operand<D>(qbh, off, db, st), pd[st], dk[db]);
                }
            order_reads_ahead<2 * C::DB * 2, 2, FA_BWD_PF_V>();
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
        }
    };

    if (n_it > 0) issue(0);
    for (int it = 0; it < n_it; it += 2) {
        tile(std::integral_constant<int, 0>{}, it);
        if (it + 1 < n_it) tile(std::integral_constant<int, 1>{}, it + 1);
    }

    char* dK = reinterpret_cast<char*>(p.dk) + kvbase;
    char* dV = reinterpret_cast<char*>(p.dv) + kvbase;
    store_rows<D>(smem, dk, p.scale, dK, k0, p.Nk, w, n, g, lane, KVSTR);
    store_rows<D>(smem, dv, 1.f, dV, k0, p.Nk, w, n, g, lane, KVSTR);
}

// ---------------------------------------------------------------- 2b. dK and dV by wave pairs (d = 128)

// The work of one key split over a pair of waves.  The P wave holds the key's
// K row and computes S = Q K^T, P and dV^T += dO^T P; the dS wave holds its V
// row and computes dP = dO V^T, takes P from the P wave through LDS, and
// forms dS = P (dP - D) and dK^T += Q^T dS.  That is four products per key and
// query tile, as in the one-wave kernel above, but each wave keeps one
// operand and one accumulator, so three workgroups fit per CU at d = 128
// (the one-wave kernel needs 474 registers there).  A workgroup owns 64
// keys: waves 0 and 1 are the P waves of keys 0-31 and 32-63, waves 2 and 3
// the dS waves of the same keys.  A second barrier per tile publishes P.
template <int D>
struct PairCfg {
    using C = BwdCfg<D>;
    static constexpr int KEYS = 64;                    // keys per workgroup
    static constexpr int TQ = 32;                      // query rows per streamed tile
    static constexpr int QSTAGE = 2 * TQ * C::ROW;     // Q tile + dO tile
    static constexpr int QTILES = 2 * QSTAGE;          // two stages
    static constexpr int PX = 2 * 32 * 32 * 4;         // P of both pairs, fp32
    static constexpr int SCRATCH = 4 * TQ * C::NW;     // per wave: one row statistic of the tile
    static constexpr int LDS = QTILES + PX + SCRATCH > C::OUT ? QTILES + PX + SCRATCH : C::OUT;
};

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(256, 3) void fa_bwd_dkv_pair_kernel(BwdParams pin) {
    BwdParams p = pin;
    using C = BwdCfg<D>;
    using K = PairCfg<D>;
    constexpr int TQ = K::TQ;
    __shared__ __attribute__((aligned(1024))) char smem_raw[K::LDS];
    lds_char* smem = (lds_char*)smem_raw;
    const uint32_t smem_u32 = (uint32_t)(uintptr_t)smem;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31;
    const int g = lane >> 5;
    const bool dsw = w >= 2;                     // dS wave (else P wave)
    const int pr = w & 1;                        // pair: keys 32 pr .. 32 pr + 31 of the workgroup

    // workgroup -> (batch, key/value head, key tile), as in fa_bwd_dkv_kernel
    int b, hkv, kt;
    if (VARLEN && p.compact_dkv) {
        const int k = blockIdx.x / p.Hkv;
        hkv = blockIdx.x - k * p.Hkv;
        if (!varlen_slot<false>(p.cu_k, p.total_k, p.B, p.n_ktiles, K::KEYS, k, b, kt)) return;
        b = __builtin_amdgcn_readfirstlane(b);
        kt = __builtin_amdgcn_readfirstlane(kt);
    } else {
        int kvflat, unused;
        bwd_order(blockIdx.x, p.B * p.Hkv, 1, p.n_ktiles, p.group_dkv, kvflat, unused, kt);
        b = kvflat / p.Hkv;
        hkv = kvflat - b * p.Hkv;
    }
    const int k0 = kt * K::KEYS;
    const int wk0 = k0 + 32 * pr;
    const int key = wk0 + n;

    const int64_t QSTR = VARLEN ? (int64_t)p.Hq * C::ROW : C::ROW;
    const int64_t KVSTR = VARLEN ? (int64_t)p.Hkv * C::ROW : C::ROW;
    int64_t q_tok0 = 0, k_tok0 = 0;
    if constexpr (VARLEN) {
        seq_bounds(p, b, q_tok0, k_tok0);
        if (k0 >= p.Nk) return;                  // past this sequence's keys: nothing to write
    }
    const int64_t kvbase = VARLEN ? k_tok0 * KVSTR + (int64_t)hkv * C::ROW
                                  : (int64_t)(b * p.Hkv + hkv) * p.Nk * C::ROW;
    // B operand of the first product: K rows (P wave) or V rows (dS wave)
    bf16x8 rf[C::KS];
    load_b_rows<D>(reinterpret_cast<const char*>(dsw ? p.v : p.k) + kvbase, key, p.Nk, g, rf, KVSTR);

    const int qs = CAUSAL ? max(0, k0 - p.causal_shift) : 0;       // first query that sees key k0
    const int qt0 = qs / TQ;
    const int nqt = qs < p.Nq ? (p.Nq + TQ - 1) / TQ - qt0 : 0;
    const int n_it = __builtin_amdgcn_readfirstlane(nqt * p.group);
    const int64_t R = VARLEN ? (int64_t)p.Hq * p.total_q : (int64_t)p.B * p.Hq * p.Nq;

    const TileOffsets<D> off(n, g);
    float* scratch = reinterpret_cast<float*>(smem_raw + K::QTILES + K::PX + w * 4 * TQ);
    float* px = reinterpret_cast<float*>(smem_raw + K::QTILES) + pr * 1024;   // this pair's P

    f32x16 acc[C::DB];                           // dV^T (P wave) or dK^T (dS wave)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

    // the statistic each wave needs: base-2 LSE (P wave) or D (dS wave)
    const int64_t stat = dsw ? 0 : R;
    float pre;
    QueryWalk qw(p, b, hkv, q_tok0, nqt, VARLEN, C::ROW);
    auto issue = [&](int stage) {
        const int qt = qt0 + qw.iq;
        copy_pair<D, TQ>(reinterpret_cast<const char*>(p.q) + qw.qbase,
                         reinterpret_cast<const char*>(p.dout) + qw.qbase, qt * TQ, p.Nq,
                         smem_u32 + stage * K::QSTAGE, w, lane, QSTR);
        pre = p.ws[stat + qw.wrow0 + min(qt * TQ + n, p.Nq - 1)];
        qw.next();
    };
    int cur_q = 0;                               // the computed tile is query tile qt0 + cur_q

    // The role is a template argument: each role runs a loop of its own, so
    // the registers of one role's values are not held live in the other's.
    auto tile = [&](auto stage_c, auto role_c, int it) {
        constexpr int STG = decltype(stage_c)::value;
        constexpr bool DSW = decltype(role_c)::value;
        FA_WAIT_VMCNT(0);
        bwd_barrier();
        scratch[n] = pre;                        // both lane halves write the same value of row n
        const int q0 = (qt0 + cur_q) * TQ;
        if (++cur_q == nqt) cur_q = 0;
        const lds_char* qb = smem + STG * K::QSTAGE;
        const lds_char* ob = qb + TQ * C::ROW;
        f32x16 s = f32x16{};                     // S (P wave) or dP (dS wave)
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) s = mfma_bf16_32x32x16(lds_b128((DSW ? ob : qb) + off.b[ks]), rf[ks], s);
        order_reads_ahead<C::KS, 1, FA_BWD_PF_S>();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        if (it + 1 < n_it) issue(STG ^ 1);

        // element i of a lane holds query row q0 + 8*(i/4) + 4g + i%4 and key `key`
        bf16x8 pk[2];                            // P (P wave) or dS (dS wave) as B operands
        if constexpr (!DSW) {
            float l2[16];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(scratch + 8 * a + 4 * g);
#pragma unroll
                for (int r = 0; r < 4; ++r) l2[4 * a + r] = x[r];
            }
            f32x16 pv;
#pragma unroll
            for (int i = 0; i < 16; ++i) pv[i] = fast_exp2(fmaf(s[i], p.c, -l2[i]));
            const bool need_mask = (q0 + 32 > p.Nq) || (CAUSAL && wk0 + 31 > q0 + p.causal_shift);
            if (need_mask) {
                // rows past Nq, and (causal) rows before the first one this
                // lane's key is visible to
                const int hi = p.Nq - q0 - 4 * g;
                const int lo = CAUSAL ? key - p.causal_shift - q0 - 4 * g : 0;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int idx = 8 * (i >> 2) + (i & 3);
                    pv[i] = (idx >= hi || idx < lo) ? 0.f : pv[i];
                }
            }
            // lane-major 16-byte pieces: conflict-free, and the dS wave's lane
            // reads back exactly what the same lane of the P wave wrote
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<f32x4*>(px + j * 256 + lane * 4) = f32x4{pv[4 * j], pv[4 * j + 1], pv[4 * j + 2], pv[4 * j + 3]};
            pack_b(pv, pk);
        }
        f32x16 sd;                               // dS wave: dP - D, ready before P arrives
        if constexpr (DSW) {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const f32x4 dl = *reinterpret_cast<const f32x4*>(scratch + 8 * a + 4 * g);
#pragma unroll
                for (int r = 0; r < 4; ++r) sd[4 * a + r] = s[4 * a + r] - dl[r];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        bwd_barrier();                           // P of the tile is in LDS
        if constexpr (DSW) {
            f32x16 ds;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const f32x4 pv = *reinterpret_cast<const f32x4*>(px + a * 256 + lane * 4);
#pragma unroll
                for (int r = 0; r < 4; ++r) ds[4 * a + r] = pv[r] * sd[4 * a + r];
            }
            pack_b(ds, pk);
        }
        // dV^T += dO^T P (P wave) or dK^T += Q^T dS (dS wave)
        const lds_char* tb = DSW ? qb : ob;
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
                acc[db] = mfma_bf16_32x32x16(tr_operand<D>(tb, off, db, st), pk[st], acc[db]);
        order_reads_ahead<2 * C::DB, 2, FA_BWD_PF_V>();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
    };

    auto run = [&](auto role_c) {
        if (n_it > 0) issue(0);
        for (int it = 0; it < n_it; it += 2) {
            tile(std::integral_constant<int, 0>{}, role_c, it);
            if (it + 1 < n_it) tile(std::integral_constant<int, 1>{}, role_c, it + 1);
        }
    };
    if (dsw)
        run(std::true_type{});
    else
        run(std::false_type{});

    // P waves write dV, dS waves dK (scaled); store_rows stages wave w's rows
    // at 32 w, so the dS waves' rows start 64 below their keys
    char* dst = reinterpret_cast<char*>(dsw ? p.dk : p.dv) + kvbase;
    store_rows<D>(smem, acc, dsw ? p.scale : 1.f, dst, dsw ? k0 - 64 : k0, p.Nk, w, n, g, lane, KVSTR);
}

// ---------------------------------------------------------------- 3. dQ

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(256, 2) void fa_bwd_dq_kernel(BwdParams pin) {
    BwdParams p = pin;
    using C = BwdCfg<D>;
    __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS];
    lds_char* smem = (lds_char*)smem_raw;
    const uint32_t smem_u32 = (uint32_t)(uintptr_t)smem;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31;
    const int g = lane >> 5;

    // workgroup -> (batch, query head, query tile): heads first, and for
    // causal problems the query tiles with the most keys first
    int b, hkv, hq, qt;
    if (VARLEN && p.compact_dq) {
        // compact grid: slot k of query head x, query tiles from the last down (varlen_slot)
        const int k = blockIdx.x / p.Hq;
        const int x = blockIdx.x - k * p.Hq;
        hkv = x % p.Hkv;
        hq = hkv * p.group + x / p.Hkv;
        if (!varlen_slot<true>(p.cu_q, p.total_q, p.B, p.n_qtiles, C::ROWS, k, b, qt)) return;
        b = __builtin_amdgcn_readfirstlane(b);
        qt = __builtin_amdgcn_readfirstlane(qt);
    } else {
        int t_ord, kvflat, gi;
        bwd_order(blockIdx.x, p.B * p.Hkv, p.group, p.n_qtiles, p.group_dq, kvflat, gi, t_ord);
        b = kvflat / p.Hkv;
        hkv = kvflat - b * p.Hkv;
        hq = hkv * p.group + gi;
        qt = CAUSAL ? p.n_qtiles - 1 - t_ord : t_ord;
    }
    const int q0 = qt * C::ROWS;
    const int wq0 = q0 + 32 * w;
    const int qrow = wq0 + n;

    const int64_t QSTR = VARLEN ? (int64_t)p.Hq * C::ROW : C::ROW;
    const int64_t KVSTR = VARLEN ? (int64_t)p.Hkv * C::ROW : C::ROW;
    int64_t q_tok0 = 0, k_tok0 = 0;
    if constexpr (VARLEN) {
        seq_bounds(p, b, q_tok0, k_tok0);
        if (q0 >= p.Nq) return;                  // past this sequence's queries
    }
    // first row of this head: bytes into q / dO / dq and K / V, and its workspace index
    const int64_t qbase = VARLEN ? q_tok0 * QSTR + (int64_t)hq * C::ROW : (int64_t)(b * p.Hq + hq) * p.Nq * C::ROW;
    const int64_t kvbase = VARLEN ? k_tok0 * KVSTR + (int64_t)hkv * C::ROW
                                  : (int64_t)(b * p.Hkv + hkv) * p.Nk * C::ROW;
    const int64_t wrow0 = VARLEN ? (int64_t)hq * p.total_q + q_tok0 : (int64_t)(b * p.Hq + hq) * p.Nq;
    const char* Kh = reinterpret_cast<const char*>(p.k) + kvbase;
    const char* Vh = reinterpret_cast<const char*>(p.v) + kvbase;

    const int kend = key_end(q0, C::ROWS, p.Nk, p.causal_shift, CAUSAL);
    const int n_tiles = __builtin_amdgcn_readfirstlane((kend + C::T - 1) / C::T);
    const int wkend = __builtin_amdgcn_readfirstlane(key_end(wq0, 32, p.Nk, p.causal_shift, CAUSAL));

    bf16x8 qf[C::KS], df[C::KS];
    load_b_rows<D>(reinterpret_cast<const char*>(p.q) + qbase, qrow, p.Nq, g, qf, QSTR);
    load_b_rows<D>(reinterpret_cast<const char*>(p.dout) + qbase, qrow, p.Nq, g, df, QSTR);
    const int64_t R = VARLEN ? (int64_t)p.Hq * p.total_q : (int64_t)p.B * p.Hq * p.Nq;
    float lse2 = INFINITY, dlt = 0.f;
    if (qrow < p.Nq) {
        dlt = p.ws[wrow0 + qrow];
        lse2 = p.ws[R + wrow0 + qrow];
    }

    const TileOffsets<D> off(n, g);
    f32x16 acc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

    auto issue = [&](int j, int stage) {
        copy_pair<D, C::T>(Kh, Vh, j * C::T, p.Nk, smem_u32 + stage * C::STAGE, w, lane, KVSTR);
    };

    auto tile = [&](auto stage_c, int j) {
        constexpr int STG = decltype(stage_c)::value;
        FA_WAIT_VMCNT(0);
        bwd_barrier();
        const int key0 = j * C::T;
        if (key0 >= wkend) {                      // every key of the tile is hidden from this wave
            if (j + 1 < n_tiles) issue(j + 1, STG ^ 1);
            return;
        }
        const lds_char* kb = smem + STG * C::STAGE;
        const lds_char* vb = kb + C::TILE;
        f32x16 s = f32x16{}, dp = f32x16{};
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            s = mfma_bf16_32x32x16(lds_b128(kb + off.b[ks]), qf[ks], s);
            dp = mfma_bf16_32x32x16(lds_b128(vb + off.b[ks]), df[ks], dp);
        }
        order_reads_ahead<2 * C::KS, 1, FA_BWD_PF_S>();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        if (j + 1 < n_tiles) issue(j + 1, STG ^ 1);

        const bool need_mask = (key0 + C::T > p.Nk) || (CAUSAL && key0 + C::T - 1 > wq0 + p.causal_shift);
        f32x16 pv, ds;
#pragma unroll
        for (int i = 0; i < 16; ++i) pv[i] = fast_exp2(fmaf(s[i], p.c, -lse2));
        // Only edge tiles mask (a wave-uniform branch); folded into every
        // element's arithmetic, the test cost two VALU instructions per score.
        if (need_mask) {
            const int lim = (CAUSAL ? min(qrow + p.causal_shift, p.Nk - 1) : p.Nk - 1) - key0 - 4 * g;
#pragma unroll
            for (int i = 0; i < 16; ++i) pv[i] = 8 * (i >> 2) + (i & 3) > lim ? 0.f : pv[i];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) ds[i] = pv[i] * (dp[i] - dlt);
        bf16x8 pd[2];
        pack_b(ds, pd);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int db = 0; db < C::DB; ++db) acc[db] = mfma_bf16_32x32x16(tr_operand<D>(kb, off, db, st), pd[st], acc[db]);
        order_reads_ahead<2 * C::DB, 2, FA_BWD_PF_V>();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
    };

    if (n_tiles > 0) issue(0, 0);
    for (int j = 0; j < n_tiles; j += 2) {
        tile(std::integral_constant<int, 0>{}, j);
        if (j + 1 < n_tiles) tile(std::integral_constant<int, 1>{}, j + 1);
    }

    store_rows<D>(smem, acc, p.scale, reinterpret_cast<char*>(p.dq) + qbase, q0, p.Nq, w, n, g, lane, QSTR);
}

// dQ with the key loop software-pipelined: the S^T and dP^T products of key
// tile j + 1 are issued in the same instruction stream as the softmax of
// tile j, so a wave keeps the MFMA pipe busy through its own exponentials.
// At two waves per SIMD (the dQ kernel's occupancy either way) the registers
// for the second pair of score blocks are free.  Three LDS stages: tile j
// (read by the dQ product), j + 1 (read by the score products) and j + 2
// (copies in flight).  Every wave computes every tile of the workgroup; the
// mask zeroes the scores of keys hidden from its rows.
template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(256, 2) void fa_bwd_dq_pipe_kernel(BwdParams pin) {
    BwdParams p = pin;
    using C = BwdCfg<D>;
    constexpr int NST = 3;
    constexpr int LDS = NST * C::STAGE > C::OUT ? NST * C::STAGE : C::OUT;
    __shared__ __attribute__((aligned(1024))) char smem_raw[LDS];
    lds_char* smem = (lds_char*)smem_raw;
    const uint32_t smem_u32 = (uint32_t)(uintptr_t)smem;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31;
    const int g = lane >> 5;

    int b, hkv, hq, qt;
    if (VARLEN && p.compact_dq) {
        const int k = blockIdx.x / p.Hq;
        const int x = blockIdx.x - k * p.Hq;
        hkv = x % p.Hkv;
        hq = hkv * p.group + x / p.Hkv;
        if (!varlen_slot<true>(p.cu_q, p.total_q, p.B, p.n_qtiles, C::ROWS, k, b, qt)) return;
        b = __builtin_amdgcn_readfirstlane(b);
        qt = __builtin_amdgcn_readfirstlane(qt);
    } else {
        int t_ord, kvflat, gi;
        bwd_order(blockIdx.x, p.B * p.Hkv, p.group, p.n_qtiles, p.group_dq, kvflat, gi, t_ord);
        b = kvflat / p.Hkv;
        hkv = kvflat - b * p.Hkv;
        hq = hkv * p.group + gi;
        qt = CAUSAL ? p.n_qtiles - 1 - t_ord : t_ord;
    }
    const int q0 = qt * C::ROWS;
    const int wq0 = q0 + 32 * w;
    const int qrow = wq0 + n;

    const int64_t QSTR = VARLEN ? (int64_t)p.Hq * C::ROW : C::ROW;
    const int64_t KVSTR = VARLEN ? (int64_t)p.Hkv * C::ROW : C::ROW;
    int64_t q_tok0 = 0, k_tok0 = 0;
    if constexpr (VARLEN) {
        seq_bounds(p, b, q_tok0, k_tok0);
        if (q0 >= p.Nq) return;
    }
    const int64_t qbase = VARLEN ? q_tok0 * QSTR + (int64_t)hq * C::ROW : (int64_t)(b * p.Hq + hq) * p.Nq * C::ROW;
    const int64_t kvbase = VARLEN ? k_tok0 * KVSTR + (int64_t)hkv * C::ROW
                                  : (int64_t)(b * p.Hkv + hkv) * p.Nk * C::ROW;
    const int64_t wrow0 = VARLEN ? (int64_t)hq * p.total_q + q_tok0 : (int64_t)(b * p.Hq + hq) * p.Nq;
    const char* Kh = reinterpret_cast<const char*>(p.k) + kvbase;
    const char* Vh = reinterpret_cast<const char*>(p.v) + kvbase;

    const int kend = key_end(q0, C::ROWS, p.Nk, p.causal_shift, CAUSAL);
    const int n_tiles = __builtin_amdgcn_readfirstlane((kend + C::T - 1) / C::T);

    bf16x8 qf[C::KS], df[C::KS];
    load_b_rows<D>(reinterpret_cast<const char*>(p.q) + qbase, qrow, p.Nq, g, qf, QSTR);
    load_b_rows<D>(reinterpret_cast<const char*>(p.dout) + qbase, qrow, p.Nq, g, df, QSTR);
    const int64_t R = VARLEN ? (int64_t)p.Hq * p.total_q : (int64_t)p.B * p.Hq * p.Nq;
    float lse2 = INFINITY, dlt = 0.f;
    if (qrow < p.Nq) {
        dlt = p.ws[wrow0 + qrow];
        lse2 = p.ws[R + wrow0 + qrow];
    }
    // last key visible to this lane's row, relative to element 0 of a tile
    const int lim0 = (CAUSAL ? min(qrow + p.causal_shift, p.Nk - 1) : p.Nk - 1) - 4 * g;

    const TileOffsets<D> off(n, g);
    f32x16 acc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

    auto issue = [&](int j, int stage) {
        copy_pair<D, C::T>(Kh, Vh, j * C::T, p.Nk, smem_u32 + stage * C::STAGE, w, lane, KVSTR);
    };
    // S^T and dP^T of the tile in `stage`
    auto scores = [&](int stage, f32x16& s, f32x16& dp) {
        const lds_char* kb = smem + stage * C::STAGE;
        const lds_char* vb = kb + C::TILE;
        s = f32x16{};
        dp = f32x16{};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            s = mfma_bf16_32x32x16(lds_b128(kb + off.b[ks]), qf[ks], s);
            dp = mfma_bf16_32x32x16(lds_b128(vb + off.b[ks]), df[ks], dp);
        }
    };

    f32x16 s0, dp0;
    if (n_tiles > 0) {
        issue(0, 0);
        if (n_tiles > 1) issue(1, 1);
        FA_WAIT_VMCNT(0);
        bwd_barrier();
        __builtin_amdgcn_s_setprio(1);
        scores(0, s0, dp0);
        __builtin_amdgcn_s_setprio(0);
    }

    // Tile j sits in stage U = j % 3 (compile time); its scores are in (s, dp).
    auto tile = [&](auto u_c, int j) {
        constexpr int U = decltype(u_c)::value;
        constexpr int NXT = (U + 1) % NST, ISS = (U + 2) % NST;
        // tile j + 1 landed; every wave is past tile j - 1, whose stage the
        // copies of tile j + 2 now overwrite
        FA_WAIT_VMCNT(0);
        bwd_barrier();
        if (j + 2 < n_tiles) issue(j + 2, ISS);
        const int key0 = j * C::T;
        const bool need_mask = (key0 + C::T > p.Nk) || (CAUSAL && key0 + C::T - 1 > wq0 + p.causal_shift);
        // One basic block: the score products of tile j + 1 (for the last
        // tile they read a stale stage and are discarded) interleaved with
        // the softmax of tile j, one MFMA, one LDS read and four VALU
        // instructions at a time.  The mask comes after, on dS, so that no
        // branch splits the block.
        f32x16 s1, dp1, pv, ds;
        __builtin_amdgcn_sched_barrier(0);
        scores(NXT, s1, dp1);
#pragma unroll
        for (int i = 0; i < 16; ++i) pv[i] = fast_exp2(fmaf(s0[i], p.c, -lse2));
#pragma unroll
        for (int i = 0; i < 16; ++i) ds[i] = pv[i] * (dp0[i] - dlt);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int m = 0; m < 2 * C::KS; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (m + 2 < 2 * C::KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 64 / (2 * C::KS), 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (need_mask) {
            const int lim = lim0 - key0;
#pragma unroll
            for (int i = 0; i < 16; ++i) ds[i] = 8 * (i >> 2) + (i & 3) > lim ? 0.f : ds[i];
        }
        bf16x8 pd[2];
        pack_b(ds, pd);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        const lds_char* kb = smem + U * C::STAGE;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int db = 0; db < C::DB; ++db) acc[db] = mfma_bf16_32x32x16(tr_operand<D>(kb, off, db, st), pd[st], acc[db]);
        order_reads_ahead<2 * C::DB, 2, FA_BWD_PF_V>();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        s0 = s1;
        dp0 = dp1;
    };

    for (int j = 0; j < n_tiles; j += NST) {
        tile(std::integral_constant<int, 0>{}, j);
        if (j + 1 < n_tiles) tile(std::integral_constant<int, 1>{}, j + 1);
        if (j + 2 < n_tiles) tile(std::integral_constant<int, 2>{}, j + 2);
    }

    store_rows<D>(smem, acc, p.scale, reinterpret_cast<char*>(p.dq) + qbase, q0, p.Nq, w, n, g, lane, QSTR);
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_bwd_d(const BwdParams& p, hipStream_t stream) {
    using C = BwdCfg<D>;
    BwdParams pp = p;
    // dK/dV workgroups stream Q and dO rows, dQ workgroups K and V rows
    const long long q_rows = VARLEN ? (long long)p.total_q : (long long)p.B * p.Nq;
    const long long k_rows = VARLEN ? (long long)p.total_k : (long long)p.B * p.Nk;
    pp.group_dkv = stream_group(q_rows * p.Hq * D * 2 * 2);
    pp.group_dq = stream_group(k_rows * p.Hkv * D * 2 * 2);
    const int64_t R = VARLEN ? (int64_t)p.total_q * p.Hq : (int64_t)p.B * p.Hq * p.Nq;
    void* args[] = {&pp};
    hipError_t e = hipSuccess;
    if (R > 0) {
        const int64_t rows_per_block = 4 * (64 / (D / 8));
        const int64_t blocks = std::min<int64_t>((R + rows_per_block - 1) / rows_per_block, 4096);
        e = hipLaunchKernel(reinterpret_cast<const void*>(&fa_bwd_prep_kernel<D, VARLEN>), dim3((unsigned)blocks),
                            dim3(256), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    // grids: Nk / Nq are the (largest) lengths; packed workgroups past their
    // sequence's end return at once.  A packed batch whose padded grid would
    // be 8 times the tiles that exist takes the compact grid instead
    // (varlen_compact in fa_varlen.hpp).
    // d = 128: wave pairs, 64 keys per workgroup; d = 64: one wave per key
    constexpr bool PAIR = D == 128;
    constexpr int KV_ROWS = PAIR ? PairCfg<D>::KEYS : C::ROWS;
    pp.n_ktiles = (p.Nk + KV_ROWS - 1) / KV_ROWS;
    pp.compact_dkv = VARLEN && varlen_compact(p.total_k, p.B, pp.n_ktiles, KV_ROWS) ? 1 : 0;
    const int64_t kv_grid = pp.compact_dkv ? varlen_slots(p.total_k, p.B, pp.n_ktiles, KV_ROWS) * p.Hkv
                                           : (int64_t)pp.n_ktiles * p.B * p.Hkv;
    if (kv_grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    if (kv_grid > 0) {
        if constexpr (PAIR) {
            const void* kpair = reinterpret_cast<const void*>(&fa_bwd_dkv_pair_kernel<D, CAUSAL, VARLEN>);
            e = hipLaunchKernel(kpair, dim3((unsigned)kv_grid), dim3(256), args, test_extra_lds(PairCfg<D>::LDS), stream);
        } else {
            const void* kboth = reinterpret_cast<const void*>(&fa_bwd_dkv_kernel<D, CAUSAL, VARLEN>);
            e = hipLaunchKernel(kboth, dim3((unsigned)kv_grid), dim3(256), args, test_extra_lds(KvCfg<D>::LDS), stream);
        }
        if (e != hipSuccess) return e;
    }
    pp.n_qtiles = (p.Nq + C::ROWS - 1) / C::ROWS;
    pp.compact_dq = VARLEN && varlen_compact(p.total_q, p.B, pp.n_qtiles, C::ROWS) ? 1 : 0;
    const int64_t q_grid = pp.compact_dq ? varlen_slots(p.total_q, p.B, pp.n_qtiles, C::ROWS) * p.Hq
                                         : (int64_t)pp.n_qtiles * p.B * p.Hq;
    if (q_grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    if (q_grid > 0) {
        if constexpr (FA_BWD_DQ_PIPE && D == 128) {
            const void* kdq = reinterpret_cast<const void*>(&fa_bwd_dq_pipe_kernel<D, CAUSAL, VARLEN>);
            e = hipLaunchKernel(kdq, dim3((unsigned)q_grid), dim3(256), args, test_extra_lds(3 * C::STAGE), stream);
        } else {
            const void* kdq = reinterpret_cast<const void*>(&fa_bwd_dq_kernel<D, CAUSAL, VARLEN>);
            e = hipLaunchKernel(kdq, dim3((unsigned)q_grid), dim3(256), args, test_extra_lds(C::LDS), stream);
        }
    }
    return e;
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int d, bool causal, hipStream_t stream) {
    if (d == 64) return causal ? launch_bwd_d<64, true, false>(p, stream) : launch_bwd_d<64, false, false>(p, stream);
    if (d == 128) return causal ? launch_bwd_d<128, true, false>(p, stream) : launch_bwd_d<128, false, false>(p, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_varlen(const BwdParams& p, int d, bool causal, hipStream_t stream) {
    if (d == 64) return causal ? launch_bwd_d<64, true, true>(p, stream) : launch_bwd_d<64, false, true>(p, stream);
    if (d == 128) return causal ? launch_bwd_d<128, true, true>(p, stream) : launch_bwd_d<128, false, true>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa
