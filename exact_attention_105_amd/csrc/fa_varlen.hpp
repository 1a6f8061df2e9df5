// Variable-length batches for the bf16 prefill kernel (fa_fwd_bf16.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"

namespace fa {

// Packed ("varlen") layout: q and o are [total_q, Hq, d], k and v are
// [total_k, Hkv, d], token-major; sequence s owns query tokens
// cu_q[s] .. cu_q[s+1]-1 and key tokens cu_k[s] .. cu_k[s+1]-1; lse is
// [Hq, total_q].  In FwdParams, B counts sequences, Nq is the largest query
// length (it sizes the grid) and Nk is unused.
struct VarlenParams {
    const int* cu_q;     // n_seqs + 1 offsets (device)
    const int* cu_k;     // n_seqs + 1 offsets (device)
    int total_q;
    int total_k;
    int compact;         // set by the launcher: 1 = compact grid (varlen_slot), 0 = padded grid
};

// Tiles of BM rows of sequence s (its token range cu[s] .. cu[s+1]-1,
// clamped to [0, total]), at most n_levels; 0 for s >= n_seqs.
__device__ __forceinline__ int varlen_ntiles(const int* cu, int total, int s, int n_seqs, int n_levels, int BM) {
    if (s >= n_seqs) return 0;
    const int a = min(max(cu[s], 0), total);
    const int e = min(max(cu[s + 1], a), total);
    return min((e - a + BM - 1) / BM, n_levels);
}

// Sum over the wave of a value in [0, 2^bits), wave-uniform: one ballot per bit.
__device__ __forceinline__ int wave_sum_bits(int v, int bits) {
    int sum = 0;
    for (int bit = 0; bit < bits; ++bit) sum += __popcll(__ballot((v >> bit) & 1)) << bit;
    return sum;
}

// The compact variable-length grid: slot k of a head -> (sequence s, tile
// t).  The slots list every tile that exists level by level -- all
// sequences' tile t = L, then all tiles at the next level -- and within a
// level the sequences in order: the order of a padded
// ceil(max_len / BM) x n_seqs grid with its empty tiles left out.  Levels
// run from the highest tile index down (DESCENDING: under a causal mask the
// last query tiles see the most keys) or from 0 up (the first key tiles are
// seen by the most queries), so that the heaviest work starts first.  Every
// wave of the workgroup computes the same answer: lane i holds the tile
// counts of sequences i, i + 64, ... (at most kVarlenChunks x 64 sequences,
// in registers); the number of slots before a level comes from ballots, a
// binary search finds the level of slot k, and a ballot rank finds its
// sequence.  Returns false for a slot past the last tile (the grid is sized
// by an upper bound).
constexpr int kVarlenChunks = 16;        // the compact grid serves up to 1024 sequences

template <bool DESCENDING>
__device__ inline bool varlen_slot(const int* cu, int total, int n_seqs, int n_levels, int BM, int k, int& s_out,
                                   int& t_out) {
    const int lane = threadIdx.x & 63;
    const int bits = 32 - __clz(n_levels);              // every per-lane term is <= n_levels < 2^bits
    int nt[kVarlenChunks];
#pragma unroll
    for (int ch = 0; ch < kVarlenChunks; ++ch) nt[ch] = varlen_ntiles(cu, total, 64 * ch + lane, n_seqs, n_levels, BM);
    const int nchunks = min((n_seqs + 63) >> 6, kVarlenChunks);
    // slots ahead of level Q: levels > Q-1 descending (sum of max(0, tiles - Q)
    // counts the levels >= Q), levels < Q ascending (sum of min(tiles, Q))
    auto before = [&](int Q) {
        int c = 0;
#pragma unroll
        for (int ch = 0; ch < kVarlenChunks; ++ch)
            if (ch < nchunks) c += wave_sum_bits(DESCENDING ? max(nt[ch] - Q, 0) : min(nt[ch], Q), bits);
        return c;
    };
    const int all = DESCENDING ? before(0) : before(n_levels);
    if (k < 0 || k >= all) return false;
    int lo = 0, hi = n_levels - 1, base;
    if (DESCENDING) {                                   // the largest Q with (slots at levels >= Q) > k
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (before(mid) > k) lo = mid;
            else hi = mid - 1;
        }
        base = lo + 1 < n_levels ? before(lo + 1) : 0;
    } else {                                            // the largest Q with (slots at levels < Q) <= k
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (before(mid) <= k) lo = mid;
            else hi = mid - 1;
        }
        base = before(lo);
    }
    int r = k - base;                                   // rank among the sequences with a tile at level lo
    int s = -1;
#pragma unroll
    for (int ch = 0; ch < kVarlenChunks; ++ch) {
        if (ch < nchunks && s < 0) {
            const uint64_t m = __ballot(nt[ch] > lo);
            const int cnt = __popcll(m);
            if (r < cnt) {
                const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
                const uint64_t sel = __ballot(nt[ch] > lo && below == r);
                s = 64 * ch + __ffsll((unsigned long long)sel) - 1;
            }
            r -= cnt;
        }
    }
    if (s < 0) return false;
    s_out = s;
    t_out = lo;
    return true;
}

// Slots per head of the compact grid: an upper bound on sum_s
// ceil(len_s / BM) that the host can compute, floor(total / BM) + n_seqs
// (each sequence adds at most one partial tile), and never more than the
// padded n_seqs x n_levels.
inline long long varlen_slots(int total, int n_seqs, int n_levels, int BM) {
    const long long bound = (long long)total / BM + n_seqs;
    const long long padded = (long long)n_seqs * n_levels;
    return bound < padded ? bound : padded;
}

// Whether a launch takes the compact grid: at most kVarlenChunks x 64
// sequences, and a padded grid at least 8 times larger.  An empty workgroup
// of the padded grid costs only its dispatch (about 0.7 ns of the launch,
// measured); the slot search costs every workgroup of the compact grid a few
// microseconds.  Measured on 16 heads, d = 128, causal: one 8192-token
// sequence among 255 of 128 tokens (padded 28x) 554 -> 373 us with the
// compact grid; 24 log-uniform lengths up to 8192 (padded 3.9x) 714 -> 745 us,
// and 1024 sequences of 1..511 tokens (1.35x) 952 -> 1618 us, so those keep
// the padded grid.
inline bool varlen_compact(int total, int n_seqs, int n_levels, int BM) {
    if (n_seqs > 64 * kVarlenChunks) return false;
    return 8 * varlen_slots(total, n_seqs, n_levels, BM) <= (long long)n_seqs * n_levels;
}

hipError_t launch_fwd_bf16_varlen(const FwdParams& p, const VarlenParams& vp, int d, bool causal,
                                  hipStream_t stream);

}  // namespace fa
