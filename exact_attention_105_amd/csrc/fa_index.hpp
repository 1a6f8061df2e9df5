// Index arithmetic of the attention kernels: workgroup -> work-unit orders
// and the clamps that keep every K/V copy inside its tensor.
//
// Kept apart from the device building blocks (fa_device.hpp) and compiled for
// both sides, so that host-side checks run this same code over whole grids
// (tests/index_replay.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define FA_HD __host__ __device__ __forceinline__

namespace fa {

__host__ __device__ constexpr int imin(int a, int b) { return a < b ? a : b; }
__host__ __device__ constexpr int imax(int a, int b) { return a > b ? a : b; }

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, Hq, Hkv, Nq, Nk;
    int group;          // Hq / Hkv
    int n_qtiles;       // ceil(Nq / rows per workgroup)
    int n_heads;        // B * Hq
    int causal_shift;   // Nk - Nq: key j visible to query i iff j <= i + causal_shift
    float c;            // |scale| (* sq * sk for fp8) * log2(e): exponent of 2 per raw score
    float o_scale;      // multiplies the normalised output (sv for fp8, 1 for bf16)
    uint32_t q_sign;    // XOR mask applied to Q bit patterns (flips the sign when scale < 0)
    int kv_group;       // causal order: 0 walks all heads together; G > 0 takes each XCD's
                        // key/value heads G at a time (stream_group)
};

// Heads are enumerated so that the Hq/Hkv query heads sharing one key/value
// head get flat indices that are congruent modulo 8 whenever B*Hkv is a
// multiple of 8; the hardware hands workgroups to the 8 XCDs round-robin, so
// those heads (and their K/V traffic) land on the same XCD and its L2.
FA_HD void head_of(const FwdParams& p, int x, int& b, int& hq, int& hkv) {
    const int kvflat = x % (p.B * p.Hkv);
    const int gi = x / (p.B * p.Hkv);
    b = kvflat / p.Hkv;
    hkv = kvflat % p.Hkv;
    hq = hkv * p.group + gi;
}

// Workgroup -> (batch, query head, key/value head, query tile) for the
// prefill kernels.  The hardware hands workgroups to the 8 XCDs round-robin
// (id mod 8).
//  * Causal problems: consecutive ids walk the heads first (head_of), the
//    query tiles heaviest first, so every head's long rows start at the
//    beginning of the launch (longest-first scheduling; the tail is made of
//    the shortest tiles).
//  * Non-causal problems, when B*Hkv is a multiple of 8: XCD x owns the
//    key/value heads congruent to x mod 8 and walks them one at a time --
//    the query heads of a key/value head next to each other, each head's
//    query tiles consecutively -- so the workgroups resident on an XCD stream
//    the same keys and values through its L2 together.  (On a causal problem
//    whose keys and values fit the memory-side cache, 16K tokens x 32 heads,
//    this order cut the fetched bytes about 8x but lost more to the late
//    start of the last heads' long rows than it gained.)
//  * Causal problems whose keys and values outgrow the 256 MB memory-side
//    cache (kv_group > 0): XCD x again owns the key/value heads congruent to
//    x mod 8, but walks them kv_group at a time, heaviest query tiles first
//    within each group.  The heads-first order streams every head's keys at
//    once; past that cache its re-reads go to HBM, and measured launches ran
//    up to 1.6x longer (2048 tokens x 1024 heads of d = 128).
template <bool CAUSAL>
FA_HD void tile_of(const FwdParams& p, int bid, int& b, int& hq, int& hkv, int& qt) {
    const int kvh = p.B * p.Hkv;
    int t_ord;
    if (CAUSAL && p.kv_group > 0 && (kvh & 7) == 0) {
        const int xcd = bid & 7;
        const int L = bid >> 3;
        const int nkv = kvh >> 3;                       // key/value heads on this XCD
        const int G = imin(p.kv_group, nkv);
        const int per = G * p.group * p.n_qtiles;       // tiles of one full group
        const int gidx = L / per;
        const int r = L - gidx * per;
        const int ge = imin(G, nkv - gidx * G) * p.group; // query heads in this group
        t_ord = r / ge;
        const int hl = gidx * G * p.group + (r - t_ord * ge);
        const int kg = hl / p.group;
        const int gi = hl - kg * p.group;
        const int kvflat = xcd + 8 * kg;
        b = kvflat / p.Hkv;
        hkv = kvflat - b * p.Hkv;
        hq = hkv * p.group + gi;
        qt = p.n_qtiles - 1 - t_ord;
        return;
    }
    if (!CAUSAL && (kvh & 7) == 0) {
        const int xcd = bid & 7;
        const int L = bid >> 3;
        const int hl = L / p.n_qtiles;          // head index within this XCD's share
        t_ord = L - hl * p.n_qtiles;
        const int kg = hl / p.group;
        const int gi = hl - kg * p.group;
        const int kvflat = xcd + 8 * kg;
        b = kvflat / p.Hkv;
        hkv = kvflat - b * p.Hkv;
        hq = hkv * p.group + gi;
    } else {
        t_ord = bid / p.n_heads;
        head_of(p, bid - t_ord * p.n_heads, b, hq, hkv);
    }
    qt = CAUSAL ? (p.n_qtiles - 1 - t_ord) : t_ord;
}

// Group size for the XCD-local orders of launches whose workgroups all
// stream one set of per-head tensors (keys and values for the forward and
// dQ kernels, queries and output gradients for dK/dV) holding `bytes` bytes
// in all: 2 above the 256 MiB memory-side cache, else 0 (heads first).
inline int stream_group(long long bytes) { return bytes > (256LL << 20) ? 2 : 0; }

// Workgroup -> (key/value head kvflat = b*Hkv + hkv, member gi of its
// `width` heads, tile rank t) over kvh*width units of n_tiles tiles.  The
// hardware hands workgroups to the 8 XCDs round-robin (id mod 8).
//  * group == 0: ranks outermost, units inner (all heads together, the
//    heaviest causal tiles first).
//  * group > 0 and kvh a multiple of 8: XCD x owns the key/value heads
//    congruent to x mod 8 and takes them `group` at a time, ranks outermost
//    within each group, so the workgroups resident on an XCD share the rows
//    they stream through its L2 (stream_group picks this once those rows
//    outgrow the memory-side cache).
FA_HD void bwd_order(int bid, int kvh, int width, int n_tiles, int group,
                      int& kvflat, int& gi, int& t) {
    if (group > 0 && (kvh & 7) == 0) {
        const int xcd = bid & 7;
        const int L = bid >> 3;
        const int nkv = kvh >> 3;                        // key/value heads on this XCD
        const int G = imin(group, nkv);
        const int per = G * width * n_tiles;             // workgroups of one full group
        const int gidx = L / per;
        const int r = L - gidx * per;
        const int ge = imin(G, nkv - gidx * G) * width;   // units in this group
        t = r / ge;
        const int hl = gidx * G * width + (r - t * ge);
        const int kg = hl / width;
        gi = hl - kg * width;
        kvflat = xcd + 8 * kg;
    } else {
        const int n = kvh * width;
        t = bid / n;
        const int x = bid - t * n;
        kvflat = x % kvh;
        gi = x / kvh;
    }
}

// Row, relative to the tile's first row r0, that copy row `row` of a tile of
// a tensor with N rows fetches: rows past the last one are clamped to it
// (their scores are masked, or their products discarded).  Needs r0 < N.
FA_HD int copy_src_row(int row, int r0, int N) { return imin(row, N - 1 - r0); }

// Keys [0, key_end) that query rows q0 .. q0 + rows - 1 need: all Nk, or
// (causal) up to the last key visible to the last row, never below 0.
FA_HD int key_end(int q0, int rows, int Nk, int causal_shift, bool causal) {
    return causal ? imin(Nk, imax(q0 + rows + causal_shift, 0)) : Nk;
}

}  // namespace fa
