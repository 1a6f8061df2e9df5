// Host-side replay of the kernels' index arithmetic (fa_index.hpp, the same
// functions the kernels call) over whole grids:
//   * every prefill order (tile_of: heads first, XCD-local, kv_group > 0) is a
//     bijection from workgroup ids onto (batch, query head, query tile), with
//     the key/value head each query head reads;
//   * every K/V tile a workgroup or wave loads lies inside the keys, and every
//     copy row, clamped or not, reads a row of the tensor;
//   * the backward orders (bwd_order) are bijections onto their work units.
// Prints one line per failure and a summary; exit status 1 on any failure.
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "fa_index.hpp"

using namespace fa;

static long long g_checks = 0, g_fail = 0;

#define CHECK(cond, ...)                                 \
    do {                                                 \
        ++g_checks;                                      \
        if (!(cond)) {                                   \
            if (g_fail < 20) {                           \
                printf("FAIL %s:%d: ", __FILE__, __LINE__); \
                printf(__VA_ARGS__);                     \
                printf("\n");                            \
            }                                            \
            ++g_fail;                                    \
        }                                                \
    } while (0)

// Rows of a tile starting at r0 (< N) fetched by the copies: tiles that end
// inside the tensor read rows r0 .. r0+T-1, the last one is clamped.
static void check_tile_rows(int r0, int T, int N, const char* what) {
    CHECK(r0 >= 0 && r0 < N, "%s tile start %d outside [0, %d)", what, r0, N);
    const bool full = r0 + T <= N;
    for (int row = 0; row < T; ++row) {
        const int src = r0 + (full ? row : copy_src_row(row, r0, N));
        CHECK(src >= 0 && src < N, "%s row %d of tile %d reads key %d of %d", what, row, r0, src, N);
    }
}

// A prefill launch: BM query rows per workgroup, RW per wave, BN keys per tile.
template <bool CAUSAL>
static void check_prefill(int B, int Hq, int Hkv, int Nq, int Nk, int kv_group, int BM, int RW, int BN) {
    FwdParams p{};
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Nq = Nq; p.Nk = Nk;
    p.group = Hq / Hkv;
    p.n_qtiles = (Nq + BM - 1) / BM;
    p.n_heads = B * Hq;
    p.causal_shift = Nk - Nq;
    p.kv_group = kv_group;
    const long long grid = (long long)p.n_qtiles * p.n_heads;
    std::vector<char> seen(grid, 0);
    for (long long bid = 0; bid < grid; ++bid) {
        int b = -1, hq = -1, hkv = -1, qt = -1;
        tile_of<CAUSAL>(p, (int)bid, b, hq, hkv, qt);
        const bool ok = b >= 0 && b < B && hq >= 0 && hq < Hq && qt >= 0 && qt < p.n_qtiles;
        CHECK(ok, "tile_of<%d>(B%d Hq%d Hkv%d Nq%d kvg%d) bid %lld -> b%d hq%d qt%d", CAUSAL, B, Hq, Hkv, Nq,
              kv_group, bid, b, hq, qt);
        if (!ok) continue;
        CHECK(hkv == hq / p.group, "bid %lld: hq %d read from kv head %d (group %d)", bid, hq, hkv, p.group);
        const long long unit = ((long long)b * Hq + hq) * p.n_qtiles + qt;
        CHECK(!seen[unit], "bid %lld: unit (b%d hq%d qt%d) mapped twice", bid, b, hq, qt);
        seen[unit] = 1;
    }
    for (long long u = 0; u < grid; ++u) CHECK(seen[u], "unit %lld never mapped", u);

    // Key tiles of every query tile (they depend only on qt), and of each wave.
    for (int qt = 0; qt < p.n_qtiles; ++qt) {
        const int q0 = qt * BM;
        const int kend = key_end(q0, BM, Nk, p.causal_shift, CAUSAL);
        CHECK(kend >= 0 && kend <= Nk, "qt %d: key end %d outside [0, %d]", qt, kend, Nk);
        const int n_tiles = (kend + BN - 1) / BN;
        for (int j = 0; j < n_tiles; ++j) check_tile_rows(j * BN, BN, Nk, "prefill K/V");
        for (int w = 0; w < BM / RW; ++w) {
            const int wkend = key_end(q0 + w * RW, RW, Nk, p.causal_shift, CAUSAL);
            CHECK(wkend <= kend, "qt %d wave %d needs keys to %d beyond the workgroup's %d", qt, w, wkend, kend);
            // the last visible key of every existing row of the wave is below wkend
            for (int r = q0 + w * RW; r < q0 + (w + 1) * RW && r < Nq; ++r) {
                const int last_visible = CAUSAL ? r + p.causal_shift : Nk - 1;
                if (last_visible >= 0)
                    CHECK(imin(last_visible, Nk - 1) < wkend, "row %d sees key %d past the wave's end %d", r,
                          last_visible, wkend);
            }
        }
    }
}

// bwd_order over kvh * width units of n_tiles tiles.
static void check_bwd_order(int kvh, int width, int n_tiles, int group) {
    const long long grid = (long long)kvh * width * n_tiles;
    std::vector<char> seen(grid, 0);
    for (long long bid = 0; bid < grid; ++bid) {
        int kvflat = -1, gi = -1, t = -1;
        bwd_order((int)bid, kvh, width, n_tiles, group, kvflat, gi, t);
        const bool ok = kvflat >= 0 && kvflat < kvh && gi >= 0 && gi < width && t >= 0 && t < n_tiles;
        CHECK(ok, "bwd_order(kvh%d w%d n%d g%d) bid %lld -> kv%d gi%d t%d", kvh, width, n_tiles, group, bid, kvflat,
              gi, t);
        if (!ok) continue;
        const long long unit = ((long long)kvflat * width + gi) * n_tiles + t;
        CHECK(!seen[unit], "bwd_order bid %lld: unit mapped twice", bid);
        seen[unit] = 1;
    }
    for (long long u = 0; u < grid; ++u) CHECK(seen[u], "bwd_order unit %lld never mapped", u);
}

static void check_shape(int B, int Hq, int Hkv, int Nq, int Nk, bool causal) {
    const int group = Hq / Hkv;
    // the launcher's choice of kv_group and the other one
    for (int kvg : {0, 2}) {
        if (causal) {
            check_prefill<true>(B, Hq, Hkv, Nq, Nk, kvg, 128, 32, 32);   // bf16 prefill
            check_prefill<true>(B, Hq, Hkv, Nq, Nk, kvg, 128, 32, 64);   // fp8 prefill
        } else {
            check_prefill<false>(B, Hq, Hkv, Nq, Nk, kvg, 128, 32, 32);
            check_prefill<false>(B, Hq, Hkv, Nq, Nk, kvg, 128, 32, 64);
        }
        check_bwd_order(B * Hkv, 1, (Nk + 127) / 128, kvg);             // dK/dV, d = 64: 128-key tiles
        check_bwd_order(B * Hkv, 1, (Nk + 63) / 64, kvg);               // dK/dV wave pairs, d = 128: 64-key tiles
        check_bwd_order(B * Hkv, group, (Nq + 127) / 128, kvg);         // dQ: query tiles
    }
    // backward query tiles (32 and 64 rows) and key tiles copied with clamps
    for (int T : {32, 64})
        for (int r0 = 0; r0 < Nq; r0 += T) check_tile_rows(r0, T, Nq, "backward Q/dO");
    for (int r0 = 0; r0 < Nk; r0 += 32) check_tile_rows(r0, 32, Nk, "backward K/V");
    for (int r0 = 0; r0 < Nk; r0 += 16) check_tile_rows(r0, 16, Nk, "decode K/V");
}

int main(int argc, char** argv) {
    const int n_random = argc > 1 ? atoi(argv[1]) : 200;
    // the five workloads at their full sizes
    check_shape(1, 2, 2, 128, 128, false);
    check_shape(16, 12, 12, 2048, 2048, false);
    check_shape(16, 12, 12, 2048, 2048, true);
    check_shape(2, 16, 16, 16384, 16384, true);
    check_shape(4, 32, 8, 8192, 8192, true);
    check_shape(64, 32, 8, 1, 8192, true);
    check_shape(4, 16, 16, 8192, 8192, false);
    // random shapes: ragged lengths, Nq != Nk both ways, GQA groups, batch
    // sizes whose key/value head count is and is not a multiple of 8
    srand(12345);
    const int hkvs[] = {1, 2, 3, 4, 8, 16};
    const int groups[] = {1, 2, 4, 8};
    for (int i = 0; i < n_random; ++i) {
        const int B = 1 + rand() % 5;
        const int Hkv = hkvs[rand() % 6];
        const int Hq = Hkv * groups[rand() % 4];
        const int Nq = 1 + rand() % (i % 4 == 0 ? 3000 : 700);
        const int Nk = 1 + rand() % (i % 4 == 1 ? 3000 : 700);
        check_shape(B, Hq, Hkv, Nq, Nk, (i & 1) != 0);
    }
    printf("%lld checks, %lld failures\n", g_checks, g_fail);
    return g_fail == 0 ? 0 : 1;
}
