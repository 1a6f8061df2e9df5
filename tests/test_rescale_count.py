"""How often the online softmax has to rescale O, on the long-context
workload's own scores (CPU, numpy only).

The standard recurrence ("FlashAttention (DE)", systems-analysis.info,
section "Online-Softmax-Berechnung") rescales a row whenever a new key tile
raises its running maximum.  The kernels move a row's exponent reference only
when a tile's maximum exceeds it by more than 2^8 (the adaptive rescaling of
page "FlashAttention 4", centron.de, on smarter online-softmax rescaling),
and a wave skips the O rescale when none of its 32 rows moved.  This test
replays both rules tile by tile on sampled 32-row waves of the 16K causal
workload (32-key tiles, the bf16 kernel's) and checks that the lazy rule
rescales far less often; the counts are printed.
"""
import numpy as np

from synth.inputs import CONFIGS, generate

RESCALE_LOG2 = 8.0
TILE = 32


def counts(s2, tile=TILE, thr=RESCALE_LOG2):
    """s2: [32, Nk_visible] scores in log2 units of one wave's rows (-inf
    where masked).  Returns (row rescales standard, row rescales lazy, wave
    rescales standard, wave rescales lazy), not counting the first tile."""
    rows, nk = s2.shape
    run = np.full(rows, -np.inf)
    ref = np.full(rows, -np.inf)
    rs = rl = ws = wl = 0
    for j0 in range(0, nk, tile):
        tm = s2[:, j0:j0 + tile].max(axis=1)
        first = np.isneginf(run)
        up = (tm > run) & ~first
        mv = (tm > ref + thr) & ~np.isneginf(ref)
        rs += int(up.sum())
        rl += int(mv.sum())
        ws += int(up.any())
        wl += int(mv.any())
        run = np.maximum(run, tm)
        ref = np.where(np.isneginf(ref) & np.isfinite(tm), tm, np.where(mv, tm, ref))
    return rs, rl, ws, wl


def test_lazy_reference_rescales_far_less_often():
    cfg = CONFIGS["long16k_causal"]
    x = generate(cfg)
    q = x["q"].view(np.uint16).astype(np.uint32) << 16
    k = x["k"].view(np.uint16).astype(np.uint32) << 16
    q = q.view(np.float32)
    k = k.view(np.float32)
    c = cfg.scale * np.log2(np.e)
    rng = np.random.default_rng(12)
    tot = np.zeros(4, dtype=np.int64)
    tiles = 0
    for _ in range(12):
        b, h = int(rng.integers(cfg.B)), int(rng.integers(cfg.Hq))
        w0 = 32 * int(rng.integers(cfg.Nq // 32 // 2, cfg.Nq // 32))   # waves in the second half: long rows
        qs = q[b, h, w0:w0 + 32].astype(np.float64)
        ks = k[b, h // (cfg.Hq // cfg.Hkv), :w0 + 32].astype(np.float64)
        s2 = (qs @ ks.T) * c
        i = np.arange(w0, w0 + 32)[:, None]
        j = np.arange(w0 + 32)[None, :]
        s2 = np.where(j <= i, s2, -np.inf)
        tot += np.array(counts(s2))
        tiles += (w0 + 32 + TILE - 1) // TILE
    rs, rl, ws, wl = (int(v) for v in tot)
    print(f"\n12 waves, {tiles} wave-tiles: row rescales standard {rs} lazy {rl}; "
          f"wave O rescales standard {ws} lazy {wl} ({ws / max(wl, 1):.1f}x fewer)")
    assert wl * 10 <= ws, (ws, wl)
