"""How often the online softmax has to rescale O, on the long-context
workload's own scores (CPU, numpy only).

The standard recurrence ("FlashAttention (DE)", systems-analysis.info,
section "Online-Softmax-Berechnung") rescales a row whenever a new key tile
raises its running maximum.  The kernels move a row's exponent reference only
when a tile's maximum exceeds it by more than 2^8 (the adaptive rescaling of
page "FlashAttention 4", centron.de, on smarter online-softmax rescaling),
and a wave skips the O rescale when none of its 32 rows moved.  The bf16
kernel only looks at the row maxima when some lane's sum of its 16
exponentials (keys with the same key index mod 8 below or above 4, against
the current reference) passes 2^12, which implies a score more than 2^8 above
the reference; rows then move by the 2^8 rule.  This test replays the rules
tile by tile on sampled 32-row waves of the 16K causal workload (32-key
tiles, the bf16 kernel's) and checks that the lazy rules rescale far less
often and that the kernel's trigger never moves more rows than the plain
lazy rule; the counts are printed.
"""
import numpy as np

from synth.inputs import CONFIGS, generate

RESCALE_LOG2 = 8.0
TILE = 32


SUM_LIMIT_LOG2 = RESCALE_LOG2 + 4


def counts(s2, tile=TILE, thr=RESCALE_LOG2):
    """s2: [32, Nk_visible] scores in log2 units of one wave's rows (-inf
    where masked).  Returns (row rescales standard, row rescales lazy, wave
    rescales standard, wave rescales lazy, row rescales with the kernel's
    sum trigger, wave rescales with it), not counting the first tile."""
    rows, nk = s2.shape
    run = np.full(rows, -np.inf)
    ref = np.full(rows, -np.inf)
    kref = np.full(rows, -np.inf)
    rs = rl = ws = wl = rk = wk = 0
    for j0 in range(0, nk, tile):
        blk = s2[:, j0:j0 + tile]
        tm = blk.max(axis=1)
        first = np.isneginf(run)
        up = (tm > run) & ~first
        mv = (tm > ref + thr) & ~np.isneginf(ref)
        rs += int(up.sum())
        rl += int(mv.sum())
        ws += int(up.any())
        wl += int(mv.any())
        run = np.maximum(run, tm)
        ref = np.where(np.isneginf(ref) & np.isfinite(tm), tm, np.where(mv, tm, ref))
        # kernel trigger: a lane's sum of exponentials over its half of the
        # tile's keys (key index mod 8 below 4, or not) passes 2^12
        if not first.all():
            half = (np.arange(blk.shape[1]) % 8) < 4
            with np.errstate(over="ignore"):
                e = np.exp2(blk - kref[:, None])
            sums = np.stack([e[:, half].sum(axis=1), e[:, ~half].sum(axis=1)])
            trig = bool((sums > 2.0 ** SUM_LIMIT_LOG2).any())
            kmv = trig & (tm > kref + thr) & ~np.isneginf(kref)
            rk += int(kmv.sum())
            wk += int(kmv.any())
        else:
            kmv = np.zeros(rows, dtype=bool)
        kref = np.where(np.isneginf(kref) & np.isfinite(tm), tm, np.where(kmv, tm, kref))
    return rs, rl, ws, wl, rk, wk


def test_lazy_reference_rescales_far_less_often():
    cfg = CONFIGS["long16k_causal"]
    x = generate(cfg)
    q = x["q"].view(np.uint16).astype(np.uint32) << 16
    k = x["k"].view(np.uint16).astype(np.uint32) << 16
    q = q.view(np.float32)
    k = k.view(np.float32)
    c = cfg.scale * np.log2(np.e)
    rng = np.random.default_rng(12)
    tot = np.zeros(6, dtype=np.int64)
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
    rs, rl, ws, wl, rk, wk = (int(v) for v in tot)
    print(f"\n12 waves, {tiles} wave-tiles: row rescales standard {rs} lazy {rl} kernel trigger {rk}; "
          f"wave O rescales standard {ws} lazy {wl} ({ws / max(wl, 1):.1f}x fewer) kernel trigger {wk}")
    assert wl * 10 <= ws, (ws, wl)
    assert rk <= rl and wk <= wl, (rk, rl, wk, wl)
