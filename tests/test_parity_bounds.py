"""CPU tests of the exactness rules the GPU parity tests use (parity_bounds.py).

The rules must (a) accept what an fp32 computation with another summation
order legitimately produces, and (b) reject planted mistakes: a code off by one
away from any midpoint, a code off by two, a Top-K entry far below the k-th
score.
"""
import numpy as np

import parity_bounds as PB
from oracle import csa_oracle as O

RNG = np.random.default_rng(20261203)


def test_e4m3_midpoints_and_grid_points():
    codes = np.arange(0x00, 0x7E, dtype=np.uint8)          # finite positive codes
    vals = O.e4m3_decode(codes)
    mids = (vals[:-1] + vals[1:]) / 2
    assert np.all(PB.near_midpoint(mids, np.full(mids.shape, 1e-12), "e4m3"))
    assert not np.any(PB.near_midpoint(vals[1:], np.full(vals.shape[0] - 1, 1e-3 * vals[1:]), "e4m3"))
    # the saturation midpoint between 416 and 448
    assert PB.near_midpoint(np.array([432.0]), np.array([1e-9]), "e4m3")[0]


def test_e2m1_and_bf16_midpoints():
    mags = O.e2m1_decode(np.arange(8))
    mids = (mags[:-1] + mags[1:]) / 2
    assert np.all(PB.near_midpoint(-mids, np.full(mids.shape, 1e-12), "e2m1"))
    assert not np.any(PB.near_midpoint(mags, np.full(8, 1e-3), "e2m1"))
    x = np.array([1.0 + 2.0 ** -8, 3.0 + 2.0 ** -7])          # bf16 midpoints (spacing 2^-7 in [1, 2), 2^-6 in [2, 4))
    assert np.all(PB.near_midpoint(x, np.full(2, 1e-12), "bf16"))
    assert not PB.near_midpoint(np.array([1.0 + 2.0 ** -7]), np.array([1e-6]), "bf16")[0]


def test_code_check_rejects_planted_mistakes():
    x = RNG.standard_normal((64, 16)) * 3
    codes, scales = O.store(x, "fp8")[1]
    band = np.full(x.shape, 1e-7)
    assert PB.check_stored(codes, x, band, "fp8") == (0, 0)
    q = (O.round_f32(x) / scales[0]).astype(np.float64)
    step, mid = PB._grid(np.abs(q), "e4m3")
    far = int(np.argmax(np.abs(np.abs(q) - mid).ravel() / step.ravel()))     # farthest from any midpoint
    bad = codes.copy().ravel()
    bad[far] = bad[far] + 1 if (bad[far] & 0x7F) < 0x7D else bad[far] - 1
    assert PB.check_stored(bad.reshape(codes.shape), x, band, "fp8")[1] == 1
    two = codes.copy().ravel()
    two[far] = two[far] + 2 if (two[far] & 0x7F) < 0x7C else two[far] - 2
    assert PB.check_stored(two.reshape(codes.shape), x, band, "fp8")[1] == 1
    # a value placed on a midpoint may take either neighbour, and a value whose
    # band spans several steps (cancellation) any code inside its band
    xm = x.copy()
    s = float(scales[0])
    lo = O.e4m3_decode(np.array([0x40], np.uint8))[0]     # 2.0
    hi = O.e4m3_decode(np.array([0x41], np.uint8))[0]     # 2.25
    xm[5, 3] = (lo + hi) / 2 * s
    cm, _ = O.store(xm, "fp8")[1]
    alt = cm.copy()
    alt[5, 3] = 0x41 if cm[5, 3] == 0x40 else 0x40
    assert PB.check_stored(alt, xm, band, "fp8") == (1, 0)
    wide = band.copy()
    wide[5, 3] = 3 * 0.25 * s                   # three E4M3 steps at 2.0
    far3 = cm.copy()
    far3[5, 3] = 0x43                           # 2.75: inside the band
    assert PB.check_stored(far3, xm, wide, "fp8") == (1, 0)
    far3[5, 3] = 0x45                           # 3.25: outside it
    assert PB.check_stored(far3, xm, wide, "fp8")[1] == 1


def _gpu_like_compress(K, V, Z, r, P):
    """fp32 compress with another summation order and fp32 exponentials:
    what a correct GPU implementation may produce."""
    K32, V32, Z32, P32 = (np.asarray(a, np.float32) for a in (K, V, Z, P))
    nb = K.shape[0] // r
    Zb = Z32[: nb * r].reshape(nb, r, -1)
    e = np.exp(Zb - Zb.max(axis=1, keepdims=True)).astype(np.float32)
    den = np.float32(0)
    for i in reversed(range(r)):
        den = den + e[:, i]
    w = (e / den[:, None]).astype(np.float32)
    kb = np.zeros((nb, K.shape[1]), np.float32)
    vb = np.zeros_like(kb)
    for i in reversed(range(r)):
        kb = kb + w[:, i] * K32[: nb * r].reshape(nb, r, -1)[:, i]
        vb = vb + w[:, i] * V32[: nb * r].reshape(nb, r, -1)[:, i]
    ki = np.zeros((nb, P.shape[1]), np.float32)
    for d in reversed(range(K.shape[1])):            # column by column, reversed
        ki = ki + kb[:, d:d + 1] * P32[d][None, :]
    return kb.astype(np.float64), vb.astype(np.float64), ki.astype(np.float64)


def test_fp32_reordered_compress_passes_the_rules():
    r, L = 4, 4 * 640
    K, V, Z = (RNG.standard_normal((L, 128)).astype(np.float32).astype(np.float64) for _ in range(3))
    P = (RNG.standard_normal((128, 64)) / np.sqrt(128)).astype(np.float32).astype(np.float64)
    kb, vb, ki = O.compress(K, V, Z, r, P)
    gk, gv, gi = _gpu_like_compress(K, V, Z, r, P)
    TK, TV, TI = PB.pooled_terms(K, V, Z, r, P)
    bk, bv, bi = PB.value_band(TK, r), PB.value_band(TV, r), PB.value_band(TI, 128 + r + 8)
    assert np.all(np.abs(gk - kb) <= bk) and np.all(np.abs(gi - ki) <= bi)
    total = 0
    for x64, g64, band in ((kb, gk, bk), (vb, gv, bv), (ki, gi, bi)):
        for dt in ("fp8", "bf16"):
            gcodes = O.store(g64, dt)[1]
            gcodes = gcodes[0] if dt == "fp8" else gcodes
            allowed, bad = PB.check_stored(gcodes, x64, band, dt)
            assert bad == 0, (dt, allowed, bad)
            total += allowed
        gc, gs = O.store(g64, "fp4")[1]
        allowed, bad = PB.check_fp4(gc, gs, x64, band)
        assert bad == 0, ("fp4", allowed, bad)
    # Top-K on the GPU-like stored keys is valid under the derived slack
    for dt in ("fp8", "bf16"):
        qi = RNG.standard_normal((4, 64))
        w = RNG.uniform(0, 1, 4)
        s = O.index_scores(qi, w, O.store(ki, dt)[0])
        sg = O.index_scores(qi, w, O.store(gi, dt)[0])
        slack = PB.key_score_slack(qi, w, ki, bi, dt)
        for k in (16, 100, 600):
            ok, msg = PB.topk_valid(O.topk(sg, k), s, k, slack)
            assert ok, (dt, k, msg)


def test_topk_valid_rules():
    s = np.sort(RNG.uniform(1, 2, 200).astype(np.float32))[::-1].copy()     # distinct, descending
    perm = RNG.permutation(200)
    s = s[perm]
    k = 20
    good = O.topk(s, k)
    assert PB.topk_valid(good, s, k)[0]
    # swap the k-th for the (k+1)-th: invalid unless within eps or slack
    order = np.argsort(-s.astype(np.float64), kind="stable")
    kth, nxt = order[k - 1], order[k]
    bad = np.sort(np.concatenate([order[: k - 1], [nxt]]))
    assert not PB.topk_valid(bad, s, k)[0]
    gap = float(s[kth] - s[nxt])
    slack = np.zeros(200)
    slack[nxt] = gap
    assert PB.topk_valid(bad, s, k, slack)[0]
    s2 = s.copy()
    s2[nxt] = np.float32(s[kth] * (1 - 5e-7))
    assert PB.topk_valid(bad, s2, k)[0]
    # a far entry is never valid, whatever the eps band
    far = np.sort(np.concatenate([order[: k - 1], [order[-1]]]))
    assert not PB.topk_valid(far, s, k)[0]
    # counts, order, padding
    assert not PB.topk_valid(good[::-1], s, k)[0]
    assert not PB.topk_valid(np.concatenate([good[:-1], [-1]]), s, k)[0]
    small = O.topk(s[:7], k)
    assert PB.topk_valid(small, s[:7], k)[0]
