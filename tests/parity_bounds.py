"""Exactness rules for parity checks where both sides round the same values.

The GPU and the oracle compute each compressed entry (and each indexer key)
from the same raw rows, the GPU in fp32, the oracle in float64 rounded once to
fp32. Their fp32 values may differ in the last bits (summation order, the
hardware exponential), by at most the forward error bound of the fp32 sums.
When both sides then round to a storage format (bf16; E4M3 codes with a page
scale; E2M1 codes with an E4M3 group scale) the codes must be equal, except
where the value sits within that error bound of a rounding midpoint: there
the two codes may be the two neighbours of the midpoint. Everything here is
derived from the oracle's float64 values alone; nothing read back from the
GPU enters an expected value or a bound.

* ``code_check`` - stored codes equal, or the rounding of some value within
  the error band of the exact value (for a band below one grid step: the
  other neighbour of a midpoint the value is provably near); returns the
  count of such allowed exceptions.
* ``key_score_slack`` - per indexer key, how far the flips its codes may take
  can move its score, plus the page-scale uncertainty.
* ``topk_valid`` - the GPU's Top-K set is a valid Top-K of some score vector
  within [s - eps|s| - B, s + eps|s| + B] of the oracle's scores s (eps: the
  fp32 accumulation-order band of 1e-6 relative; B: the slack above, zero for
  keys with no code near a midpoint).
"""
from __future__ import annotations

import numpy as np

from oracle import csa_oracle as O

U32 = 2.0 ** -24          # unit roundoff of fp32
E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


# --------------------------------------------------------------------------- forward error bounds

def pooled_terms(K: np.ndarray, V: np.ndarray, Z: np.ndarray, r: int, P: np.ndarray | None = None):
    """Sums of absolute terms of each pooled value, float64: T_K[j, d] =
    sum_i w_i |K_i,d| over block j (likewise T_V), and for the indexer keys
    T_I[j, e] = sum_d T_K[j, d] |P_d,e| (which also carries the entries' own
    error into the projection). The fp32 error of a value is a small multiple
    of its T."""
    K, V, Z = (np.asarray(a, np.float64) for a in (K, V, Z))
    nb = K.shape[0] // r
    n = nb * r
    Zb = Z[:n].reshape(nb, r, -1)
    e = np.exp(Zb - Zb.max(axis=1, keepdims=True))
    w = e / e.sum(axis=1, keepdims=True)
    TK = (w * np.abs(K[:n].reshape(nb, r, -1))).sum(axis=1)
    TV = (w * np.abs(V[:n].reshape(nb, r, -1))).sum(axis=1)
    TI = None if P is None else TK @ np.abs(np.asarray(P, np.float64))
    return TK, TV, TI


def value_band(T: np.ndarray, n_terms: int) -> np.ndarray:
    """Bound on |fp32 value (GPU) - fp32 rounding of the exact value (oracle)|
    for a value computed as a sum of n_terms products with absolute sum T:
    (n_terms + 8) unit roundoffs of T for the sum, the weights' exponentials
    and the final rounding, doubled for margin."""
    return 2.0 * (n_terms + 8) * U32 * np.asarray(T, np.float64)


# --------------------------------------------------------------------------- rounding grids

def _grid(qa: np.ndarray, fmt: str):
    """(spacing, nearest midpoint) of the format's grid around |q| = qa."""
    qa = np.asarray(qa, np.float64)
    if fmt == "e2m1":
        mids = (E2M1_MAGS[:-1] + E2M1_MAGS[1:]) / 2
        i = np.argmin(np.abs(qa[..., None] - mids), axis=-1)
        return (E2M1_MAGS[1:] - E2M1_MAGS[:-1])[i], mids[i]
    _, e = np.frexp(qa)
    if fmt == "e4m3":
        step = np.ldexp(1.0, np.maximum(e, -5) - 4)
    elif fmt == "bf16":
        step = np.ldexp(1.0, np.maximum(e, -125) - 8)
    else:
        raise ValueError(fmt)
    return step, (np.floor(qa / step) + 0.5) * step


def near_midpoint(q: np.ndarray, band: np.ndarray, fmt: str) -> np.ndarray:
    """|q| lies within `band` of a midpoint between two neighbouring codes."""
    qa = np.abs(np.asarray(q, np.float64))
    _, mid = _grid(qa, fmt)
    return np.abs(qa - mid) <= band


def _magnitudes(codes: np.ndarray, fmt: str):
    """(magnitude, lower neighbour magnitude, upper neighbour magnitude, sign)
    of each code; the top finite code's upper neighbour is +inf (saturation),
    zero's lower neighbour is its own negative mirror (the interval of +-0 is
    symmetric)."""
    c = np.asarray(codes).astype(np.int64)
    if fmt == "e4m3":
        m = c & 0x7F
        dec = lambda v: O.e4m3_decode(np.clip(v, 0, 0x7E).astype(np.uint8))
        top, sign = 0x7E, (c & 0x80) != 0
    elif fmt == "bf16":
        m = c & 0x7FFF
        dec = lambda v: O.decode_bf16(np.clip(v, 0, 0x7F7F).astype(np.uint16))
        top, sign = 0x7F7F, (c & 0x8000) != 0
    elif fmt == "e2m1":
        m = c & 0x7
        dec = lambda v: E2M1_MAGS[np.clip(v, 0, 7)]
        top, sign = 7, (c & 0x8) != 0
    else:
        raise ValueError(fmt)
    mag = dec(m)
    up = np.where(m >= top, np.inf, dec(m + 1))
    lo = np.where(m <= 0, -dec(np.ones_like(m)), dec(m - 1))
    return mag, lo, up, sign


def code_ok(got: np.ndarray, q: np.ndarray, band: np.ndarray, fmt: str) -> np.ndarray:
    """The code is the correct rounding (to nearest) of some value within
    `band` of q: its rounding interval [midpoint below, midpoint above]
    (signed) meets [q - band, q + band]."""
    mag, lo, up, sign = _magnitudes(got, fmt)
    a = (lo + mag) / 2                      # interval of the magnitude
    b = (mag + up) / 2
    lo_v = np.where(sign & (mag > 0), -b, a)
    hi_v = np.where(sign & (mag > 0), -a, b)
    q = np.asarray(q, np.float64)
    return (hi_v >= q - band) & (lo_v <= q + band)


def code_check(got: np.ndarray, want: np.ndarray, q: np.ndarray, band_q: np.ndarray, fmt: str):
    """(n_allowed, n_bad): a code that differs from the oracle's is allowed
    when it is the rounding of some value within band_q of the oracle's
    pre-rounding value q (which, for band_q below one grid step, means q sits
    at a midpoint and the code is its other neighbour); otherwise it is bad."""
    got = np.asarray(got)
    want = np.asarray(want)
    diff = got != want
    if not np.any(diff):
        return 0, 0
    ok = code_ok(got, np.broadcast_to(q, got.shape), np.broadcast_to(band_q, got.shape), fmt)
    return int(np.sum(diff & ok)), int(np.sum(diff & ~ok))


# --------------------------------------------------------------------------- stored entries

def fp8_pages(x64: np.ndarray, band_x: np.ndarray, page: int = 64):
    """The oracle's E4M3 page quantisation of x64 with, per value, the
    quotient x/s it rounds and that quotient's band (value band plus the page
    scale's own uncertainty, from the band of the page's amax element).
    Returns (codes, scales, q, band_q, rel_scale_band per page)."""
    _, (codes, scales) = O.store(x64, "fp8")
    x32 = O.round_f32(x64).astype(np.float64)
    E = x64.shape[0]
    pidx = np.arange(E) // page
    s = scales.astype(np.float64)[pidx][:, None]
    q = (O.round_f32(x64) / scales[pidx][:, None]).astype(np.float64)
    n_pages = scales.shape[0]
    rel_s = np.zeros(n_pages)
    for p in range(n_pages):
        sl = slice(p * page, min(E, (p + 1) * page))
        a = np.abs(x32[sl])
        if a.size and a.max() > 0:
            i = np.unravel_index(np.argmax(a), a.shape)
            rel_s[p] = (band_x[sl][i] + U32 * a.max()) / a.max()
    band_q = band_x / s + np.abs(q) * (rel_s[pidx][:, None] + 2 * U32)
    return codes, scales, q, band_q, rel_s


def check_stored(got_codes, x64, band_x, dtype: str, page: int = 64):
    """(n_allowed, n_bad) for GPU codes of entries whose oracle values are x64."""
    if dtype == "bf16":
        want = O.round_bf16(x64)
        return code_check(np.asarray(got_codes).view(np.uint16), want, O.round_f32(x64), band_x + U32 * np.abs(x64),
                          "bf16")
    if dtype == "fp8":
        codes, _, q, band_q, _ = fp8_pages(x64, band_x, page)
        return code_check(got_codes, codes, q, band_q, "e4m3")
    raise ValueError(dtype)


def check_fp4(got_codes, got_gsc, x64, band_x):
    """E2M1 entries: group scale codes equal or adjacent across an E4M3
    midpoint of amax/6; element codes checked against the quotient by the
    GPU's own group scale where that scale legitimately differs (the scale is
    then itself a checked, allowed value). Returns (n_allowed, n_bad)."""
    x32 = O.round_f32(x64)
    E, D = x64.shape
    g = x32.reshape(E, D // 16, 16).astype(np.float64)
    bg = np.asarray(band_x, np.float64).reshape(E, D // 16, 16)
    amax = np.abs(g).max(axis=-1)
    amax_band = np.take_along_axis(bg, np.abs(g).argmax(axis=-1)[..., None], -1)[..., 0] + U32 * amax
    _, (oc, osc) = O.store(x64, "fp4")
    q6 = (amax.astype(np.float32) / np.float32(6.0)).astype(np.float64)
    a_s, b_s = code_check(got_gsc, osc, q6, amax_band / 6 + 2 * U32 * q6, "e4m3")
    # element codes against the quotient by the scale the GPU stored (the oracle's when equal)
    sc = np.where(np.asarray(got_gsc) == osc, osc, np.asarray(got_gsc))
    s = O.e4m3_decode(sc).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0))
    q = (g.astype(np.float32) / safe[..., None]).astype(np.float64)
    want = np.where(s[..., None] > 0, O.e2m1_encode(q.astype(np.float32)), 0).astype(np.uint8)
    band_q = bg / safe[..., None] + 2 * U32 * np.abs(q)
    a_e, b_e = code_check(np.asarray(got_codes).reshape(E, D // 16, 16), want, q, band_q, "e2m1")
    return a_s + a_e, b_s + b_e


# --------------------------------------------------------------------------- indexer scores

def key_slack_parts(x64: np.ndarray, band_x: np.ndarray, dtype: str, page: int = 64):
    """The query-independent parts of key_score_slack: per key j and dimension
    d, how far the stored key's dequantised value may move (M[j, d]: one grid
    step plus the band where the code may flip, else 0), and the relative
    uncertainty of its page scale (rel[j], fp8 only). The slack of a query
    (q_idx, w) is then M @ sum_h w_h |q_h| + rel * |score|."""
    E = x64.shape[0]
    if dtype == "f32":
        return np.zeros((E, x64.shape[1])), np.zeros(E)
    if dtype == "bf16":
        x32 = O.round_f32(x64).astype(np.float64)
        b = band_x + U32 * np.abs(x64)
        near = near_midpoint(x32, b, "bf16")
        step, _ = _grid(np.abs(x32) + b, "bf16")
        return near * (step + b), np.zeros(E)
    if dtype == "fp8":
        codes, scales, q, band_q, rel_s = fp8_pages(x64, band_x, page)
        near = near_midpoint(q, band_q, "e4m3")
        step, _ = _grid(np.abs(q) + band_q, "e4m3")
        pidx = np.arange(E) // page
        return near * (step + band_q) * scales.astype(np.float64)[pidx][:, None], rel_s[pidx]
    raise ValueError(dtype)


def key_score_slack(qi: np.ndarray, w: np.ndarray, x64: np.ndarray, band_x: np.ndarray, dtype: str,
                    page: int = 64) -> np.ndarray:
    """Per key j: the most its indexer score can move between the oracle's
    stored key and any stored key the GPU may legitimately hold. A dimension
    whose code may flip moves the dequantised key by one grid step (times the
    page scale), which moves the score by at most sum_h w_h |q_h,d| times that
    (ReLU is 1-Lipschitz, w >= 0); a page scale known to relative s_rel moves
    every score of its page by s_rel times the score."""
    qi = np.asarray(qi, np.float64)
    w = np.asarray(w, np.float64)
    coef = (w[:, None] * np.abs(qi)).sum(axis=0)          # [D_I]
    M, rel = key_slack_parts(x64, band_x, dtype, page)
    if not np.any(rel):
        return M @ coef
    stored = O.store(x64, dtype)[0]
    score = np.maximum(stored @ qi.T, 0.0) @ w
    return M @ coef + rel * np.abs(score)


def topk_valid(gpu_row: np.ndarray, s: np.ndarray, k: int, slack: np.ndarray | None = None, eps: float = 1e-6):
    """The GPU's row is a valid Top-k of the n = len(s) visible entries for some
    scores within eps relative plus `slack` of the oracle's scores s: the right
    count, ascending, -1 padded, and no selected entry's upper bound below an
    unselected entry's lower bound. Returns (ok, message)."""
    row = np.asarray(gpu_row).astype(np.int64)
    n = s.shape[0]
    m = min(k, n)
    sel = row[row >= 0]
    if sel.shape[0] != m or np.any(row[m:] != -1):
        return False, f"count {sel.shape[0]} != {m} or bad padding"
    if np.any(np.diff(sel) <= 0) or (m and (sel[0] < 0 or sel[-1] >= n)):
        return False, "row not strictly ascending inside the visible range"
    if m == n:
        return True, ""
    sf = np.asarray(s, np.float64)
    sl = np.zeros(n) if slack is None else np.asarray(slack, np.float64)
    hi = sf + eps * np.abs(sf) + sl
    lo = sf - eps * np.abs(sf) - sl
    inside = np.zeros(n, dtype=bool)
    inside[sel] = True
    worst_in = int(sel[np.argmin(hi[sel])])
    out_idx = np.flatnonzero(~inside)
    best_out = int(out_idx[np.argmax(lo[~inside])])
    if hi[worst_in] < lo[best_out]:
        return False, (f"selected {worst_in} (score {sf[worst_in]:.7g}, slack {sl[worst_in]:.3g}) ranks below "
                       f"unselected {best_out} (score {sf[best_out]:.7g}, slack {sl[best_out]:.3g})")
    o = O.topk(s.astype(np.float32), k)
    nd = len(set(sel.tolist()) ^ set(o[o >= 0].tolist()))
    return True, f"{nd // 2} swaps against the oracle's own Top-K" if nd else ""
