"""CPU oracle for the Compressed Sparse Attention (CSA) decode / prefill-chunk step.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module. The product path (the
HIP library and its Python binding) never imports it and shares no code with
it.

Plain, slow, obviously-correct NumPy in float64. Each function follows one
step of the method as the source pages describe it; where the pages leave a
step open, the reading taken is stated in the docstring. Sources, cited by
page title and section:

* [Walkthrough] "DeepSeek-V4.1-Flash technical report" chaptered walkthrough
  (astryx-dracula ``templates/tech-report.tsx``), chapters "Compressed Sparse
  Attention 2", "Causal Encoder-Decoder", "SWA Bounded Replay" and the FP4
  section "FP4 main KV cache".
* [Atlas] "Model architectures" atlas, entries on compressed KV (CSA/HCA),
  sliding-window attention, MQA/GQA, trained sparse attention (lightning
  indexer) and IndexCache.
* [Explainer] Illustrated DeepSeek-V4.1-Flash explainer (definitions of the
  compression ratio, indexer and Top-K).

Parity status per function (what pins it in ``tests/test_oracle.py``):
  round_bf16 ............ torch's bf16 conversion; hand-worked tie cases
  e4m3_encode/decode .... OCP E4M3 code table fixture; round-trip of all codes
  fp8_quantize_page ..... amax element -> +-448 code (the 448 maximum printed
                          in the FP4 section); exact-value round trip
  compress .............. r = 1 identity; equal gates -> mean; dominant gate;
                          r = 2 closed form; in-block permutation; linearity
  index_scores .......... pure-Python brute force; H_I = 1, w = 1 -> ReLU(q.k)
  topk .................. brute-force full sort with hand-made tie fixtures
  attend / attend_step .. r = 1, k = all, W = 0 -> torch SDPA causal; k = 0 ->
                          banded SDPA; single key; equal logits -> mean; with
                          V = identity the output rows are the softmax weights,
                          equal to torch.softmax of the same logits and summing
                          to one
  hca_attend_step ....... r = 1, W = 0 -> torch SDPA causal; a pure-Python
                          loop softmax over the explicit key list
  e2m1_encode/decode .... the E2M1 value set from its bit layout; hand-worked
                          ties; saturation at 6; the pages' 448 x 6 = 2688 range
  fp4_quantize_rows ..... exact round trip of on-grid groups; amax -> +-6 when
                          amax/6 is an E4M3 value; groups independent; the
                          E2M1 half-step plus scale-rounding error bound
  store_ring_rows ....... each row's amax element -> +-448 code; E4M3 relative
                          error bound; exact round trip of on-grid rows
  candidate_pool ........ pure-Python brute force with tie fixtures; block = 1
                          -> the entry Top-K; all blocks kept when few are
                          visible; the pages' 2,048 x 8 = 16,384 pool size
  reindex_topk .......... pure-Python brute force; a pool covering every block
                          -> the full Top-K; the Full layer's own query -> its
                          own Top-K (k <= pool blocks, distinct scores)
None is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0  # largest finite OCP E4M3 value; the FP4 section quotes its range as 448 * 6


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns, round-to-nearest-even, straight from float64.

    bf16 keeps 8 significant bits; for |x| in [2**(e-1), 2**e) the spacing is
    2**(e-8), and below the smallest normal (2**-126) it is fixed at 2**-133.
    Dividing by a power of two is exact, so ``np.round`` (ties to even) on the
    scaled value is the correctly rounded result.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    ulp = np.ldexp(1.0, np.maximum(e, -125) - 8)
    y = np.round(x / ulp) * ulp
    y32 = y.astype(np.float32)  # exact: y has at most 8 significant bits
    return (y32.view(np.uint32) >> 16).astype(np.uint16)


def round_f32(x: np.ndarray) -> np.ndarray:
    """float64 -> float32, round-to-nearest-even (IEEE conversion)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 (e4m3fn: bias 7, 3 mantissa bits, no infinities) -> float64.

    Exponent field 0 is subnormal: M/8 * 2**-6. Field 1..15 is normal:
    (1 + M/8) * 2**(E-7). S.1111.111 is NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    M = (c & 7).astype(np.float64)
    mag = np.where(E == 0, M / 8.0 * 2.0 ** -6, (1.0 + M / 8.0) * np.ldexp(1.0, E - 7))
    mag = np.where((E == 15) & ((c & 7) == 7), np.nan, mag)
    return s * mag


def e4m3_encode(x32: np.ndarray) -> np.ndarray:
    """float32 values -> OCP E4M3 codes, round-to-nearest-even, saturating at +-448.

    E4M3 keeps 4 significant bits: spacing 2**(e-4) for |x| in
    [2**(e-1), 2**e) and 2**-9 below the smallest normal 2**-6. Anything that
    rounds above 448 saturates to 448. The sign bit is the IEEE sign of the
    input (so a negative value that rounds to zero encodes as 0x80).
    """
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)
    ulp = np.ldexp(1.0, np.maximum(e, -5) - 4)
    y = np.minimum(np.round(a / ulp) * ulp, E4M3_MAX)
    sub = y < 2.0 ** -6
    _, ey = np.frexp(np.where(sub, 1.0, y))
    E = np.where(sub, 0, ey - 1 + 7)
    M = np.where(sub, np.round(y / 2.0 ** -9), np.round((y / np.ldexp(1.0, ey - 1) - 1.0) * 8.0))
    code = (E.astype(np.int64) << 3) | M.astype(np.int64)
    code = code | np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)


def fp8_quantize_page(x32: np.ndarray) -> tuple[np.ndarray, np.float32]:
    """One 64-entry page of one stream -> (E4M3 codes, float32 scale).

    Reading (the pages give FP8 for caches and 448 as the E4M3 ceiling, but
    no scaling rule for an FP8 main-KV page): one float32 scale per page and
    stream, ``s = amax|x| / 448`` in float32 (``s = 1`` when the page is all
    zero), codes = E4M3(x / s) with an IEEE float32 division, over the page's
    filled entries only. Dequantised value = E4M3 value * s.
    """
    x32 = np.asarray(x32, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0.0)
    s = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(E4M3_MAX))
    codes = e4m3_encode((x32 / s).astype(np.float32))
    return codes, s


# ---------------------------------------------------------------------------
# a1: gated-pooling compressor
# ---------------------------------------------------------------------------

def compress(K: np.ndarray, V: np.ndarray, Z: np.ndarray, r: int,
             P: np.ndarray | None = None):
    """Fold every r consecutive raw rows into one compressed entry.

    Follows [Atlas] compressed-KV entry (every m KV tokens squeezed into one
    entry with learned compression weights), [Walkthrough] "Causal
    Encoder-Decoder" > "One hidden state feeds the decoder" (global KV entries
    C and compression weights Z are both projected from hidden states) and
    "Compressed Sparse Attention 2" > "A simpler compressor" (groups do not
    overlap, no absolute positional embedding, indexer K is a projection of
    the main-KV entry).

    Readings: block j covers rows [j*r, (j+1)*r); per channel d the weights
    are a softmax over the block's r gate logits Z[i, d]; the same weights
    pool K and V (one Z per layer); a trailing incomplete block yields no
    entry; indexer K = Kbar @ P in float64, before any rounding.

    Returns float64 (Kbar [E, D], Vbar [E, D], KI [E, D_I] or None).
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Z = np.asarray(Z, dtype=np.float64)
    n_blocks = K.shape[0] // r
    D = K.shape[1]
    n = n_blocks * r
    Kb = K[:n].reshape(n_blocks, r, D)
    Vb = V[:n].reshape(n_blocks, r, D)
    Zb = Z[:n].reshape(n_blocks, r, D)
    m = Zb.max(axis=1, keepdims=True)
    e = np.exp(Zb - m)
    w = e / e.sum(axis=1, keepdims=True)
    kbar = (w * Kb).sum(axis=1)
    vbar = (w * Vb).sum(axis=1)
    kidx = None if P is None else kbar @ np.asarray(P, dtype=np.float64)
    return kbar, vbar, kidx


# ---------------------------------------------------------------------------
# FP4 main KV: E2M1 elements, one E4M3 scale per 16 channels
# ---------------------------------------------------------------------------

E2M1_MAX = 6.0      # the FP4 section's range 2688 = 448 (E4M3) x 6 (E2M1)
FP4_GROUP = 16      # channels sharing one scale


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit E2M1 codes -> float64: bit 3 sign, bits 2-1 exponent (bias 1),
    bit 0 mantissa; exponent 0 is subnormal (0 or 0.5)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(c & 8, -mag, mag)


def e2m1_encode(x32: np.ndarray) -> np.ndarray:
    """float32 values -> E2M1 codes: nearest of the 8 magnitudes, a tie going
    to the even code, saturating at 6; the sign bit is the input's IEEE sign."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    a = np.abs(x)
    mags = e2m1_decode(np.arange(8))                       # 0, .5, 1, 1.5, 2, 3, 4, 6
    d = np.abs(a[..., None] - mags)                         # [..., 8]
    best = d.min(axis=-1, keepdims=True)
    cand = np.where(d == best, np.arange(8), 99)
    even = np.where(cand % 2 == 0, cand, 99).min(axis=-1)
    code = np.where(even < 99, even, cand.min(axis=-1))
    code = np.where(a >= E2M1_MAX, 7, code)
    return (code | np.where(np.signbit(x), 8, 0)).astype(np.uint8)


def fp4_quantize_rows(x32: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Entries [E, D] float32 -> (E2M1 codes [E, D], E4M3 scale codes [E, D/16]).

    [Walkthrough] "FP4 main KV cache" (E2M1 elements, one E4M3 scale per 16
    channels, no second-level scale). Reading (the scale rule is not given):
    the scale is amax/6 of the 16 values (fp32 division) rounded to the
    nearest E4M3 value; elements are E2M1(x / scale) with an IEEE fp32
    division; a group whose scale rounds to 0 stores all-zero codes.
    """
    x32 = np.asarray(x32, dtype=np.float32)
    E, D = x32.shape
    g = x32.reshape(E, D // FP4_GROUP, FP4_GROUP)
    amax = np.abs(g).max(axis=-1)
    sc = e4m3_encode((amax / np.float32(E2M1_MAX)).astype(np.float32))
    s = e4m3_decode(sc).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0))
    q = (g / safe[..., None]).astype(np.float32)
    codes = np.where(s[..., None] > 0, e2m1_encode(q), 0).astype(np.uint8)
    return codes.reshape(E, D), sc


def fp4_dequantize_rows(codes: np.ndarray, scale_codes: np.ndarray) -> np.ndarray:
    E, D = codes.shape
    s = e4m3_decode(scale_codes)
    return (e2m1_decode(codes).reshape(E, D // FP4_GROUP, FP4_GROUP) * s[..., None]).reshape(E, D)


def store(x64: np.ndarray, dtype: str, page_entries: int = 64):
    """Round compressed entries [E, width] to the cache format, page by page.

    Returns (values as float64 exactly as the cache holds them, raw payload):
    raw is float32 array ('f32'), uint16 bf16 bits ('bf16') or
    (uint8 codes [E, width], float32 scales [n_pages]) ('fp8'), or
    (E2M1 codes [E, width], E4M3 scale codes [E, width/16]) ('fp4', every entry
    on its own). Page p holds entries [64p, 64p+64) of the sequence; the last
    page may be partly filled and its fp8 scale covers its filled entries only.
    """
    x64 = np.asarray(x64, dtype=np.float64)
    if dtype == "f32":
        raw = round_f32(x64)
        return raw.astype(np.float64), raw
    if dtype == "bf16":
        raw = round_bf16(x64)
        return decode_bf16(raw), raw
    if dtype == "fp8":
        E = x64.shape[0]
        x32 = round_f32(x64)
        codes = np.zeros(x64.shape, dtype=np.uint8)
        n_pages = (E + page_entries - 1) // page_entries
        scales = np.ones(n_pages, dtype=np.float32)
        vals = np.zeros(x64.shape, dtype=np.float64)
        for p in range(n_pages):
            sl = slice(p * page_entries, min(E, (p + 1) * page_entries))
            c, s = fp8_quantize_page(x32[sl])
            codes[sl] = c
            scales[p] = s
            vals[sl] = e4m3_decode(c) * np.float64(s)
        return vals, (codes, scales)
    if dtype == "fp4":
        codes, sc = fp4_quantize_rows(round_f32(x64))
        return fp4_dequantize_rows(codes, sc), (codes, sc)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# a2 / a3: lightning-indexer scores and Top-K
# ---------------------------------------------------------------------------

def store_ring_rows(x64: np.ndarray, dtype: str):
    """Raw window rows [n, D] as the ring holds them: unchanged for the
    activation dtype, or E4M3 codes with one fp32 scale amax/448 per row.

    The FP4 section keeps SWA KV in FP8 for its sensitivity to quantization;
    the scale granularity is not given, so the reading is one scale per row
    (rows enter the ring one token at a time) with the same codec as a page.
    Returns (float64 values as stored, raw payload)."""
    x64 = np.asarray(x64, dtype=np.float64)
    if dtype != "fp8":
        return x64.copy(), None
    x32 = round_f32(x64)
    codes = np.zeros(x64.shape, dtype=np.uint8)
    scales = np.ones(x64.shape[0], dtype=np.float32)
    vals = np.zeros(x64.shape, dtype=np.float64)
    for i in range(x64.shape[0]):
        c, sc = fp8_quantize_page(x32[i:i + 1])
        codes[i] = c[0]
        scales[i] = sc
        vals[i] = e4m3_decode(c[0]) * np.float64(sc)
    return vals, (codes, scales)


def visible_entries(t: int, r: int) -> int:
    """Number of compressed entries a query at raw position t may see.

    Causality ([Explainer] definition of causal; [Walkthrough] CSA2 "The
    Hierarchical Sparse Indexer" scores all causally visible positions):
    entry j is visible iff its whole block lies at or before t, i.e.
    (j+1)*r <= t+1.
    """
    return (t + 1) // r


def index_scores(q_idx: np.ndarray, w: np.ndarray, kidx: np.ndarray) -> np.ndarray:
    """s_j = sum_h w_h * max(0, q_h . k_j) in float64, rounded once to float32.

    [Walkthrough] CSA2 "The indexer selects, SWA covers the rest" (indexer
    query against indexer key); [Atlas] trained-sparse-attention entries (a
    lightning indexer, run as MQA: several indexer query heads over one shared
    key). The ReLU-weighted head sum is the reading taken here of the
    lightning-indexer score; no extra scale is applied (with ReLU and w >= 0 a
    positive scale would not change the ranking).

    q_idx [H_I, D_I], w [H_I], kidx [N, D_I] -> float32 [N].
    """
    q = np.asarray(q_idx, dtype=np.float64)
    k = np.asarray(kidx, dtype=np.float64)
    dots = k @ q.T                      # [N, H_I]
    s = np.maximum(dots, 0.0) @ np.asarray(w, dtype=np.float64)
    return s.astype(np.float32)


def topk(scores: np.ndarray, k: int) -> np.ndarray:
    """The k visible entries with the largest scores, ascending by index.

    [Explainer] (Top-K picks the most relevant positions); [Walkthrough] CSA2
    "The indexer selects, SWA covers the rest" (top entries per query).
    Readings: ties go to the lower index; when fewer than k entries are
    visible all are taken and the row is padded with -1.
    """
    s = np.asarray(scores, dtype=np.float32)
    n = s.shape[0]
    if k <= 0:
        return np.zeros(0, dtype=np.int32)
    j = np.arange(n)
    order = np.lexsort((j, -s.astype(np.float64)))   # by score desc, then index asc
    sel = np.sort(order[:k]).astype(np.int32)
    out = np.full(k, -1, dtype=np.int32)
    out[:sel.shape[0]] = sel
    return out


# ---------------------------------------------------------------------------
# a5 - a7: sparse branch + SWA branch under one softmax
# ---------------------------------------------------------------------------

def attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of H query heads over one shared key/value set (MQA).

    [Atlas] MQA/GQA entry (many query heads over a single shared K/V head).
    q [H, D], keys/vals [n, D] -> [H, D] float64. An empty key set gives 0.
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    vals = np.asarray(vals, dtype=np.float64)
    if keys.shape[0] == 0:
        return np.zeros((q.shape[0], vals.shape[1]))
    logits = scale * (q @ keys.T)                  # [H, n]
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p /= p.sum(axis=1, keepdims=True)
    return p @ vals


def key_set(T: np.ndarray, t: int, W: int, swa_start: int = 0):
    """Which keys a query at raw position t attends to.

    [Walkthrough] CSA2 "The indexer selects, SWA covers the rest": the query
    attends to the selected main-KV entries together with the layer-local
    sliding-window KV. "SWA Bounded Replay" > "Replay only the window": the
    window keys of a query at i are [max(s, i - W + 1), i] (s = 0 without a
    replay). Readings: one softmax over the union; no de-duplication between
    the branches; the window includes the current token; W = 0 disables it.

    Returns (entry indices into the compressed cache, raw row indices).
    """
    ent = np.asarray([int(j) for j in T if j >= 0], dtype=np.int64)
    lo = max(swa_start, t - W + 1)
    rows = np.arange(lo, t + 1, dtype=np.int64) if W > 0 else np.zeros(0, dtype=np.int64)
    return ent, rows


def attend_step(q: np.ndarray, T: np.ndarray, t: int, W: int, scale: float,
                kbar: np.ndarray, vbar: np.ndarray, rawk: np.ndarray, rawv: np.ndarray,
                swa_start: int = 0) -> np.ndarray:
    """One query's CSA attention output (all heads): sparse + SWA, one softmax."""
    ent, rows = key_set(T, t, W, swa_start)
    keys = np.concatenate([np.asarray(kbar, np.float64)[ent], np.asarray(rawk, np.float64)[rows]], axis=0)
    vals = np.concatenate([np.asarray(vbar, np.float64)[ent], np.asarray(rawv, np.float64)[rows]], axis=0)
    return attend(q, keys, vals, scale)


def hca_attend_step(q: np.ndarray, t: int, r: int, W: int, scale: float,
                    kbar: np.ndarray, vbar: np.ndarray, rawk: np.ndarray, rawv: np.ndarray,
                    swa_start: int = 0) -> np.ndarray:
    """Heavily compressed attention for one query: no indexer, every visible
    compressed entry takes part.

    [Atlas] compressed-KV entry: HCA uses the same compression primitive far
    more aggressively (large r) and then runs ordinary dense attention over
    the resulting short stream. Reading: the layer keeps the sliding-window
    branch of the CSA layers (W = 0 drops it), and the softmax runs over the
    union exactly as in attend_step.
    """
    T = np.arange(visible_entries(t, r), dtype=np.int64)
    return attend_step(q, T, t, W, scale, kbar, vbar, rawk, rawv, swa_start)


# ---------------------------------------------------------------------------
# hierarchical sparse indexer: the Full layer's candidate pool, Reindex mode
# ---------------------------------------------------------------------------

POOL_BLOCK = 8  # positions per pool block ("blocks of 8 positions")


def candidate_pool(scores: np.ndarray, n_blocks: int, block: int = POOL_BLOCK) -> np.ndarray:
    """The candidate pool a Full-mode layer builds for one query.

    [Walkthrough] CSA2 "The Hierarchical Sparse Indexer": the Full layer's
    scores over every visible position are grouped into blocks of `block`
    positions, a block scores the maximum of its positions, and the best
    `n_blocks` blocks are kept; every position of a kept block is a candidate.
    Readings: positions are compressed entries (what the indexer scores);
    blocks are aligned, [b*block, (b+1)*block), the last one cut at the
    visible count; equal block scores go to the lower block; the block list
    is ascending and padded with -1 when fewer blocks are visible (the same
    rules as the entry Top-K, which this reuses on the block scores).

    scores float32 [N] -> int32 [n_blocks] block ids.
    """
    s = np.asarray(scores, dtype=np.float32)
    nb = (s.shape[0] + block - 1) // block
    bs = np.array([s[b * block:(b + 1) * block].max() for b in range(nb)], dtype=np.float32)
    return topk(bs, n_blocks)


def pool_entries(pool: np.ndarray, n_vis: int, block: int = POOL_BLOCK) -> np.ndarray:
    """Entries covered by a pool's blocks, ascending, visible ones only."""
    b = np.asarray([int(x) for x in pool if x >= 0], dtype=np.int64)
    e = (b[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    return e[e < n_vis]


def reindex_topk(q_idx: np.ndarray, w: np.ndarray, kidx: np.ndarray, pool: np.ndarray, k: int,
                 n_vis: int, block: int = POOL_BLOCK) -> np.ndarray:
    """Top-K of a Reindex-mode layer.

    [Walkthrough] CSA2 "Full, Reindex, and Reuse" (a Reindex layer reuses the
    shared indexer keys and rescores them with its own indexer query) and
    "The Hierarchical Sparse Indexer" (deeper indexers score only inside the
    candidate pool). Scores as index_scores over the pool's visible entries;
    Top-K as topk (ties to the lower entry, ascending, -1 padding when the
    pool holds fewer than k entries).
    """
    e = pool_entries(pool, n_vis, block)
    s = index_scores(q_idx, w, np.asarray(kidx)[e])
    sel = topk(s, k)                      # positions into e; e ascending keeps the rules
    out = np.full(k, -1, dtype=np.int32)
    m = sel >= 0
    out[m] = e[sel[m]]
    return out


# ---------------------------------------------------------------------------
# whole step: one index pass reused by a group of layers
# ---------------------------------------------------------------------------

def decode_step(q_idx, w, kidx, r, k, t, layers):
    """Index once, attend with every layer of the group using the same Top-K.

    [Walkthrough] CSA2 "Full, Reindex, and Reuse": a Reuse layer runs no
    indexer and follows the latest selection; [Atlas] IndexCache ('shared'
    layers borrow the nearest 'full' layer's top-k). Each entry of ``layers``
    is a dict with q, W, scale, kbar, vbar, rawk, rawv (each layer keeps its
    own main KV and window here, as in IndexCache).
    Returns (T, [out per layer]).
    """
    n = visible_entries(t, r)
    s = index_scores(q_idx, w, kidx[:n])
    T = topk(s, k)
    outs = [attend_step(L["q"], T, t, L["W"], L["scale"], L["kbar"], L["vbar"],
                        L["rawk"], L["rawv"], L.get("swa_start", 0)) for L in layers]
    return T, outs
