"""Full-size parity in the launch configurations the benchmark times.

Every Top-K row of every full-size workload is checked against the oracle to
the exact rule (a valid Top-K of scores within 1e-6 relative of the oracle's,
plus the per-key slack of codes that sit at a rounding boundary), with the
oracle's indexer keys recomputed from the same seeded raw rows:

* decode, batch 4 x 1,048,576 tokens, fp8 cache, Top-1024, W = 128, 64 heads,
  4 layers sharing one Top-K: all 4 rows; stored indexer keys and layer-0
  compressed keys of every sequence; attention of layer 0 and of one more
  layer per sequence (layers 1, 2, 3, and 3 again for sequence 0);
* decode, batch 32 x 65,536 bf16 tokens, Top-512: all 32 rows and outputs;
* serving, 64 requests of 4K-256K tokens on a paged fp8 pool, one appended
  token each: all 64 rows and outputs;
* prefill, a 2,048-token chunk after 131,072 tokens: all 2,048 rows, the
  attention of every 16th query and of the last;
* the fp4 and fp8-ring decode variants, the hierarchical indexer (its pool
  checked on block scores; the GPU's Reindex run on the oracle's own pool)
  and the HCA layer on sampled sequences.

Attention references use the oracle's own Top-K; outputs are bf16, compared
at 2e-2 max-abs.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

from compressed_sparse_attention_csa_amd import binding as B
from compressed_sparse_attention_csa_amd import synth as Sy
from oracle import csa_oracle as O

import parity_bounds as PB
from gpu_helpers import TopkRows, check_stored_pool, max_abs, oracle_entries, to64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ATOL = 2e-2


@pytest.fixture(scope="module")
def bench_mod():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sys.path.insert(0, ROOT)
    import bench
    return bench


def _rows(seed, kind, layer, seq, r0, n, dev):
    return Sy.normal_rows(seed, Sy.stream_id(kind, layer, seq), r0, n, 128, dev, torch.bfloat16)


def _entries(seed, layer, seq, n_rows, dev, with_proj, r=4, step=1 << 18):
    """The oracle's compressed entries of (layer, seq) from the seeded raw rows,
    float64 before rounding, with their fp32 error bands:
    (kbar, vbar, kidx, band_kbar, band_kidx); kidx and its band are None
    without the projection."""
    P = to64(Sy.proj_matrix(seed, 128, 64)) if with_proj else None
    E = n_rows // r
    kb, vb, bk = np.empty((E, 128)), np.empty((E, 128)), np.empty((E, 128))
    ki, bi = (np.empty((E, 64)), np.empty((E, 64))) if with_proj else (None, None)
    for r0 in range(0, E * r, step):
        n = min(step, E * r - r0)
        K, V, Z = (to64(_rows(seed, kind, layer, seq, r0, n, dev)) for kind in (Sy.KIND_K, Sy.KIND_V, Sy.KIND_Z))
        a, b_, c_, ba, _, bc = oracle_entries(K, V, Z, r, P)
        sl = slice(r0 // r, (r0 + n) // r)
        kb[sl], vb[sl], bk[sl] = a, b_, ba
        if with_proj:
            ki[sl], bi[sl] = c_, bc
    return kb, vb, ki, bk, bi


def _window(seed, layer, seq, t, W, dev, swa=""):
    """Raw K/V rows as the window ring holds them: rows (t - W, t] filled, the
    rest zero (never read)."""
    lo = max(0, t - W + 1)
    Kw, Vw = np.zeros((t + 1, 128)), np.zeros((t + 1, 128))
    Kw[lo:] = O.store_ring_rows(to64(_rows(seed, Sy.KIND_K, layer, seq, lo, t + 1 - lo, dev)), swa)[0]
    Vw[lo:] = O.store_ring_rows(to64(_rows(seed, Sy.KIND_V, layer, seq, lo, t + 1 - lo, dev)), swa)[0]
    return Kw, Vw


def _check_attention(got, q64, To, t, W, scale, kbs, vbs, Kw, Vw, what):
    ref = O.attend_step(q64, To, t, W, scale, kbs, vbs, Kw, Vw)
    err = max_abs(got, ref)
    assert err <= ATOL, f"{what}: max-abs {err}"


# --------------------------------------------------------------------------- batch-4 1M decode

@pytest.fixture(scope="module")
def decode_1m(bench_mod):
    """One decode step of the benchmark's cache (built as the benchmark builds it)."""
    bm = bench_mod
    seed, dev = 0, torch.device("cuda:0")
    c = bm.build_cache(seed, 1, dev)[0]
    q_seq, q_pos = list(range(bm.BATCH)), [bm.CONTEXT - 1] * bm.BATCH
    qi = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_QI), 0, bm.BATCH * bm.IDX_HEADS, 64, dev,
                        torch.bfloat16).view(bm.BATCH, bm.IDX_HEADS, 64)
    w = Sy.uniform_rows(seed, Sy.stream_id(Sy.KIND_W), 0, bm.BATCH, bm.IDX_HEADS, dev)
    qs = [Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_Q, l), 0, bm.BATCH * bm.HEADS, 128, dev,
                         torch.bfloat16).view(bm.BATCH, bm.HEADS, 128) for l in range(bm.LAYERS)]
    T = c.index_topk(q_seq, q_pos, qi, w, bm.TOPK)
    scale = 1.0 / math.sqrt(128)
    outs = [to64(c.attend(l, q_seq, q_pos, qs[l], T, bm.TOPK, scale)) for l in range(bm.LAYERS)]
    assert c.read_errors() == 0
    yield dict(cache=c, T=T.cpu().numpy(), qi=to64(qi), w=to64(w), q=[to64(x) for x in qs], outs=outs,
               scale=scale, seed=seed, dev=dev)
    c.close()


@pytest.mark.parametrize("b", range(4))
def test_decode_1m_every_sequence(bench_mod, decode_1m, b):
    bm, d = bench_mod, decode_1m
    seed, dev, c = d["seed"], d["dev"], d["cache"]
    E, t = bm.CONTEXT // bm.RATIO, bm.CONTEXT - 1
    kb, vb, ki, bk, bi = _entries(seed, 0, b, bm.CONTEXT, dev, True)
    check_stored_pool(c, c.kidx, c.kidx_scale, b, E, ki, bi, "fp8", f"sequence {b} indexer keys")
    check_stored_pool(c, c.kbar[0], c.kbar_scale[0], b, E, kb, bk, "fp8", f"sequence {b} layer-0 keys")
    s = TopkRows(ki, bi, "fp8").check(d["T"][b], d["qi"][b], d["w"][b], E, bm.TOPK, f"sequence {b}")
    To = O.topk(s, bm.TOPK)
    Kw, Vw = _window(seed, 0, b, t, bm.WINDOW, dev)
    _check_attention(d["outs"][0][b], d["q"][0][b], To, t, bm.WINDOW, d["scale"], O.store(kb, "fp8")[0],
                     O.store(vb, "fp8")[0], Kw, Vw, f"sequence {b} layer 0")
    layer = b if b else 3       # every layer's own K/V once (layer 3 twice)
    kl, vl, _, _, _ = _entries(seed, layer, b, bm.CONTEXT, dev, False)
    Kw, Vw = _window(seed, layer, b, t, bm.WINDOW, dev)
    _check_attention(d["outs"][layer][b], d["q"][layer][b], To, t, bm.WINDOW, d["scale"],
                     O.store(kl, "fp8")[0], O.store(vl, "fp8")[0], Kw, Vw, f"sequence {b} layer {layer}")


# --------------------------------------------------------------------------- batch-32 64K bf16 decode

def test_decode_batch32_64k_bf16_every_row():
    """32 sequences of 65,536 bf16 tokens (16,384 entries each), 64 heads,
    Top-512, W = 128: one decode step; every row's Top-K and output against the
    oracle."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from compressed_sparse_attention_csa_amd.cache import CacheSpec, CsaCache
    seed, dev, B_, L, k, W, H = 1, torch.device("cuda:0"), 32, 1 << 16, 512, 128, 64
    pages = L // 4 // 64
    spec = CacheSpec(ratio=4, q_heads=H, idx_heads=4, window=W, ring_rows=W, n_layers=1, max_seqs=B_,
                     max_pages_per_seq=pages, pool_pages=B_ * pages, kv_dtype="bf16", act_dtype="bf16",
                     max_queries=B_, max_k=k)
    bt = torch.tensor(Sy.permutation(seed, B_ * pages, salt=9), dtype=torch.int32).view(B_, pages).to(dev)
    c = CsaCache(spec, dev, block_table=bt)
    P = Sy.proj_matrix(seed, 128, 64, device=dev)
    for b in range(B_):
        K, V, Z = (_rows(seed, kind, 0, b, 0, L, dev) for kind in (Sy.KIND_K, Sy.KIND_V, Sy.KIND_Z))
        c.compress(0, [b], [L], K, V, Z, P)
    ids, pos = list(range(B_)), [L - 1] * B_
    qi = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_QI), 0, B_ * 4, 64, dev, torch.bfloat16).view(B_, 4, 64)
    w = Sy.uniform_rows(seed, Sy.stream_id(Sy.KIND_W), 0, B_, 4, dev)
    q = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_Q), 0, B_ * H, 128, dev, torch.bfloat16).view(B_, H, 128)
    T = c.index_topk(ids, pos, qi, w, k)
    out = to64(c.attend(0, ids, pos, q, T, k, 1.0 / math.sqrt(128)))
    assert c.read_errors() == 0
    Tg, qi64, w64, q64 = T.cpu().numpy(), to64(qi), to64(w), to64(q)
    E, t = L // 4, L - 1
    for b in range(B_):
        kb, vb, ki, _, bi = _entries(seed, 0, b, L, dev, True, step=L)
        s = TopkRows(ki, bi, "bf16").check(Tg[b], qi64[b], w64[b], E, k, f"sequence {b}")
        Kw, Vw = _window(seed, 0, b, t, W, dev)
        _check_attention(out[b], q64[b], O.topk(s, k), t, W, 1.0 / math.sqrt(128), O.store(kb, "bf16")[0],
                         O.store(vb, "bf16")[0], Kw, Vw, f"sequence {b}")
    c.close()


# --------------------------------------------------------------------------- 64 ragged serving requests

@pytest.fixture(scope="module")
def serving_64():
    """64 requests with log-uniform contexts from 4K to 256K tokens on one
    shared paged fp8 pool (shuffled free list): bulk build, then one serving
    step that appends one token per request (compress), indexes (Top-512) and
    attends (W = 128, 64 heads)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from compressed_sparse_attention_csa_amd.cache import CacheSpec, CsaCache
    seed, dev, nreq, k, W, H = 2, torch.device("cuda:0"), 64, 512, 128, 64
    lens = Sy.log_uniform_lengths(seed, nreq, 4096, 262144)
    final = [L + 1 for L in lens]
    pages = [(L // 4 + 63) // 64 for L in final]
    pool = sum(pages) + 16
    perm = Sy.permutation(seed, pool, salt=13)
    max_pages = max(pages)
    bt = torch.full((nreq, max_pages), -1, dtype=torch.int32)
    off = 0
    for b, p in enumerate(pages):
        bt[b, :p] = torch.tensor(perm[off:off + p], dtype=torch.int32)
        off += p
    spec = CacheSpec(ratio=4, q_heads=H, idx_heads=4, window=W, ring_rows=W, n_layers=1, max_seqs=nreq,
                     max_pages_per_seq=max_pages, pool_pages=pool, kv_dtype="fp8", act_dtype="bf16",
                     max_queries=nreq, max_k=k)
    c = CsaCache(spec, dev, block_table=bt.to(dev))
    P = Sy.proj_matrix(seed, 128, 64, device=dev)
    for b in range(nreq):
        K, V, Z = (_rows(seed, kind, 0, b, 0, lens[b], dev) for kind in (Sy.KIND_K, Sy.KIND_V, Sy.KIND_Z))
        c.compress(0, [b], [lens[b]], K, V, Z, P)
    ids = list(range(nreq))
    new = [torch.cat([_rows(seed, kind, 0, b, lens[b], 1, dev) for b in ids]) for kind in (Sy.KIND_K, Sy.KIND_V, Sy.KIND_Z)]
    c.compress(0, ids, [1] * nreq, *new, P)
    pos = lens[:]          # the appended token's position
    qi = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_QI), 0, nreq * 4, 64, dev, torch.bfloat16).view(nreq, 4, 64)
    w = Sy.uniform_rows(seed, Sy.stream_id(Sy.KIND_W), 0, nreq, 4, dev)
    q = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_Q), 0, nreq * H, 128, dev, torch.bfloat16).view(nreq, H, 128)
    T = c.index_topk(ids, pos, qi, w, k)
    out = to64(c.attend(0, ids, pos, q, T, k, 1.0 / math.sqrt(128)))
    assert c.read_errors() == 0
    yield dict(cache=c, T=T.cpu().numpy(), out=out, qi=to64(qi), w=to64(w), q=to64(q), pos=pos, final=final, k=k,
               W=W, seed=seed, dev=dev)
    c.close()


@pytest.mark.parametrize("part", range(4))
def test_serving_64_requests_every_row(serving_64, part):
    """A quarter of the 64 requests (b = part mod 4): Top-K and output of the
    step against the oracle run on each request's raw rows, including the
    appended token's (its entry closes a block for some requests)."""
    d = serving_64
    seed, dev, k, W = d["seed"], d["dev"], d["k"], d["W"]
    for b in range(part, 64, 4):
        t, n_rows = d["pos"][b], d["final"][b]
        N = O.visible_entries(t, 4)
        kb, vb, ki, bk, bi = _entries(seed, 0, b, n_rows, dev, True, step=1 << 16)
        if b % 16 == part:
            check_stored_pool(d["cache"], d["cache"].kidx, d["cache"].kidx_scale, b, N, ki, bi, "fp8",
                              f"request {b} indexer keys")
        s = TopkRows(ki, bi, "fp8").check(d["T"][b], d["qi"][b], d["w"][b], N, k, f"request {b}")
        Kw, Vw = _window(seed, 0, b, t, W, dev)
        _check_attention(d["out"][b], d["q"][b], O.topk(s, k), t, W, 1.0 / math.sqrt(128), O.store(kb, "fp8")[0],
                         O.store(vb, "fp8")[0], Kw, Vw, f"request {b}")


# --------------------------------------------------------------------------- hierarchical indexer at 1M

def _block_view(s, slack):
    """Block scores (maximum over each aligned 8 entries) and block slack (the
    largest entry slack in the block): a block's score moves by at most that."""
    idx = np.arange(0, s.shape[0], 8)
    return (np.maximum.reduceat(np.asarray(s, np.float64), idx), np.maximum.reduceat(slack, idx))


def test_hierarchical_indexer_1m(bench_mod):
    """The benchmark's 1M-token batch-4 cache: the Full layer's Top-1024 with a
    2,048-block pool, then a Reindex layer's Top-1024 inside a pool. For
    sequence 0: the Full Top-K and the GPU pool are valid selections of the
    oracle's scores (blocks scored by their maximum); the GPU Reindex, run on
    the oracle's own pool, is a valid Top-K of the oracle's Reindex scores over
    that pool. Every row: the pool is ascending and covers its Full Top-K, and
    the Reindex rows lie inside their pools."""
    bm = bench_mod
    seed, dev, nb = 0, torch.device("cuda:0"), bm.POOL_BLOCKS
    c = bm.build_cache(seed, 1, dev)[0]
    q_seq, q_pos = list(range(bm.BATCH)), [bm.CONTEXT - 1] * bm.BATCH
    qi = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_QI), 0, bm.BATCH * 4, 64, dev, torch.bfloat16).view(bm.BATCH, 4, 64)
    w = Sy.uniform_rows(seed, Sy.stream_id(Sy.KIND_W), 0, bm.BATCH, 4, dev)
    qi2 = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_QI, 1), 0, bm.BATCH * 4, 64, dev, torch.bfloat16).view(bm.BATCH, 4, 64)
    w2 = Sy.uniform_rows(seed, Sy.stream_id(Sy.KIND_W, 1), 0, bm.BATCH, 4, dev)
    T, P = c.index_topk_pool(q_seq, q_pos, qi, w, bm.TOPK, nb)
    T2 = c.index_reindex(q_seq, q_pos, qi2, w2, P, bm.TOPK)
    assert c.read_errors() & ~B.ERR_FALLBACK == 0
    Tg, Pg, T2g = T.cpu().numpy(), P.cpu().numpy(), T2.cpu().numpy()
    E = bm.CONTEXT // bm.RATIO
    for b in range(bm.BATCH):
        assert np.all(np.diff(Pg[b]) > 0) and Pg[b][0] >= 0 and Pg[b][-1] < E // 8
        ents = set(O.pool_entries(Pg[b], E).tolist())
        assert set(T2g[b].tolist()) <= ents and np.all(np.diff(T2g[b]) > 0)
        assert set(Tg[b].tolist()) <= ents            # the Full Top-K lies in its own pool
    _, _, ki, _, bi = _entries(seed, 0, 0, bm.CONTEXT, dev, True)
    rows = TopkRows(ki, bi, "fp8")
    qa, wa, qb, wb = to64(qi[0]), to64(w[0]), to64(qi2[0]), to64(w2[0])
    s = rows.check(Tg[0], qa, wa, E, bm.TOPK, "Full Top-K")
    bs, bsl = _block_view(s, rows.slack(qa, wa, s, E))
    ok, msg = PB.topk_valid(Pg[0], bs, nb, bsl)
    assert ok, "pool: " + msg
    # the GPU's Reindex over the oracle's pool
    Po = O.candidate_pool(s, nb)
    Pt = torch.from_numpy(np.tile(Po.astype(np.int32), (bm.BATCH, 1))).to(dev)
    T3 = c.index_reindex(q_seq, q_pos, qi2, w2, Pt, bm.TOPK).cpu().numpy()
    assert c.read_errors() & ~B.ERR_FALLBACK == 0
    e = O.pool_entries(Po, E)
    s2 = rows.scores(qb, wb, E)
    sl2 = rows.slack(qb, wb, s2, E)
    pos = np.searchsorted(e, T3[0])
    assert np.array_equal(e[pos], T3[0]), "Reindex row outside the oracle's pool"
    ok, msg = PB.topk_valid(pos, s2[e], bm.TOPK, sl2[e])
    assert ok, "reindex: " + msg
    want = O.reindex_topk(qb, wb, rows.kis, Po, bm.TOPK, E)
    print(f"[reindex] {len(set(T3[0].tolist()) ^ set(want.tolist())) // 2} swaps against the oracle's own")
    c.close()


# --------------------------------------------------------------------------- 1M decode variants

@pytest.mark.parametrize("kv,swa", [("fp4", ""), ("fp8", "fp8")])
def test_decode_1m_variant_sampled(bench_mod, kv, swa):
    """The benchmark's decode-step variants: fp4 K/V (E2M1, E4M3 scale per 16
    channels) with a bf16 window ring, and fp8 K/V pages with an fp8 window ring
    (one scale per row); fp8 indexer keys in both. Sequence 0's Top-K and
    layer-0 attention against the oracle's entries and ring rows."""
    bm = bench_mod
    seed, dev = 0, torch.device("cuda:0")
    c = bm.build_cache(seed, 1, dev, swa=swa, kv=kv)[0]
    q_seq, q_pos = list(range(bm.BATCH)), [bm.CONTEXT - 1] * bm.BATCH
    qi = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_QI), 0, bm.BATCH * 4, 64, dev, torch.bfloat16).view(bm.BATCH, 4, 64)
    w = Sy.uniform_rows(seed, Sy.stream_id(Sy.KIND_W), 0, bm.BATCH, 4, dev)
    q = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_Q, 0), 0, bm.BATCH * bm.HEADS, 128, dev, torch.bfloat16).view(bm.BATCH, bm.HEADS, 128)
    T = c.index_topk(q_seq, q_pos, qi, w, bm.TOPK)
    scale = 1.0 / math.sqrt(128)
    out = to64(c.attend(0, q_seq, q_pos, q, T, bm.TOPK, scale))
    assert c.read_errors() == 0
    E, t = bm.CONTEXT // bm.RATIO, bm.CONTEXT - 1
    kb, vb, ki, _, bi = _entries(seed, 0, 0, bm.CONTEXT, dev, True)
    s = TopkRows(ki, bi, kv).check(T.cpu().numpy()[0], to64(qi[0]), to64(w[0]), E, bm.TOPK, "sequence 0")
    Kw, Vw = _window(seed, 0, 0, t, bm.WINDOW, dev, swa)
    _check_attention(out[0], to64(q[0]), O.topk(s, bm.TOPK), t, bm.WINDOW, scale, O.store(kb, kv)[0],
                     O.store(vb, kv)[0], Kw, Vw, "sequence 0")
    c.close()


# --------------------------------------------------------------------------- prefill chunk

def test_prefill_chunk_2048_on_131k_every_row(bench_mod):
    """The benchmark's prefill chunk (2,048 bf16 tokens after a 131,072-token
    context, pages in permuted order, Top-1024, W = 128, 64 heads), one step
    through the C ABI: every query's Top-K against the oracle (the chunk's own
    entries are visible to its later queries), and the attention of every 16th
    query and of the last."""
    bm = bench_mod
    seed, dev = 0, torch.device("cuda:0")
    W_ = bm.build_prefill(seed, dev)
    c = W_["cache"]
    B.csa_seq_set_len(c.handle, 0, 0, bm.PF_PRIOR)
    W_["chunk_step"](torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert c.read_errors() & ~B.ERR_FALLBACK == 0
    T, out = W_["T"].cpu().numpy(), to64(W_["out"])
    qi64, w64, q64 = to64(W_["qi"]), to64(W_["w"]), to64(W_["q"])
    n_rows = bm.PF_PRIOR + bm.PF_CHUNK
    kb, vb, ki, _, bi = _entries(seed, 0, 0, n_rows, dev, True, step=1 << 16)
    rows = TopkRows(ki, bi, "bf16")
    kbs, vbs = O.store(kb, "bf16")[0], O.store(vb, "bf16")[0]
    Kw, Vw = _window(seed, 0, 0, n_rows - 1, bm.WINDOW + bm.PF_CHUNK, dev)
    for i in range(bm.PF_CHUNK):
        t = bm.PF_PRIOR + i
        N = O.visible_entries(t, bm.RATIO)
        s = rows.check(T[i], qi64[i], w64[i], N, bm.PF_K, f"chunk query {i}")
        if i % 16 == 0 or i == bm.PF_CHUNK - 1:
            _check_attention(out[i], q64[i], O.topk(s, bm.PF_K), t, bm.WINDOW, W_["scale"], kbs, vbs, Kw, Vw,
                             f"chunk query {i}")
    c.close()


# --------------------------------------------------------------------------- HCA layer

def test_hca_1m_dense_sampled(bench_mod):
    """The benchmark's HCA layer (batch 4, 1,048,576 tokens at r = 128: 8,192
    fp8 entries per sequence, all attended, with the 128-token window, 64
    heads), one call through the C ABI; sequences 0 and 3 against the oracle
    from the same seeded raw rows."""
    bm = bench_mod
    seed, dev = 0, torch.device("cuda:0")
    c, _, _ = bm.build_hca(seed, dev)
    q = bm.hca_q(seed, dev)
    t = bm.CONTEXT - 1
    out = to64(c.attend_dense(0, list(range(bm.BATCH)), [t] * bm.BATCH, q, 1.0 / math.sqrt(128)))
    assert c.read_errors() == 0
    step = 1 << 18
    for b in (0, 3):
        E = bm.CONTEXT // bm.HCA_RATIO
        kb, vb = np.empty((E, 128)), np.empty((E, 128))
        for r0 in range(0, bm.CONTEXT, step):
            K, V, Z = (to64(_rows(seed, kind, 7, b, r0, step, dev)) for kind in (Sy.KIND_K, Sy.KIND_V, Sy.KIND_Z))
            a, v_, _ = O.compress(K, V, Z, bm.HCA_RATIO)
            kb[r0 // bm.HCA_RATIO:(r0 + step) // bm.HCA_RATIO], vb[r0 // bm.HCA_RATIO:(r0 + step) // bm.HCA_RATIO] = a, v_
        Kw, Vw = _window(seed, 7, b, t, bm.WINDOW, dev)
        ref = O.hca_attend_step(to64(q[b]), t, bm.HCA_RATIO, bm.WINDOW, 1.0 / math.sqrt(128),
                                O.store(kb, "fp8")[0], O.store(vb, "fp8")[0], Kw, Vw)
        err = max_abs(out[b], ref)
        assert err <= ATOL, f"sequence {b}: max-abs {err}"
    c.close()
