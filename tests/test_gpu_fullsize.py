"""Full-size parity in the launch configuration the benchmark times.

The 1,048,576-token batch-4 decode (fp8 cache, 4 layers sharing one Top-1024,
W = 128, 64 heads) is built on the GPU exactly as bench.py builds it; one step
runs through the C ABI. The oracle recomputes, for sequence 0, the indexer
keys of all 262,144 entries from the same seeded raw rows, its Top-K, and the
attention of layers 0 and 3. The fp4 and fp8-ring decode variants, the HCA
layer (r = 128, every entry attended) and the prefill chunk (2,048 tokens on a
131,072-token context) are checked the same way on sampled sequences or
query tokens.
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

from gpu_helpers import max_abs, to64, topk_matches

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench_mod():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sys.path.insert(0, ROOT)
    import bench
    return bench


def _rows(seed, kind, layer, seq, r0, n, dev):
    return Sy.normal_rows(seed, Sy.stream_id(kind, layer, seq), r0, n, 128, dev, torch.bfloat16)


def test_decode_1m_context_sampled(bench_mod):
    bm = bench_mod
    seed, dev = 0, torch.device("cuda:0")
    caches = bm.build_cache(seed, 1, dev)
    c = caches[0]
    q_seq, q_pos = list(range(bm.BATCH)), [bm.CONTEXT - 1] * bm.BATCH
    qi = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_QI), 0, bm.BATCH * bm.IDX_HEADS, 64, dev, torch.bfloat16).view(bm.BATCH, bm.IDX_HEADS, 64)
    w = Sy.uniform_rows(seed, Sy.stream_id(Sy.KIND_W), 0, bm.BATCH, bm.IDX_HEADS, dev)
    qs = [Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_Q, l), 0, bm.BATCH * bm.HEADS, 128, dev, torch.bfloat16).view(bm.BATCH, bm.HEADS, 128)
          for l in range(bm.LAYERS)]
    T = c.index_topk(q_seq, q_pos, qi, w, bm.TOPK)
    scale = 1.0 / math.sqrt(128)
    outs = [to64(c.attend(l, q_seq, q_pos, qs[l], T, bm.TOPK, scale)) for l in range(bm.LAYERS)]
    assert c.read_errors() == 0
    Tg = T.cpu().numpy()
    # every row is a valid, ascending, distinct set of visible entries
    E = bm.CONTEXT // bm.RATIO
    for b in range(bm.BATCH):
        row = Tg[b]
        assert np.all(np.diff(row) > 0) and row[0] >= 0 and row[-1] < E

    # oracle for sequence 0, from the same seeded raw rows (generated on the
    # device by the seeded generator, copied out, then all arithmetic in fp64)
    P = to64(Sy.proj_matrix(seed, 128, 64))

    def layer_entries(layer):
        kb, vb, ki = (np.empty((E, 128)), np.empty((E, 128)), np.empty((E, 64)) if layer == 0 else None)
        step = 1 << 18
        for r0 in range(0, bm.CONTEXT, step):
            K, V, Z = (to64(_rows(seed, kind, layer, 0, r0, step, dev)) for kind in (Sy.KIND_K, Sy.KIND_V, Sy.KIND_Z))
            a, b_, c_ = O.compress(K, V, Z, bm.RATIO, P if layer == 0 else None)
            sl = slice(r0 // bm.RATIO, (r0 + step) // bm.RATIO)
            kb[sl], vb[sl] = a, b_
            if layer == 0:
                ki[sl] = c_
        return O.store(kb, "fp8")[0], O.store(vb, "fp8")[0], (O.store(ki, "fp8")[0] if layer == 0 else None)

    kb0, vb0, kis = layer_entries(0)
    s = O.index_scores(to64(qi[0]), to64(w[0]), kis)
    To = O.topk(s, bm.TOPK)
    ok, msg = topk_matches(Tg[0], To, s, rel=2e-2)
    assert ok, msg

    # attention of layers 0 and 3 with the oracle's own Top-K
    t = bm.CONTEXT - 1
    lo = t - bm.WINDOW + 1
    for layer in (0, 3):
        kbs, vbs, _ = (kb0, vb0, None) if layer == 0 else layer_entries(layer)
        Kw = np.zeros((bm.CONTEXT, 128))
        Vw = np.zeros((bm.CONTEXT, 128))
        Kw[lo:] = to64(_rows(seed, Sy.KIND_K, layer, 0, lo, bm.WINDOW, dev))
        Vw[lo:] = to64(_rows(seed, Sy.KIND_V, layer, 0, lo, bm.WINDOW, dev))
        ref = O.attend_step(to64(qs[layer][0]), To, t, bm.WINDOW, scale, kbs, vbs, Kw, Vw)
        err = max_abs(outs[layer][0], ref)
        assert err <= 2e-2, f"layer {layer}: max-abs {err}"
    for cc in caches:
        cc.close()


def _oracle_entries(seed, layer, seq, n_rows, dev, with_proj, kv, r=4, step=1 << 16):
    """Oracle compressed entries of (layer, seq) from the seeded raw rows, stored in `kv`."""
    P = to64(Sy.proj_matrix(seed, 128, 64)) if with_proj else None
    E = n_rows // r
    kb, vb = np.empty((E, 128)), np.empty((E, 128))
    ki = np.empty((E, 64)) if with_proj else None
    for r0 in range(0, E * r, step):
        n = min(step, E * r - r0)
        K, V, Z = (to64(_rows(seed, kind, layer, seq, r0, n, dev)) for kind in (Sy.KIND_K, Sy.KIND_V, Sy.KIND_Z))
        a, b_, c_ = O.compress(K, V, Z, r, P)
        sl = slice(r0 // r, (r0 + n) // r)
        kb[sl], vb[sl] = a, b_
        if with_proj:
            ki[sl] = c_
    return (O.store(kb, kv)[0], O.store(vb, kv)[0], O.store(ki, kv)[0] if with_proj else None)


def _check_query(seed, dev, seq, t, qi_row, w_row, q_row, T_row, out_row, k, W, kv, tol, n_rows):
    kbs, vbs, kis = _oracle_entries(seed, 0, seq, n_rows, dev, True, kv)
    N = O.visible_entries(t, 4)
    s = O.index_scores(to64(qi_row), to64(w_row), kis[:N])
    To = O.topk(s, k)
    ok, msg = topk_matches(T_row, To, s, rel=2e-2)
    assert ok, f"sequence {seq}: {msg}"
    lo = max(0, t - W + 1)
    Kw = np.zeros((t + 1, 128))
    Vw = np.zeros((t + 1, 128))
    Kw[lo:] = to64(_rows(seed, Sy.KIND_K, 0, seq, lo, t + 1 - lo, dev))
    Vw[lo:] = to64(_rows(seed, Sy.KIND_V, 0, seq, lo, t + 1 - lo, dev))
    ref = O.attend_step(to64(q_row), To, t, W, 1.0 / math.sqrt(128), kbs, vbs, Kw, Vw)
    err = max_abs(out_row, ref)
    assert err <= tol, f"sequence {seq}: max-abs {err}"


def test_decode_batch32_64k_bf16_sampled():
    """32 sequences of 65,536 bf16 tokens (16,384 entries each), 64 heads,
    Top-512, W = 128: one decode step for all 32; sequences 0 and 31 checked
    against the oracle, every row checked for validity."""
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
    Tg = T.cpu().numpy()
    for b in range(B_):
        assert np.all(np.diff(Tg[b]) > 0) and Tg[b][0] >= 0 and Tg[b][-1] < L // 4
    for b in (0, B_ - 1):
        _check_query(seed, dev, b, L - 1, qi[b], w[b], q[b], Tg[b], out[b], k, W, "bf16", 2e-2, L)
    c.close()


def test_serving_64_requests_4k_to_256k_sampled():
    """64 requests with log-uniform contexts from 4K to 256K tokens on one
    shared paged fp8 pool (shuffled free list): bulk build, then one serving
    step that appends one token per request (compress), indexes (Top-512) and
    attends (W = 128, 64 heads). The longest and the shortest request are
    checked against the oracle."""
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
    Tg = T.cpu().numpy()
    for b in ids:
        N = final[b] // 4
        row = Tg[b][Tg[b] >= 0]
        assert len(row) == min(k, N) and np.all(np.diff(row) > 0) and row[-1] < N
    for b in (int(np.argmax(lens)), int(np.argmin(lens))):
        _check_query(seed, dev, b, pos[b], qi[b], w[b], q[b], Tg[b], out[b], k, W, "fp8", 2e-2, final[b])
    c.close()


def _seq0_entries(bm, seed, dev, layer, kv):
    """Oracle compressed entries of sequence 0 of `layer` at the benchmark's
    1M-token size, stored in `kv` (indexer keys fp8 for fp8 and fp4 caches)."""
    E = bm.CONTEXT // bm.RATIO
    P = to64(Sy.proj_matrix(seed, 128, 64)) if layer == 0 else None
    kb, vb = np.empty((E, 128)), np.empty((E, 128))
    ki = np.empty((E, 64)) if layer == 0 else None
    step = 1 << 18
    for r0 in range(0, bm.CONTEXT, step):
        K, V, Z = (to64(_rows(seed, kind, layer, 0, r0, step, dev)) for kind in (Sy.KIND_K, Sy.KIND_V, Sy.KIND_Z))
        a, b_, c_ = O.compress(K, V, Z, bm.RATIO, P)
        sl = slice(r0 // bm.RATIO, (r0 + step) // bm.RATIO)
        kb[sl], vb[sl] = a, b_
        if layer == 0:
            ki[sl] = c_
    return O.store(kb, kv)[0], O.store(vb, kv)[0], (O.store(ki, "fp8")[0] if layer == 0 else None)


def _block_scores(s):
    nb = (s.shape[0] + 7) // 8
    return np.maximum.reduceat(s.astype(np.float32), np.arange(0, s.shape[0], 8))[:nb]


def test_hierarchical_indexer_1m_sampled(bench_mod):
    """The benchmark's 1M-token batch-4 cache: the Full layer's Top-1024 with a
    2,048-block pool, then a Reindex layer's Top-1024 inside the pool; sequence
    0 against the oracle's pool and Reindex selection (2e-2 tie band: the fp8
    indexer keys are compressed on each side), every row checked for validity."""
    bm = bench_mod
    seed, dev, nb = 0, torch.device("cuda:0"), 2048
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
    _, _, kis = _seq0_entries(bm, seed, dev, 0, "fp8")
    s = O.index_scores(to64(qi[0]), to64(w[0]), kis)
    Po = O.candidate_pool(s, nb)
    ok, msg = topk_matches(Pg[0], Po, _block_scores(s), rel=2e-2)
    assert ok, "pool: " + msg
    s2 = O.index_scores(to64(qi2[0]), to64(w2[0]), kis)
    ok, msg = topk_matches(T2g[0], O.reindex_topk(to64(qi2[0]), to64(w2[0]), kis, Po, bm.TOPK, E), s2, rel=2e-2)
    assert ok, "reindex: " + msg
    c.close()


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
    kb, vb, kis = _seq0_entries(bm, seed, dev, 0, kv)
    s = O.index_scores(to64(qi[0]), to64(w[0]), kis)
    To = O.topk(s, bm.TOPK)
    ok, msg = topk_matches(T.cpu().numpy()[0], To, s, rel=2e-2)
    assert ok, msg
    t = bm.CONTEXT - 1
    lo = t - bm.WINDOW + 1
    Kw, Vw = np.zeros((bm.CONTEXT, 128)), np.zeros((bm.CONTEXT, 128))
    Kw[lo:] = O.store_ring_rows(to64(_rows(seed, Sy.KIND_K, 0, 0, lo, bm.WINDOW, dev)), swa)[0]
    Vw[lo:] = O.store_ring_rows(to64(_rows(seed, Sy.KIND_V, 0, 0, lo, bm.WINDOW, dev)), swa)[0]
    ref = O.attend_step(to64(q[0]), To, t, bm.WINDOW, scale, kb, vb, Kw, Vw)
    assert max_abs(out[0], ref) <= 2e-2
    c.close()


def test_prefill_chunk_2048_on_131k_sampled(bench_mod):
    """The benchmark's prefill chunk (2,048 bf16 tokens after a 131,072-token
    context, pages in permuted order, Top-1024, W = 128, 64 heads), one step
    through the C ABI: its first, a middle and its last query against the
    oracle, whose entries come from the same seeded raw rows (the chunk's own
    entries are visible to its later queries)."""
    bm = bench_mod
    seed, dev = 0, torch.device("cuda:0")
    W_ = bm.build_prefill(seed, dev)
    c = W_["cache"]
    B.csa_seq_set_len(c.handle, 0, 0, bm.PF_PRIOR)
    W_["chunk_step"](torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert c.read_errors() & ~B.ERR_FALLBACK == 0
    T, out = W_["T"].cpu().numpy(), W_["out"]
    n_rows = bm.PF_PRIOR + bm.PF_CHUNK
    kbs, vbs, kis = _oracle_entries(seed, 0, 0, n_rows, dev, True, "bf16")
    for i in (0, 777, bm.PF_CHUNK - 1):
        t = bm.PF_PRIOR + i
        N = O.visible_entries(t, bm.RATIO)
        s = O.index_scores(to64(W_["qi"][i]), to64(W_["w"][i]), kis[:N])
        To = O.topk(s, bm.PF_K)
        ok, msg = topk_matches(T[i], To, s)
        assert ok, f"chunk query {i}: {msg}"
        lo = t - bm.WINDOW + 1
        Kw = np.zeros((t + 1, 128))
        Vw = np.zeros((t + 1, 128))
        Kw[lo:] = to64(_rows(seed, Sy.KIND_K, 0, 0, lo, bm.WINDOW, dev))
        Vw[lo:] = to64(_rows(seed, Sy.KIND_V, 0, 0, lo, bm.WINDOW, dev))
        ref = O.attend_step(to64(W_["q"][i]), To, t, bm.WINDOW, W_["scale"], kbs, vbs, Kw, Vw)
        err = max_abs(to64(out[i]), ref)
        assert err <= 2e-2, f"chunk query {i}: max-abs {err}"
    c.close()


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
    lo = t - bm.WINDOW + 1
    for b in (0, 3):
        E = bm.CONTEXT // bm.HCA_RATIO
        kb, vb = np.empty((E, 128)), np.empty((E, 128))
        for r0 in range(0, bm.CONTEXT, step):
            K, V, Z = (to64(_rows(seed, kind, 7, b, r0, step, dev)) for kind in (Sy.KIND_K, Sy.KIND_V, Sy.KIND_Z))
            a, v_, _ = O.compress(K, V, Z, bm.HCA_RATIO)
            kb[r0 // bm.HCA_RATIO:(r0 + step) // bm.HCA_RATIO], vb[r0 // bm.HCA_RATIO:(r0 + step) // bm.HCA_RATIO] = a, v_
        Kw = np.zeros((bm.CONTEXT, 128))
        Vw = np.zeros((bm.CONTEXT, 128))
        Kw[lo:] = to64(_rows(seed, Sy.KIND_K, 7, b, lo, bm.WINDOW, dev))
        Vw[lo:] = to64(_rows(seed, Sy.KIND_V, 7, b, lo, bm.WINDOW, dev))
        ref = O.hca_attend_step(to64(q[b]), t, bm.HCA_RATIO, bm.WINDOW, 1.0 / math.sqrt(128),
                                O.store(kb, "fp8")[0], O.store(vb, "fp8")[0], Kw, Vw)
        err = max_abs(out[b], ref)
        assert err <= 2e-2, f"sequence {b}: max-abs {err}"
    c.close()
