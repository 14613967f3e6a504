"""GPU parity: every ABI call of the HIP library against the oracle.

Inputs are seeded (compressed_sparse_attention_csa_amd.synth). Isolated tests
write oracle-made cache contents into the device pools, so index and attend
are compared on identical inputs; chain tests run the whole step on each side
from the same raw rows. Bars: Top-K sets exact except near-ties within 1e-6
relative of the k-th oracle score; outputs max-abs 2e-3 (fp32) / 2e-2
(bf16, fp8). Where both sides compress the same raw rows, stored codes must
equal the oracle's rounding except at rounding boundaries within the fp32
error band (tests/parity_bounds.py), and a chained Top-K row must be a valid
Top-K of the oracle's scores within 1e-6 relative plus the score slack of
exactly those keys.
"""
import math

import numpy as np
import pytest
import torch

from compressed_sparse_attention_csa_amd import binding as B
from compressed_sparse_attention_csa_amd import synth as Sy
from compressed_sparse_attention_csa_amd.cache import CacheSpec, CsaCache
from oracle import csa_oracle as O

import parity_bounds as PB
from gpu_helpers import (TOL, TORCH_ACT, check_topk_chain, fill_index_keys, fill_main_kv, fill_ring, make_cache,
                         max_abs, oracle_entries, raw_rows, to64, topk_matches, unpack_fp4,
                         check_stored_pool)

pytestmark = pytest.mark.gpu

DT_CASES = [("f32", "f32"), ("bf16", "bf16"), ("fp8", "bf16")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.synchronize()


# --------------------------------------------------------------------------- number formats

def test_device_codecs_match_oracle(golden_dir):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    ref = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    out = torch.empty(256, dtype=torch.float32, device="cuda")
    B.csa_debug_convert(0, codes.cuda(), out)
    got = out.cpu().numpy().astype(np.float64)
    assert np.array_equal(got[finite], ref[finite])
    outb = torch.empty(256, dtype=torch.int16, device="cuda")
    B.csa_debug_convert(1, codes.cuda(), outb)
    gotb = outb.cpu().numpy().view(np.uint16)
    assert np.array_equal(gotb[finite], O.round_bf16(ref[finite]))
    # encoder: random values over the whole range, exact midpoints, the fixture table
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * 40, rng.standard_normal(5000) * 0.01,
                        (O.e4m3_decode(finite.astype(np.uint8))[:-1] + O.e4m3_decode(finite.astype(np.uint8))[1:]) / 2,
                        [0.0, -0.0, 448.0, 464.0, 500.0, -1e9, 2 ** -10, 1.5 * 2 ** -9]]).astype(np.float32)
    x = x[np.isfinite(x)]
    xt = torch.from_numpy(x).cuda()
    o8 = torch.empty(x.shape[0], dtype=torch.uint8, device="cuda")
    B.csa_debug_convert(2, xt, o8)
    assert np.array_equal(o8.cpu().numpy(), O.e4m3_encode(x))
    ob = torch.empty(x.shape[0], dtype=torch.int16, device="cuda")
    B.csa_debug_convert(3, xt, ob)
    assert np.array_equal(ob.cpu().numpy().view(np.uint16), O.round_bf16(x.astype(np.float64)))


# --------------------------------------------------------------------------- compress

def _compress_case(kv, act, r, lens, seed=3, n_layers=1, chunks=None, swa=""):
    """Compress seeded rows for each sequence of `lens` on the GPU (in one call,
    or in the given per-call chunk sizes) and return (cache, raw inputs)."""
    max_pages = max(1, max(L // r for L in lens) // 64 + 2)
    cache = make_cache(seed, ratio=r, q_heads=16, window=8, ring_rows=max(16, r), n_layers=n_layers,
                       max_seqs=len(lens), max_pages_per_seq=max_pages, pool_pages=len(lens) * max_pages + 3,
                       kv_dtype=kv, act_dtype=act, max_queries=len(lens), max_k=64, swa_dtype=swa)
    P = Sy.proj_matrix(seed, 128, 64)
    raw = {}
    for layer in range(n_layers):
        per = [(raw_rows(seed, Sy.KIND_K, layer, b, 0, L, act), raw_rows(seed, Sy.KIND_V, layer, b, 0, L, act),
                raw_rows(seed, Sy.KIND_Z, layer, b, 0, L, act)) for b, L in enumerate(lens)]
        raw[layer] = per
        steps = chunks or [None]
        pos = [0] * len(lens)
        for ch in steps:
            ids, nn, ks, vs, zs = [], [], [], [], []
            for b, L in enumerate(lens):
                n = L - pos[b] if ch is None else min(ch, L - pos[b])
                if n <= 0:
                    continue
                ids.append(b)
                nn.append(n)
                ks.append(per[b][0][pos[b]:pos[b] + n])
                vs.append(per[b][1][pos[b]:pos[b] + n])
                zs.append(per[b][2][pos[b]:pos[b] + n])
                pos[b] += n
            if not ids:
                continue
            cache.compress(layer, ids, nn, torch.cat(ks).cuda(), torch.cat(vs).cuda(), torch.cat(zs).cuda(),
                           P.cuda() if layer == 0 else None)
        if chunks:
            while any(pos[b] < L for b, L in enumerate(lens)):
                ids = [b for b, L in enumerate(lens) if pos[b] < L]
                nn = [lens[b] - pos[b] for b in ids]
                cache.compress(layer, ids, nn, torch.cat([per[b][0][pos[b]:] for b in ids]).cuda(),
                               torch.cat([per[b][1][pos[b]:] for b in ids]).cuda(),
                               torch.cat([per[b][2][pos[b]:] for b in ids]).cuda(), P.cuda() if layer == 0 else None)
                for b in ids:
                    pos[b] = lens[b]
    torch.cuda.synchronize()
    return cache, raw, P


_check_stored = check_stored_pool


@pytest.mark.parametrize("kv,act", DT_CASES)
@pytest.mark.parametrize("r", [1, 4])
def test_compress_matches_oracle(kv, act, r):
    lens = [64 * 4 * 3 + 21, 517, 5] if r == 4 else [300, 129, 64]
    cache, raw, P = _compress_case(kv, act, r, lens)
    for b, L in enumerate(lens):
        K, V, Z = (to64(t) for t in raw[0][b])
        kb, vb, ki, bk, bv, bi = oracle_entries(K, V, Z, r, to64(P))
        n = L // r
        if n == 0:
            continue
        sc = kv == "fp8"
        _check_stored(cache, cache.kbar[0], cache.kbar_scale[0] if sc else None, b, n, kb, bk, kv, f"kbar seq {b}")
        _check_stored(cache, cache.vbar[0], cache.vbar_scale[0] if sc else None, b, n, vb, bv, kv, f"vbar seq {b}")
        _check_stored(cache, cache.kidx, cache.kidx_scale, b, n, ki, bi, kv, f"kidx seq {b}")
        # ring holds the last R raw rows, bit for bit
        R = cache.cfg.ring_rows
        rows = np.arange(max(0, L - R), L)
        assert torch.equal(cache.ring_k[0][b, rows % R].cpu(), raw[0][b][0][rows])
        assert torch.equal(cache.ring_v[0][b, rows % R].cpu(), raw[0][b][1][rows])
        assert cache.seq_len(0, b) == L
    assert cache.read_errors() == 0


@pytest.mark.parametrize("kv,act", DT_CASES)
def test_compress_incremental_equals_bulk(kv, act):
    lens = [64 * 4 * 2 + 13, 301]
    bulk, _, _ = _compress_case(kv, act, 4, lens, seed=9)
    inc, _, _ = _compress_case(kv, act, 4, lens, seed=9, chunks=[1, 3, 2, 1, 7, 64, 1, 1, 200, 5])
    for b, L in enumerate(lens):
        n = L // 4
        for pa, pb in ((bulk.kbar[0], inc.kbar[0]), (bulk.vbar[0], inc.vbar[0]), (bulk.kidx, inc.kidx)):
            assert torch.equal(bulk.logical(pa, b, n).cpu(), inc.logical(pb, b, n).cpu())
        if kv == "fp8":
            for sa, sb in ((bulk.kbar_scale[0], inc.kbar_scale[0]), (bulk.kidx_scale, inc.kidx_scale)):
                assert torch.equal(bulk.logical_scales(sa, b, n).cpu(), inc.logical_scales(sb, b, n).cpu())
        R = bulk.cfg.ring_rows
        assert torch.equal(bulk.ring_k[0][b].cpu(), inc.ring_k[0][b].cpu())
        assert torch.equal(bulk.block_stage[0][b, :, : (L % 4)].cpu(), inc.block_stage[0][b, :, : (L % 4)].cpu())


# --------------------------------------------------------------------------- index (isolated)

def _index_case(kv, act, lens, k, q_pos=None, seed=11, h_i=4, dup_keys=False, chunk=None, exact=False):
    r = 4
    max_pages = max(L // r for L in lens) // 64 + 2
    nq = len(lens) if chunk is None else chunk[1]
    cache = make_cache(seed, ratio=r, q_heads=16, idx_heads=h_i, window=0, ring_rows=8, max_seqs=len(lens),
                       max_pages_per_seq=max_pages, pool_pages=len(lens) * max_pages + 1, kv_dtype=kv, act_dtype=act,
                       max_queries=nq, max_k=k)
    keys = []
    for b, L in enumerate(lens):
        n = L // r
        if dup_keys and n:
            # many exact ties: every indexer key repeats one of 7 rows
            x = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_KI, 0, b), 0, 7, 64).double().numpy()
            x = x[np.arange(n) % 7]
            vals, rawv = O.store(x, kv)
            from gpu_helpers import store_raw_to_torch, write_logical, write_scales
            write_logical(cache, cache.kidx, b, store_raw_to_torch(rawv, kv))
            if kv == "fp8":
                write_scales(cache, cache.kidx_scale, b, rawv[1])
            keys.append(vals)
        else:
            keys.append(fill_index_keys(cache, seed, b, n))
        B.csa_seq_set_len(cache.handle, 0, b, L)
    if chunk is None:
        q_seq = list(range(len(lens)))
        q_pos = q_pos or [L - 1 for L in lens]
    else:
        q_seq = [chunk[0]] * chunk[1]
        q_pos = [lens[chunk[0]] - chunk[1] + i for i in range(chunk[1])]
    n_q = len(q_seq)
    qi = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_QI), 0, n_q * h_i, 64, dtype=TORCH_ACT[act]).view(n_q, h_i, 64)
    w = Sy.uniform_rows(seed, Sy.stream_id(Sy.KIND_W), 0, n_q, h_i)
    T = cache.index_topk(q_seq, q_pos, qi.cuda(), w.cuda(), k).cpu().numpy()
    assert cache.read_errors() & ~B.ERR_FALLBACK == 0
    q64, w64 = to64(qi), to64(w)
    for i in range(n_q):
        N = O.visible_entries(q_pos[i], r)
        s = O.index_scores(q64[i], w64[i], keys[q_seq[i]][:N])
        To = O.topk(s, k)
        if exact:
            assert T[i].tolist() == To.tolist(), f"query {i}: exact ties must resolve to the lower index"
        ok, msg = topk_matches(T[i], To, s)
        assert ok, f"query {i} (seq {q_seq[i]}, pos {q_pos[i]}, N={N}): {msg}"
    return cache


@pytest.mark.parametrize("kv,act", DT_CASES)
def test_index_decode_matches_oracle(kv, act):
    # ragged visible counts: several scan tiles, partial pages, N < k, N == k, N == 0
    _index_case(kv, act, lens=[4096, 4 * 3000 + 3, 4 * 70, 4 * 64, 2, 4 * 20000 + 1], k=64)


@pytest.mark.parametrize("kv,act", [("bf16", "bf16"), ("fp8", "bf16")])
@pytest.mark.parametrize("k", [512, 1024, 2048])
def test_index_decode_large_k(kv, act, k):
    _index_case(kv, act, lens=[4 * 65536, 4 * 9000 + 2, 4 * 3 * k], k=k)


@pytest.mark.parametrize("kv,act", [("bf16", "bf16"), ("fp8", "bf16")])
@pytest.mark.parametrize("n,k", [(300000, 16), (50000, 64)])
def test_index_decode_wide_groups(kv, act, n, k):
    """Many entries and a small k: threshold groups of 256 entries (two scan
    waves, combined through LDS) and of 128 entries (both pages of a wave)."""
    _index_case(kv, act, lens=[4 * n + 3, 4 * (n // 4)], k=k)


@pytest.mark.parametrize("h_i", [1, 2, 3])
def test_index_fewer_heads(h_i):
    _index_case("bf16", "bf16", lens=[4 * 5000, 4 * 777], k=100, h_i=h_i)


@pytest.mark.parametrize("kv,act", DT_CASES)
def test_index_exact_ties_go_to_lower_index(kv, act):
    _index_case(kv, act, lens=[4 * 3000, 4 * 200], k=96, dup_keys=True, exact=True)
    # rows past the one-workgroup limit go through scan, filter and final
    _index_case(kv, act, lens=[4 * 9000, 4 * 5000], k=96, dup_keys=True, exact=True)


@pytest.mark.parametrize("kv,act", DT_CASES)
def test_index_chunk_matches_oracle(kv, act):
    # a 300-token prefill chunk at the end of a 12,000-token sequence (causal over its own entries)
    _index_case(kv, act, lens=[12000, 40], k=256, chunk=(0, 300))


def test_index_chunk_short_context():
    # early chunk queries see fewer than k entries
    _index_case("bf16", "bf16", lens=[1000], k=200, chunk=(0, 600))
    _index_case("fp8", "bf16", lens=[4 * 5000 + 2], k=1024, chunk=(0, 257))


# --------------------------------------------------------------------------- attend (isolated)

def _attend_case(kv, act, lens, k, W, seed=21, n_layers=1, H=64, chunk=None, topk_mode="random", ones_col=False,
                 swa="", swa_start=None):
    r = 4
    max_pages = max(L // r for L in lens) // 64 + 2
    n_q = len(lens) if chunk is None else chunk[1]
    R = max(W, r, 8) if chunk is None else max(W, r) + chunk[1]
    cache = make_cache(seed, ratio=r, q_heads=H, window=W, ring_rows=R, n_layers=n_layers, max_seqs=len(lens),
                       max_pages_per_seq=max_pages, pool_pages=len(lens) * max_pages + 2, kv_dtype=kv, act_dtype=act,
                       max_queries=n_q, max_k=max(k, 1), swa_dtype=swa)
    starts = swa_start or [0] * len(lens)
    for b, s0 in enumerate(starts):
        cache.set_swa_start(b, s0)
    kvs, rings = {}, {}
    for layer in range(n_layers):
        for b, L in enumerate(lens):
            kvs[layer, b] = fill_main_kv(cache, seed, layer, b, L // r)
            rings[layer, b] = fill_ring(cache, seed, layer, b, L)
            if ones_col:
                kvs[layer, b][1][:, 5] = 1.0
                rings[layer, b][1][:, 5] = 1.0
            B.csa_seq_set_len(cache.handle, layer, b, L)
    if ones_col:
        # rewrite column 5 of every V pool row / ring row to exactly 1.0 on the device
        for layer in range(n_layers):
            if kv == "fp8":
                # 1.0 is not representable under an amax/448 scale in general: set code so value == scale*code
                pass
            else:
                cache.vbar[layer][:, :, 5] = 1.0
            cache.ring_v[layer][:, :, 5] = 1.0
    if chunk is None:
        q_seq = list(range(len(lens)))
        q_pos = [L - 1 for L in lens]
    else:
        q_seq = [chunk[0]] * chunk[1]
        q_pos = [lens[chunk[0]] - chunk[1] + i for i in range(chunk[1])]
    rng = np.random.default_rng(seed)
    T = np.full((n_q, max(k, 1)), -1, dtype=np.int32)
    for i in range(n_q):
        N = O.visible_entries(q_pos[i], r)
        m = min(k, N)
        if topk_mode == "random" and m > 0:
            sel = np.sort(rng.choice(N, size=m, replace=False))
            T[i, :m] = sel
    Tt = torch.from_numpy(T).cuda()
    scale = 1.0 / math.sqrt(128)
    q = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_Q), 0, n_q * H, 128, dtype=TORCH_ACT[act]).view(n_q, H, 128)
    q64 = to64(q)
    for layer in range(n_layers):
        out = cache.attend(layer, q_seq, q_pos, q.cuda(), Tt, k, scale)
        got = to64(out)
        assert cache.read_errors() == 0
        for i in range(n_q):
            kb, vb = kvs[layer, q_seq[i]]
            K, V = rings[layer, q_seq[i]]
            ref = O.attend_step(q64[i], T[i, :k], q_pos[i], W, scale, kb, vb, K, V, starts[q_seq[i]])
            err = max_abs(got[i], ref)
            assert err <= TOL[act], f"layer {layer} query {i}: max-abs {err}"
            if ones_col and kv != "fp8" and swa != "fp8":
                assert np.max(np.abs(got[i][:, 5] - 1.0)) <= (1e-5 if act == "f32" else 2 ** -8)
    return cache


@pytest.mark.parametrize("kv,act", DT_CASES)
def test_attend_decode_matches_oracle(kv, act):
    _attend_case(kv, act, lens=[4096, 4 * 3000 + 3, 300, 131], k=256, W=128)


@pytest.mark.parametrize("kv,act", DT_CASES)
@pytest.mark.parametrize("H", [16, 32, 128])
def test_attend_head_counts(kv, act, H):
    _attend_case(kv, act, lens=[4 * 700, 999], k=70, W=100, H=H)


@pytest.mark.parametrize("kv,act,k", [("bf16", "bf16", 256), ("fp8", "bf16", 1024), ("f32", "f32", 256)])
def test_attend_many_pairs_merge(kv, act, k):
    """16 queries x 64 heads = 1,024 (query, head) pairs with 6 or 18 splits
    each: the merge kernel that takes 8 pairs per workgroup."""
    _attend_case(kv, act, lens=[4 * (1100 + 37 * i) + i % 4 for i in range(16)], k=k, W=128)


def test_attend_merge_many_splits():
    """A decode query with a 4,096-row window: 80 splits of 64 keys, the merge
    that stages each split's (m, l) through LDS."""
    _attend_case("bf16", "bf16", lens=[4 * 5000 + 1], k=1024, W=4096, H=16)


@pytest.mark.parametrize("k,W", [(0, 128), (64, 0), (1, 1), (1024, 128), (33, 200)])
def test_attend_branch_edges(k, W):
    _attend_case("bf16", "bf16", lens=[4 * 5000, 4 * 20 + 3, 17], k=k, W=W)


@pytest.mark.parametrize("kv,act", DT_CASES)
def test_attend_chunk_matches_oracle(kv, act):
    _attend_case(kv, act, lens=[4 * 2000, 64], k=128, W=64, chunk=(0, 150))


@pytest.mark.parametrize("kv,act", [("f32", "f32"), ("bf16", "bf16")])
def test_attend_weights_sum_to_one(kv, act):
    _attend_case(kv, act, lens=[4 * 900, 4 * 50], k=200, W=64, ones_col=True)


def test_attend_reuse_group_two_layers():
    _attend_case("fp8", "bf16", lens=[4 * 4000, 4 * 100], k=512, W=128, n_layers=2)


# --------------------------------------------------------------------------- whole step

def _chain(kv, act, lens, k, W, seed=31, n_layers=1, H=16, r=4, dense=False, swa=""):
    """Compress -> index -> attend on the GPU, and the same on the oracle, from the same raw rows."""
    max_pages = max(1, max(L // r for L in lens) // 64 + 2)
    R = max(W, r, 8)
    cache = make_cache(seed, ratio=r, q_heads=H, window=W, ring_rows=R, n_layers=n_layers, max_seqs=len(lens),
                       max_pages_per_seq=max_pages, pool_pages=len(lens) * max_pages + 5, kv_dtype=kv,
                       act_dtype=act, max_queries=len(lens), max_k=k, swa_dtype=swa)
    P = Sy.proj_matrix(seed, 128, 64)
    raws = {}
    for layer in range(n_layers):
        ks, vs, zs = [], [], []
        for b, L in enumerate(lens):
            ks.append(raw_rows(seed, Sy.KIND_K, layer, b, 0, L, act))
            vs.append(raw_rows(seed, Sy.KIND_V, layer, b, 0, L, act))
            zs.append(raw_rows(seed, Sy.KIND_Z, layer, b, 0, L, act))
            raws[layer, b] = (to64(ks[-1]), to64(vs[-1]), to64(zs[-1]))
        cache.compress(layer, list(range(len(lens))), lens, torch.cat(ks).cuda(), torch.cat(vs).cuda(),
                       torch.cat(zs).cuda(), P.cuda() if layer == 0 else None)
    n_q = len(lens)
    q_seq, q_pos = list(range(n_q)), [L - 1 for L in lens]
    qi = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_QI), 0, n_q * 4, 64, dtype=TORCH_ACT[act]).view(n_q, 4, 64)
    w = Sy.uniform_rows(seed, Sy.stream_id(Sy.KIND_W), 0, n_q, 4)
    T = cache.index_topk(q_seq, q_pos, qi.cuda(), w.cuda(), k)
    scale = 1.0 / math.sqrt(128)
    outs = []
    for layer in range(n_layers):
        q = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_Q, layer), 0, n_q * H, 128, dtype=TORCH_ACT[act]).view(n_q, H, 128)
        outs.append((q, to64(cache.attend(layer, q_seq, q_pos, q.cuda(), T, k, scale))))
    Tg = T.cpu().numpy()
    assert cache.read_errors() == 0
    # oracle chain
    P64 = to64(P)
    for b, L in enumerate(lens):
        comp = {}
        for layer in range(n_layers):
            K, V, Z = raws[layer, b]
            kb, vb, ki, _, _, bi = oracle_entries(K, V, Z, r, P64 if layer == 0 else None)
            comp[layer] = (O.store(kb, kv)[0], O.store(vb, kv)[0], O.store_ring_rows(K, swa)[0],
                           O.store_ring_rows(V, swa)[0])
            if layer == 0:
                kis = O.store(ki, "fp8" if kv == "fp4" else kv)[0]   # fp4 caches keep fp8 indexer keys
                ki0, bi0 = ki, bi
        layers = [dict(q=to64(outs[l][0][b]), W=W, scale=scale, kbar=comp[l][0], vbar=comp[l][1], rawk=comp[l][2],
                       rawv=comp[l][3]) for l in range(n_layers)]
        To, oo = O.decode_step(to64(qi[b]), to64(w[b]), kis, r, k, L - 1, layers)
        N = O.visible_entries(L - 1, r)
        check_topk_chain(Tg[b], to64(qi[b]), to64(w[b]), ki0, bi0, kv, N, k, f"seq {b}")
        for l in range(n_layers):
            err = max_abs(outs[l][1][b], oo[l])
            assert err <= TOL[act], f"seq {b} layer {l}: max-abs {err}"


def test_step_decode_fp32_small_config():
    """The 4,096-token fp32 decode configuration: B = 1, r = 4, 16 heads, k = 64, W = 128."""
    _chain("f32", "f32", [4096], k=64, W=128, H=16)


@pytest.mark.parametrize("kv,act", [("bf16", "bf16"), ("fp8", "bf16")])
def test_step_decode_chain(kv, act):
    _chain(kv, act, [4 * 3000 + 2, 4100, 777], k=256, W=128, H=64, n_layers=2)


def test_ratio1_all_selected_no_window_is_causal_attention():
    """r = 1, k >= visible, W = 0 reduces to dense causal attention (torch SDPA)."""
    L, H = 200, 16
    cache = make_cache(41, ratio=1, q_heads=H, window=0, ring_rows=8, max_seqs=1, max_pages_per_seq=4,
                       pool_pages=5, kv_dtype="f32", act_dtype="f32", max_queries=L, max_k=256)
    K = raw_rows(41, Sy.KIND_K, 0, 0, 0, L, "f32")
    V = raw_rows(41, Sy.KIND_V, 0, 0, 0, L, "f32")
    Z = raw_rows(41, Sy.KIND_Z, 0, 0, 0, L, "f32")
    P = Sy.proj_matrix(41, 128, 64)
    cache.compress(0, [0], [L], K.cuda(), V.cuda(), Z.cuda(), P.cuda())
    qi = Sy.normal_rows(41, Sy.stream_id(Sy.KIND_QI), 0, L * 4, 64).view(L, 4, 64)
    w = Sy.uniform_rows(41, Sy.stream_id(Sy.KIND_W), 0, L, 4)
    T = cache.index_topk([0] * L, list(range(L)), qi.cuda(), w.cuda(), 256)
    Tc = T.cpu()
    for t in range(L):
        assert sorted(x for x in Tc[t].tolist() if x >= 0) == list(range(t + 1))
    q = Sy.normal_rows(41, Sy.stream_id(Sy.KIND_Q), 0, L * H, 128).view(L, H, 128)
    out = cache.attend(0, [0] * L, list(range(L)), q.cuda(), T, 256, 1 / math.sqrt(128)).cpu()
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.permute(1, 0, 2).double().unsqueeze(0), K.double()[None, None].expand(1, H, L, 128),
        V.double()[None, None].expand(1, H, L, 128), is_causal=True, scale=1 / math.sqrt(128))[0].permute(1, 0, 2)
    assert max_abs(out.double().numpy(), ref.numpy()) <= 2e-3


def test_page_placement_does_not_change_results():
    """Same logical contents under two physical page orders give bit-identical outputs."""
    outs = []
    for seed in (51, 52):
        cache = make_cache(seed, ratio=4, q_heads=64, window=128, ring_rows=128, max_seqs=2, max_pages_per_seq=40,
                           pool_pages=90, kv_dtype="fp8", act_dtype="bf16", max_queries=2, max_k=512)
        for b, L in enumerate([4 * 2500, 4 * 1000]):
            fill_main_kv(cache, 7, 0, b, L // 4)
            fill_index_keys(cache, 7, b, L // 4)
            fill_ring(cache, 7, 0, b, L)
            B.csa_seq_set_len(cache.handle, 0, b, L)
        qi = Sy.normal_rows(7, Sy.stream_id(Sy.KIND_QI), 0, 8, 64, dtype=torch.bfloat16).view(2, 4, 64).cuda()
        w = Sy.uniform_rows(7, Sy.stream_id(Sy.KIND_W), 0, 2, 4).cuda()
        q = Sy.normal_rows(7, Sy.stream_id(Sy.KIND_Q), 0, 128, 128, dtype=torch.bfloat16).view(2, 64, 128).cuda()
        T = cache.index_topk([0, 1], [9999, 3999], qi, w, 512)
        o = cache.attend(0, [0, 1], [9999, 3999], q, T, 512, 0.088)
        outs.append((T.cpu(), o.cpu()))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])


def test_pool_at_the_32bit_offset_limit():
    """Attention gathers address a pool with 32-bit byte offsets. A pool just
    under the 0xfffff000-byte limit, holding the sequences' pages at its top
    end (row offsets above 2^31 and up to the limit), gives the same Top-K and
    bit-identical outputs as the same contents at the start of a small pool."""
    big = 0xFFFFF000 // (64 * 128)        # fp8 rows of 128 B
    lens = [4 * 2500, 4 * 1000]
    outs = []
    for pool_pages, top in ((90, False), (big, True)):
        spec = CacheSpec(ratio=4, q_heads=64, window=128, ring_rows=128, max_seqs=2, max_pages_per_seq=40,
                         pool_pages=pool_pages, kv_dtype="fp8", act_dtype="bf16", max_queries=2, max_k=512)
        first = pool_pages - 80 if top else 0
        bt = torch.arange(first, first + 80, dtype=torch.int32).flip(0).view(2, 40).cuda()
        cache = CsaCache(spec, "cuda", block_table=bt)
        assert B.csa_buffer_sizes_for(spec.config()).kv_pool <= 0xFFFFF000
        for b, L in enumerate(lens):
            fill_main_kv(cache, 7, 0, b, L // 4)
            fill_index_keys(cache, 7, b, L // 4)
            fill_ring(cache, 7, 0, b, L)
            B.csa_seq_set_len(cache.handle, 0, b, L)
        qi = Sy.normal_rows(7, Sy.stream_id(Sy.KIND_QI), 0, 8, 64, dtype=torch.bfloat16).view(2, 4, 64).cuda()
        w = Sy.uniform_rows(7, Sy.stream_id(Sy.KIND_W), 0, 2, 4).cuda()
        q = Sy.normal_rows(7, Sy.stream_id(Sy.KIND_Q), 0, 128, 128, dtype=torch.bfloat16).view(2, 64, 128).cuda()
        T = cache.index_topk([0, 1], [lens[0] - 1, lens[1] - 1], qi, w, 512)
        o = cache.attend(0, [0, 1], [lens[0] - 1, lens[1] - 1], q, T, 512, 0.088)
        assert cache.read_errors() == 0
        outs.append((T.cpu(), o.cpu()))
        cache.close()
        del cache
        torch.cuda.empty_cache()
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])


def test_bad_page_ids_are_flagged_not_faulting():
    cache = make_cache(61, ratio=4, q_heads=16, window=16, ring_rows=16, max_seqs=1, max_pages_per_seq=8,
                       pool_pages=10, kv_dtype="bf16", act_dtype="bf16", max_queries=1, max_k=64)
    fill_index_keys(cache, 61, 0, 400)
    fill_main_kv(cache, 61, 0, 0, 400)
    fill_ring(cache, 61, 0, 0, 1600)
    B.csa_seq_set_len(cache.handle, 0, 0, 1600)
    cache.block_table[0, 3] = 1000      # outside the 10-page pool
    cache.block_table[0, 5] = -7
    qi = torch.zeros((1, 4, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.ones((1, 4), device="cuda")
    T = cache.index_topk([0], [1599], qi, w, 64)
    q = torch.zeros((1, 16, 128), dtype=torch.bfloat16, device="cuda")
    Tbad = torch.arange(64, dtype=torch.int32, device="cuda").view(1, 64) * 6
    cache.attend(0, [0], [1599], q, Tbad, 64, 0.1)
    flags = cache.read_errors()
    assert flags & B.ERR_PAGE
    Tvis = torch.full((1, 64), 500, dtype=torch.int32, device="cuda")   # 500 >= 400 visible entries
    cache.block_table[0, 3] = 3
    cache.block_table[0, 5] = 5
    cache.attend(0, [0], [1599], q, Tvis, 64, 0.1)
    assert cache.read_errors() & B.ERR_TOPK


@pytest.mark.parametrize("n_tok,n", [(1, 16000), (8, 16000), (1, 2000)])
def test_bad_pages_lose_the_exact_fallback(n_tok, n):
    """All-zero indexer queries tie every real entry at score 0, which sends the
    decode select (n_tok = 1; a short row, n = 2,000, in the one-workgroup
    kernel) and the chunk select (n_tok = 8) to the exact fallback. There the
    entries of pages whose ids lie outside the pool score below every real
    entry, so the Top-K is the lowest-index real entries and skips those pages."""
    r, k = 4, 64
    L = r * n
    cache = make_cache(62, ratio=r, q_heads=16, window=16, ring_rows=32, max_seqs=1, max_pages_per_seq=n // 64 + 2,
                       pool_pages=n // 64 + 4, kv_dtype="bf16", act_dtype="bf16", max_queries=n_tok, max_k=k)
    fill_index_keys(cache, 62, 0, n)
    B.csa_seq_set_len(cache.handle, 0, 0, L)
    cache.block_table[0, 0] = 1000      # outside the pool
    cache.block_table[0, 2] = -7
    qi = torch.zeros((n_tok, 4, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.ones((n_tok, 4), device="cuda")
    T = cache.index_topk([0] * n_tok, list(range(L - n_tok, L)), qi, w, k).cpu().numpy()
    flags = cache.read_errors()
    assert flags & B.ERR_PAGE and flags & B.ERR_FALLBACK, flags
    want = np.arange(64, 64 + k, dtype=np.int32)     # page 1, the first page with a valid id
    for i in range(n_tok):
        assert np.array_equal(T[i], want), f"query {i}: {T[i][:8]}..."


def test_graph_replay_matches_eager():
    """The decode step captured in a HIP graph: every replay, with eager work in
    between, reproduces the eager outputs bit for bit."""
    cache = make_cache(71, ratio=4, q_heads=64, window=128, ring_rows=128, max_seqs=3, max_pages_per_seq=40,
                       pool_pages=121, kv_dtype="fp8", act_dtype="bf16", max_queries=3, max_k=512)
    lens = [4 * 2500, 4 * 1000 + 3, 4 * 300]
    for b, L in enumerate(lens):
        fill_main_kv(cache, 71, 0, b, L // 4)
        fill_index_keys(cache, 71, b, L // 4)
        fill_ring(cache, 71, 0, b, L)
        B.csa_seq_set_len(cache.handle, 0, b, L)
    q_seq, q_pos = [0, 1, 2], [L - 1 for L in lens]
    qi = Sy.normal_rows(71, Sy.stream_id(Sy.KIND_QI), 0, 12, 64, dtype=torch.bfloat16).view(3, 4, 64).cuda()
    w = Sy.uniform_rows(71, Sy.stream_id(Sy.KIND_W), 0, 3, 4).cuda()
    q = Sy.normal_rows(71, Sy.stream_id(Sy.KIND_Q), 0, 192, 128, dtype=torch.bfloat16).view(3, 64, 128).cuda()
    T = torch.empty((3, 512), dtype=torch.int32, device="cuda")
    out = torch.empty((3, 64, 128), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.current_stream()
    B.csa_index_topk(cache.handle, q_seq, q_pos, qi, w, 512, T, s)
    B.csa_attend(cache.handle, 0, q_seq, q_pos, q, T, 512, 0.088, out, s)
    torch.cuda.synchronize()
    T_ref, out_ref = T.clone(), out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream()
        B.csa_index_topk(cache.handle, q_seq, q_pos, qi, w, 512, T, cs)
        B.csa_attend(cache.handle, 0, q_seq, q_pos, q, T, 512, 0.088, out, cs)
    for rep in range(4):
        T.zero_()
        out.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()       # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(T, T_ref), f"replay {rep}: Top-K differs"
        assert torch.equal(out, out_ref), f"replay {rep}: output differs"
        del junk
    assert cache.read_errors() == 0


@pytest.mark.parametrize("kv,swa", [("fp8", "fp8"), ("fp4", "")])
def test_graph_replay_hierarchical_step_matches_eager(kv, swa):
    """Full layer with a candidate pool, a Reindex layer, attention of both
    (fp4 K/V, or fp8 pages with an fp8 ring) and a window-ring rewrite, captured
    in one HIP graph: every replay reproduces the eager outputs bit for bit."""
    cache = make_cache(73, ratio=4, q_heads=64, window=128, ring_rows=128, n_layers=2, max_seqs=3,
                       max_pages_per_seq=40, pool_pages=121, kv_dtype=kv, act_dtype="bf16", max_queries=3, max_k=512,
                       swa_dtype=swa)
    lens = [4 * 2500, 4 * 1000 + 3, 4 * 300]
    for b, L in enumerate(lens):
        for layer in range(2):
            fill_main_kv(cache, 73, layer, b, L // 4)
            fill_ring(cache, 73, layer, b, L)
            B.csa_seq_set_len(cache.handle, layer, b, L)
        fill_index_keys(cache, 73, b, L // 4)
    q_seq, q_pos = [0, 1, 2], [L - 1 for L in lens]
    qi = [Sy.normal_rows(73, Sy.stream_id(Sy.KIND_QI, l), 0, 12, 64, dtype=torch.bfloat16).view(3, 4, 64).cuda() for l in range(2)]
    w = [Sy.uniform_rows(73, Sy.stream_id(Sy.KIND_W, l), 0, 3, 4).cuda() for l in range(2)]
    q = [Sy.normal_rows(73, Sy.stream_id(Sy.KIND_Q, l), 0, 192, 128, dtype=torch.bfloat16).view(3, 64, 128).cuda() for l in range(2)]
    newk = raw_rows(74, Sy.KIND_K, 0, 0, 0, 8, "bf16").cuda()
    T = [torch.empty((3, 512), dtype=torch.int32, device="cuda") for _ in range(2)]
    P = torch.empty((3, 64), dtype=torch.int32, device="cuda")
    out = [torch.empty((3, 64, 128), dtype=torch.bfloat16, device="cuda") for _ in range(2)]

    def step(st):
        B.csa_ring_write(cache.handle, 1, [0], [lens[0] - 8], [8], newk, newk, st)
        B.csa_index_topk_pool(cache.handle, q_seq, q_pos, qi[0], w[0], 512, T[0], 64, P, st)
        B.csa_index_reindex(cache.handle, q_seq, q_pos, qi[1], w[1], 64, P, 512, T[1], st)
        for l in range(2):
            B.csa_attend(cache.handle, l, q_seq, q_pos, q[l], T[l], 512, 0.088, out[l], st)
    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    refs = [x.clone() for x in (T[0], T[1], P, out[0], out[1])]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    for rep in range(4):
        for x in (T[0], T[1], P, out[0], out[1]):
            x.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()       # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for x, r in zip((T[0], T[1], P, out[0], out[1]), refs):
            assert torch.equal(x, r), f"replay {rep} differs"
        del junk
    assert cache.read_errors() & ~B.ERR_FALLBACK == 0


@pytest.mark.parametrize("kv,act", DT_CASES)
def test_index_chunk_threshold_fallback_is_exact(kv, act):
    """Adversarial prefill chunk: only the entries the threshold pass samples
    (every 16th) carry signal, so the sampled threshold admits fewer than k
    candidates; the exact full-row fallback must still return the oracle's Top-K."""
    from gpu_helpers import store_raw_to_torch, write_logical, write_scales
    r, L, k, n_tok, seed = 4, 4 * 6000, 512, 96, 13
    cache = make_cache(seed, ratio=r, q_heads=16, window=0, ring_rows=8, max_seqs=1,
                       max_pages_per_seq=L // r // 64 + 2, pool_pages=L // r // 64 + 3, kv_dtype=kv,
                       act_dtype=act, max_queries=n_tok, max_k=k)
    n = L // r
    x = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_KI, 0, 0), 0, n, 64).double().numpy()
    mask = (np.arange(n) % 16) == 15
    x[~mask] *= 1e-3
    vals, raw = O.store(x, kv)
    write_logical(cache, cache.kidx, 0, store_raw_to_torch(raw, kv))
    if kv == "fp8":
        write_scales(cache, cache.kidx_scale, 0, raw[1])
    B.csa_seq_set_len(cache.handle, 0, 0, L)
    q_pos = list(range(L - n_tok, L))
    qi = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_QI), 0, n_tok * 4, 64, dtype=TORCH_ACT[act]).view(n_tok, 4, 64)
    w = Sy.uniform_rows(seed, Sy.stream_id(Sy.KIND_W), 0, n_tok, 4)
    T = cache.index_topk([0] * n_tok, q_pos, qi.cuda(), w.cuda(), k).cpu().numpy()
    flags = cache.read_errors()
    assert flags & B.ERR_FALLBACK, "the adversarial case should take the exact fallback"
    assert flags & ~B.ERR_FALLBACK == 0
    q64, w64 = to64(qi), to64(w)
    for i in range(0, n_tok, 7):
        N = O.visible_entries(q_pos[i], r)
        s = O.index_scores(q64[i], w64[i], vals[:N])
        ok, msg = topk_matches(T[i], O.topk(s, k), s)
        assert ok, f"token {i}: {msg}"


@pytest.mark.parametrize("kv,act", [("fp8", "bf16"), ("f32", "f32")])
def test_index_decode_candidates_crowd_one_slice(kv, act):
    """The decode final select reads every filter slice's first slots together
    with the slice counts; a slice with more candidates than those slots sends
    the query down the two-step path (counts, then candidates). Keys of one
    4,096-entry slice are scaled up so that nearly all of the Top-512 (and so
    hundreds of candidates) sit in it; the result must still be the oracle's
    Top-K, without the exact full-row fallback."""
    from gpu_helpers import store_raw_to_torch, write_logical, write_scales
    r, k, seed = 4, 512, 19
    lens = [4 * 65536, 4 * 40000 + 1]
    max_pages = max(L // r for L in lens) // 64 + 2
    cache = make_cache(seed, ratio=r, q_heads=16, idx_heads=4, window=0, ring_rows=8, max_seqs=len(lens),
                       max_pages_per_seq=max_pages, pool_pages=len(lens) * max_pages + 1, kv_dtype=kv,
                       act_dtype=act, max_queries=len(lens), max_k=k)
    keys = []
    for b, L in enumerate(lens):
        n = L // r
        x = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_KI, 0, b), 0, n, 64).double().numpy()
        x[3 * 4096: 4 * 4096] *= 3.0           # slice 3 holds nearly every large score
        vals, rawv = O.store(x, kv)
        write_logical(cache, cache.kidx, b, store_raw_to_torch(rawv, kv))
        if kv == "fp8":
            write_scales(cache, cache.kidx_scale, b, rawv[1])
        keys.append(vals)
        B.csa_seq_set_len(cache.handle, 0, b, L)
    q_seq, q_pos = [0, 1], [L - 1 for L in lens]
    qi = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_QI), 0, 2 * 4, 64, dtype=TORCH_ACT[act]).view(2, 4, 64)
    w = Sy.uniform_rows(seed, Sy.stream_id(Sy.KIND_W), 0, 2, 4)
    T = cache.index_topk(q_seq, q_pos, qi.cuda(), w.cuda(), k).cpu().numpy()
    assert cache.read_errors() == 0, "no fallback and no error expected"
    q64, w64 = to64(qi), to64(w)
    for i in range(2):
        N = O.visible_entries(q_pos[i], r)
        s = O.index_scores(q64[i], w64[i], keys[i][:N])
        To = O.topk(s, k)
        in_slice = int(np.sum((To >= 3 * 4096) & (To < 4 * 4096)))
        assert in_slice > 64, f"query {i}: only {in_slice} of the Top-{k} in the crowded slice"
        ok, msg = topk_matches(T[i], To, s)
        assert ok, f"query {i}: {msg}"


def test_index_chunk_exact_ties():
    _index_case("bf16", "bf16", lens=[4 * 3000], k=96, dup_keys=True, exact=True, chunk=(0, 130))


# --------------------------------------------------------------------------- ragged serving step

def test_serving_steps_ragged_paged_fp8():
    """Ragged requests (log-uniform lengths) on a shared paged fp8 pool with a
    shuffled free list: bulk build, then steps that append one token to every
    request (compress re-quantises open pages), index and attend; the final step
    is compared with the oracle run on each request's full raw rows."""
    seed, r, k, W, H = 17, 4, 128, 32, 16
    lens = Sy.log_uniform_lengths(seed, 8, 1024, 16384)
    steps = 3
    final = [L + steps for L in lens]
    pages = [(L // r + 63) // 64 + 1 for L in final]
    max_pages = max(pages)
    pool = sum(pages) + 3
    perm = Sy.permutation(seed, pool, salt=11)
    bt = torch.full((len(lens), max_pages), -1, dtype=torch.int32)
    off = 0
    for b, p in enumerate(pages):
        bt[b, :p] = torch.tensor(perm[off:off + p], dtype=torch.int32)
        off += p
    from compressed_sparse_attention_csa_amd.cache import CacheSpec, CsaCache
    spec = CacheSpec(ratio=r, q_heads=H, idx_heads=4, window=W, ring_rows=W, n_layers=1, max_seqs=len(lens),
                     max_pages_per_seq=max_pages, pool_pages=pool, kv_dtype="fp8", act_dtype="bf16",
                     max_queries=len(lens), max_k=k)
    cache = CsaCache(spec, "cuda", block_table=bt.cuda())
    P = Sy.proj_matrix(seed, 128, 64)
    raw = [[raw_rows(seed, kind, 0, b, 0, final[b], "bf16") for kind in (Sy.KIND_K, Sy.KIND_V, Sy.KIND_Z)]
           for b in range(len(lens))]
    ids = list(range(len(lens)))
    cache.compress(0, ids, lens, *(torch.cat([raw[b][a][:lens[b]] for b in ids]).cuda() for a in range(3)), P.cuda())
    scale = 1 / math.sqrt(128)
    for st in range(steps):
        cur = [L + st for L in lens]
        cache.compress(0, ids, [1] * len(ids), *(torch.cat([raw[b][a][cur[b]:cur[b] + 1] for b in ids]).cuda()
                                                  for a in range(3)), P.cuda())
        qpos = [c for c in cur]
        qi = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_QI, 0, st), 0, len(ids) * 4, 64, dtype=torch.bfloat16).view(-1, 4, 64)
        w = Sy.uniform_rows(seed, Sy.stream_id(Sy.KIND_W, 0, st), 0, len(ids), 4)
        q = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_Q, 0, st), 0, len(ids) * H, 128, dtype=torch.bfloat16).view(-1, H, 128)
        T = cache.index_topk(ids, qpos, qi.cuda(), w.cuda(), k)
        out = to64(cache.attend(0, ids, qpos, q.cuda(), T, k, scale))
    assert cache.read_errors() == 0
    Tg = T.cpu().numpy()
    for b in ids:
        K, V, Z = (to64(t) for t in raw[b])
        kb, vb, ki, bk, bv, bi = oracle_entries(K, V, Z, r, to64(P))
        kis, kbs, vbs = O.store(ki, "fp8")[0], O.store(kb, "fp8")[0], O.store(vb, "fp8")[0]
        t = final[b] - 1
        N = O.visible_entries(t, r)
        s = check_topk_chain(Tg[b], to64(qi[b]), to64(w[b]), ki, bi, "fp8", N, k, f"request {b}")
        To = O.topk(s, k)
        ref = O.attend_step(to64(q[b]), To, t, W, scale, kbs, vbs, K, V)
        assert max_abs(out[b], ref) <= 2e-2, f"request {b}: max-abs {max_abs(out[b], ref)}"
        # the device pages after one-token appends equal a one-shot quantisation of the same entries
        n = final[b] // r
        _check_stored(cache, cache.kidx, cache.kidx_scale, b, n, ki, bi, "fp8", f"request {b} kidx")
        _check_stored(cache, cache.kbar[0], cache.kbar_scale[0], b, n, kb, bk, "fp8", f"request {b} kbar")
        _check_stored(cache, cache.vbar[0], cache.vbar_scale[0], b, n, vb, bv, "fp8", f"request {b} vbar")


# --------------------------------------------------------------------------- heavily compressed attention (no indexer)

def _hca_case(kv, act, lens, r, W, H=64, seed=57, chunk=None, swa=""):
    """Compress with a large ratio and no indexer, then csa_attend_dense; the
    oracle compresses the same raw rows and attends to every visible entry."""
    max_pages = max(1, max(L // r for L in lens) // 64 + 2)
    n_q = len(lens) if chunk is None else chunk[1]
    R = max(W, r, 8) + (0 if chunk is None else chunk[1])
    cache = make_cache(seed, ratio=r, q_heads=H, idx_heads=0, window=W, ring_rows=R, n_layers=1,
                       max_seqs=len(lens), max_pages_per_seq=max_pages, pool_pages=len(lens) * max_pages + 3,
                       kv_dtype=kv, act_dtype=act, max_queries=n_q, max_k=1, swa_dtype=swa)
    assert cache.kidx is None
    raws = []
    for b, L in enumerate(lens):
        rows = [raw_rows(seed, kind, 0, b, 0, L, act) for kind in (Sy.KIND_K, Sy.KIND_V, Sy.KIND_Z)]
        raws.append(tuple(to64(x) for x in rows))
        cache.compress(0, [b], [L], *(x.cuda() for x in rows))
    if chunk is None:
        q_seq, q_pos = list(range(len(lens))), [L - 1 for L in lens]
    else:
        q_seq = [chunk[0]] * chunk[1]
        q_pos = [lens[chunk[0]] - chunk[1] + i for i in range(chunk[1])]
    q = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_Q), 0, n_q * H, 128, dtype=TORCH_ACT[act]).view(n_q, H, 128)
    scale = 1.0 / math.sqrt(128)
    got = to64(cache.attend_dense(0, q_seq, q_pos, q.cuda(), scale))
    assert cache.read_errors() == 0
    ents = {}
    for i in range(n_q):
        b = q_seq[i]
        if b not in ents:
            K, V, Z = raws[b]
            kb, vb, _ = O.compress(K, V, Z, r)
            ents[b] = (O.store(kb, kv)[0], O.store(vb, kv)[0])
        K, V = (O.store_ring_rows(x, swa)[0] for x in raws[b][:2])
        ref = O.hca_attend_step(to64(q[i]), q_pos[i], r, W, scale, ents[b][0], ents[b][1], K, V)
        err = max_abs(got[i], ref)
        assert err <= TOL[act], f"query {i} (seq {b}, t {q_pos[i]}): max-abs {err}"


@pytest.mark.parametrize("kv,act", DT_CASES)
def test_hca_decode_matches_oracle(kv, act):
    _hca_case(kv, act, lens=[128 * 300 + 77, 128 * 64, 200, 127], r=128, W=128)


@pytest.mark.parametrize("r,W", [(16, 0), (16, 64), (64, 128), (4, 32)])
def test_hca_ratios_and_windows(r, W):
    _hca_case("fp8", "bf16", lens=[r * 1500 + 3, r * 70 + r - 1, 9], r=r, W=W)


def test_hca_many_splits():
    """4,096 entries (64 blocks) per query: the split-and-merge path."""
    _hca_case("bf16", "bf16", lens=[16 * 4096, 16 * 4000 + 5], r=16, W=128, H=16)


def test_hca_three_rounds():
    """8,192 entries (130 blocks with the window): 44 splits of three 64-key
    rounds each, merged by the 48-split merge."""
    _hca_case("fp8", "bf16", lens=[4 * 8192 + 3, 4 * 300], r=4, W=128, H=16)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_hca_more_blocks_than_splits(kv):
    """12,000 entries (188 blocks) for one query: more blocks than a query may
    be split into, so every workgroup walks several blocks in sequence."""
    _hca_case(kv, "bf16", lens=[4 * 12000 + 1, 4 * 2500], r=4, W=128, H=16)


@pytest.mark.parametrize("kv,act", [("bf16", "bf16"), ("fp8", "bf16")])
def test_hca_chunk_queries(kv, act):
    _hca_case(kv, act, lens=[64 * 900 + 10, 300], r=64, W=128, chunk=(0, 96))


def test_hca_ratio1_no_window_is_causal_attention():
    """r = 1, W = 0: dense causal attention (torch SDPA)."""
    L, H = 160, 16
    cache = make_cache(43, ratio=1, q_heads=H, idx_heads=0, window=0, ring_rows=8, max_seqs=1, max_pages_per_seq=4,
                       pool_pages=5, kv_dtype="f32", act_dtype="f32", max_queries=L, max_k=1)
    K, V, Z = (raw_rows(43, kind, 0, 0, 0, L, "f32") for kind in (Sy.KIND_K, Sy.KIND_V, Sy.KIND_Z))
    cache.compress(0, [0], [L], K.cuda(), V.cuda(), Z.cuda())
    q = Sy.normal_rows(43, Sy.stream_id(Sy.KIND_Q), 0, L * H, 128).view(L, H, 128)
    out = cache.attend_dense(0, [0] * L, list(range(L)), q.cuda(), 1 / math.sqrt(128)).cpu()
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.permute(1, 0, 2).double().unsqueeze(0), K.double()[None, None].expand(1, H, L, 128),
        V.double()[None, None].expand(1, H, L, 128), is_causal=True, scale=1 / math.sqrt(128))[0].permute(1, 0, 2)
    assert max_abs(out.double().numpy(), ref.numpy()) <= 2e-3


def test_hca_group_rejects_indexer_calls():
    cache = make_cache(3, ratio=32, q_heads=16, idx_heads=0, window=32, ring_rows=32, max_seqs=1,
                       max_pages_per_seq=2, pool_pages=2, kv_dtype="bf16", act_dtype="bf16", max_queries=1, max_k=1)
    K = raw_rows(3, Sy.KIND_K, 0, 0, 0, 64, "bf16").cuda()
    with pytest.raises(RuntimeError):
        cache.compress(0, [0], [64], K, K, K, Sy.proj_matrix(3, 128, 64).cuda())
    cache.compress(0, [0], [64], K, K, K)
    with pytest.raises(RuntimeError):
        cache.index_topk([0], [63], torch.zeros((1, 1, 64), dtype=torch.bfloat16, device="cuda"),
                         torch.ones((1, 1), device="cuda"), 1)


# --------------------------------------------------------------------------- window ring: fp8 rows, bounded replay

def _ring_bytes(cache, layer, seq):
    out = [cache.ring_k[layer][seq].cpu(), cache.ring_v[layer][seq].cpu()]
    if cache.spec.swa_dtype == "fp8":
        out += [cache.ring_k_scale[layer][seq].cpu(), cache.ring_v_scale[layer][seq].cpu()]
    return out


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_fp8_ring_rows_match_oracle_codec(kv):
    """Compress writes the newest R raw rows as E4M3 codes with one amax/448
    scale per row: codes and scales equal the oracle's, byte for byte."""
    lens = [4 * 200 + 3, 77, 5]
    cache, raw, _ = _compress_case(kv, "bf16", 4, lens, swa="fp8")
    R = cache.cfg.ring_rows
    for b, L in enumerate(lens):
        rows = np.arange(max(0, L - R), L)
        for x, ring, sc in ((raw[0][b][0], cache.ring_k[0], cache.ring_k_scale[0]),
                            (raw[0][b][1], cache.ring_v[0], cache.ring_v_scale[0])):
            _, (codes, scales) = O.store_ring_rows(to64(x)[rows], "fp8")
            assert np.array_equal(ring[b, rows % R].cpu().numpy(), codes)
            assert np.array_equal(sc[b, rows % R].cpu().numpy(), scales)
    assert cache.read_errors() == 0


def test_fp8_ring_incremental_equals_bulk():
    """Appending one row at a time or in uneven chunks leaves the same ring
    codes, ring scales and open-block staging as one bulk append."""
    lens = [4 * 70 + 3, 150]
    bulk, _, _ = _compress_case("fp8", "bf16", 4, lens, seed=19, swa="fp8")
    inc, _, _ = _compress_case("fp8", "bf16", 4, lens, seed=19, chunks=[1, 1, 5, 2, 30, 1, 64, 3], swa="fp8")
    for b, L in enumerate(lens):
        for x, y in zip(_ring_bytes(bulk, 0, b), _ring_bytes(inc, 0, b)):
            assert torch.equal(x, y)
        assert torch.equal(bulk.block_stage[0][b, :, : (L % 4)].cpu(), inc.block_stage[0][b, :, : (L % 4)].cpu())
        n = L // 4
        assert torch.equal(bulk.logical(bulk.kbar[0], b, n).cpu(), inc.logical(inc.kbar[0], b, n).cpu())


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_attend_fp8_ring_decode_matches_oracle(kv):
    _attend_case(kv, "bf16", lens=[4 * 700 + 2, 4 * 64, 37, 4], k=256, W=128, swa="fp8")


@pytest.mark.parametrize("kv", ["bf16", "fp8", "fp4"])
def test_attend_fp8_ring_chunk_matches_oracle(kv):
    _attend_case(kv, "bf16", lens=[4 * 600 + 1, 400], k=128, W=128, chunk=(0, 48), swa="fp8")


@pytest.mark.parametrize("kv,act", DT_CASES)
def test_attend_chunk_head_counts(kv, act):
    # 32 and 128 heads in a prefill chunk, with a ragged last Top-K block
    for H in (32, 128):
        _attend_case(kv, act, lens=[4 * 900 + 2, 64], k=150, W=64, H=H, chunk=(0, 40))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_step_decode_chain_fp8_ring(kv):
    _chain(kv, "bf16", [4 * 2000 + 3, 999, 130], k=128, W=128, H=64, n_layers=2, swa="fp8")


def test_hca_fp8_ring():
    _hca_case("fp8", "bf16", lens=[64 * 500 + 7, 100], r=64, W=128, swa="fp8")


@pytest.mark.parametrize("swa", ["", "fp8"])
def test_window_bounded_by_replay_start(swa):
    """With replay start s, the window of a query at t is [max(s, t - W + 1), t]:
    s inside the window, at the query itself, before the window (no effect)."""
    lens = [4 * 900 + 1, 4 * 300 + 2, 4 * 50, 4 * 64 + 3]
    starts = [lens[0] - 40, lens[1] - 1, 10, lens[3] - 127]
    _attend_case("bf16", "bf16", lens=lens, k=64, W=128, swa=swa, swa_start=starts)


def test_window_replay_start_bounds_chunk_queries():
    """A prefill chunk after a replay start: queries before s + W - 1 see a
    truncated window, later ones the full W rows."""
    L = 4 * 500
    _attend_case("fp8", "bf16", lens=[L, 90], k=64, W=128, chunk=(0, 96), swa_start=[L - 96 - 20, 0])


@pytest.mark.parametrize("swa", ["", "fp8"])
def test_ring_replay_rewrites_window_only(swa):
    """Bounded replay: rewrite the ring rows [s, L) of a sequence from a second
    seeded stream. The compressed pages, indexer keys and open-block staging
    stay byte-identical; attention with replay start s uses the new window
    rows and the old compressed entries (the oracle gets exactly that)."""
    r, W, H, k = 4, 128, 16, 64
    lens = [4 * 400 + 2, 4 * 100]
    cache, raw, P = _compress_case("fp8", "bf16", r, lens, seed=23, swa=swa)
    # _compress_case sizes the ring at max(16, r) rows; rebuild with the window here
    cache = make_cache(23, ratio=r, q_heads=H, window=W, ring_rows=W, max_seqs=2, max_pages_per_seq=cache.spec.max_pages_per_seq,
                       pool_pages=cache.spec.pool_pages, kv_dtype="fp8", act_dtype="bf16", max_queries=2, max_k=k,
                       swa_dtype=swa)
    for b, L in enumerate(lens):
        cache.compress(0, [b], [L], *(x.cuda() for x in raw[0][b]), P.cuda())
    torch.cuda.synchronize()
    before = [t.clone() for t in (cache.kbar[0], cache.vbar[0], cache.kidx, cache.kbar_scale[0], cache.vbar_scale[0],
                                  cache.kidx_scale, cache.block_stage[0])]
    s0 = [lens[0] - 50, lens[1] - W]
    newk = [raw_rows(99, Sy.KIND_K, 0, b, s0[b], L - s0[b], "bf16") for b, L in enumerate(lens)]
    newv = [raw_rows(99, Sy.KIND_V, 0, b, s0[b], L - s0[b], "bf16") for b, L in enumerate(lens)]
    cache.ring_write(0, [1, 0], [s0[1], s0[0]], [lens[1] - s0[1], lens[0] - s0[0]],
                     torch.cat([newk[1], newk[0]]).cuda(), torch.cat([newv[1], newv[0]]).cuda())
    for b in range(2):
        cache.set_swa_start(b, s0[b])
    torch.cuda.synchronize()
    for x, y in zip(before, (cache.kbar[0], cache.vbar[0], cache.kidx, cache.kbar_scale[0], cache.vbar_scale[0],
                              cache.kidx_scale, cache.block_stage[0])):
        assert torch.equal(x, y)
    assert [cache.seq_len(0, b) for b in range(2)] == lens
    # ring contents: the oracle codec of the new rows
    for b, L in enumerate(lens):
        rows = np.arange(s0[b], L)
        for x, ring in ((newk[b], cache.ring_k[0]), (newv[b], cache.ring_v[0])):
            got = ring[b, rows % W].cpu()
            if swa == "fp8":
                assert np.array_equal(got.numpy(), O.store_ring_rows(to64(x), "fp8")[1][0])
            else:
                assert torch.equal(got, x)
    # attention against the oracle: old entries, old window rows before s (masked by s), new rows from s
    qi = Sy.normal_rows(23, Sy.stream_id(Sy.KIND_QI), 0, 2 * 4, 64, dtype=torch.bfloat16).view(2, 4, 64)
    w = Sy.uniform_rows(23, Sy.stream_id(Sy.KIND_W), 0, 2, 4)
    q_pos = [L - 1 for L in lens]
    T = cache.index_topk([0, 1], q_pos, qi.cuda(), w.cuda(), k)
    q = Sy.normal_rows(23, Sy.stream_id(Sy.KIND_Q), 0, 2 * H, 128, dtype=torch.bfloat16).view(2, H, 128)
    scale = 1 / math.sqrt(128)
    out = to64(cache.attend(0, [0, 1], q_pos, q.cuda(), T, k, scale))
    assert cache.read_errors() == 0
    Tg = T.cpu().numpy()
    for b, L in enumerate(lens):
        K, V, Z = (to64(x) for x in raw[0][b])
        kb, vb, ki, _, _, bi = oracle_entries(K, V, Z, r, to64(P))
        N = O.visible_entries(L - 1, r)
        To = O.topk(check_topk_chain(Tg[b], to64(qi[b]), to64(w[b]), ki, bi, "fp8", N, k, f"seq {b}"), k)
        Kr, Vr = K.copy(), V.copy()
        Kr[s0[b]:], Vr[s0[b]:] = to64(newk[b]), to64(newv[b])
        Kr, Vr = O.store_ring_rows(Kr, swa)[0], O.store_ring_rows(Vr, swa)[0]
        ref = O.attend_step(to64(q[b]), To, L - 1, W, scale, O.store(kb, "fp8")[0],
                            O.store(vb, "fp8")[0], Kr, Vr, s0[b])
        assert max_abs(out[b], ref) <= TOL["bf16"]


def test_ring_write_rejects_rows_outside_the_ring():
    cache = make_cache(5, ratio=4, q_heads=16, window=32, ring_rows=32, max_seqs=1, max_pages_per_seq=2, pool_pages=2,
                       kv_dtype="bf16", act_dtype="bf16", max_queries=1, max_k=1)
    K = raw_rows(5, Sy.KIND_K, 0, 0, 0, 100, "bf16").cuda()
    cache.compress(0, [0], [100], K, K, K, Sy.proj_matrix(5, 128, 64).cuda())
    with pytest.raises(B.CsaError):
        cache.ring_write(0, [0], [60], [8], K[:8], K[:8])       # row 60 left the 32-row ring
    with pytest.raises(B.CsaError):
        cache.ring_write(0, [0], [95], [8], K[:8], K[:8])       # rows 100.. not appended
    cache.ring_write(0, [0], [68], [32], K[:32], K[:32])
    torch.cuda.synchronize()
    assert torch.equal(cache.ring_k[0][0, (np.arange(68, 100) % 32)].cpu(), K[:32].cpu())


# --------------------------------------------------------------------------- FP4 main KV

def test_device_fp4_codecs():
    """E2M1 decode as the attention kernel unpacks a row (low nibble first) and
    the compressor's encoder, against the oracle's format definition."""
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    out = torch.empty(512, dtype=torch.float32, device="cuda")
    B.csa_debug_convert(4, b.cuda(), out)
    got = out.cpu().numpy().astype(np.float64).reshape(256, 2)
    bb = np.arange(256)
    np.testing.assert_array_equal(got[:, 0], O.e2m1_decode(bb & 0xF))
    np.testing.assert_array_equal(got[:, 1], O.e2m1_decode(bb >> 4))
    rng = np.random.default_rng(71)
    mags = O.e2m1_decode(np.arange(8))
    mids = (mags[:-1] + mags[1:]) / 2
    x = np.concatenate([rng.standard_normal(20000) * 3, rng.uniform(-8, 8, 5000), mids, -mids, mags, -mags,
                        [0.0, -0.0, 6.0, 6.5, 100.0, -1e9, 1e-30]]).astype(np.float32)
    codes = torch.empty(x.shape[0], dtype=torch.uint8, device="cuda")
    B.csa_debug_convert(5, torch.from_numpy(x).cuda(), codes)
    np.testing.assert_array_equal(codes.cpu().numpy(), O.e2m1_encode(x))


def _check_fp4(cache, pool, gpool, seq, n, x64, band, what, exact):
    """GPU fp4 entries of one stream vs the oracle's quantisation of x64: every
    code and group scale equal when the GPU's fp32 entries are the oracle's
    (exact); otherwise equal except where a group amax / 6 or an element's
    quotient lies within its error band of a rounding boundary (counted)."""
    codes = unpack_fp4(cache.logical(pool, seq, n).cpu().numpy())
    gsc = cache.logical(gpool, seq, n).cpu().numpy()
    _, (oc, osc) = O.store(x64[:n], "fp4")
    if exact:
        assert np.array_equal(codes, oc) and np.array_equal(gsc, osc), what
        return
    allowed, bad = PB.check_fp4(codes, gsc, x64[:n], band[:n])
    assert bad == 0, f"{what}: {bad} fp4 codes differ from the oracle's quantisation outside every error band"
    if allowed:
        print(f"[codes] {what}: {allowed} fp4 codes at a rounding boundary take the other neighbour")


@pytest.mark.parametrize("r", [1, 4])
def test_compress_fp4_matches_oracle(r):
    """r = 1: entries are the raw bf16 rows, so the fp4 bytes equal the oracle's
    exactly; r = 4: pooled fp32 entries may differ from the oracle's by an ulp."""
    lens = [64 * 4 * 3 + 21, 517, 5] if r == 4 else [300, 129, 64]
    cache, raw, P = _compress_case("fp4", "bf16", r, lens)
    for b, L in enumerate(lens):
        K, V, Z = (to64(t) for t in raw[0][b])
        kb, vb, ki, bk, bv, bi = oracle_entries(K, V, Z, r, to64(P))
        n = L // r
        if n == 0:
            continue
        _check_fp4(cache, cache.kbar[0], cache.kbar_gscale[0], b, n, kb, bk, f"kbar seq {b}", exact=r == 1)
        _check_fp4(cache, cache.vbar[0], cache.vbar_gscale[0], b, n, vb, bv, f"vbar seq {b}", exact=r == 1)
        _check_stored(cache, cache.kidx, cache.kidx_scale, b, n, ki, bi, "fp8", f"kidx seq {b}")
    assert cache.read_errors() == 0


def test_compress_fp4_incremental_equals_bulk():
    lens = [64 * 4 * 2 + 13, 301]
    bulk, _, _ = _compress_case("fp4", "bf16", 4, lens, seed=9)
    inc, _, _ = _compress_case("fp4", "bf16", 4, lens, seed=9, chunks=[1, 3, 2, 1, 7, 64, 1, 1, 200, 5])
    for b, L in enumerate(lens):
        n = L // 4
        for pa, pb in ((bulk.kbar[0], inc.kbar[0]), (bulk.vbar[0], inc.vbar[0]), (bulk.kbar_gscale[0], inc.kbar_gscale[0]),
                       (bulk.vbar_gscale[0], inc.vbar_gscale[0]), (bulk.kidx, inc.kidx)):
            assert torch.equal(bulk.logical(pa, b, n).cpu(), inc.logical(pb, b, n).cpu())
        assert torch.equal(bulk.logical_scales(bulk.kidx_scale, b, n).cpu(), inc.logical_scales(inc.kidx_scale, b, n).cpu())


@pytest.mark.parametrize("swa", ["", "fp8"])
def test_attend_fp4_decode_matches_oracle(swa):
    _attend_case("fp4", "bf16", lens=[4 * 700 + 2, 4 * 64, 37, 4], k=256, W=128, swa=swa)


@pytest.mark.parametrize("H", [16, 128])
def test_attend_fp4_head_counts(H):
    _attend_case("fp4", "bf16", lens=[4 * 500 + 3, 4 * 90], k=200, W=64, H=H)


def test_attend_fp4_chunk_matches_oracle():
    _attend_case("fp4", "bf16", lens=[4 * 600 + 1, 400], k=128, W=128, chunk=(0, 48))


def test_step_decode_chain_fp4():
    _chain("fp4", "bf16", [4 * 3000 + 2, 4100, 777], k=256, W=128, H=64, n_layers=2)


def test_hca_fp4():
    _hca_case("fp4", "bf16", lens=[64 * 500 + 7, 100], r=64, W=128)
