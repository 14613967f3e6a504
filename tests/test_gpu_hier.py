"""GPU parity for the hierarchical sparse indexer: the Full-mode layer's
candidate pool (csa_index_topk_pool) and the Reindex-mode Top-K inside a pool
(csa_index_reindex), against the oracle on identical stored indexer keys.

Bars: Top-K and pool sets exact except near-ties within 1e-6 relative of the
oracle's k-th entry score (or n_pool-th block maximum); bit-exact where the
inputs force exact ties.
"""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_csa_amd import binding as B
from compressed_sparse_attention_csa_amd import synth as Sy
from oracle import csa_oracle as O

from gpu_helpers import TORCH_ACT, fill_index_keys, make_cache, store_raw_to_torch, to64, topk_matches, write_logical, \
    write_scales

pytestmark = pytest.mark.gpu

DT_CASES = [("f32", "f32"), ("bf16", "bf16"), ("fp8", "bf16")]
R = 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.synchronize()


def _keys_cache(kv, act, lens, seed, n_q, k, h_i=4, dup_keys=False):
    """A cache whose indexer keys are seeded rows stored through the oracle's codec."""
    max_pages = max(L // R for L in lens) // 64 + 2
    cache = make_cache(seed, ratio=R, q_heads=16, idx_heads=h_i, window=0, ring_rows=8, max_seqs=len(lens),
                       max_pages_per_seq=max_pages, pool_pages=len(lens) * max_pages + 1, kv_dtype=kv, act_dtype=act,
                       max_queries=n_q, max_k=k)
    keys = []
    for b, L in enumerate(lens):
        n = L // R
        if dup_keys and n:
            x = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_KI, 0, b), 0, 5, 64).double().numpy()[np.arange(n) % 5]
            vals, raw = O.store(x, kv)
            write_logical(cache, cache.kidx, b, store_raw_to_torch(raw, kv))
            if kv == "fp8":
                write_scales(cache, cache.kidx_scale, b, raw[1])
            keys.append(vals)
        else:
            keys.append(fill_index_keys(cache, seed, b, n))
        B.csa_seq_set_len(cache.handle, 0, b, L)
    return cache, keys


def _queries(seed, layer, n_q, h_i, act):
    qi = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_QI, layer), 0, n_q * h_i, 64, dtype=TORCH_ACT[act]).view(n_q, h_i, 64)
    w = Sy.uniform_rows(seed, Sy.stream_id(Sy.KIND_W, layer), 0, n_q, h_i)
    return qi, w


def _block_scores(s):
    nb = (s.shape[0] + O.POOL_BLOCK - 1) // O.POOL_BLOCK
    return np.array([s[b * O.POOL_BLOCK:(b + 1) * O.POOL_BLOCK].max() for b in range(nb)], dtype=np.float32)


def _pool_case(kv, act, lens, k, n_blocks, seed=41, chunk=None, dup_keys=False, exact=False):
    n_q = len(lens) if chunk is None else chunk[1]
    cache, keys = _keys_cache(kv, act, lens, seed, n_q, k, dup_keys=dup_keys)
    if chunk is None:
        q_seq, q_pos = list(range(len(lens))), [L - 1 for L in lens]
    else:
        q_seq = [chunk[0]] * chunk[1]
        q_pos = [lens[chunk[0]] - chunk[1] + i for i in range(chunk[1])]
    qi, w = _queries(seed, 0, n_q, 4, act)
    T, P = cache.index_topk_pool(q_seq, q_pos, qi.cuda(), w.cuda(), k, n_blocks)
    # the plain entry point gives the same Top-K
    T2 = cache.index_topk(q_seq, q_pos, qi.cuda(), w.cuda(), k) if chunk is None else None
    T, P = T.cpu().numpy(), P.cpu().numpy()
    assert cache.read_errors() & ~B.ERR_FALLBACK == 0
    q64, w64 = to64(qi), to64(w)
    for i in range(n_q):
        N = O.visible_entries(q_pos[i], R)
        s = O.index_scores(q64[i], w64[i], keys[q_seq[i]][:N])
        ok, msg = topk_matches(T[i], O.topk(s, k), s)
        assert ok, f"query {i} Top-K (N={N}): {msg}"
        Po = O.candidate_pool(s, n_blocks)
        if exact:
            assert P[i].tolist() == Po.tolist(), f"query {i}: equal block maxima go to the lower block"
        ok, msg = topk_matches(P[i], Po, _block_scores(s))
        assert ok, f"query {i} pool (N={N}, blocks {n_blocks}): {msg}"
    if T2 is not None:
        assert np.array_equal(T2.cpu().numpy(), T)
    return cache, keys, (q_seq, q_pos, qi, w), T, P


@pytest.mark.parametrize("kv,act", DT_CASES)
def test_pool_matches_oracle(kv, act):
    # 8,751 blocks (last one partial), fewer blocks than the pool, a pool-sized context, N < k, N = 0
    _pool_case(kv, act, lens=[4 * 70005 + 1, 4 * 3000 + 2, 4 * 16384, 4 * 100, 3], k=512, n_blocks=2048)


@pytest.mark.parametrize("n_blocks", [1, 7, 256, 1024])
def test_pool_sizes(n_blocks):
    _pool_case("fp8", "bf16", lens=[4 * 262144, 4 * 20000 + 3], k=1024, n_blocks=n_blocks)


@pytest.mark.parametrize("kv,act", DT_CASES)
def test_pool_exact_ties_go_to_lower_block(kv, act):
    # five distinct keys repeat: many blocks share the same maximum
    _pool_case(kv, act, lens=[4 * 4000, 4 * 900 + 1], k=64, n_blocks=100, dup_keys=True, exact=True)


def test_pool_for_chunk_queries():
    _pool_case("bf16", "bf16", lens=[4 * 12000, 40], k=256, n_blocks=512, chunk=(0, 150))


@pytest.mark.parametrize("kv,act", DT_CASES)
def test_pool_chunk_kernels_match_oracle(kv, act):
    """Chunk queries take the score GEMM, which also writes the block maxima:
    a 600-token chunk whose early queries see fewer blocks than the pool."""
    _pool_case(kv, act, lens=[4 * 20000 + 3, 50], k=512, n_blocks=2048, chunk=(0, 600))


def test_pool_chunk_long_context():
    """More visible blocks than the pool select holds in LDS (7,500 > 6,144)."""
    _pool_case("fp8", "bf16", lens=[4 * 60000 + 1], k=1024, n_blocks=2048, chunk=(0, 64))


def test_pool_chunk_exact_ties():
    _pool_case("bf16", "bf16", lens=[4 * 3000], k=64, n_blocks=50, dup_keys=True, exact=True, chunk=(0, 200))


def _random_pool(rng, n_ent, n_blocks, force_last=False):
    nb = (n_ent + 7) // 8
    if nb <= n_blocks:
        return np.concatenate([np.arange(nb), -np.ones(n_blocks - nb)]).astype(np.int32)
    pick = rng.choice(nb - 1, size=n_blocks - 1 if force_last else n_blocks, replace=False)
    if force_last:
        pick = np.append(pick, nb - 1)
    return np.sort(pick).astype(np.int32)


def _reindex_case(kv, act, lens, k, n_blocks, seed=47, force_last=True, dup_keys=False, exact=False, q_pos=None):
    n_q = len(lens)
    cache, keys = _keys_cache(kv, act, lens, seed, n_q, k, dup_keys=dup_keys)
    q_seq = list(range(n_q))
    q_pos = q_pos or [L - 1 for L in lens]
    rng = np.random.default_rng(seed)
    pools = np.stack([_random_pool(rng, O.visible_entries(q_pos[i], R), n_blocks, force_last) for i in range(n_q)])
    qi, w = _queries(seed, 1, n_q, 4, act)
    T = cache.index_reindex(q_seq, q_pos, qi.cuda(), w.cuda(), torch.from_numpy(pools).cuda(), k).cpu().numpy()
    assert cache.read_errors() & ~B.ERR_FALLBACK == 0
    q64, w64 = to64(qi), to64(w)
    for i in range(n_q):
        N = O.visible_entries(q_pos[i], R)
        To = O.reindex_topk(q64[i], w64[i], keys[i], pools[i], k, N)
        if exact:
            assert T[i].tolist() == To.tolist()
        s = O.index_scores(q64[i], w64[i], keys[i][:N])
        ok, msg = topk_matches(T[i], To, s)
        assert ok, f"query {i} (N={N}): {msg}"
        assert set(int(j) for j in T[i] if j >= 0) <= set(O.pool_entries(pools[i], N).tolist())


@pytest.mark.parametrize("kv,act", DT_CASES)
def test_reindex_matches_oracle(kv, act):
    # a 2,048-block pool that includes the partial last block; whole-context pools; N = 0
    _reindex_case(kv, act, lens=[4 * 70005 + 1, 4 * 9000, 4 * 1000 + 3, 4 * 20, 2], k=512, n_blocks=2048)


def test_reindex_pool_smaller_than_k():
    # 16 blocks with the 5-entry tail: 125 entries for k = 127 (two -1 pads) and for k = 300
    _reindex_case("bf16", "bf16", lens=[4 * 10005, 4 * 10005], k=127, n_blocks=16)
    _reindex_case("fp8", "bf16", lens=[4 * 10005, 4 * 3001], k=300, n_blocks=16)


@pytest.mark.parametrize("kv,act", DT_CASES)
def test_reindex_exact_ties(kv, act):
    _reindex_case(kv, act, lens=[4 * 30000, 4 * 5000], k=200, n_blocks=300, dup_keys=True, exact=True)


@pytest.mark.parametrize("k", [64, 1024, 2048])
def test_reindex_k_range(k):
    _reindex_case("fp8", "bf16", lens=[4 * 262144, 4 * 50000 + 1], k=k, n_blocks=2048)


def test_reindex_with_full_query_recovers_full_topk():
    """The Full layer's Top-K lies in its own pool (k <= pool blocks), so
    rescoring the pool with the Full layer's query returns that Top-K."""
    cache, keys, (q_seq, q_pos, qi, w), T, P = _pool_case("fp8", "bf16", lens=[4 * 200000, 4 * 30000 + 2], k=1024,
                                                           n_blocks=2048)
    T2 = cache.index_reindex(q_seq, q_pos, qi.cuda(), w.cuda(), torch.from_numpy(P).cuda(), 1024).cpu().numpy()
    assert np.array_equal(T2, T)


def test_full_reindex_reuse_chain():
    """Full builds the pool, a Reindex layer selects inside it with its own
    query, and the oracle does the same from the same keys."""
    lens = [4 * 150000 + 3, 4 * 40000]
    cache, keys, (q_seq, q_pos, _, _), T, P = _pool_case("fp8", "bf16", lens=lens, k=512, n_blocks=2048)
    qi2, w2 = _queries(53, 1, len(lens), 4, "bf16")
    T2 = cache.index_reindex(q_seq, q_pos, qi2.cuda(), w2.cuda(), torch.from_numpy(P).cuda(), 512).cpu().numpy()
    qf, wf = _queries(41, 0, len(lens), 4, "bf16")      # the Full layer's query of _pool_case
    q64, w64 = to64(qi2), to64(w2)
    for i in range(len(lens)):
        N = O.visible_entries(q_pos[i], R)
        Po = O.candidate_pool(O.index_scores(to64(qf[i]), to64(wf[i]), keys[i][:N]), 2048)
        assert np.array_equal(P[i], Po)                 # no near-tie block at this seed
        To = O.reindex_topk(q64[i], w64[i], keys[i], Po, 512, N)
        s = O.index_scores(q64[i], w64[i], keys[i][:N])
        ok, msg = topk_matches(T2[i], To, s)
        assert ok, msg
