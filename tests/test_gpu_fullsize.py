"""Full-size parity in the launch configuration the benchmark times.

The 1,048,576-token batch-4 decode (fp8 cache, 4 layers sharing one Top-1024,
W = 128, 64 heads) is built on the GPU exactly as bench.py builds it; one step
runs through the C ABI. The oracle recomputes, for sequence 0, the indexer
keys of all 262,144 entries from the same seeded raw rows, its Top-K, and the
attention of layers 0 and 3.
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
