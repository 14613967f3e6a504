"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
its host-side validation rejects bad calls before touching the GPU.

No call here launches a kernel: every device call below is built to fail
validation, and the handle is created over placeholder pointers that the
library never dereferences on the host.
"""
import ctypes as C
import os
import re

import pytest

from compressed_sparse_attention_csa_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "csa.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = B.lib()
    declared = _declared_functions()
    assert set(declared) == set(B.EXPORTS), (declared, B.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def _spec(**kw):
    c = B.Config()
    c.ratio, c.head_dim, c.q_heads, c.idx_heads, c.idx_dim = 4, 128, 64, 4, 64
    c.window, c.ring_rows, c.n_layers = 128, 128, 2
    c.max_seqs, c.max_pages_per_seq, c.pool_pages = 4, 16, 64
    c.kv_dtype, c.act_dtype, c.swa_dtype = B.CSA_FP8_E4M3, B.CSA_BF16, B.CSA_BF16
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _fake_handle(cfg, n_layers=None, workspace_bytes=None):
    """A handle over placeholder (never dereferenced) addresses."""
    b = B.Buffers()
    n = n_layers or cfg.n_layers
    fake = 0x10000
    for l in range(n):
        for f in ("kbar", "vbar", "kbar_scale", "vbar_scale", "kbar_stage", "vbar_stage", "ring_k", "ring_v", "block_stage",
                  "ring_k_scale", "ring_v_scale", "kbar_gscale", "vbar_gscale"):
            getattr(b, f)[l] = fake
    b.kidx = b.kidx_scale = b.kidx_stage = b.block_table = fake
    b.workspace = 0x100000
    b.workspace_bytes = workspace_bytes or B.csa_workspace_size(cfg, 8, 512)
    return B.csa_cache_create(cfg, b)


def test_status_strings_and_sizes():
    L = B.lib()
    assert L.csa_status_string(0) == b"CSA_OK"
    assert L.csa_status_string(4) == b"CSA_ERR_CAPACITY"
    cfg = _spec()
    sz = B.csa_buffer_sizes_for(cfg)
    assert sz.kv_pool == 64 * 64 * 128 * 1
    assert sz.idx_pool == 64 * 64 * 64
    assert sz.page_scale == 64 * 4
    assert sz.kv_stage == 4 * 64 * 128 * 4
    assert sz.ring == 4 * 128 * 128 * 2
    assert sz.block_stage == 4 * 3 * 4 * 128 * 2
    assert sz.ring_scale == 0
    fp8_ring = B.csa_buffer_sizes_for(_spec(swa_dtype=B.CSA_FP8_E4M3))
    assert fp8_ring.ring == 4 * 128 * 128 and fp8_ring.ring_scale == 4 * 128 * 4
    assert sz.block_table == 4 * 16 * 4
    assert B.csa_workspace_size(cfg, 8, 512) > 0
    # workspace grows with the number of queries and with k
    assert B.csa_workspace_size(cfg, 64, 512) > B.csa_workspace_size(cfg, 8, 512)
    assert B.csa_workspace_size(cfg, 8, 2048) >= B.csa_workspace_size(cfg, 8, 512)


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, 5), ("idx_dim", 32, 5), ("q_heads", 48, 5), ("idx_heads", 5, 5), ("idx_heads", -1, 5), ("ratio", 0, 5), ("ratio", 257, 5),
    ("window", -1, 2), ("ring_rows", 64, 2), ("n_layers", 9, 2), ("pool_pages", 0, 2),
    ("kv_dtype", B.CSA_BF16, 3),                      # bf16 cache with... bf16 act is fine, so flip act below
])
def test_bad_configs_rejected(field, value, status):
    cfg = _spec(**{field: value})
    if field == "kv_dtype":
        cfg.act_dtype = B.CSA_F32
    with pytest.raises(B.CsaError) as e:
        B.csa_buffer_sizes_for(cfg)
    assert e.value.status == status
    assert B.csa_workspace_size(cfg, 8, 512) == 0


def test_pool_and_ring_byte_limits():
    """Attention addresses each K/V pool and window ring with 32-bit byte
    offsets: configs whose pool or ring passes 0xfffff000 bytes are refused."""
    lim = 0xFFFFF000
    fits = _spec(pool_pages=lim // (64 * 128))           # fp8 rows of 128 B: just inside
    assert B.csa_buffer_sizes_for(fits).kv_pool <= lim
    for cfg in (_spec(pool_pages=lim // (64 * 128) + 1),  # one page more
                _spec(kv_dtype=B.CSA_BF16, pool_pages=lim // (64 * 256) + 1),
                _spec(max_seqs=lim // (128 * 2 * 128) + 1, max_pages_per_seq=1, pool_pages=64)):
        with pytest.raises(B.CsaError) as e:
            B.csa_buffer_sizes_for(cfg)
        assert e.value.status == 5   # CSA_ERR_UNSUPPORTED
    # an fp4 pool of the same page count is half the bytes of an fp8 one
    assert B.csa_buffer_sizes_for(_spec(kv_dtype=B.CSA_FP4_E2M1, pool_pages=lim // (64 * 128) + 1)).kv_pool <= lim


def test_stream_read_validates_before_launch():
    """The streaming-read reference rejects bad arguments on the host (status 1,
    CSA_ERR_INVALID_ARG): no buffers, a null or misaligned buffer, a size that
    is not a positive multiple of 16, no launches."""
    L = B.lib()
    us = C.c_float(0.0)
    for bufs, nbytes, reps in (([], 1 << 20, 4), ([0], 1 << 20, 4), ([0x10008], 1 << 20, 4), ([0x10000], 100, 4),
                               ([0x10000], 1 << 20, 0), ([0x10000], 0, 4)):
        ptrs = (C.c_void_p * max(1, len(bufs)))(*bufs)
        assert L.csa_debug_stream_read(ptrs, len(bufs), nbytes, reps, C.c_void_p(0), C.byref(us)) == 1


def test_create_requires_buffers():
    cfg = _spec()
    b = B.Buffers()
    with pytest.raises(B.CsaError) as e:
        B.csa_cache_create(cfg, b)
    assert e.value.status == 1
    h = _fake_handle(cfg)
    B.csa_cache_destroy(h)


def test_unaligned_workspace_rejected():
    cfg = _spec()
    b = B.Buffers()
    for l in range(cfg.n_layers):
        for f in ("kbar", "vbar", "kbar_scale", "vbar_scale", "kbar_stage", "vbar_stage", "ring_k", "ring_v", "block_stage",
                  "ring_k_scale", "ring_v_scale", "kbar_gscale", "vbar_gscale"):
            getattr(b, f)[l] = 0x10000
    b.kidx = b.kidx_scale = b.kidx_stage = b.block_table = 0x10000
    b.workspace = 0x100010
    b.workspace_bytes = 1 << 20
    with pytest.raises(B.CsaError) as e:
        B.csa_cache_create(cfg, b)
    assert e.value.status == 1


def test_sequence_bookkeeping():
    cfg = _spec()
    h = _fake_handle(cfg)
    try:
        assert B.csa_seq_len(h, 0, 0) == 0
        B.csa_seq_set_len(h, 1, 2, 1000)
        assert B.csa_seq_len(h, 1, 2) == 1000
        assert B.csa_seq_len(h, 0, 2) == 0
        B.csa_seq_reset(h, 2)
        assert B.csa_seq_len(h, 1, 2) == 0
        assert B.csa_seq_len(h, 5, 0) == -1
        assert B.csa_seq_len(h, 0, 9) == -1
        with pytest.raises(B.CsaError) as e:
            B.csa_seq_set_len(h, 0, 0, 16 * 64 * 4 + 4)     # beyond the block-table row
        assert e.value.status == 4
        with pytest.raises(B.CsaError):
            B.csa_seq_reset(h, -1)
    finally:
        B.csa_cache_destroy(h)


def test_device_calls_validate_before_launch():
    cfg = _spec()
    h = _fake_handle(cfg)
    L = B.lib()
    fake = C.c_void_p(0x10000)
    s = C.c_void_p(0)
    i32 = B._i32
    try:
        # compress: layer 0 needs proj_idx; other layers must not pass it
        assert L.csa_compress(C.c_void_p(h), 0, 1, i32([0]), i32([4]), fake, fake, fake, None, s) == 1
        assert L.csa_compress(C.c_void_p(h), 1, 1, i32([0]), i32([4]), fake, fake, fake, fake, s) == 1
        assert L.csa_compress(C.c_void_p(h), 2, 1, i32([0]), i32([4]), fake, fake, fake, None, s) == 1
        assert L.csa_compress(C.c_void_p(h), 1, 2, i32([0, 0]), i32([4, 4]), fake, fake, fake, None, s) == 1
        assert L.csa_compress(C.c_void_p(h), 1, 1, i32([7]), i32([4]), fake, fake, fake, None, s) == 1
        assert L.csa_compress(C.c_void_p(h), 1, 1, i32([0]), i32([-1]), fake, fake, fake, None, s) == 2
        assert L.csa_compress(C.c_void_p(h), 1, 1, i32([0]), i32([16 * 64 * 4 + 4]), fake, fake, fake, None, s) == 4
        assert L.csa_compress(C.c_void_p(h), 1, 1, i32([0]), i32([8]), None, fake, fake, None, s) == 1
        # nothing was appended by the failed calls
        assert B.csa_seq_len(h, 1, 0) == 0
        # a zero-row append is a no-op that needs no pointers
        assert L.csa_compress(C.c_void_p(h), 1, 1, i32([0]), i32([0]), None, None, None, None, s) == 0
        # index: positions must lie inside the indexing layer's sequence
        assert L.csa_index_topk(C.c_void_p(h), 1, i32([0]), i32([0]), fake, fake, 16, fake, s) == 1
        B.csa_seq_set_len(h, 0, 0, 4096)
        assert L.csa_index_topk(C.c_void_p(h), 1, i32([0]), i32([4096]), fake, fake, 16, fake, s) == 1
        assert L.csa_index_topk(C.c_void_p(h), 1, i32([0]), i32([4095]), fake, fake, 0, fake, s) == 5
        assert L.csa_index_topk(C.c_void_p(h), 1, i32([0]), i32([4095]), fake, fake, 4096, fake, s) == 5
        assert L.csa_index_topk(C.c_void_p(h), 1, i32([0]), i32([4095]), None, fake, 16, fake, s) == 1
        assert L.csa_index_topk(C.c_void_p(h), 0, i32([0]), i32([4095]), fake, fake, 16, fake, s) == 1
        # attend: per-layer lengths; the window must still be in the ring
        assert L.csa_attend(C.c_void_p(h), 1, 1, i32([0]), i32([0]), fake, fake, 16, C.c_float(0.1), fake, s) == 1
        assert L.csa_attend(C.c_void_p(h), 0, 1, i32([0]), i32([100]), fake, fake, 16, C.c_float(0.1), fake, s) == 4
        assert L.csa_attend(C.c_void_p(h), 0, 1, i32([0]), i32([4095]), fake, None, 16, C.c_float(0.1), fake, s) == 1
        assert L.csa_attend(C.c_void_p(h), 0, 1, i32([0]), i32([4095]), fake, fake, -1, C.c_float(0.1), fake, s) == 5
        assert L.csa_attend(C.c_void_p(h), 3, 1, i32([0]), i32([4095]), fake, fake, 16, C.c_float(0.1), fake, s) == 1
        assert b"ring" in L.csa_last_error() or True
    finally:
        B.csa_cache_destroy(h)


def test_pool_and_reindex_calls_validate():
    """Pool sizes must lie in [1, CSA_MAX_POOL_BLOCKS] with a pool buffer; the
    query checks are those of csa_index_topk; an indexer-less group refuses."""
    cfg = _spec()
    h = _fake_handle(cfg)
    L = B.lib()
    fake = C.c_void_p(0x10000)
    s = C.c_void_p(0)
    i32 = B._i32
    try:
        B.csa_seq_set_len(h, 0, 0, 4096)
        tp = lambda pos, k, nb, pool=fake: L.csa_index_topk_pool(C.c_void_p(h), 1, i32([0]), i32([pos]), fake, fake, k,
                                                                 fake, nb, pool, s)
        ri = lambda pos, k, nb, pool=fake: L.csa_index_reindex(C.c_void_p(h), 1, i32([0]), i32([pos]), fake, fake, nb,
                                                               pool, k, fake, s)
        for f in (tp, ri):
            assert f(4095, 16, 0) == 5
            assert f(4095, 16, B.CSA_MAX_POOL_BLOCKS + 1) == 5
            assert f(4095, 16, 8, None) == 1
            assert f(4096, 16, 8) == 1          # position past the sequence
            assert f(4095, 0, 8) == 5
    finally:
        B.csa_cache_destroy(h)
    h = _fake_handle(_spec(idx_heads=0))
    try:
        B.csa_seq_set_len(h, 0, 0, 4096)
        assert L.csa_index_reindex(C.c_void_p(h), 1, i32([0]), i32([4095]), fake, fake, 8, fake, 16, fake, s) == 5
        assert L.csa_index_topk_pool(C.c_void_p(h), 1, i32([0]), i32([4095]), fake, fake, 16, fake, 8, fake, s) == 5
    finally:
        B.csa_cache_destroy(h)


def test_window_replay_calls_validate():
    """csa_seq_set_swa_start takes s >= 0 for a valid sequence; csa_ring_write
    only rewrites rows that were appended and are still inside the ring."""
    cfg = _spec()
    h = _fake_handle(cfg)
    L = B.lib()
    fake = C.c_void_p(0x10000)
    s = C.c_void_p(0)
    i32 = B._i32
    try:
        B.csa_seq_set_swa_start(h, 0, 100)
        for seq, start in ((-1, 0), (cfg.max_seqs, 0), (0, -1)):
            with pytest.raises(B.CsaError):
                B.csa_seq_set_swa_start(h, seq, start)
        B.csa_seq_set_len(h, 1, 0, 1000)
        R = cfg.ring_rows
        w = lambda seqs, p0, n, k=fake: L.csa_ring_write(C.c_void_p(h), 1, len(seqs), i32(seqs), i32(p0), i32(n), k, fake, s)
        assert w([0], [990], [11]) == 1                  # row 1000 not appended yet
        assert w([0], [1000 - R - 1], [2]) == 4          # row already left the ring
        assert w([0, 0], [995, 996], [1, 1]) == 1        # a sequence listed twice
        assert w([0], [-1], [1]) == 1
        assert w([0], [995], [-1]) == 1
        assert w([0], [995], [5], None) == 1             # rows need data
        assert w([0], [995], [0], None) == 0             # nothing to write needs none
        assert L.csa_ring_write(C.c_void_p(h), 7, 1, i32([0]), i32([995]), i32([1]), fake, fake, s) == 1
        assert B.csa_seq_len(h, 1, 0) == 1000            # rewrites never change lengths
    finally:
        B.csa_cache_destroy(h)


def test_destroyed_handle_rejected():
    cfg = _spec()
    h = _fake_handle(cfg)
    B.csa_cache_destroy(h)
    L = B.lib()
    assert L.csa_seq_reset(C.c_void_p(0), 0) == 1
    assert L.csa_cache_destroy(C.c_void_p(0)) == 1
    assert L.csa_debug_convert(7, C.c_void_p(0x10), C.c_void_p(0x10), 4, C.c_void_p(0)) == 1


def test_profile_masks_validated():
    """Kernel-timing calls take a mask of CSA_PROFILE_INDEX (1) / CSA_PROFILE_ATTEND (2);
    with nothing launched, ending a kind returns zero launches."""
    cfg = _spec()
    h = _fake_handle(cfg)
    L = B.lib()
    try:
        assert L.csa_profile_begin(C.c_void_p(h), 0) == 1
        assert L.csa_profile_begin(C.c_void_p(h), 4) == 1
        assert L.csa_profile_begin(C.c_void_p(h), 3) == 0
        ms, n = C.c_double(-1.0), C.c_int32(-1)
        assert L.csa_profile_end(C.c_void_p(h), 3, C.byref(ms), C.byref(n)) == 1
        assert L.csa_profile_end(C.c_void_p(h), 2, C.byref(ms), C.byref(n)) == 0
        assert n.value == 0 and ms.value == 0.0
        assert B.csa_profile_end(h, B.PROFILE_INDEX) == (0.0, 0)
    finally:
        B.csa_cache_destroy(h)


def test_indexerless_group_accepted_and_sized():
    """idx_heads = 0 (a heavily compressed group): no indexer buffers needed."""
    cfg = _spec(idx_heads=0, ratio=128)
    sz = B.csa_buffer_sizes_for(cfg)
    assert sz.idx_pool == 0 and sz.idx_stage == 0 and sz.kv_pool > 0
    b = B.Buffers()
    fake = 0x10000
    for f in ("kbar", "vbar", "kbar_scale", "vbar_scale", "kbar_stage", "vbar_stage", "ring_k", "ring_v", "block_stage",
                  "ring_k_scale", "ring_v_scale", "kbar_gscale", "vbar_gscale"):
        for l in range(cfg.n_layers):
            getattr(b, f)[l] = fake
    b.block_table = fake
    b.workspace = 0x20000
    b.workspace_bytes = B.csa_workspace_size(cfg, 4, 1)
    h = B.csa_cache_create(cfg, b)
    try:
        L = B.lib()
        i32 = lambda xs: (C.c_int32 * len(xs))(*xs)
        s = C.c_void_p(0)
        f = C.c_void_p(fake)
        assert L.csa_index_topk(C.c_void_p(h), 1, i32([0]), i32([0]), f, f, 16, f, s) == 5
        assert L.csa_compress(C.c_void_p(h), 0, 1, i32([0]), i32([4]), f, f, f, f, s) == 1
    finally:
        B.csa_cache_destroy(h)


def test_fp4_config_sizes_and_buffers():
    """FP4 main KV: packed E2M1 rows (64 bytes), one E4M3 code per 16 channels of
    an entry, fp8 indexer keys with page scales and staging, no K/V staging."""
    cfg = _spec(kv_dtype=B.CSA_FP4_E2M1)
    sz = B.csa_buffer_sizes_for(cfg)
    P, S = cfg.pool_pages, cfg.max_seqs
    assert sz.kv_pool == P * 64 * 64
    assert sz.group_scale == P * 64 * 8
    assert sz.idx_pool == P * 64 * 64
    assert sz.page_scale == P * 4 and sz.idx_stage == S * 64 * 64 * 4 and sz.kv_stage == 0
    assert B.csa_buffer_sizes_for(_spec()).group_scale == 0
    with pytest.raises(B.CsaError) as e:
        B.csa_buffer_sizes_for(_spec(kv_dtype=B.CSA_FP4_E2M1, act_dtype=B.CSA_F32, swa_dtype=B.CSA_F32))
    assert e.value.status == 3
    # group scales are required
    b = B.Buffers()
    for l in range(cfg.n_layers):
        for f in ("kbar", "vbar", "ring_k", "ring_v", "block_stage"):
            getattr(b, f)[l] = 0x10000
    b.kidx = b.kidx_scale = b.kidx_stage = b.block_table = 0x10000
    b.workspace, b.workspace_bytes = 0x100000, B.csa_workspace_size(cfg, 8, 512)
    with pytest.raises(B.CsaError):
        B.csa_cache_create(cfg, b)
    for l in range(cfg.n_layers):
        b.kbar_gscale[l] = b.vbar_gscale[l] = 0x10000
    B.csa_cache_destroy(B.csa_cache_create(cfg, b))


def test_long_chunks_are_indexed_query_by_query():
    """A chunk whose last query sees more entries than the chunk select takes
    (262,144) is planned by the per-query index path, which scans up to 2M
    entries a query; a shorter chunk by the chunk path. A 1 MiB workspace fits
    neither plan, so each shows itself through its own capacity error, raised
    on the host before anything is enqueued."""
    cfg = _spec(n_layers=1, max_seqs=1, max_pages_per_seq=4300, pool_pages=4300)
    h = _fake_handle(cfg, workspace_bytes=1 << 20)
    L = B.lib()
    fake = C.c_void_p(0x10000)
    s = C.c_void_p(0)
    i32 = B._i32
    try:
        for n_vis, plan in ((4200 * 64, b"one by one"), (262144, b"-token chunk"), (200000, b"-token chunk")):
            length = 4 * n_vis + 3
            B.csa_seq_set_len(h, 0, 0, length)
            pos = list(range(length - 8, length))
            assert L.csa_index_topk(C.c_void_p(h), 8, i32([0] * 8), i32(pos), fake, fake, 16, fake, s) == 4
            assert plan in L.csa_last_error(), (n_vis, L.csa_last_error())
            assert L.csa_index_topk_pool(C.c_void_p(h), 8, i32([0] * 8), i32(pos), fake, fake, 16, fake, 64,
                                         fake, s) == 4
            assert plan in L.csa_last_error(), (n_vis, L.csa_last_error())
    finally:
        B.csa_cache_destroy(h)
