"""Device buffers of one CSA layer group, allocated with torch, plus the handle.

The library never allocates device memory; this class sizes every buffer
from the library's own size query, allocates it as a torch tensor on the
chosen device and creates the handle over those pointers. The tensors are
plain views of the cache so tests can read (and, for isolated tests, write)
pages directly.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import binding as B

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8, "fp4": torch.uint8}


@dataclass
class CacheSpec:
    ratio: int = 4
    q_heads: int = 64
    idx_heads: int = 4
    window: int = 128
    ring_rows: int = 0            # 0: max(window, ratio)
    n_layers: int = 1
    max_seqs: int = 1
    max_pages_per_seq: int = 1
    pool_pages: int = 1
    kv_dtype: str = "bf16"
    act_dtype: str = "bf16"
    swa_dtype: str = ""           # "": act_dtype; "fp8": E4M3 window ring with per-row scales
    max_queries: int = 1
    max_k: int = 512

    def config(self) -> B.Config:
        c = B.Config()
        c.ratio = self.ratio
        c.head_dim = B.CSA_HEAD_DIM
        c.q_heads = self.q_heads
        c.idx_heads = self.idx_heads
        c.idx_dim = B.CSA_IDX_DIM
        c.window = self.window
        c.ring_rows = self.ring_rows or max(self.window, self.ratio, 1)
        c.n_layers = self.n_layers
        c.max_seqs = self.max_seqs
        c.max_pages_per_seq = self.max_pages_per_seq
        c.pool_pages = self.pool_pages
        c.kv_dtype = B.DTYPE_CODES[self.kv_dtype]
        c.act_dtype = B.DTYPE_CODES[self.act_dtype]
        c.swa_dtype = B.DTYPE_CODES[self.swa_dtype or self.act_dtype]
        return c


class CsaCache:
    """A handle plus its torch-owned device buffers."""

    def __init__(self, spec: CacheSpec, device="cuda", block_table: torch.Tensor | None = None):
        self.spec = spec
        self.cfg = spec.config()
        self.device = torch.device(device)
        sz = B.csa_buffer_sizes_for(self.cfg)
        kvt = _TORCH_DT[spec.kv_dtype]
        actt = _TORCH_DT[spec.act_dtype]
        P, S, D, DI, L = spec.pool_pages, spec.max_seqs, B.CSA_HEAD_DIM, B.CSA_IDX_DIM, spec.n_layers
        R = self.cfg.ring_rows
        dev = self.device
        fp8, fp4 = spec.kv_dtype == "fp8", spec.kv_dtype == "fp4"
        row = D // 2 if fp4 else D           # fp4: two E2M1 codes per byte
        self.kbar = [torch.zeros((P, 64, row), dtype=kvt, device=dev) for _ in range(L)]
        self.vbar = [torch.zeros((P, 64, row), dtype=kvt, device=dev) for _ in range(L)]
        # fp4: one E4M3 scale code per 16 channels of every entry
        self.kbar_gscale = [torch.zeros((P, 64, D // 16), dtype=torch.uint8, device=dev) for _ in range(L)] if fp4 else []
        self.vbar_gscale = [torch.zeros((P, 64, D // 16), dtype=torch.uint8, device=dev) for _ in range(L)] if fp4 else []
        idx = spec.idx_heads > 0   # an HCA group (idx_heads = 0) has no indexer keys
        idx8 = fp8 or fp4          # fp4 main KV keeps fp8 indexer keys
        self.kidx = torch.zeros((P, 64, DI), dtype=kvt, device=dev) if idx else None
        self.kbar_scale = [torch.ones(P, dtype=torch.float32, device=dev) for _ in range(L)] if fp8 else []
        self.vbar_scale = [torch.ones(P, dtype=torch.float32, device=dev) for _ in range(L)] if fp8 else []
        self.kidx_scale = torch.ones(P, dtype=torch.float32, device=dev) if idx8 and idx else None
        self.kbar_stage = [torch.zeros((S, 64, D), dtype=torch.float32, device=dev) for _ in range(L)] if fp8 else []
        self.vbar_stage = [torch.zeros((S, 64, D), dtype=torch.float32, device=dev) for _ in range(L)] if fp8 else []
        self.kidx_stage = torch.zeros((S, 64, DI), dtype=torch.float32, device=dev) if idx8 and idx else None
        ring_fp8 = spec.swa_dtype == "fp8"
        ringt = torch.uint8 if ring_fp8 else actt
        self.ring_k = [torch.zeros((S, R, D), dtype=ringt, device=dev) for _ in range(L)]
        self.ring_v = [torch.zeros((S, R, D), dtype=ringt, device=dev) for _ in range(L)]
        self.ring_k_scale = [torch.ones((S, R), dtype=torch.float32, device=dev) for _ in range(L)] if ring_fp8 else []
        self.ring_v_scale = [torch.ones((S, R), dtype=torch.float32, device=dev) for _ in range(L)] if ring_fp8 else []
        # gate logits, raw keys and raw values of each sequence's open r-block
        self.block_stage = [torch.zeros((S, 3, spec.ratio, D), dtype=actt, device=dev) for _ in range(L)]
        if block_table is None:
            block_table = torch.full((S, spec.max_pages_per_seq), -1, dtype=torch.int32, device=dev)
        assert block_table.shape == (S, spec.max_pages_per_seq) and block_table.dtype == torch.int32
        self.block_table = block_table
        ws = B.csa_workspace_size(self.cfg, spec.max_queries, spec.max_k)
        if ws == 0:
            raise ValueError("invalid cache spec")
        self.workspace = torch.zeros(ws, dtype=torch.uint8, device=dev)
        assert sz.kv_pool == self.kbar[0].numel() * self.kbar[0].element_size()
        assert sz.ring == self.ring_k[0].numel() * self.ring_k[0].element_size()
        assert sz.block_stage == self.block_stage[0].numel() * self.block_stage[0].element_size()

        b = B.Buffers()
        for l in range(L):
            b.kbar[l] = self.kbar[l].data_ptr()
            b.vbar[l] = self.vbar[l].data_ptr()
            b.ring_k[l] = self.ring_k[l].data_ptr()
            b.ring_v[l] = self.ring_v[l].data_ptr()
            b.block_stage[l] = self.block_stage[l].data_ptr()
            if ring_fp8:
                b.ring_k_scale[l] = self.ring_k_scale[l].data_ptr()
                b.ring_v_scale[l] = self.ring_v_scale[l].data_ptr()
            if fp4:
                b.kbar_gscale[l] = self.kbar_gscale[l].data_ptr()
                b.vbar_gscale[l] = self.vbar_gscale[l].data_ptr()
            if fp8:
                b.kbar_scale[l] = self.kbar_scale[l].data_ptr()
                b.vbar_scale[l] = self.vbar_scale[l].data_ptr()
                b.kbar_stage[l] = self.kbar_stage[l].data_ptr()
                b.vbar_stage[l] = self.vbar_stage[l].data_ptr()
        if idx:
            b.kidx = self.kidx.data_ptr()
            if idx8:
                b.kidx_scale = self.kidx_scale.data_ptr()
                b.kidx_stage = self.kidx_stage.data_ptr()
        b.block_table = self.block_table.data_ptr()
        b.workspace = self.workspace.data_ptr()
        b.workspace_bytes = ws
        self._bufs = b
        self._swa = {}
        self.handle = B.csa_cache_create(self.cfg, b)

    def clone(self) -> "CsaCache":
        """Another cache with this one's contents: every device buffer copied,
        the same block table, sequence lengths and replay starts (replicas of
        one workload)."""
        c = CsaCache(self.spec, self.device, block_table=self.block_table)
        for name in ("kbar", "vbar", "kbar_gscale", "vbar_gscale", "kbar_scale", "vbar_scale", "kbar_stage",
                     "vbar_stage", "ring_k", "ring_v", "ring_k_scale", "ring_v_scale", "block_stage"):
            for src, dst in zip(getattr(self, name), getattr(c, name)):
                dst.copy_(src)
        for name in ("kidx", "kidx_scale", "kidx_stage"):
            if getattr(self, name) is not None:
                getattr(c, name).copy_(getattr(self, name))
        for layer in range(self.cfg.n_layers):
            for seq in range(self.cfg.max_seqs):
                n = B.csa_seq_len(self.handle, layer, seq)
                if n:
                    B.csa_seq_set_len(c.handle, layer, seq, n)
        for seq, start in self._swa.items():
            c.set_swa_start(seq, start)
        return c

    # ----------------------------------------------------------------- calls
    def compress(self, layer, seq_ids, n_new, raw_k, raw_v, gate, proj_idx=None, stream=None):
        B.csa_compress(self.handle, layer, seq_ids, n_new, raw_k, raw_v, gate, proj_idx, stream)

    def index_topk(self, q_seq, q_pos, q_idx, w_idx, k, topk=None, stream=None):
        if topk is None:
            topk = torch.empty((len(q_seq), k), dtype=torch.int32, device=self.device)
        B.csa_index_topk(self.handle, q_seq, q_pos, q_idx, w_idx, k, topk, stream)
        return topk

    def index_topk_pool(self, q_seq, q_pos, q_idx, w_idx, k, n_pool_blocks, topk=None, pool=None, stream=None):
        if topk is None:
            topk = torch.empty((len(q_seq), k), dtype=torch.int32, device=self.device)
        if pool is None:
            pool = torch.empty((len(q_seq), n_pool_blocks), dtype=torch.int32, device=self.device)
        B.csa_index_topk_pool(self.handle, q_seq, q_pos, q_idx, w_idx, k, topk, n_pool_blocks, pool, stream)
        return topk, pool

    def index_reindex(self, q_seq, q_pos, q_idx, w_idx, pool, k, topk=None, stream=None):
        if topk is None:
            topk = torch.empty((len(q_seq), k), dtype=torch.int32, device=self.device)
        B.csa_index_reindex(self.handle, q_seq, q_pos, q_idx, w_idx, pool.shape[1], pool, k, topk, stream)
        return topk

    def attend(self, layer, q_seq, q_pos, q, topk, k, scale, out=None, stream=None):
        if out is None:
            out = torch.empty_like(q)
        B.csa_attend(self.handle, layer, q_seq, q_pos, q, topk, k, scale, out, stream)
        return out

    def attend_noalloc(self, layer, q_seq, q_pos, q, topk, k, scale, out=None, stream=None):
        if out is None:
            out = torch.empty_like(q)
        B.csa_attend_noalloc(self.handle, layer, q_seq, q_pos, q, topk, k, scale, out, stream)
        return out

    def attend_dense(self, layer, q_seq, q_pos, q, scale, out=None, stream=None):
        if out is None:
            out = torch.empty_like(q)
        B.csa_attend_dense(self.handle, layer, q_seq, q_pos, q, scale, out, stream)
        return out

    def set_swa_start(self, seq, start):
        B.csa_seq_set_swa_start(self.handle, seq, start)
        self._swa[seq] = start

    def ring_write(self, layer, seq_ids, pos0, n_rows, raw_k, raw_v, stream=None):
        B.csa_ring_write(self.handle, layer, seq_ids, pos0, n_rows, raw_k, raw_v, stream)

    def seq_len(self, layer, seq):
        return B.csa_seq_len(self.handle, layer, seq)

    def read_errors(self, stream=None):
        return B.csa_read_errors(self.handle, stream)

    def close(self):
        if getattr(self, "handle", None):
            B.csa_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ----------------------------------------------------------------- views
    def logical(self, pool: torch.Tensor, seq: int, n_entries: int) -> torch.Tensor:
        """Entries [0, n_entries) of `seq` from a page pool, in logical order."""
        n_pages = (n_entries + 63) // 64
        pages = self.block_table[seq, :n_pages].long()
        return pool[pages].reshape(n_pages * 64, *pool.shape[2:])[:n_entries]

    def logical_scales(self, scales: torch.Tensor, seq: int, n_entries: int) -> torch.Tensor:
        n_pages = (n_entries + 63) // 64
        return scales[self.block_table[seq, :n_pages].long()]
