"""Shared helpers for the GPU parity tests: build caches from seeded inputs,
write oracle-made cache contents into device pools, and compare results.

The oracle side only ever sees values generated here or computed by the
oracle itself; nothing read back from the GPU is fed to it.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from compressed_sparse_attention_csa_amd import binding as B
from compressed_sparse_attention_csa_amd import synth as Sy
from compressed_sparse_attention_csa_amd.cache import CacheSpec, CsaCache
from oracle import csa_oracle as O

import parity_bounds as PB

TORCH_ACT = {"f32": torch.float32, "bf16": torch.bfloat16}
TOL = {"f32": 2e-3, "bf16": 2e-2}


def to64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a CPU/GPU tensor's values."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def shuffled_block_table(seed: int, max_seqs: int, max_pages: int, pool_pages: int, device="cuda") -> torch.Tensor:
    perm = Sy.permutation(seed, pool_pages, salt=7)
    assert pool_pages >= max_seqs * max_pages
    bt = torch.tensor(perm[: max_seqs * max_pages], dtype=torch.int32).view(max_seqs, max_pages)
    return bt.to(device)


def make_cache(seed=0, **kw) -> CsaCache:
    spec = CacheSpec(**kw)
    bt = shuffled_block_table(seed, spec.max_seqs, spec.max_pages_per_seq, spec.pool_pages)
    return CsaCache(spec, "cuda", block_table=bt)


def raw_rows(seed, kind, layer, seq, row0, n, act, device="cpu"):
    return Sy.normal_rows(seed, Sy.stream_id(kind, layer, seq), row0, n, 128, device=device, dtype=TORCH_ACT[act])


# --------------------------------------------------------------------------- writing oracle contents

def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """E2M1 codes [E, D] -> bytes [E, D/2], channel 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8) & 0xF
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def store_raw_to_torch(raw, dtype: str):
    """Oracle cache payload -> torch tensor of the pool's element type (CPU)."""
    if dtype == "fp4":
        return torch.from_numpy(np.ascontiguousarray(pack_fp4(raw[0])))
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(raw))
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16)
    codes, _ = raw
    return torch.from_numpy(np.ascontiguousarray(codes))


def write_logical(cache: CsaCache, pool: torch.Tensor, seq: int, values: torch.Tensor):
    """Write logical entries [0, E) of `seq` into their physical pages."""
    E = values.shape[0]
    if E == 0:
        return
    n_pages = (E + 63) // 64
    padded = torch.zeros((n_pages * 64, *values.shape[1:]), dtype=values.dtype)
    padded[:E] = values
    pages = cache.block_table[seq, :n_pages].long()
    pool[pages] = padded.view(n_pages, 64, *values.shape[1:]).to(pool.device)


def write_scales(cache: CsaCache, scales_t: torch.Tensor, seq: int, scales: np.ndarray):
    n = scales.shape[0]
    if n == 0:
        return
    pages = cache.block_table[seq, :n].long()
    scales_t[pages] = torch.from_numpy(scales.astype(np.float32)).to(scales_t.device)


def fill_index_keys(cache: CsaCache, seed: int, seq: int, n_entries: int):
    """Seeded indexer keys for `seq`, stored through the oracle's codec. Returns decoded float64 values."""
    x = Sy.normal_rows(seed, Sy.stream_id(Sy.KIND_KI, 0, seq), 0, n_entries, 64).double().numpy()
    dt = "fp8" if cache.spec.kv_dtype == "fp4" else cache.spec.kv_dtype   # fp4 caches keep fp8 indexer keys
    vals, raw = O.store(x, dt)
    write_logical(cache, cache.kidx, seq, store_raw_to_torch(raw, dt))
    if dt == "fp8":
        write_scales(cache, cache.kidx_scale, seq, raw[1])
    return vals


def fill_main_kv(cache: CsaCache, seed: int, layer: int, seq: int, n_entries: int):
    """Seeded compressed K/V for (layer, seq) stored through the oracle's codec."""
    dt = cache.spec.kv_dtype
    out = []
    for kind, pool, scales, gsc in ((Sy.KIND_KBAR, cache.kbar[layer], cache.kbar_scale, cache.kbar_gscale),
                                    (Sy.KIND_VBAR, cache.vbar[layer], cache.vbar_scale, cache.vbar_gscale)):
        x = Sy.normal_rows(seed, Sy.stream_id(kind, layer, seq), 0, n_entries, 128).double().numpy()
        vals, raw = O.store(x, dt)
        write_logical(cache, pool, seq, store_raw_to_torch(raw, dt))
        if dt == "fp8":
            write_scales(cache, scales[layer], seq, raw[1])
        if dt == "fp4":
            write_logical(cache, gsc[layer], seq, torch.from_numpy(np.ascontiguousarray(raw[1])))
        out.append(vals)
    return out


def fill_ring(cache: CsaCache, seed: int, layer: int, seq: int, length: int):
    """Raw K/V rows of (layer, seq) for positions [length - R, length) into the ring.
    Returns float64 (K, V) for rows [0, length) — rows older than the ring are
    returned too (the oracle may index them; the GPU must not need them)."""
    act = cache.spec.act_dtype
    K = raw_rows(seed, Sy.KIND_K, layer, seq, 0, length, act)
    V = raw_rows(seed, Sy.KIND_V, layer, seq, 0, length, act)
    return write_ring_rows(cache, layer, seq, 0, K, V)


def write_ring_rows(cache: CsaCache, layer: int, seq: int, row0: int, K: torch.Tensor, V: torch.Tensor):
    """Raw rows [row0, row0 + n) into the ring slots of the newest R of them,
    through the oracle's ring codec (per-row E4M3 for an fp8 ring). Returns
    float64 (K, V) as the ring holds them (older rows: the raw values)."""
    R = cache.cfg.ring_rows
    n = K.shape[0]
    lo = max(0, n - R)
    rows = torch.arange(row0 + lo, row0 + n)
    out = []
    for x, ring, scales in ((K, cache.ring_k[layer], cache.ring_k_scale), (V, cache.ring_v[layer], cache.ring_v_scale)):
        x64 = to64(x)
        if cache.spec.swa_dtype == "fp8":
            vals, (codes, sc) = O.store_ring_rows(x64[lo:], "fp8")
            ring[seq, rows % R] = torch.from_numpy(codes).to(cache.device)
            scales[layer][seq, rows % R] = torch.from_numpy(sc).to(cache.device)
            x64[lo:] = vals
        else:
            ring[seq, rows % R] = x[lo:].to(cache.device)
        out.append(x64)
    return tuple(out)


# --------------------------------------------------------------------------- comparisons

def topk_matches(gpu_T: np.ndarray, oracle_T: np.ndarray, oracle_scores: np.ndarray, rel=1e-6):
    """Index sets equal, except entries whose oracle score is within `rel` of the
    oracle's k-th score (near-ties that fp32 accumulation order may swap).
    Returns (ok, message)."""
    g = [int(x) for x in gpu_T if x >= 0]
    o = [int(x) for x in oracle_T if x >= 0]
    if len(g) != len(o):
        return False, f"count {len(g)} != {len(o)}"
    if list(gpu_T) != sorted(g) + [-1] * (len(gpu_T) - len(g)):
        return False, "gpu row not ascending / badly padded"
    diff = set(g) ^ set(o)
    if not diff:
        return True, ""
    kth = min(float(oracle_scores[j]) for j in o)
    bad = [j for j in diff if abs(float(oracle_scores[j]) - kth) > rel * max(abs(kth), 1e-30)]
    if bad:
        return False, f"{len(diff)} differing, {len(bad)} outside the tie band, e.g. {bad[:5]} (kth={kth})"
    return True, f"{len(diff)} near-tie swaps"


def max_abs(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


# --------------------------------------------------------------------------- oracle entries with error bands

def oracle_entries(K64, V64, Z64, r, P64=None):
    """The oracle's compressed entries (float64, before rounding) and, for each
    value, the band within which a correct fp32 implementation may differ
    (parity_bounds.value_band of its absolute terms). Returns
    (kbar, vbar, kidx, band_kbar, band_vbar, band_kidx); kidx and its band are
    None without a projection."""
    kb, vb, ki = O.compress(K64, V64, Z64, r, P64)
    TK, TV, TI = PB.pooled_terms(K64, V64, Z64, r, P64)
    bi = None if TI is None else PB.value_band(TI, 128 + r + 8)
    return kb, vb, ki, PB.value_band(TK, r), PB.value_band(TV, r), bi


def check_topk_chain(gpu_row, qi64, w64, ki64, band_ki, kdtype, n_vis, k, what=""):
    """A Top-K row the GPU computed from keys it compressed itself, against the
    oracle's keys (ki64, all stored entries of the sequence): exact within the
    1e-6 relative band, except that keys whose stored codes may legitimately
    differ (parity_bounds.key_score_slack) carry their score slack."""
    return TopkRows(ki64, band_ki, kdtype).check(gpu_row, qi64, w64, n_vis, k, what)


def check_stored_pool(cache, pool, scales, seq, n, x64, band, kv, what):
    """GPU pool contents of one stream vs the oracle's rounding of x64: fp32
    values within the fp32 error band of the exact values; bf16 and E4M3
    codes equal, except where a value lies within its error band of a rounding
    boundary (then the other rounding is allowed, and counted); E4M3 page
    scales within the uncertainty of their page's amax."""
    got_raw = cache.logical(pool, seq, n).cpu()
    x64, band = x64[:n], band[:n]
    if kv == "f32":
        err = np.abs(got_raw.double().numpy() - x64)
        assert np.all(err <= band), (what, float(np.max(err / band)))
        return
    if kv == "bf16":
        allowed, bad = PB.check_stored(got_raw.view(torch.int16).numpy().view(np.uint16), x64, band, "bf16")
    else:
        codes, oscales, _, _, rel_s = PB.fp8_pages(x64, band)
        gs = cache.logical_scales(scales, seq, n).cpu().double().numpy()
        os64 = oscales.astype(np.float64)
        assert np.all(np.abs(gs - os64) <= os64 * (rel_s + 2 * PB.U32)), (what, "page scales")
        allowed, bad = PB.check_stored(got_raw.numpy(), x64, band, "fp8")
    assert bad == 0, f"{what}: {bad} codes differ from the oracle's rounding outside every error band"
    if allowed:
        print(f"[codes] {what}: {allowed} of {x64.size} codes at a rounding boundary take the other neighbour")


class TopkRows:
    """The oracle's indexer keys of one sequence (float64 before rounding, with
    their fp32 error bands), stored as the cache stores them, against which
    many Top-K rows are checked: scores of the stored keys, and per key the
    slack that legitimate code flips allow (parity_bounds.key_slack_parts)."""

    def __init__(self, ki64, band_ki, kdtype):
        self.dt = "fp8" if kdtype == "fp4" else kdtype   # fp4 caches keep fp8 indexer keys
        self.kis = O.store(ki64, self.dt)[0]
        self.M, self.rel = PB.key_slack_parts(ki64, band_ki, self.dt)

    def scores(self, qi64, w64, n_vis):
        return O.index_scores(qi64, w64, self.kis[:n_vis])

    def slack(self, qi64, w64, s, n_vis):
        coef = (np.asarray(w64, np.float64)[:, None] * np.abs(np.asarray(qi64, np.float64))).sum(axis=0)
        return self.M[:n_vis] @ coef + self.rel[:n_vis] * np.abs(np.asarray(s, np.float64))

    def check(self, gpu_row, qi64, w64, n_vis, k, what=""):
        """Assert the GPU row is a valid Top-k; returns the oracle's scores."""
        s = self.scores(qi64, w64, n_vis)
        ok, msg = PB.topk_valid(gpu_row, s, k, self.slack(qi64, w64, s, n_vis))
        assert ok, f"{what}: {msg}"
        if msg:
            print(f"[topk] {what}: {msg}")
        return s
