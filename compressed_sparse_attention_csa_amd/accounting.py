"""Byte and FLOP accounting for the CSA step (algorithmic, not measured).

These are the quantities a roofline compares against: bytes the method must
move from HBM, FLOPs it must perform. Written per unit so the totals can be
re-derived by hand.
"""
from __future__ import annotations

DTYPE_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}


def kv_cache_bytes_per_token(n_layers: int, n_kv_heads: int, d_head: int, elem_bytes: int) -> int:
    """Uncompressed K+V cache per token: 2 x layers x KV heads x head dim x bytes.

    The formula the Model-architectures atlas gives in its MQA/GQA entry.
    """
    return 2 * n_layers * n_kv_heads * d_head * elem_bytes


def index_scan_bytes(n_entries: int, d_i: int, kv_dtype: str, page_entries: int = 64) -> int:
    """Bytes one query's indexer scan reads: its visible indexer keys (+ page
    scales). Caches with fp4 K/V keep fp8 indexer keys."""
    kv_dtype = "fp8" if kv_dtype == "fp4" else kv_dtype
    b = n_entries * d_i * DTYPE_BYTES[kv_dtype]
    if kv_dtype == "fp8":
        b += -(-n_entries // page_entries) * 4
    return b


def attend_bytes(k_sel: int, window: int, d: int, h_q: int, kv_dtype: str, act_dtype: str,
                 swa_dtype: str | None = None) -> int:
    """Bytes one query's attention reads and writes for one layer.

    Gathered compressed K and V rows (plus one K and one V page scale per
    gathered entry for fp8), the window's K and V rows in the ring's format
    (plus one K and one V row scale each for an fp8 ring), the query, the
    output, and the Top-K row it reads.
    """
    ab = DTYPE_BYTES[act_dtype]
    sd = swa_dtype or act_dtype
    if kv_dtype == "fp4":                 # d/2 code bytes + d/16 E4M3 group-scale bytes per row
        b = k_sel * 2 * (d // 2 + d // 16)
    else:
        b = k_sel * 2 * d * DTYPE_BYTES[kv_dtype]
    if kv_dtype == "fp8":
        b += k_sel * 2 * 4
    b += window * 2 * d * DTYPE_BYTES[sd]
    if sd == "fp8":
        b += window * 2 * 4
    b += 2 * h_q * d * ab
    b += k_sel * 4
    return b


def compress_bytes(old_len: int, n_new: int, r: int, d: int, d_i: int, kv_dtype: str, act_dtype: str,
                   ring_rows: int, swa_dtype: str | None = None, with_index: bool = True, page: int = 64) -> int:
    """Bytes one sequence's append of n_new raw rows after old_len moves in one
    layer (csa_compress).

    Read: the new rows' gate logits, keys and values; the open block's earlier
    rows from block staging when that block closes now; for fp8 pages, the
    fp32 staging of each touched page's earlier entries (a page's scale is its
    amax, so its earlier entries are re-encoded) and, with the indexer, the
    projection matrix once. Written: the newest min(n_new, R) keys and values
    into the window ring (plus one scale per row for an fp8 ring); the rows
    of the block still open afterwards into block staging; the new entries'
    K, V (and indexer key) codes - for fp8 pages every filled slot of each
    touched page, its scales, and the fp32 staging of the new entries while
    the page stays open; for fp4 K/V, the new entries' codes and group scales
    with fp8 indexer keys handled as an fp8 page.
    """
    ab = DTYPE_BYTES[act_dtype]
    sd = swa_dtype or act_dtype
    di = d_i if with_index else 0
    new_len = old_len + n_new
    nb_old, nb_new = old_len // r, new_len // r
    b = n_new * 3 * d * ab
    if nb_new > nb_old:
        b += (old_len - nb_old * r) * 3 * d * ab
    b += (new_len - max(old_len, nb_new * r)) * 3 * d * ab
    ring = min(n_new, ring_rows)
    b += ring * 2 * d * (1 if sd == "fp8" else DTYPE_BYTES[sd]) + (ring * 2 * 4 if sd == "fp8" else 0)
    if nb_new == nb_old:
        return b
    if di:
        b += d * di * 4
    for p in range(nb_old // page, (nb_new - 1) // page + 1):
        p0 = p * page
        e0, e1 = max(p0, nb_old), min(p0 + page, nb_new)
        filled, new = e1 - p0, e1 - e0
        still_open = filled < page
        if kv_dtype == "fp8":
            b += (e0 - p0) * (2 * d + di) * 4
            b += filled * (2 * d + di) + (3 if di else 2) * 4
            if still_open:
                b += new * (2 * d + di) * 4
        elif kv_dtype == "fp4":
            b += new * 2 * (d // 2 + d // 16)
            if di:
                b += (e0 - p0) * di * 4 + filled * di + 4
                if still_open:
                    b += new * di * 4
        else:
            b += new * (2 * d + di) * DTYPE_BYTES[kv_dtype]
    return b


def reindex_bytes(pool_entries: int, n_blocks: int, d_i: int, kv_dtype: str) -> int:
    """Bytes one query's Reindex scores read: the pool's indexer keys, its
    block ids and (fp8) one page scale per block (an aligned 8-entry block
    lies inside one 64-entry page)."""
    b = pool_entries * d_i * DTYPE_BYTES[kv_dtype] + n_blocks * 4
    if kv_dtype == "fp8":
        b += n_blocks * 4
    return b


def decode_step_bytes(n_seq: int, entries: list[int] | int, d: int, d_i: int, h_q: int, h_i: int,
                      k: int, window: int, group: int, kv_dtype: str, act_dtype: str,
                      swa_dtype: str | None = None) -> int:
    """Algorithmic HBM bytes of one decode step: one index pass + `group` attends.

    entries: visible compressed entries per sequence (one int for all, or a list).
    """
    if isinstance(entries, int):
        entries = [entries] * n_seq
    ab = DTYPE_BYTES[act_dtype]
    total = 0
    for n in entries:
        total += index_scan_bytes(n, d_i, kv_dtype)
        total += h_i * d_i * ab + h_i * 4 + k * 4          # q_idx, w, Top-K row written
        k_sel = min(k, n)
        total += group * attend_bytes(k_sel, window, d, h_q, kv_dtype, act_dtype, swa_dtype)
    return total


def index_flops(n_scores: int, h_i: int, d_i: int) -> int:
    """Multiply-adds of the indexer, counted as 2 FLOP each, per visible score."""
    return n_scores * h_i * d_i * 2


def attend_flops(n_queries: int, h_q: int, n_keys: int, d: int) -> int:
    """QK^T and PV: 2 x 2 x heads x keys x dim per query."""
    return n_queries * h_q * n_keys * d * 4


def prefill_visible_scores(prior_tokens: int, chunk: int, r: int) -> int:
    """Visible (query, entry) pairs of a prefill chunk: query t sees (t+1)//r entries."""
    return sum((prior_tokens + tau + 1) // r for tau in range(chunk))
