"""Oracle: the compact draft KV built from the selected context chunks and the recent window.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: DiffSpec (vllm-diffspec README).
  - "What DiffSpec Does", item 2: the draft model keeps the important long-range context inside a
    bounded working set.
  - The paragraph after that list: the chunks chosen from the target's paged KV are joined with a
    rolling window of recent tokens and rebuilt as a compact draft cache at local positions.
  - "Architecture": the draft cache has two views.  The canonical view is pre-RoPE K/V at absolute
    positions; the compact view is rebuilt with RoPE at local draft positions.
  - "Configuration": chunk size 64 and a token budget of 2048 for the compact draft context.

Readings (the pages give no formula; these are the plainest ones that fit the passages):
  - Selection.  Take sequence b with L committed tokens and recent window W, and let w0 = max(0, L - W).
    Token t in [0, L) is kept iff t >= w0 or its chunk t // chunk_size is in the selected list.
    Ids that are out of range, -1 padding and repeated ids select nothing more.
  - Order.  Kept tokens keep their context order.  Compact slot j holds the j-th kept token, so
    local positions are 0, 1, 2, ... with no gaps.
  - RoPE.  K is rotated at local position j and V is copied unchanged.
    rope = 0 copies K as stored (the compact cache stays pre-RoPE; position j is implicit).
    rope = 1 rotates each pair (d, d + D/2).
    rope = 2 rotates each pair (2i, 2i + 1).
    Pair i is turned by the angle j * inv_freq[i]; inv_freq is given by the caller.
  - Budget.  The caller's capacity must hold num_select * chunk_size + W tokens, which bounds every
    possible selection.

Pools are bf16 bit patterns (uint16) [pages][kv_heads][page_size][head_dim].  A dim-major V pool is
[pages][kv_heads][head_dim][page_size].
"""

from __future__ import annotations

import numpy as np

from .attention import bf16_to_f64


def selected_positions(L: int, chunk_ids, chunk_size: int, window: int) -> np.ndarray:
    """Context positions kept for the draft, in increasing order."""
    w0 = max(0, L - window)
    keep = set(range(w0, L))
    for c in chunk_ids:
        c = int(c)
        if c >= 0 and c * chunk_size < L:
            keep.update(range(c * chunk_size, min((c + 1) * chunk_size, L)))
    return np.array(sorted(keep), dtype=np.int64)


def rope(x: np.ndarray, positions: np.ndarray, inv_freq: np.ndarray, style: int) -> np.ndarray:
    """x float64 [n][heads][D], rotated at positions[n]; style as in the module docstring."""
    if style == 0:
        return x.copy()
    D = x.shape[-1]
    ang = np.asarray(positions, dtype=np.float64)[:, None] * np.asarray(inv_freq, dtype=np.float64)[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    out = np.empty_like(x)
    if style == 1:
        a, b = x[..., :D // 2], x[..., D // 2:]
        out[..., :D // 2] = a * c - b * s
        out[..., D // 2:] = b * c + a * s
    elif style == 2:
        a, b = x[..., 0::2], x[..., 1::2]
        out[..., 0::2] = a * c - b * s
        out[..., 1::2] = b * c + a * s
    else:
        raise ValueError(f"rope style {style}")
    return out


def draft_gather(k_pool, v_pool, block_table, ctx_lens, chunk_index, page_size: int, chunk_size: int,
                 window: int, capacity: int, inv_freq=None, rope_style: int = 1, v_layout: int = 0):
    """Returns (out_k, out_v, out_pos, out_len).

    out_k and out_v are float64 [batch][capacity][kv_heads][D]; slots at or past out_len are NaN.
    out_pos is int32 [batch][capacity] (the absolute position of each slot, -1 past out_len).
    out_len is int32 [batch].  chunk_index is [batch][num_select]."""
    bt = np.asarray(block_table)
    B = len(ctx_lens)
    H, D = k_pool.shape[1], k_pool.shape[3]
    vpool = np.swapaxes(v_pool, 2, 3) if v_layout else v_pool
    out_k = np.full((B, capacity, H, D), np.nan)
    out_v = np.full((B, capacity, H, D), np.nan)
    out_pos = np.full((B, capacity), -1, dtype=np.int32)
    out_len = np.zeros(B, dtype=np.int32)
    for b in range(B):
        L = int(ctx_lens[b])
        pos = selected_positions(L, chunk_index[b], chunk_size, window)
        n = len(pos)
        if n > capacity:
            raise ValueError(f"sequence {b}: {n} kept tokens exceed the capacity {capacity}")
        pages, rows = bt[b, pos // page_size], pos % page_size
        kr = bf16_to_f64(k_pool[pages, :, rows, :])          # [n][H][D]
        vr = bf16_to_f64(vpool[pages, :, rows, :])
        out_k[b, :n] = rope(kr, np.arange(n), inv_freq, rope_style) if n else kr
        out_v[b, :n] = vr
        out_pos[b, :n] = pos
        out_len[b] = n
    return out_k, out_v, out_pos, out_len
