"""Oracle: committing the accepted path of a verified draft tree into the paged KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Adaptive Speculative Decoding", section Layout: each row of the batch keeps its own
length, writes go to the row's own offset, and rollback is a length update, because the cache mask
never lets a query read past the row's length.  Read here for a tree: the verification forward
wrote node i of sequence b at slot ctx_len + i; after acceptance the committed tokens are the root
(already at slot ctx_len) followed by the accepted drafts, so the draft at depth i (node path[i])
must sit at slot ctx_len + i, and the new length is ctx_len + 1 + number accepted.  Everything past
the new length is stale and unreadable.  ("The controller": k accepted drafts add k + 1 tokens, the
last of them the bonus token, whose K/V the next verification writes as its root.)

Pools are bf16 bit patterns (uint16) [pages][kv_heads][page_size][head_dim], or for a dim-major V
pool [pages][kv_heads][head_dim][page_size]; one pool per layer.
"""

from __future__ import annotations

import numpy as np


def _slot_view(pool, v_layout: int):
    """The pool as [pages][kv_heads][page_size][head_dim] (a view; writes go to the pool)."""
    return np.swapaxes(pool, 2, 3) if v_layout else pool


def kv_commit(k_pools, v_pools, block_table, ctx_lens, num_accepted, path_nodes, page_size: int,
              v_layout: int = 0, max_nodes: int | None = None):
    """Returns (new k pools, new v pools, new ctx_lens); the inputs are not modified.

    For every sequence b with num_accepted[b] = n >= 0 and every layer, K and V of slot
    ctx_lens[b] + path_nodes[b][i] are copied to slot ctx_lens[b] + i for i = 1..n, in increasing i
    (each row's source is read before any later row overwrites it: path[i] >= i).  A sequence with
    n < 0 keeps its cache and length."""
    k_new = [np.array(k, copy=True) for k in k_pools]
    v_new = [np.array(v, copy=True) for v in v_pools]
    bt = np.asarray(block_table)
    lens = np.asarray(ctx_lens).astype(np.int64).copy()
    for b in range(len(lens)):
        n = int(num_accepted[b])
        if n < 0:
            continue
        L = int(lens[b])
        path = [int(x) for x in path_nodes[b][:n + 1]]
        for i in range(1, n + 1):
            node = path[i]
            if node == i:
                continue
            if not (i < node and (max_nodes is None or node < max_nodes)):
                raise ValueError(f"path node {node} at depth {i}: a node at depth i has index >= i")
            src, dst = L + node, L + i
            ps, rs = bt[b, src // page_size], src % page_size
            pd, rd = bt[b, dst // page_size], dst % page_size
            for layer in range(len(k_new)):
                k_new[layer][pd, :, rd, :] = k_new[layer][ps, :, rs, :]
                vv = _slot_view(v_new[layer], v_layout)
                vv[pd, :, rd, :] = vv[ps, :, rs, :].copy()
        lens[b] = L + 1 + n
    return k_new, v_new, lens.astype(np.int32)
