"""Oracle: tree-masked attention over a paged KV cache, and the per-chunk attention mass.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (the pages are cited by title and section):

* "DiffSpec: Accelerating Long Sequence Generation with Differential Speculative
  Decoding" (vllm-diffspec README), section "What DiffSpec Does", item 5: all
  candidates of the speculative structure are verified together, exploiting their
  shared prefix.  Read here as: every draft-tree node is a query of one target
  forward; it attends to the whole committed context and to its own ancestors in
  the tree (itself included), and to nothing else.
* "Adaptive Speculative Decoding", section Layout (specdec/kvcache.py): a row's
  query j may read cache slots s <= lengths[b] + j; a chain of drafts is the
  special case of the tree in which the ancestors of node j are nodes 0..j.
* same DiffSpec README, sections "What DiffSpec Does" (item 2) and Architecture
  ("Target-guided retrieval"): context chunks are scored from the paged target KV
  by an attention-derived signal.  Read here as the attention probability mass that
  the verification queries put on each chunk of the committed context, averaged
  over all tree nodes and query heads.
* DiffSpec README (CGCL-codes), section Features ("Chunk Arena and Paged KV"): K/V
  live in fixed-size pages addressed through a per-sequence block table.

Conventions: K/V pools are bf16 bit patterns [pages][kv_heads][page_size][head_dim]
(a dim-major V pool, [pages][kv_heads][head_dim][page_size], is read through the same
indices with the last two swapped); logical slot t of sequence b lives in page
block_table[b][t // page_size] at row t % page_size.  Node i of sequence b owns slot ctx_len[b] + i.  Query head h reads
KV head h // (num_q_heads // num_kv_heads).  Everything is computed in float64.
"""

from __future__ import annotations

import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64; exact."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def ancestor_matrix(parents) -> np.ndarray:
    """anc[i, j] is True iff node j is node i or one of its ancestors.

    The tree is given by sequence-local parents with parents[0] = -1 (the root, i.e. the last
    committed token) and 0 <= parents[i] < i, so each row is its parent's row plus itself."""
    parents = np.asarray(parents, dtype=np.int64)
    n = len(parents)
    if n == 0:
        return np.zeros((0, 0), dtype=bool)
    if parents[0] != -1:
        raise ValueError("node 0 must be the root (parent -1)")
    anc = np.zeros((n, n), dtype=bool)
    for i in range(n):
        if i > 0 and not (0 <= parents[i] < i):
            raise ValueError(f"parents[{i}] = {parents[i]} must satisfy 0 <= parent < {i}")
        if i > 0:
            anc[i] = anc[parents[i]]
        anc[i, i] = True
    return anc


def gather_kv(pool, block_table_row, n_slots: int, page_size: int, kv_head=None) -> np.ndarray:
    """Logical K or V rows 0..n_slots-1 of one sequence, through its block table -> float64
    [n_slots][kv_heads][head_dim] (or [n_slots][head_dim] for one ``kv_head``)."""
    t = np.arange(n_slots)
    pages = np.asarray(block_table_row)[t // page_size]
    if n_slots and pages.min() < 0:
        raise ValueError("block table has no page for a needed slot")
    if kv_head is None:
        return bf16_to_f64(pool[pages, :, t % page_size, :])
    return bf16_to_f64(pool[pages, kv_head, t % page_size, :])


def tree_attention(q_bits, k_pool, v_pool, block_table, ctx_lens, node_offsets, parents, scale: float,
                   num_kv_heads: int, page_size: int = 16, chunk_size: int = 0, kv_heads=None, seqs=None,
                   v_layout: int = 0):
    """Tree verification attention (float64).

    For sequence b with committed context length L and tree node i, query head h with KV head g, the
    visible keys are {0..L-1} U {L + j : j ancestor-or-self of i}.  out = softmax(scale * q k^T) v over
    exactly those keys; lse is the natural log of the softmax denominator.

    With ``chunk_size`` > 0 it also returns, per sequence, the attention mass of context chunk c
    (tokens [c*chunk_size, min((c+1)*chunk_size, L))), summed over the chunk's keys and averaged over
    all N nodes and all query heads of the sequence; tree keys belong to no chunk.

    ``kv_heads`` / ``seqs`` restrict the work to a subset (other outputs stay NaN; a mass computed
    over a KV-head subset averages over that subset's query heads only).  ``v_layout`` 1: ``v_pool`` is
    dim-major, [pages][kv_heads][head_dim][page_size].

    Returns (out [T][Hq][D], lse [T][Hq], masses: list of [n_chunks] arrays or None)."""
    q = np.asarray(q_bits)
    T, Hq, D = q.shape
    if v_layout:
        v_pool = np.swapaxes(np.asarray(v_pool), 2, 3)     # back to [pages][kv_heads][page_size][head_dim]
    G = Hq // num_kv_heads
    out = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    masses = [] if chunk_size else None
    kv_heads = range(num_kv_heads) if kv_heads is None else list(kv_heads)
    seqs = range(len(ctx_lens)) if seqs is None else list(seqs)
    for b in seqs:
        L = int(ctx_lens[b])
        n0, n1 = int(node_offsets[b]), int(node_offsets[b + 1])
        N = n1 - n0
        if N == 0:
            if chunk_size:
                masses.append(np.zeros((L + chunk_size - 1) // chunk_size))
            continue
        anc = ancestor_matrix(parents[n0:n1])
        visible = np.concatenate([np.ones((N, L), dtype=bool), anc], axis=1)   # [N][L+N]
        mass = np.zeros((L + chunk_size - 1) // chunk_size) if chunk_size else None
        for g in kv_heads:
            k = gather_kv(k_pool, block_table[b], L + N, page_size, g)
            v = gather_kv(v_pool, block_table[b], L + N, page_size, g)
            qg = bf16_to_f64(q[n0:n1, g * G:(g + 1) * G, :]).reshape(N * G, D)   # row = node*G + head
            s = scale * (qg @ k.T)
            vis = np.repeat(visible, G, axis=0)
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.where(vis, np.exp(s - m), 0.0)
            z = e.sum(axis=1, keepdims=True)
            p = e / z
            o = p @ v
            out[n0:n1, g * G:(g + 1) * G, :] = o.reshape(N, G, D)
            lse[n0:n1, g * G:(g + 1) * G] = (m + np.log(z)).reshape(N, G)
            if chunk_size:
                pc = p[:, :L].sum(axis=0)                       # mass of every context key over rows
                for c in range(len(mass)):
                    mass[c] += pc[c * chunk_size:min((c + 1) * chunk_size, L)].sum()
        if chunk_size:
            masses.append(mass / (N * G * len(kv_heads)))
    return out, lse, masses


def topk_chunks(mass, k: int):
    """The k chunks of largest mass, ordered by (mass descending, chunk index ascending); padded with
    index -1 and mass 0 when there are fewer than k chunks."""
    mass = np.asarray(mass, dtype=np.float64)
    order = sorted(range(len(mass)), key=lambda c: (-mass[c], c))[:k]
    idx = np.full(k, -1, dtype=np.int64)
    val = np.zeros(k)
    idx[:len(order)] = order
    val[:len(order)] = mass[order]
    return idx, val
