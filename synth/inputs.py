"""Seeded synthetic workloads for the verification step of tree speculative decoding.

Everything here is input generation: random draws, bf16 rounding of the draws,
page pools and block tables, draft-tree shapes, logits with a planted maximum,
the draft model's proposal distribution and uniforms.  Nothing here evaluates
the verification step itself.

Shapes follow the workloads the DiffSpec pages measure on (Llama-3.1-8B, batch
1, 32K to 128K input; "DiffSpec: Accelerating Long Sequence Generation with
Differential Speculative Decoding", section Key Results) and the Qwen3-8B
target of "Adaptive Speculative Decoding" (8 KV heads x 128 head_dim x bf16,
section "What made it tractable").  No real text, KV or weights are used.

Random streams: every draw comes from
``numpy.random.Generator(PCG64(SeedSequence([case, layer, stream])))`` with the
stream ids below, so each tensor can be regenerated on its own.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

PAGE_SIZE = 16

# stream ids for SeedSequence([case, layer, stream])
S_Q, S_K, S_V, S_BLOCKS, S_TREE, S_TARGET, S_DRAFT, S_TOKENS, S_UNIFORM, S_CTX = range(10)

BF16_QNAN = np.uint16(0x7FC0)

__all__ = [
    "PAGE_SIZE", "BF16_QNAN", "rng_for", "bf16_bits", "bf16_to_f32",
    "S_Q", "S_K", "S_V", "S_BLOCKS", "S_TREE", "S_TARGET", "S_DRAFT", "S_TOKENS", "S_UNIFORM", "S_CTX",
    "chain_tree", "random_tree", "tree_depths", "children_lists",
    "PagedKV", "paged_kv", "dim_major", "AttentionCase", "attention_case",
    "GreedyCase", "greedy_case", "RejectionCase", "rejection_case",
    "uniforms24", "ragged_ctx_lens", "rope_inv_freq", "chunk_selection", "WORKLOADS",
]


def rng_for(case: int, layer: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(case), int(layer), int(stream)])))


def bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = BF16_QNAN
    return r


def bf16_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def uniforms24(rng: np.random.Generator, n: int) -> np.ndarray:
    """Uniforms in [0, 1) on the 2^-24 grid, so that they are exact in float32 and float64."""
    return (rng.integers(0, 1 << 24, size=n, dtype=np.int64).astype(np.float64) * 2.0 ** -24).astype(np.float32)


# ----------------------------------------------------------------------------------------------
# draft trees (parents are sequence-local, parents[0] = -1, parents[i] < i)
# ----------------------------------------------------------------------------------------------

def chain_tree(n: int) -> np.ndarray:
    return np.arange(-1, n - 1, dtype=np.int32)


def tree_depths(parents) -> np.ndarray:
    parents = np.asarray(parents)
    d = np.zeros(len(parents), dtype=np.int32)
    for i in range(1, len(parents)):
        d[i] = d[parents[i]] + 1
    return d


def children_lists(parents):
    ch = [[] for _ in range(len(parents))]
    for i in range(1, len(parents)):
        ch[int(parents[i])].append(i)
    return ch


def random_tree(rng: np.random.Generator, n_nodes: int, depth: int, max_children: int = 4) -> np.ndarray:
    """Root 0, a spine 1..depth (so the depth is exactly ``depth``), then every further node picks a
    uniform parent among the nodes that are shallower than ``depth`` and have < ``max_children`` children."""
    if n_nodes < 1:
        raise ValueError("n_nodes >= 1")
    depth = min(depth, n_nodes - 1)
    parents = np.full(n_nodes, -1, dtype=np.int32)
    dep = np.zeros(n_nodes, dtype=np.int32)
    nch = np.zeros(n_nodes, dtype=np.int32)
    for i in range(1, depth + 1):
        parents[i] = i - 1
        dep[i] = i
        nch[i - 1] += 1
    for i in range(depth + 1, n_nodes):
        elig = np.nonzero((dep[:i] < depth) & (nch[:i] < max_children))[0]
        if len(elig) == 0:
            raise ValueError("tree too wide for depth/max_children")
        p = int(elig[rng.integers(len(elig))])
        parents[i] = p
        dep[i] = dep[p] + 1
        nch[p] += 1
    return parents


# ----------------------------------------------------------------------------------------------
# paged KV
# ----------------------------------------------------------------------------------------------

@dataclasses.dataclass
class PagedKV:
    k_pool: np.ndarray        # uint16 bf16 bits [pool_pages][Hkv][page_size][D]
    v_pool: np.ndarray        # same
    block_table: np.ndarray   # int32 [B][max_blocks], -1 past the sequence's pages
    slots: np.ndarray         # int32 [B] logical slots in use (context + tree nodes)
    page_size: int = PAGE_SIZE


def _normal_bf16(rng, shape, std=1.0):
    return bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def paged_kv(case: int, layer: int, slots, num_kv_heads: int, head_dim: int, *,
             page_size: int = PAGE_SIZE, pool_factor: float = 1.25, poison: bool = True,
             max_blocks: Optional[int] = None, perm_stream: int = S_BLOCKS, kv_std: float = 1.0) -> PagedKV:
    """K and V ~ N(0, kv_std) rounded to bf16, stored in a pool of ceil(pool_factor * pages) pages that a
    seeded permutation maps to the sequences.  Values are drawn in logical order, so a different
    ``perm_stream`` moves the same logical KV to other physical pages.  Unused pages and the tail slots
    of each sequence's last page are NaN when ``poison`` is set."""
    slots = np.asarray(slots, dtype=np.int64)
    B = len(slots)
    npages = [(int(s) + page_size - 1) // page_size for s in slots]
    total = int(sum(npages))
    pool = max(total, int(math.ceil(pool_factor * total)))
    perm = rng_for(case, layer, perm_stream).permutation(pool)[:total].astype(np.int32)
    mb = max(npages) if max_blocks is None else max_blocks
    bt = np.full((B, max(mb, 1)), -1, dtype=np.int32)
    shape = (pool, num_kv_heads, page_size, head_dim)
    fill = BF16_QNAN if poison else np.uint16(0)
    k_pool = np.full(shape, fill, dtype=np.uint16)
    v_pool = np.full(shape, fill, dtype=np.uint16)
    rk, rv = rng_for(case, layer, S_K), rng_for(case, layer, S_V)
    off = 0
    for b in range(B):
        n = npages[b]
        bt[b, :n] = perm[off:off + n]
        # logical order: token-major [slot][head][dim] so values do not depend on the page size
        kl = _normal_bf16(rk, (n * page_size, num_kv_heads, head_dim), kv_std)
        vl = _normal_bf16(rv, (n * page_size, num_kv_heads, head_dim), kv_std)
        if poison:
            kl[slots[b]:] = BF16_QNAN
            vl[slots[b]:] = BF16_QNAN
        kl = kl.reshape(n, page_size, num_kv_heads, head_dim).transpose(0, 2, 1, 3)
        vl = vl.reshape(n, page_size, num_kv_heads, head_dim).transpose(0, 2, 1, 3)
        k_pool[bt[b, :n]] = kl
        v_pool[bt[b, :n]] = vl
        off += n
    return PagedKV(k_pool, v_pool, bt, slots.astype(np.int32), page_size)


def dim_major(pool: np.ndarray) -> np.ndarray:
    """A [pages][kv_heads][page_size][head_dim] pool rewritten as [pages][kv_heads][head_dim][page_size]
    (each dim's page_size tokens contiguous): the dim-major V cache layout.  Only moves values."""
    return np.ascontiguousarray(np.asarray(pool).transpose(0, 1, 3, 2))


def ragged_ctx_lens(case: int, batch: int, lo: int, hi: int) -> np.ndarray:
    return rng_for(case, 0, S_CTX).integers(lo, hi + 1, size=batch).astype(np.int32)


# ----------------------------------------------------------------------------------------------
# attention case
# ----------------------------------------------------------------------------------------------

@dataclasses.dataclass
class AttentionCase:
    q: np.ndarray             # uint16 bf16 bits [T][Hq][D]
    kv: PagedKV
    ctx_lens: np.ndarray      # int32 [B]
    node_offsets: np.ndarray  # int32 [B+1]
    parents: np.ndarray       # int32 [T], sequence-local
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    needle_chunks: Optional[np.ndarray] = None   # [B][n] chunk ids holding a planted key (needle variant)


def attention_case(case: int, *, ctx_lens, trees, num_q_heads: int, num_kv_heads: int, head_dim: int,
                   layer: int = 0, poison: bool = True, kv_std: float = 1.0, q_std: float = 1.0,
                   perm_stream: int = S_BLOCKS, needle: Optional[dict] = None,
                   page_size: int = PAGE_SIZE) -> AttentionCase:
    """One layer of tree verification.  ``trees`` is a list of parent arrays (one per sequence).
    Node i of sequence b owns logical KV slot ctx_lens[b] + i.

    ``needle`` = {"count": n, "chunk": c, "score": s}: queries share a per-head direction z_h
    (q = (z_h + e)/sqrt(2)) and in ``n`` seeded chunks of ``c`` tokens one context key points along the
    KV group's mean direction, scaled so that its scaled score is about ``s`` above the typical one."""
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    B = len(ctx_lens)
    assert len(trees) == B
    sizes = [len(t) for t in trees]
    node_offsets = np.zeros(B + 1, dtype=np.int32)
    node_offsets[1:] = np.cumsum(sizes)
    T = int(node_offsets[-1])
    parents = np.concatenate([np.asarray(t, dtype=np.int32) for t in trees]) if T else np.zeros(0, np.int32)
    # block-table rows sized for the batch's largest context plus its largest tree
    max_blocks = (int(ctx_lens.max(initial=0)) + max(sizes, default=0) + page_size - 1) // page_size
    kv = paged_kv(case, layer, ctx_lens + np.asarray(sizes, np.int32), num_kv_heads, head_dim,
                  poison=poison, perm_stream=perm_stream, kv_std=kv_std, page_size=page_size, max_blocks=max_blocks)
    rq = rng_for(case, layer, S_Q)
    G = num_q_heads // num_kv_heads
    needle_chunks = None
    if needle is None:
        q = _normal_bf16(rq, (T, num_q_heads, head_dim), q_std)
    else:
        z = rq.standard_normal((num_q_heads, head_dim), dtype=np.float32)
        e = rq.standard_normal((T, num_q_heads, head_dim), dtype=np.float32)
        q = bf16_bits((z[None] + e) / np.float32(math.sqrt(2.0)))
        rn = rng_for(case, layer, S_TREE + 100)
        cs = int(needle["chunk"])
        beta = float(needle["score"]) * 2.0 * math.sqrt(2.0)
        needle_chunks = []
        for b in range(B):
            nch = int(ctx_lens[b]) // cs
            cnt = min(int(needle["count"]), nch)
            chosen = np.sort(rn.choice(nch, size=cnt, replace=False)) if cnt else np.zeros(0, np.int64)
            needle_chunks.append(chosen)
            for g in range(num_kv_heads):
                zg = z[g * G:(g + 1) * G].sum(0)
                dirn = zg / np.linalg.norm(zg)
                for c in chosen:
                    t = int(c) * cs + int(rn.integers(cs))
                    page = kv.block_table[b, t // page_size]
                    kv.k_pool[page, g, t % page_size] = bf16_bits(dirn * beta)
        needle_chunks = np.array(needle_chunks, dtype=object) if B else None
    return AttentionCase(q=q, kv=kv, ctx_lens=ctx_lens, node_offsets=node_offsets, parents=parents,
                         num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                         scale=1.0 / math.sqrt(head_dim), needle_chunks=needle_chunks)


# ----------------------------------------------------------------------------------------------
# acceptance cases
# ----------------------------------------------------------------------------------------------

PLANT_VALUE = np.float32(16.0)   # bf16-exact; every unplanted logit is clipped below it
CLIP_VALUE = np.float32(15.0)


@dataclasses.dataclass
class GreedyCase:
    node_offsets: np.ndarray     # int32 [B+1]
    parents: np.ndarray          # int32 [T] sequence-local
    draft_tokens: np.ndarray     # int32 [T]; entry of each root is the last committed token
    logits: np.ndarray           # uint16 bf16 bits or float32, [T][V]
    dtype: str                   # "bf16" | "f32"
    vocab: int
    planted: np.ndarray          # int32 [T]: the token the generator made the row's largest logit, or -1


def _logit_rows(rng, T, V, std):
    x = rng.standard_normal((T, V), dtype=np.float32) * np.float32(std)
    return x


def greedy_case(case: int, trees, vocab: int, *, dtype: str = "bf16", std: float = 2.0,
                plant_frac: float = 0.9, tie_frac: float = 0.25, alpha: float = 0.8,
                layer: int = 0) -> GreedyCase:
    """Target logits ~ N(0, std).  In a ``plant_frac`` share of rows one random token is lifted to 16.0
    (all other logits are clipped to [-15, 15]); in a ``tie_frac`` share of those a second token gets
    the same 16.0, so the row has an exact tie and the planted token is the lower index of the two.
    With probability ``alpha`` one random child of a planted node drafts the planted token; in tied
    rows another child may draft the higher-index tie partner.  Every other child drafts a distinct
    random token.  Unplanted rows keep their natural maximum (exact bf16 ties happen there too)."""
    sizes = [len(t) for t in trees]
    B = len(trees)
    node_offsets = np.zeros(B + 1, dtype=np.int32)
    node_offsets[1:] = np.cumsum(sizes)
    T = int(node_offsets[-1])
    parents = np.concatenate([np.asarray(t, np.int32) for t in trees])
    rl = rng_for(case, layer, S_TARGET)
    rt = rng_for(case, layer, S_TOKENS)
    x = _logit_rows(rl, T, vocab, std)
    planted = np.full(T, -1, dtype=np.int32)
    partner = np.full(T, -1, dtype=np.int32)
    plant_u = rt.random(T)
    tie_u = rt.random(T)
    for u in range(T):
        if plant_u[u] < plant_frac:
            row = x[u]
            np.clip(row, -CLIP_VALUE, CLIP_VALUE, out=row)
            a = int(rt.integers(vocab))
            row[a] = PLANT_VALUE
            if tie_u[u] < tie_frac and vocab > 1:
                b = int(rt.integers(vocab - 1))
                b = b + 1 if b >= a else b
                row[b] = PLANT_VALUE
                planted[u], partner[u] = min(a, b), max(a, b)
            else:
                planted[u] = a
    tokens = np.zeros(T, dtype=np.int32)
    for b in range(B):
        n0 = int(node_offsets[b])
        par = parents[n0:n0 + sizes[b]]
        tokens[n0] = int(rt.integers(vocab))
        for u_loc, kids in enumerate(children_lists(par)):
            if not kids:
                continue
            u = n0 + u_loc
            used = set()
            order = list(rt.permutation(len(kids)))
            assign = {}
            if planted[u] >= 0 and rt.random() < alpha:
                assign[kids[order.pop(0)]] = int(planted[u])
                used.add(int(planted[u]))
                if partner[u] >= 0 and order and rt.random() < 0.5:
                    assign[kids[order.pop(0)]] = int(partner[u])
                    used.add(int(partner[u]))
            if planted[u] >= 0:
                used.add(int(planted[u]))
            for k in kids:
                if k in assign:
                    continue
                while True:
                    t = int(rt.integers(vocab))
                    if t not in used:
                        break
                used.add(t)
                assign[k] = t
            for k, t in assign.items():
                tokens[n0 + k] = t
    logits = bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)
    return GreedyCase(node_offsets, parents, tokens, logits, dtype, vocab, planted)


@dataclasses.dataclass
class RejectionCase:
    node_offsets: np.ndarray
    parents: np.ndarray
    draft_tokens: np.ndarray      # int32 [T]; children of u drawn i.i.d. from draft_probs[u]
    logits: np.ndarray            # target logits, uint16 bf16 bits or float32 [T][V]
    dtype: str
    draft_probs: np.ndarray       # float32 [T][V]: the draft model's proposal distribution at each node
    u_accept: np.ndarray          # float32 [T] in [0,1) on the 2^-24 grid
    u_sample: np.ndarray          # float32 [T]
    vocab: int


def rejection_case(case: int, trees, vocab: int, *, dtype: str = "bf16", std: float = 2.0,
                   draft: str = "independent", draft_noise: float = 0.5, layer: int = 0) -> RejectionCase:
    """Target logits ~ N(0, std).  The draft model's proposal q_u is the softmax of its own logits:
    independent N(0, std) draws (``draft="independent"``), or the target logits plus N(0, draft_noise)
    (``draft="close"``, which makes deep acceptance likely).  Children of each node are drawn i.i.d.
    from q_u, as a sampling draft model would propose them."""
    sizes = [len(t) for t in trees]
    B = len(trees)
    node_offsets = np.zeros(B + 1, dtype=np.int32)
    node_offsets[1:] = np.cumsum(sizes)
    T = int(node_offsets[-1])
    parents = np.concatenate([np.asarray(t, np.int32) for t in trees])
    x = _logit_rows(rng_for(case, layer, S_TARGET), T, vocab, std)
    logits = bf16_bits(x) if dtype == "bf16" else x
    xt = bf16_to_f32(logits) if dtype == "bf16" else x
    rd = rng_for(case, layer, S_DRAFT)
    if draft == "independent":
        dl = rd.standard_normal((T, vocab)) * std
    elif draft == "close":
        dl = xt.astype(np.float64) + rd.standard_normal((T, vocab)) * draft_noise
    else:
        raise ValueError(draft)
    # the draft model's own sampling distribution (an input of verification, not part of it)
    dl = dl - dl.max(axis=1, keepdims=True)
    qd = np.exp(dl)
    qd /= qd.sum(axis=1, keepdims=True)
    q32 = qd.astype(np.float32)
    rt = rng_for(case, layer, S_TOKENS)
    tokens = np.zeros(T, dtype=np.int32)
    for b in range(B):
        n0 = int(node_offsets[b])
        par = parents[n0:n0 + sizes[b]]
        tokens[n0] = int(rt.integers(vocab))
        for u_loc, kids in enumerate(children_lists(par)):
            if kids:
                w = q32[n0 + u_loc].astype(np.float64)
                draws = rt.choice(vocab, size=len(kids), p=w / w.sum())
                for k, t in zip(kids, draws):
                    tokens[n0 + k] = int(t)
    ru = rng_for(case, layer, S_UNIFORM)
    u_acc = uniforms24(ru, T)
    u_smp = uniforms24(ru, T)
    return RejectionCase(node_offsets, parents, tokens, logits, dtype, q32, u_acc, u_smp, vocab)


# ----------------------------------------------------------------------------------------------
# compact draft KV inputs
# ----------------------------------------------------------------------------------------------

def rope_inv_freq(head_dim: int, theta: float = 500000.0) -> np.ndarray:
    """Rotary frequencies theta^(-2i/D), i < D/2, as float32 (a model constant; 500000 is Llama 3's base)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return (theta ** (-2.0 * i / head_dim)).astype(np.float32)


def chunk_selection(case: int, n_chunks, num_select: int, *, pad_frac: float = 0.0, dup_frac: float = 0.0,
                    bad_frac: float = 0.0) -> np.ndarray:
    """int32 [B][num_select] chunk ids in random order, distinct within a row, like a top-k list.  A fraction
    of the entries is replaced by -1 (padding), by a repeat of another entry of the row, or by an id at or
    past the row's chunk count."""
    rng = rng_for(case, 0, S_TOKENS)
    out = np.full((len(n_chunks), num_select), -1, dtype=np.int32)
    for b, n in enumerate(n_chunks):
        n = int(n)
        k = min(num_select, n)
        if k:
            out[b, :k] = rng.choice(n, size=k, replace=False)
        for j in range(num_select):
            r = rng.random()
            if r < pad_frac:
                out[b, j] = -1
            elif r < pad_frac + dup_frac and j > 0:
                out[b, j] = out[b, rng.integers(j)]
            elif r < pad_frac + dup_frac + bad_frac:
                out[b, j] = n + int(rng.integers(0, 4))
    return out


# ----------------------------------------------------------------------------------------------
# named workloads (shapes of the measured configurations)
# ----------------------------------------------------------------------------------------------

WORKLOADS = {
    # 1 layer, 1 sequence, 512 context, 4 q / 2 kv heads, D=64, 8-node tree of depth <= 4, chunk 64, vocab 32
    "tiny": dict(batch=1, ctx=512, hq=4, hkv=2, d=64, nodes=8, depth=4, chunk=64, vocab=32, logits="f32"),
    # Llama-3.1-8B layer at 32K, 64-node tree of depth 8, chunk 64, greedy over 128256 (bf16)
    "llama8b-32k": dict(batch=1, ctx=32768, hq=32, hkv=8, d=128, nodes=64, depth=8, chunk=64, vocab=128256,
                        logits="bf16"),
    # same at 64K with rejection sampling
    "llama8b-64k": dict(batch=1, ctx=65536, hq=32, hkv=8, d=128, nodes=64, depth=8, chunk=64, vocab=128256,
                        logits="bf16"),
    # same at 128K, 128-node tree of depth 10, top-256 chunks, 32 layers
    "llama8b-128k": dict(batch=1, ctx=131072, hq=32, hkv=8, d=128, nodes=128, depth=10, chunk=64,
                         vocab=128256, logits="bf16", layers=32, topk=256),
    # 16 ragged sequences, contexts U[4K, 64K], Qwen3-8B shape, chains of k=4 drafts (5 nodes)
    "qwen3-8b-ragged": dict(batch=16, ctx=(4096, 65536), hq=32, hkv=8, d=128, nodes=5, depth=4, chunk=64,
                            vocab=151936, logits="bf16"),
}
