"""Pins for the attention / chunk-mass oracle, each against something other than the oracle itself:
torch's CPU scaled_dot_product_attention and softmax (library routines), scipy's logsumexp, closed
forms, a transitive-closure construction of the ancestor relation, invariances."""

import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth


def _dense_kv(case: synth.AttentionCase, b: int):
    """Logical K/V of sequence b as float64 [slots][Hkv][D], read straight from the pool by page."""
    kv = case.kv
    n = int(kv.slots[b])
    ks, vs = [], []
    for t in range(n):
        page = kv.block_table[b, t // kv.page_size]
        ks.append(kv.k_pool[page, :, t % kv.page_size, :])
        vs.append(kv.v_pool[page, :, t % kv.page_size, :])
    conv = lambda a: torch.from_numpy(synth.bf16_to_f32(np.stack(a)).astype(np.float64))
    return conv(ks), conv(vs)


def _root_path(parents, i):
    path = [i]
    while parents[path[-1]] >= 0:
        path.append(int(parents[path[-1]]))
    return path[::-1]


def _sdpa_node(case, b, i, kd, vd):
    """Node i of sequence b by torch SDPA over the explicit key list: the whole context, then the
    tree slots of the nodes on the root->i path."""
    L = int(case.ctx_lens[b])
    n0 = int(case.node_offsets[b])
    par = case.parents[n0:int(case.node_offsets[b + 1])]
    keys = list(range(L)) + [L + j for j in _root_path(par, i)]
    G = case.num_q_heads // case.num_kv_heads
    q = torch.from_numpy(synth.bf16_to_f32(case.q[n0 + i]).astype(np.float64))          # [Hq][D]
    k = kd[keys].permute(1, 0, 2).repeat_interleave(G, dim=0)                             # [Hq][n][D]
    v = vd[keys].permute(1, 0, 2).repeat_interleave(G, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(q[:, None, :], k, v, scale=case.scale)[:, 0]
    s = (q[:, None, :] @ k.transpose(1, 2))[:, 0] * case.scale
    return o.numpy(), scipy.special.logsumexp(s.numpy(), axis=1)


def _run(case, chunk=0, **kw):
    return oracle.tree_attention(case.q, case.kv.k_pool, case.kv.v_pool, case.kv.block_table, case.ctx_lens,
                                 case.node_offsets, case.parents, case.scale, case.num_kv_heads,
                                 case.kv.page_size, chunk, **kw)


def test_ancestor_matrix_is_transitive_closure():
    rng = synth.rng_for(11, 0, 0)
    for n, d in [(1, 0), (2, 1), (8, 4), (40, 6), (64, 8), (128, 10)]:
        par = synth.random_tree(rng, n, d)
        A = np.zeros((n, n), dtype=np.int64)           # A[i, j] = 1 iff j is i's parent
        for i in range(1, n):
            A[i, par[i]] = 1
        reach = np.eye(n, dtype=np.int64)
        step = np.eye(n, dtype=np.int64)
        for _ in range(n):
            step = np.minimum(step @ A, 1)
            reach = np.minimum(reach + step, 1)
        assert np.array_equal(oracle.ancestor_matrix(par), reach.astype(bool))


def test_ancestor_matrix_rejects_bad_trees():
    for bad in ([0, 0], [-1, 1], [-1, 0, 3], [-1, -1]):
        with pytest.raises(ValueError):
            oracle.ancestor_matrix(np.array(bad))


@pytest.mark.parametrize("cfg", ["tiny", "medium", "multi"])
def test_tree_attention_matches_sdpa_over_root_paths(cfg):
    rng = synth.rng_for(12, 0, 0)
    if cfg == "tiny":      # the tiny verification shape: 512 context, 4/2 heads, D=64, 8 nodes depth 4
        case = synth.attention_case(1, ctx_lens=[512], trees=[synth.random_tree(rng, 8, 4)], num_q_heads=4,
                                    num_kv_heads=2, head_dim=64)
    elif cfg == "medium":  # GQA 4, D=128, ragged context (not a page multiple), 24-node tree depth 5
        case = synth.attention_case(2, ctx_lens=[333], trees=[synth.random_tree(rng, 24, 5)], num_q_heads=8,
                                    num_kv_heads=2, head_dim=128)
    else:                  # three sequences: a chain, a single node, a bushy tree
        case = synth.attention_case(3, ctx_lens=[100, 17, 64],
                                    trees=[synth.chain_tree(5), synth.chain_tree(1), synth.random_tree(rng, 12, 3)],
                                    num_q_heads=4, num_kv_heads=1, head_dim=64)
    out, lse, _ = _run(case)
    for b in range(len(case.ctx_lens)):
        kd, vd = _dense_kv(case, b)
        n0 = int(case.node_offsets[b])
        for i in range(int(case.node_offsets[b + 1]) - n0):
            o_ref, lse_ref = _sdpa_node(case, b, i, kd, vd)
            np.testing.assert_allclose(out[n0 + i], o_ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[n0 + i], lse_ref, rtol=0, atol=1e-12)


def test_chain_equals_causal_decode_rule():
    """A chain of N drafts is ordinary causal decode: query j reads slots s <= L + j
    (the per-row cache mask of the Adaptive Speculative Decoding kvcache)."""
    L, N, Hq, Hkv, D = 200, 6, 4, 2, 64
    case = synth.attention_case(4, ctx_lens=[L], trees=[synth.chain_tree(N)], num_q_heads=Hq, num_kv_heads=Hkv,
                                head_dim=D)
    out, lse, _ = _run(case)
    kd, vd = _dense_kv(case, 0)
    G = Hq // Hkv
    q = torch.from_numpy(synth.bf16_to_f32(case.q).astype(np.float64)).permute(1, 0, 2)      # [Hq][N][D]
    k = kd.permute(1, 0, 2).repeat_interleave(G, 0)
    v = vd.permute(1, 0, 2).repeat_interleave(G, 0)
    s_idx = torch.arange(L + N)[None, :]
    j_idx = torch.arange(N)[:, None]
    mask = s_idx <= L + j_idx
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=case.scale)
    np.testing.assert_allclose(out, o.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    # and the chain equals N separate single-node trees over the growing context
    for j in range(N):
        single = synth.AttentionCase(q=case.q[j:j + 1], kv=case.kv, ctx_lens=np.array([L + j], np.int32),
                                     node_offsets=np.array([0, 1], np.int32), parents=np.array([-1], np.int32),
                                     num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, scale=case.scale)
        o1, l1, _ = _run(single)
        np.testing.assert_allclose(o1[0], out[j], rtol=0, atol=1e-13)
        np.testing.assert_allclose(l1[0], lse[j], rtol=0, atol=1e-13)


def test_closed_forms():
    L, N, Hq, Hkv, D = 130, 9, 4, 2, 64
    rng = synth.rng_for(13, 0, 0)
    par = synth.random_tree(rng, N, 4)
    case = synth.attention_case(5, ctx_lens=[L], trees=[par], num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D)
    depth = synth.tree_depths(par)
    # K == 0: every visible key scores 0, so out is the plain mean of the visible V rows and lse = log(count)
    k0 = case.kv.k_pool.copy()
    k0[~np.isnan(synth.bf16_to_f32(k0))] = 0
    zc = synth.AttentionCase(**{**case.__dict__, "kv": synth.PagedKV(k0, case.kv.v_pool, case.kv.block_table,
                                                                       case.kv.slots)})
    out, lse, masses = _run(zc, chunk=64)
    kd, vd = _dense_kv(case, 0)
    for i in range(N):
        keys = list(range(L)) + [L + j for j in _root_path(par, i)]
        mean_v = vd[keys].mean(0).numpy()                      # [Hkv][D]
        np.testing.assert_allclose(out[i], np.repeat(mean_v, Hq // Hkv, 0), atol=1e-12)
        np.testing.assert_allclose(lse[i], math.log(L + depth[i] + 1), atol=1e-12)
    # chunk mass with K == 0: chunk c holds |c| / (L + depth_i + 1) for node i, averaged over nodes
    sizes = np.array([64, 64, 2])
    expect = np.array([np.mean([s / (L + depth[i] + 1) for i in range(N)]) for s in sizes])
    np.testing.assert_allclose(masses[0], expect, atol=1e-13)
    # V == c: out == c exactly (up to rounding)
    vc = case.kv.v_pool.copy()
    vc[~np.isnan(synth.bf16_to_f32(vc))] = synth.bf16_bits(np.float32(0.75))
    cc = synth.AttentionCase(**{**case.__dict__, "kv": synth.PagedKV(case.kv.k_pool, vc, case.kv.block_table,
                                                                       case.kv.slots)})
    out, _, _ = _run(cc)
    np.testing.assert_allclose(out, 0.75, atol=1e-12)


def test_needle_key_dominates():
    """One context key scoring far above the rest: output ~ that key's V row, and its chunk holds the mass."""
    L, N, Hq, Hkv, D = 256, 4, 2, 1, 64
    case = synth.attention_case(6, ctx_lens=[L], trees=[synth.chain_tree(N)], num_q_heads=Hq, num_kv_heads=Hkv,
                                head_dim=D)
    qf = synth.bf16_to_f32(case.q).astype(np.float64)
    t = 77
    page = case.kv.block_table[0, t // 16]
    # key along the sum of all queries, large enough that its score beats all others by > 40
    dirn = qf.reshape(-1, D).sum(0)
    dirn /= np.linalg.norm(dirn)
    case.kv.k_pool[page, 0, t % 16] = synth.bf16_bits(dirn * 400.0)
    out, _, masses = _run(case, chunk=64)
    kd, vd = _dense_kv(case, 0)
    scores = (qf @ kd[t, 0].numpy()) * case.scale
    assert scores.min() > 40
    np.testing.assert_allclose(out, np.broadcast_to(vd[t, 0].numpy(), out.shape), atol=1e-9)
    np.testing.assert_allclose(masses[0], [0, 1, 0, 0], atol=1e-9)


def test_block_table_and_pool_invariance():
    """The same logical KV moved to other physical pages (another permutation, a bigger pool) gives
    bit-identical results."""
    rng = synth.rng_for(14, 0, 0)
    trees = [synth.random_tree(rng, 10, 4), synth.chain_tree(3)]
    a = synth.attention_case(7, ctx_lens=[190, 45], trees=trees, num_q_heads=4, num_kv_heads=2, head_dim=64)
    b = synth.attention_case(7, ctx_lens=[190, 45], trees=trees, num_q_heads=4, num_kv_heads=2, head_dim=64,
                             perm_stream=50)
    assert not np.array_equal(a.kv.block_table, b.kv.block_table)
    ra, rb = _run(a, chunk=64), _run(b, chunk=64)
    assert np.array_equal(ra[0], rb[0]) and np.array_equal(ra[1], rb[1])
    for ma, mb in zip(ra[2], rb[2]):
        assert np.array_equal(ma, mb)
    # the same V pool handed over dim-major reads the same values
    vt = synth.dim_major(a.kv.v_pool)
    assert vt.shape == (a.kv.v_pool.shape[0], 2, 64, a.kv.page_size)
    rc = oracle.tree_attention(a.q, a.kv.k_pool, vt, a.kv.block_table, a.ctx_lens, a.node_offsets, a.parents,
                               a.scale, a.num_kv_heads, a.kv.page_size, 64, v_layout=1)
    assert np.array_equal(ra[0], rc[0]) and np.array_equal(ra[1], rc[1])


def test_chunk_mass_against_torch_softmax():
    """Chunk masses equal torch.softmax probabilities of the explicit masked scores summed per chunk,
    and context mass + tree mass = 1 for every row."""
    rng = synth.rng_for(15, 0, 0)
    par = synth.random_tree(rng, 16, 5)
    L, Hq, Hkv, D, cs = 300, 8, 2, 64, 64
    case = synth.attention_case(8, ctx_lens=[L], trees=[par], num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D)
    _, _, masses = _run(case, chunk=cs)
    kd, vd = _dense_kv(case, 0)
    G = Hq // Hkv
    q = torch.from_numpy(synth.bf16_to_f32(case.q).astype(np.float64))                   # [N][Hq][D]
    k = kd.permute(1, 0, 2).repeat_interleave(G, 0)                                        # [Hq][n][D]
    s = torch.einsum("nhd,hkd->nhk", q, k) * case.scale
    anc = torch.zeros(16, 16, dtype=torch.bool)
    for i in range(16):
        anc[i, _root_path(par, i)] = True
    vis = torch.cat([torch.ones(16, L, dtype=torch.bool), anc], 1)[:, None, :]
    p = torch.softmax(s.masked_fill(~vis, float("-inf")), dim=-1)
    ctx = p[..., :L]
    ref = torch.stack([ctx[..., c * cs:(c + 1) * cs].sum(-1).mean() for c in range(math.ceil(L / cs))])
    np.testing.assert_allclose(masses[0], ref.numpy(), atol=1e-14)
    tree_mass = p[..., L:].sum(-1).mean().item()
    assert abs(masses[0].sum() + tree_mass - 1.0) < 1e-12


def test_topk_chunks_order_and_padding():
    m = np.array([0.1, 0.3, 0.3, 0.05, 0.3, 0.2])
    idx, val = oracle.topk_chunks(m, 4)
    assert idx.tolist() == [1, 2, 4, 5]
    np.testing.assert_array_equal(val, [0.3, 0.3, 0.3, 0.2])
    idx, val = oracle.topk_chunks(m[:2], 4)
    assert idx.tolist() == [1, 0, -1, -1] and val.tolist() == [0.3, 0.1, 0.0, 0.0]
    # agrees with a stable numpy argsort on the negated masses (a library routine)
    r = synth.rng_for(16, 0, 0)
    for _ in range(20):
        m = np.round(r.random(50), 1)
        idx, _ = oracle.topk_chunks(m, 17)
        assert idx.tolist() == np.argsort(-m, kind="stable")[:17].tolist()


def test_bf16_to_f64_known_bit_patterns():
    """bf16 decoding against values fixed by the format: sign, 8-bit exponent (bias 127), 7-bit fraction."""
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xC000, 0x4049, 0x7F80, 0xFF80, 0x0001, 0x7F7F, 0x3E80],
                    dtype=np.uint16)
    want = [0.0, -0.0, 1.0, -2.0, 3.140625, math.inf, -math.inf, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, 0.25]
    got = oracle.bf16_to_f64(bits)
    assert got.dtype == np.float64
    for g, w in zip(got, want):
        assert g == w and math.copysign(1.0, g) == math.copysign(1.0, w)
    assert np.isnan(oracle.bf16_to_f64(np.array([0x7FC0], dtype=np.uint16)))[0]


def test_gather_kv_reads_each_slot_from_its_page():
    """Every logical slot t comes from page block_table[t // page_size], row t % page_size: the pool is
    filled with a code of (page, head, row, dim) so each gathered value names where it was read."""
    pages, H, ps, D = 7, 3, 4, 2
    pool = np.zeros((pages, H, ps, D), dtype=np.uint16)
    for p in range(pages):
        for h in range(H):
            for r in range(ps):
                for d in range(D):
                    val = np.float32(((p * H + h) * ps + r) * D + d)   # integers < 2^8: exact in bf16
                    pool[p, h, r, d] = np.frombuffer(val.tobytes(), dtype=np.uint32)[0] >> 16
    table = np.array([5, 0, 3, 6])
    n = 13
    allh = oracle.gather_kv(pool, table, n, ps)
    assert allh.shape == (n, H, D)
    for t in range(n):
        for h in range(H):
            for d in range(D):
                assert allh[t, h, d] == ((table[t // ps] * H + h) * ps + t % ps) * D + d
    np.testing.assert_array_equal(oracle.gather_kv(pool, table, n, ps, kv_head=2), allh[:, 2])
    with pytest.raises(ValueError):
        oracle.gather_kv(pool, np.array([1, -1]), 6, ps)


def test_argmax_lowest_and_target_probs():
    """argmax with exact ties goes to the lowest index (numpy's argmax has the same rule); softmax equals
    scipy's, -inf logits get probability 0, and a row without a finite maximum is refused."""
    rng = np.random.default_rng(5)
    for _ in range(50):
        row = rng.integers(-3, 4, 40).astype(np.float64)
        assert oracle.argmax_lowest(row) == int(np.argmax(row))
    assert oracle.argmax_lowest([1.0, 3.0, -0.0, 3.0]) == 1
    assert oracle.argmax_lowest([-0.0, 0.0]) == 0
    with pytest.raises(ValueError):
        oracle.argmax_lowest([1.0, float("nan")])
    lg = rng.normal(0, 2, 1000)
    lg[::7] = -np.inf
    p = oracle.target_probs(lg)
    np.testing.assert_allclose(p, scipy.special.softmax(lg), rtol=1e-12, atol=1e-300)
    assert (p[::7] == 0).all() and abs(p.sum() - 1.0) < 1e-14
    with pytest.raises(ValueError):
        oracle.target_probs(np.full(4, -np.inf))
