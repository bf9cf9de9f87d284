"""GPU parity for trees in bundle (preorder) order and for wide trees (more than 256 nodes).

- The interval mask (subtree_end) gives the same bytes as the ancestor bit masks on the same tree.
- Wide trees up to 2048 nodes match the oracle: attention outputs, LSE and chunk masses at the
  attention tolerances; greedy and rejection acceptance bit-exactly.
The trees come from the seeded generator, renumbered by the oracle's bundle order; the oracle's
subtree ends are the input of both sides."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import compare_mass, compare_out, dev, oracle_attention, run_attention
from oracle.bundle import bundle_order
from synth import device as sdev

pytestmark = pytest.mark.gpu


def _preorder_tree(seed, n, depth, kids=4):
    parents = synth.random_tree(synth.rng_for(seed, 0, synth.S_TREE), n, depth, kids)
    _, new_parents, end, _ = bundle_order(parents)
    return new_parents, end


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("v_layout", [0, 1])
def test_interval_mask_equals_bit_masks(v_layout, chunk):
    trees, ends = zip(*[_preorder_tree(500 + i, n, d) for i, (n, d) in enumerate([(100, 8), (37, 5), (1, 0)])])
    case = synth.attention_case(500, ctx_lens=[700, 64, 5], trees=list(trees), num_q_heads=8, num_kv_heads=2,
                                head_dim=128)
    se = np.concatenate(ends)
    a = run_attention(case, chunk_size=chunk, v_layout=v_layout)
    b = run_attention(case, chunk_size=chunk, v_layout=v_layout, subtree_end=se)
    import long_context_tree_amd as lt
    ma = torch.zeros((3, -(-700 // chunk)), dtype=torch.float32, device=dev())
    mb = torch.zeros_like(ma)
    lt.chunk_salience(a[2], ma)
    lt.chunk_salience(b[2], mb)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1]) and torch.equal(ma, mb)
    o_ref, l_ref, _ = oracle_attention(case)
    compare_out(b[0], b[1], o_ref, l_ref)


@pytest.mark.parametrize("n,split", [(12, 64), (16, 0), (30, 48)])
def test_interval_mask_narrow_trees_with_ring_write_outs(n, split):
    """Preorder trees of <= 32 nodes at 4 query heads per KV head (4-wave work-groups; <= 64 rows take the
    variant whose last wave writes the chunk values out), with splits long enough that the LDS ring of chunk
    values is written out inside a split: interval and bit masks give the same bytes, and both match the
    oracle."""
    tree, end = _preorder_tree(530 + n, n, 5)
    case = synth.attention_case(530 + n, ctx_lens=[5000], trees=[tree], num_q_heads=8, num_kv_heads=2,
                                head_dim=128)
    print(f"nodes={n} split={split}", flush=True)
    a = run_attention(case, chunk_size=64, split_tiles=split)
    b = run_attention(case, chunk_size=64, split_tiles=split, subtree_end=end)
    import long_context_tree_amd as lt
    ma = torch.zeros((1, -(-5000 // 64)), dtype=torch.float32, device=dev())
    mb = torch.zeros_like(ma)
    lt.chunk_salience(a[2], ma)
    lt.chunk_salience(b[2], mb)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1]) and torch.equal(ma, mb)
    o_ref, l_ref, m_ref = oracle_attention(case, 64)
    compare_out(b[0], b[1], o_ref, l_ref)
    compare_mass(mb.cpu().numpy()[0].astype(np.float64), m_ref[0])


@pytest.mark.parametrize("n,depth,L,hq,hkv,d", [(300, 12, 1000, 8, 2, 128), (1000, 16, 3000, 4, 1, 128),
                                                (2048, 20, 500, 4, 2, 64), (700, 40, 5000, 32, 8, 128)])
def test_wide_tree_attention_matches_oracle(n, depth, L, hq, hkv, d):
    tree, end = _preorder_tree(510 + n, n, depth)
    case = synth.attention_case(510 + n, ctx_lens=[L], trees=[tree], num_q_heads=hq, num_kv_heads=hkv, head_dim=d)
    print(f"nodes={n} L={L} heads={hq}/{hkv} D={d}", flush=True)
    out, lse, h, _ = run_attention(case, chunk_size=64, subtree_end=end)
    import long_context_tree_amd as lt
    mass = torch.zeros((1, -(-L // 64)), dtype=torch.float32, device=dev())
    lt.chunk_salience(h, mass)
    torch.cuda.synchronize()
    o_ref, l_ref, m_ref = oracle_attention(case, 64)
    compare_out(out, lse, o_ref, l_ref)
    compare_mass(mass.cpu().numpy()[0].astype(np.float64), m_ref[0])


def test_wide_tree_two_sequences_and_small_splits():
    """Two wide trees of different sizes in one call with short splits, so that many work-groups stop at
    their last node's tree slot and several splits hold only tree slots."""
    t1, e1 = _preorder_tree(520, 600, 10)
    t2, e2 = _preorder_tree(521, 257, 6)
    case = synth.attention_case(520, ctx_lens=[100, 1300], trees=[t1, t2], num_q_heads=8, num_kv_heads=4,
                                head_dim=128)
    out, lse, _, _ = run_attention(case, split_tiles=2, subtree_end=np.concatenate([e1, e2]))
    torch.cuda.synchronize()
    o_ref, l_ref, _ = oracle_attention(case)
    compare_out(out, lse, o_ref, l_ref)


def _expected(res, B, max_path):
    n = np.full(B, -1, np.int32)
    path = np.full((B, max_path), -1, np.int32)
    toks = np.full((B, max_path), -1, np.int32)
    for b, r in enumerate(res):
        if len(r[1]) > max_path:
            continue
        n[b] = r[0]
        path[b, :len(r[1])] = r[1]
        toks[b, :len(r[2])] = r[2]
    return n, path, toks


def _check(outs, exp):
    for g, e, name in zip(outs, exp, ("num_accepted", "path_nodes", "tokens")):
        assert np.array_equal(g.cpu().numpy(), e), name


@pytest.mark.parametrize("n,depth,V", [(1024, 14, 2000), (2048, 24, 300)])
def test_wide_tree_greedy_matches_oracle(n, depth, V):
    import long_context_tree_amd as lt
    trees = [_preorder_tree(530 + n, n, depth)[0], synth.random_tree(synth.rng_for(531, 0, 0), 50, 6)]
    case = synth.greedy_case(530 + n, trees, V, dtype="bf16", plant_frac=1.0, alpha=1.0)
    t = sdev.greedy_tensors(case, dev())
    max_path = depth + 1
    outs = lt.accept_greedy(t["node_offsets"], t["parents"], t["draft_tokens"], t["target_logits"], max_nodes=n,
                            max_path=max_path)
    torch.cuda.synchronize()
    ref = oracle.accept_greedy(case.node_offsets, case.parents, case.draft_tokens, case.logits, "bf16")
    assert ref[0][0] >= 2 and ref[1][0] >= 2               # real paths were accepted
    _check(outs, _expected(ref, 2, max_path))


def test_wide_tree_rejection_matches_oracle():
    import long_context_tree_amd as lt
    n, depth, V = 600, 12, 256
    trees = [_preorder_tree(540, n, depth)[0]]
    case = synth.rejection_case(540, trees, V, dtype="bf16", draft="close", draft_noise=0.3)
    t = sdev.rejection_tensors(case, dev())
    max_children = max(len(c) for c in synth.children_lists(trees[0]))
    outs = lt.accept_rejection(t["node_offsets"], t["parents"], t["draft_tokens"], t["target_logits"],
                               t["draft_probs"], t["u_accept"], t["u_sample"], max_nodes=n, max_path=depth + 1,
                               max_children=max_children)
    torch.cuda.synchronize()
    ref = oracle.accept_rejection(case.node_offsets, case.parents, case.draft_tokens, case.logits, case.draft_probs,
                                  case.u_accept, case.u_sample, "bf16", return_margins=True)
    assert ref[0][3] >= 1e-9, "decision within the tie band"
    _check(outs, _expected([x[:3] for x in ref], 1, depth + 1))


@pytest.mark.parametrize("chunk", [16, 32])
def test_wide_tree_small_chunks_dim_major(chunk):
    """A 300-node preorder tree with 16- and 32-slot chunk partials and dim-major V, against the oracle."""
    tree, end = _preorder_tree(525, 300, 10)
    case = synth.attention_case(525, ctx_lens=[900], trees=[tree], num_q_heads=8, num_kv_heads=2, head_dim=128)
    out, lse, h, _ = run_attention(case, chunk_size=chunk, subtree_end=end, v_layout=1)
    import long_context_tree_amd as lt
    mass = torch.zeros((1, -(-900 // chunk)), dtype=torch.float32, device=dev())
    lt.chunk_salience(h, mass)
    torch.cuda.synchronize()
    o_ref, l_ref, m_ref = oracle_attention(case, chunk)
    compare_out(out, lse, o_ref, l_ref)
    compare_mass(mass.cpu().numpy()[0].astype(np.float64), m_ref[0])
