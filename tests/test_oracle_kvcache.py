"""Pins of oracle.kv_commit (the commit of an accepted path into the paged cache)."""

import numpy as np
import pytest

import oracle
import synth


def _logical(pool, bt_row, slots, page_size, v_layout=0):
    """Logical rows [len(slots)][heads][dim] read straight through the block table."""
    p = np.swapaxes(pool, 2, 3) if v_layout else pool
    return np.stack([p[bt_row[s // page_size], :, s % page_size, :] for s in slots])


def _root_path(parents, f):
    path = [f]
    while parents[path[-1]] >= 0:
        path.append(int(parents[path[-1]]))
    return path[::-1]


def _case(seed, page_size=16, layers=3, v_layout=0):
    r = synth.rng_for(seed, 0, 0)
    trees = [synth.random_tree(r, 20, 6), synth.chain_tree(5), synth.random_tree(r, 9, 3)]
    ctx = np.array([100, 37, 5], dtype=np.int32)
    slots = ctx + np.array([len(t) for t in trees], dtype=np.int32)
    kv0 = synth.paged_kv(seed, 0, slots, 2, 64, page_size=page_size)
    ks, vs = [], []
    for layer in range(layers):
        kv = synth.paged_kv(seed, layer, slots, 2, 64, page_size=page_size)
        ks.append(kv.k_pool)
        vs.append(synth.dim_major(kv.v_pool) if v_layout else kv.v_pool)
    max_path = 8
    paths = np.full((3, max_path), -1, dtype=np.int32)
    nacc = np.zeros(3, dtype=np.int32)
    for b, t in enumerate(trees):
        f = int(r.integers(len(t)))
        pth = _root_path(t, f)
        paths[b, :len(pth)] = pth
        nacc[b] = len(pth) - 1
    return trees, ctx, kv0.block_table, ks, vs, paths, nacc


@pytest.mark.parametrize("v_layout", [0, 1])
@pytest.mark.parametrize("page_size", [8, 16])
def test_commit_moves_path_rows_and_keeps_the_rest(v_layout, page_size):
    trees, ctx, bt, ks, vs, paths, nacc = _case(31 + page_size, page_size, v_layout=v_layout)
    k2, v2, lens = oracle.kv_commit(ks, vs, bt, ctx, nacc, paths, page_size, v_layout)
    assert lens.tolist() == (ctx + 1 + nacc).tolist()
    for layer in range(len(ks)):
        for pool_old, pool_new, vl in ((ks[layer], k2[layer], 0), (vs[layer], v2[layer], v_layout)):
            touched = set()
            for b in range(3):
                n, L = int(nacc[b]), int(ctx[b])
                want = _logical(pool_old, bt[b], [L + int(paths[b, i]) for i in range(n + 1)], page_size, vl)
                got = _logical(pool_new, bt[b], [L + i for i in range(n + 1)], page_size, vl)
                assert np.array_equal(got, want)
                for i in range(n + 1):
                    s = L + i
                    touched.add((int(bt[b, s // page_size]), s % page_size))
            # every other (page, row) keeps its bits
            po = np.swapaxes(pool_old, 2, 3) if vl else pool_old
            pn = np.swapaxes(pool_new, 2, 3) if vl else pool_new
            for page in range(po.shape[0]):
                for row in range(page_size):
                    if (page, row) not in touched:
                        assert np.array_equal(po[page, :, row], pn[page, :, row])


def test_chain_all_accepted_is_a_no_op_and_flagged_rows_are_untouched():
    trees, ctx, bt, ks, vs, paths, nacc = _case(40)
    paths[1, :5] = [0, 1, 2, 3, 4]            # the chain, every draft accepted
    nacc[1] = 4
    nacc[2] = -1                              # a path that did not fit: nothing moves
    k2, v2, lens = oracle.kv_commit(ks, vs, bt, ctx, nacc, paths, 16)
    assert lens[1] == ctx[1] + 5 and lens[2] == ctx[2]
    for b in (1, 2):
        L = int(ctx[b])
        slots = list(range(L, L + len(trees[b])))
        for layer in range(len(ks)):
            assert np.array_equal(_logical(k2[layer], bt[b], slots, 16), _logical(ks[layer], bt[b], slots, 16))
            assert np.array_equal(_logical(v2[layer], bt[b], slots, 16), _logical(vs[layer], bt[b], slots, 16))


def test_committed_cache_reproduces_the_tree_pass_for_the_last_accepted_node():
    """The accepted node f saw the context plus its root path in the tree pass; after the commit that
    is exactly the plain causal prefix of length L + n + 1, so ordinary decode attention of f's query
    at slot L + n over the committed cache gives the same output."""
    r = synth.rng_for(41, 0, 0)
    tree = synth.random_tree(r, 24, 6)
    depths = synth.tree_depths(tree)
    f = int(np.argmax(depths))
    path = _root_path(tree, f)
    n = len(path) - 1
    case = synth.attention_case(41, ctx_lens=[150], trees=[tree], num_q_heads=4, num_kv_heads=2, head_dim=64,
                                poison=False)
    out_tree, lse_tree, _ = oracle.tree_attention(case.q, case.kv.k_pool, case.kv.v_pool, case.kv.block_table,
                                                  case.ctx_lens, case.node_offsets, case.parents, case.scale, 2,
                                                  case.kv.page_size)
    paths = np.full((1, 8), -1, dtype=np.int32)
    paths[0, :n + 1] = path
    k2, v2, lens = oracle.kv_commit([case.kv.k_pool], [case.kv.v_pool], case.kv.block_table, case.ctx_lens,
                                    np.array([n], np.int32), paths, case.kv.page_size)
    # decode: one query (f's) whose own slot is L + n, context L + n
    out_dec, lse_dec, _ = oracle.tree_attention(case.q[f:f + 1], k2[0], v2[0], case.kv.block_table,
                                                np.array([150 + n]), np.array([0, 1]), np.array([-1]), case.scale,
                                                2, case.kv.page_size)
    assert lens[0] == 150 + n + 1
    np.testing.assert_allclose(out_dec[0], out_tree[f], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_dec[0], lse_tree[f], rtol=0, atol=1e-12)


def test_commit_rejects_a_path_that_is_not_a_root_path():
    trees, ctx, bt, ks, vs, paths, nacc = _case(42)
    paths[0, :3] = [0, 5, 1]                  # node 1 at depth 2 is impossible (index < depth)
    nacc[0] = 2
    with pytest.raises(ValueError):
        oracle.kv_commit(ks, vs, bt, ctx, nacc, paths, 16)
