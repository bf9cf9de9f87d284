"""Pins for the bundle-order oracle.  The order is checked against an independent definition of
preorder: the lexicographic order of each node's root path of original indices.  Subtree ranges and
bundles are checked against brute force over the ancestor relation."""

import numpy as np
import pytest

import oracle
import synth
from oracle.bundle import bundle_order


def _root_path(parents, u):
    path = [u]
    while parents[path[-1]] >= 0:
        path.append(int(parents[path[-1]]))
    return path[::-1]


def _trees():
    r = synth.rng_for(400, 0, 0)
    out = [synth.chain_tree(1), synth.chain_tree(7), np.array([-1, 0, 0, 0], dtype=np.int32)]
    for n, d, c in ((16, 4, 4), (64, 8, 4), (128, 10, 4), (300, 12, 6), (40, 3, 8)):
        out.append(synth.random_tree(r, n, d, c))
    return out


@pytest.mark.parametrize("ti", range(8))
def test_order_is_lexicographic_root_paths(ti):
    parents = _trees()[ti]
    order, new_par, end, bundle = bundle_order(parents)
    want = sorted(range(len(parents)), key=lambda u: _root_path(parents, u))
    assert order.tolist() == want
    inv = np.empty_like(order)
    inv[order] = np.arange(len(order))
    assert all(new_par[i] == (inv[parents[u]] if parents[u] >= 0 else -1) for i, u in enumerate(order))


@pytest.mark.parametrize("ti", range(8))
def test_subtree_ranges_and_ancestors(ti):
    parents = _trees()[ti]
    n = len(parents)
    order, new_par, end, bundle = bundle_order(parents)
    anc_old = oracle.ancestor_matrix(parents)                  # anc[i][j]: j is an ancestor-or-self of i
    anc_new = anc_old[np.ix_(order, order)]
    for j in range(n):
        desc = np.flatnonzero(anc_new[:, j])                   # nodes having j as ancestor-or-self
        assert desc.tolist() == list(range(j, int(end[j])))
    # the interval test is the ancestor relation
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    assert np.array_equal((j <= i) & (i < end[j]), anc_new)
    assert np.array_equal(oracle.ancestor_matrix(new_par), anc_new)


@pytest.mark.parametrize("ti", range(8))
def test_bundles(ti):
    parents = _trees()[ti]
    order, new_par, end, bundle = bundle_order(parents)
    n = len(parents)
    nch = np.bincount(new_par[1:], minlength=n) if n > 1 else np.zeros(n, dtype=int)
    assert bundle[0] == 0
    for v in range(1, n):
        path = _root_path(new_par, v)[:-1]                     # proper ancestors, root first
        branching = [a for a in path if nch[a] >= 2]
        assert bundle[v] == (branching[-1] if branching else 0)
        assert bundle[v] <= v < end[bundle[v]]
    # leaves of one bundle form contiguous runs inside the bundle node's subtree
    leaves = [v for v in range(n) if nch[v] == 0]
    for bnode in set(bundle[leaves].tolist()):
        ls = [v for v in leaves if bundle[v] == bnode]
        assert all(bnode <= v < end[bnode] for v in ls)


def test_chain_and_star_orders():
    o, p, e, b = bundle_order(synth.chain_tree(6))
    assert o.tolist() == list(range(6)) and e.tolist() == [6] * 6 and b.tolist() == [0] * 6
    o, p, e, b = bundle_order([-1, 0, 0, 1, 2, 1])
    assert o.tolist() == [0, 1, 3, 5, 2, 4]
    assert p.tolist() == [-1, 0, 1, 1, 0, 4] and e.tolist() == [6, 4, 3, 4, 6, 6]
    assert b.tolist() == [0, 0, 1, 1, 0, 0]
    with pytest.raises(ValueError):
        bundle_order([-1, 2, 0])
