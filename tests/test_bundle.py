"""spec_tree_bundle_order (host code in the library) against the oracle: identical arrays on random
trees up to the largest supported size, and refusals of non-topological parent arrays."""

import numpy as np
import pytest

import synth
from oracle.bundle import bundle_order


def _spec():
    from long_context_tree_amd import spec
    try:
        spec.lib()
    except Exception as e:
        pytest.skip(f"libspec_verify not built: {e}")
    return spec


@pytest.mark.parametrize("n,depth,kids", [(1, 0, 4), (2, 1, 4), (9, 8, 4), (64, 8, 4), (128, 10, 4), (500, 12, 6),
                                          (2048, 16, 4), (2048, 2047, 1), (300, 2, 200)])
def test_library_matches_oracle(n, depth, kids):
    spec = _spec()
    r = synth.rng_for(410, n, depth)
    parents = synth.random_tree(r, n, depth, kids)
    got = spec.tree_bundle_order(parents)
    want = bundle_order(parents)
    for g, w, name in zip(got, want, ("order", "new_parents", "subtree_end", "bundle")):
        assert np.array_equal(g, w), name


def test_library_refuses_bad_trees():
    spec = _spec()
    with pytest.raises(spec.SpecError, match=r"parents\[0\]"):
        spec.tree_bundle_order([0, 0])
    with pytest.raises(spec.SpecError, match=r"parents\[2\] = 2"):
        spec.tree_bundle_order([-1, 0, 2])
    with pytest.raises(spec.SpecError, match="SPEC_MAX_TREE_NODES"):
        spec.tree_bundle_order(np.arange(-1, 2048, dtype=np.int32))
    assert all(len(a) == 0 for a in spec.tree_bundle_order(np.zeros(0, dtype=np.int32)))
