"""Oracle: bundle order of a draft tree.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: DiffSpec README (CGCL-codes), "Features": the bundle scheduler groups the draft tree's leaves
by their branching ancestor, so that target verification runs prefix-coherent.

Readings (the page names the grouping, not an algorithm):
  - Order.  The order is the depth-first preorder from the root, with the children of a node
    visited in increasing original index.  Every subtree then is one contiguous index range, and
    leaves under the same branching node are adjacent: the rows of one bundle share their prefix.
  - Bundle.  The bundle of a node is its nearest proper ancestor with two or more children; it is
    the root when there is none, and the root's own bundle is the root.
  - Ancestors in preorder.  Node j is an ancestor-or-self of node i exactly when
    j <= i < subtree_end[j], which is the visibility test the attention uses for such trees.
"""

from __future__ import annotations

import numpy as np


def bundle_order(parents):
    """parents: sequence-local, parents[0] = -1, 0 <= parents[i] < i.

    Returns (order, new_parents, subtree_end, bundle), all int32 [N], in the new numbering:
      order[i]        original index of the node placed at position i
      new_parents[i]  position of its parent (-1 for the root)
      subtree_end[i]  one past the last position of its subtree
      bundle[i]       position of its nearest proper ancestor with >= 2 children (0 if none)"""
    parents = [int(p) for p in parents]
    n = len(parents)
    if n == 0:
        z = np.zeros(0, dtype=np.int32)
        return z, z, z, z
    if parents[0] != -1 or any(not (0 <= parents[i] < i) for i in range(1, n)):
        raise ValueError("parents must be topological with parents[0] = -1")
    children = [[] for _ in range(n)]
    for i in range(1, n):
        children[parents[i]].append(i)          # increasing index
    order = []
    stack = [0]
    while stack:
        u = stack.pop()
        order.append(u)
        stack.extend(reversed(children[u]))     # the smallest child is visited first
    pos = {u: i for i, u in enumerate(order)}
    new_parents = np.array([pos[parents[u]] if parents[u] >= 0 else -1 for u in order], dtype=np.int32)
    size = [1] * n
    for u in range(n - 1, 0, -1):
        size[parents[u]] += size[u]
    subtree_end = np.array([pos[u] + size[u] for u in order], dtype=np.int32)
    bundle = np.zeros(n, dtype=np.int32)
    for i, u in enumerate(order):
        a = parents[u]
        while a >= 0 and len(children[a]) < 2:
            a = parents[a]
        bundle[i] = pos[a] if a >= 0 else 0
    return np.array(order, dtype=np.int32), new_parents, subtree_end, bundle
