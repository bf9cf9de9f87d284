"""Oracle: greedy and rejection-sampling acceptance over a draft tree.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (pages cited by title and section):

* vllm.cpp "Speculative decoding" documentation, section MTP: greedy verification
  accepts a draft token exactly when it equals the target's own greedy choice, so
  the emitted tokens do not depend on the draft depth.
* "Adaptive Speculative Decoding", section "Correctness first" (G1, G2) and section
  "The controller": a draft x ~ q is accepted with probability min(1, p(x)/q(x)); on
  rejection the replacement is drawn from the normalised residual max(0, p - q)
  (the Leviathan et al. / Chen et al. scheme); temperature 0 turns p into a one-hot
  and the same sampler then is greedy verification; k drafts yield up to k+1 tokens
  (the last one is the target's own token at the stopping point).
* "DiffSpec: Accelerating Long Sequence Generation with Differential Speculative
  Decoding", section "What DiffSpec Does" (item 5): candidates form a tree with
  shared prefixes.

Readings where the pages are silent (the pages give the chain rule only):

* Greedy on a tree: node j is accepted iff its parent is accepted and its token equals
  the target's argmax at the parent (lowest token id among exactly equal maxima).  The
  result is the deepest accepted node (lowest node index among equally deep ones); the
  emitted tokens are the drafts on the root->node path followed by the argmax there.
* Rejection on a tree (recursive residual over siblings): at the current node u start
  with res = p_u; test the children c of u in increasing index with their token x:
  accept iff u_accept[c] * q_u(x) < res(x) and move to c; otherwise replace res by the
  normalised max(0, res - q_u) (keeping it if that is identically zero) and try the next
  child.  If no child is accepted, emit x* = the smallest v with
  sum_{w<=v} res(w) > u_sample[u] * sum_w res(w).  With one child per node this is the
  pages' chain rule; with i.i.d. children from q_u the emitted token has law p_u.

Precision: logits are read exactly (bf16 or fp32 -> float64) and every probability,
residual and cumulative sum is float64.
"""

from __future__ import annotations

import math

import numpy as np

from .attention import bf16_to_f64


def _rows_f64(logits, dtype: str) -> np.ndarray:
    return bf16_to_f64(logits) if dtype == "bf16" else np.asarray(logits, dtype=np.float64)


def _children(parents):
    ch = [[] for _ in range(len(parents))]
    for i in range(1, len(parents)):
        ch[int(parents[i])].append(i)
    return ch


def _depths(parents):
    d = [0] * len(parents)
    for i in range(1, len(parents)):
        d[i] = d[int(parents[i])] + 1
    return d


def _path_to(parents, node):
    path = [node]
    while parents[path[-1]] >= 0:
        path.append(int(parents[path[-1]]))
    return path[::-1]


def argmax_lowest(row) -> int:
    """Index of the largest value; the lowest index among exactly equal maxima."""
    row = np.asarray(row, dtype=np.float64)
    if np.isnan(row).any():
        raise ValueError("NaN logit")
    m = row.max()
    return int(np.flatnonzero(row == m)[0])


def accept_greedy(node_offsets, parents, draft_tokens, logits, dtype: str = "bf16"):
    """Greedy longest-accepted-path acceptance, per sequence.

    Returns a list of (num_accepted, path_nodes, tokens): path_nodes are the sequence-local nodes from
    the root to the last accepted node, tokens are their draft tokens (root excluded) followed by the
    target's argmax at the last accepted node."""
    rows = _rows_f64(logits, dtype)
    res = []
    for b in range(len(node_offsets) - 1):
        n0, n1 = int(node_offsets[b]), int(node_offsets[b + 1])
        par = [int(x) for x in parents[n0:n1]]
        a = [argmax_lowest(rows[n0 + u]) for u in range(n1 - n0)]
        accepted = [False] * (n1 - n0)
        accepted[0] = True
        for j in range(1, n1 - n0):
            accepted[j] = accepted[par[j]] and int(draft_tokens[n0 + j]) == a[par[j]]
        dep = _depths(par)
        f = 0
        for j in range(1, n1 - n0):
            if accepted[j] and dep[j] > dep[f]:
                f = j
        path = _path_to(par, f)
        toks = [int(draft_tokens[n0 + j]) for j in path[1:]] + [a[f]]
        res.append((dep[f], path, toks))
    return res


def target_probs(row_f64) -> np.ndarray:
    """p = softmax(logits) in float64 (a -inf logit gets probability 0)."""
    m = row_f64.max()
    if not np.isfinite(m):
        raise ValueError("a row of target logits must have a finite maximum")
    e = np.exp(row_f64 - m)
    return e / math.fsum(e)


def _residual(res, q):
    d = np.maximum(0.0, res - q)
    z = math.fsum(d)
    return res if z == 0.0 else d / z


def accept_rejection(node_offsets, parents, draft_tokens, logits, draft_probs, u_accept, u_sample,
                     dtype: str = "bf16", return_margins: bool = False, _mutant: str = None):
    """Rejection-sampling acceptance over a draft tree (recursive residual over siblings).

    Returns a list of (num_accepted, path_nodes, tokens) per sequence; with ``return_margins`` each entry
    also carries the smallest relative distance of any decision to its threshold (accept tests relative
    to max(u*q(x), res(x)); the final draw relative to sum(res)).

    ``_mutant`` plants a known mistake ("skip_accept": accept every draft; "resample_p": draw the
    correction from p instead of the residual) so tests can show they detect it."""
    rows = _rows_f64(logits, dtype)
    out = []
    for b in range(len(node_offsets) - 1):
        n0, n1 = int(node_offsets[b]), int(node_offsets[b + 1])
        par = [int(x) for x in parents[n0:n1]]
        kids = _children(par)
        u = 0
        margin = math.inf
        path = [0]
        while True:
            p = target_probs(rows[n0 + u])
            q = np.asarray(draft_probs[n0 + u], dtype=np.float64)
            res = p
            nxt = None
            for c in kids[u]:
                x = int(draft_tokens[n0 + c])
                lhs = float(u_accept[n0 + c]) * q[x]
                rhs = res[x]
                scale = max(lhs, rhs)
                if scale > 0:
                    margin = min(margin, abs(lhs - rhs) / scale)
                if lhs < rhs or _mutant == "skip_accept":
                    nxt = c
                    break
                res = _residual(res, q)
            if nxt is None:
                dist = p if _mutant == "resample_p" else res
                cdf = np.cumsum(dist)
                total = cdf[-1]
                thr = float(u_sample[n0 + u]) * total
                xs = int(np.searchsorted(cdf, thr, side="right"))
                lo = cdf[xs - 1] if xs > 0 else 0.0
                margin = min(margin, (cdf[xs] - thr) / total, (thr - lo) / total)
                toks = [int(draft_tokens[n0 + j]) for j in path[1:]] + [xs]
                entry = (len(path) - 1, path, toks)
                out.append(entry + (margin,) if return_margins else entry)
                break
            u = nxt
            path.append(u)
    return out
