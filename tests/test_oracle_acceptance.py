"""Pins for the acceptance oracle: brute force over all root paths, the chain and all/none special
cases, planted exact ties, the exact output law of the rejection walk (by closed form and by treating
the oracle as a black box over its uniforms), the acceptance-rate identity, p = q, the one-hot (T -> 0)
reduction to greedy, and the page's G1 statistical gate with planted mutants."""

import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
import oracle.acceptance as acc
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def _root_path(parents, i):
    path = [i]
    while parents[path[-1]] >= 0:
        path.append(int(parents[path[-1]]))
    return path[::-1]


def _brute_greedy(parents, tokens, rows):
    """Enumerate every root->node path; keep the longest whose every edge matches the target's argmax
    (numpy.argmax: first index of the maximum) at the edge's parent; earlier node wins ties."""
    a = [int(np.argmax(r)) for r in rows]
    best = [0]
    for node in range(len(parents)):
        path = _root_path(parents, node)
        if all(int(tokens[path[k]]) == a[path[k - 1]] for k in range(1, len(path))) and len(path) > len(best):
            best = path
    return len(best) - 1, best, [int(tokens[j]) for j in best[1:]] + [a[best[-1]]]


def _f64(case):
    return synth.bf16_to_f32(case.logits).astype(np.float64) if case.dtype == "bf16" else case.logits.astype(
        np.float64)


@pytest.mark.parametrize("seed", range(6))
def test_greedy_matches_bruteforce(seed):
    rng = synth.rng_for(20, seed, 0)
    trees = [synth.random_tree(rng, n, d) for n, d in [(8, 4), (64, 8), (1, 0), (20, 3), (5, 4)]]
    case = synth.greedy_case(20 + seed, trees, vocab=4099, dtype="bf16" if seed % 2 else "f32")
    rows = _f64(case)
    got = oracle.accept_greedy(case.node_offsets, case.parents, case.draft_tokens, case.logits, case.dtype)
    for b, (n_acc, path, toks) in enumerate(got):
        n0, n1 = case.node_offsets[b], case.node_offsets[b + 1]
        ref = _brute_greedy(case.parents[n0:n1], case.draft_tokens[n0:n1], rows[n0:n1])
        assert (n_acc, path, toks) == ref


def test_greedy_chain_is_longest_matching_prefix():
    """Accept-if-equal on a chain (vllm.cpp MTP verification): the accepted count is the longest prefix
    of drafts equal to the target's greedy choice at the previous position."""
    rng = np.random.default_rng(3)
    V, N = 50, 9
    for trial in range(50):
        rows = rng.normal(0, 2, (N, V)).astype(np.float32)
        a = rows.argmax(1)
        toks = a[np.maximum(np.arange(N) - 1, 0)].astype(np.int32)
        cut = rng.integers(1, N + 1)
        if cut < N:
            toks[cut] = (a[cut - 1] + 1) % V
        got = oracle.accept_greedy(np.array([0, N]), synth.chain_tree(N), toks, rows, "f32")[0]
        k = cut - 1 if cut < N else N - 1
        assert got[0] == k and got[1] == list(range(k + 1))
        assert got[2] == [int(t) for t in toks[1:k + 1]] + [int(a[k])]


def test_greedy_all_and_none_match():
    rng = synth.rng_for(21, 0, 0)
    par = synth.random_tree(rng, 30, 6)
    V = 97
    rows = rng.normal(0, 2, (30, V)).astype(np.float32)
    a = rows.argmax(1)
    toks = np.array([0] + [a[p] for p in par[1:]], dtype=np.int32)
    n_acc, path, t = oracle.accept_greedy(np.array([0, 30]), par, toks, rows, "f32")[0]
    depth = synth.tree_depths(par)
    deepest = int(np.flatnonzero(depth == depth.max())[0])
    assert n_acc == depth.max() and path[-1] == deepest and t[-1] == a[deepest]
    toks2 = np.array([0] + [(a[p] + 1) % V for p in par[1:]], dtype=np.int32)
    assert oracle.accept_greedy(np.array([0, 30]), par, toks2, rows, "f32")[0] == (0, [0], [int(a[0])])


def test_greedy_exact_ties_take_lowest_index():
    rng = synth.rng_for(22, 0, 0)
    trees = [synth.random_tree(rng, 64, 8) for _ in range(4)]
    case = synth.greedy_case(22, trees, vocab=128256, tie_frac=0.5)
    rows = _f64(case)
    tied = 0
    for u in range(len(case.parents)):
        if case.planted[u] >= 0:
            assert oracle.argmax_lowest(rows[u]) == case.planted[u]
            tied += int((rows[u] == rows[u].max()).sum() > 1)
    assert tied > 20
    # the walk follows the lower-index tie token: a child carrying the higher partner is never accepted
    got = oracle.accept_greedy(case.node_offsets, case.parents, case.draft_tokens, case.logits, "bf16")
    for b, (n_acc, path, toks) in enumerate(got):
        n0 = case.node_offsets[b]
        for k in range(1, len(path)):
            assert case.draft_tokens[n0 + path[k]] == oracle.argmax_lowest(rows[n0 + path[k - 1]])


def _single_node(p_logits, q, kid_tokens, u_acc, u_smp):
    m = len(kid_tokens)
    par = np.array([-1] + [0] * m, np.int32)
    V = len(q)
    logits = np.tile(p_logits, (m + 1, 1))
    qs = np.tile(q, (m + 1, 1)).astype(np.float32)
    toks = np.array([0] + list(kid_tokens), np.int32)
    ua = np.array([0.0] + list(u_acc), np.float64)
    us = np.full(m + 1, u_smp, np.float64)
    return oracle.accept_rejection(np.array([0, m + 1]), par, toks, logits.astype(np.float64), qs, ua, us,
                                   dtype="f64")[0]


def test_rejection_exact_law_closed_form():
    """For a node whose m children are i.i.d. from q, the first emitted token has law p exactly:
    sum_j prod_{i<j}(1-alpha_i) min(q, res_{j-1}) + prod_i(1-alpha_i) res_m, alpha_i = sum min(q, res_{i-1}),
    with res_i the oracle's residual sequence."""
    rng = np.random.default_rng(5)
    V = 32
    for trial in range(40):
        p = oracle.target_probs(rng.normal(0, 2, V))
        q = scipy.special.softmax(rng.normal(0, 2, V) if trial % 3 else np.log(p) + rng.normal(0, .3, V))
        m = 1 + trial % 3
        res, law, reach = p, np.zeros(V), 1.0
        for _ in range(m):
            hit = np.minimum(q, res)
            law += reach * hit
            reach *= 1.0 - hit.sum()
            res = acc._residual(res, q)
        law += reach * res
        np.testing.assert_allclose(law, p, rtol=0, atol=1e-12)


def test_rejection_exact_law_black_box():
    """Same law, measured by running the oracle itself: the accept decision and the final draw are
    threshold functions of their uniforms, so bisection over the 2^-24 grid recovers each probability;
    the law of the first emitted token, over all child-token tuples, must equal softmax(logits)."""
    rng = np.random.default_rng(6)
    V = 6
    G = 1 << 24

    def bisect(pred):      # smallest grid k with pred(k * 2^-24) True (pred monotone False..True)
        lo, hi = 0, G
        while lo < hi:
            mid = (lo + hi) // 2
            if pred(mid / G):
                hi = mid
            else:
                lo = mid + 1
        return lo

    for trial in range(4):
        lg = rng.normal(0, 1.5, V)
        p = scipy.special.softmax(lg)
        q = scipy.special.softmax(rng.normal(0, 1.5, V)).astype(np.float32).astype(np.float64)
        q = q / q.sum()
        for m in (1, 2):
            law = np.zeros(V)
            for tup in np.ndindex(*([V] * m)):
                w = np.prod([q[x] for x in tup])
                reach = 1.0
                top = (G - 1) / G          # the largest uniform: rejects every child that can be rejected
                for j in range(m):
                    # probability that child j is accepted once children < j were rejected: the walk moves
                    # to child j exactly for u below a threshold
                    pre = [top] * j
                    first_rej = bisect(lambda u: _single_node(lg, q, tup, pre + [u] + [top] * (m - j - 1),
                                                              0.5)[1] != [0, 1 + j])
                    t = first_rej / G
                    law[tup[j]] += w * reach * t
                    reach *= 1.0 - t
                # all rejected: the draw's law from the boundaries of the inverse CDF over u_sample
                rej = [top] * m
                prev = 0
                for v in range(V):
                    bnd = bisect(lambda u: _single_node(lg, q, tup, rej, u)[2][0] > v) if v < V - 1 else G
                    law[v] += w * reach * (bnd - prev) / G
                    prev = bnd
            np.testing.assert_allclose(law, p, atol=5e-6)


def test_rejection_acceptance_rate_identity():
    """One child: P(accept) = sum_x min(p(x), q(x)) = 1 - TV(p, q)."""
    rng = np.random.default_rng(7)
    V, n = 32, 20000
    lg = rng.normal(0, 2, V)
    p = scipy.special.softmax(lg)
    q = scipy.special.softmax(rng.normal(0, 2, V)).astype(np.float32)
    r = synth.rng_for(23, 0, 0)
    B = n
    toks = np.zeros(2 * B, np.int32)
    toks[1::2] = r.choice(V, size=B, p=q.astype(np.float64) / q.astype(np.float64).sum())
    offs = np.arange(0, 2 * B + 1, 2, dtype=np.int32)
    par = np.tile(np.array([-1, 0], np.int32), B)
    ua = synth.uniforms24(r, 2 * B)
    us = synth.uniforms24(r, 2 * B)
    out = oracle.accept_rejection(offs, par, toks, np.tile(lg, (2 * B, 1)), np.tile(q, (2 * B, 1)), ua, us, "f64")
    rate = np.mean([o[0] for o in out])
    alpha = np.minimum(p, q).sum()
    assert abs(rate - alpha) < 4 * math.sqrt(alpha * (1 - alpha) / n)


def test_rejection_p_equals_q_always_accepts():
    rng = np.random.default_rng(8)
    V = 40
    lg = rng.normal(0, 2, V)
    q = oracle.target_probs(lg)
    for t in range(200):
        x = int(rng.integers(V))
        got = _single_node(lg, q, [x, (x + 1) % V], [rng.random() * (1 - 1e-9), 0.0], rng.random())
        assert got[0] == 1 and got[1] == [0, 1]


def test_rejection_one_hot_equals_greedy():
    """Temperature 0: a one-hot target turns the rejection walk into greedy verification
    (distinct sibling tokens, so both readings of longest-accepted-path coincide)."""
    rng = synth.rng_for(24, 0, 0)
    trees = [synth.random_tree(rng, 40, 6) for _ in range(3)]
    g = synth.greedy_case(24, trees, vocab=300, dtype="f32")
    rows = g.logits.astype(np.float64)
    one_hot = np.full_like(rows, -np.inf)
    for u in range(len(rows)):
        one_hot[u, oracle.argmax_lowest(rows[u])] = 0.0
    q = scipy.special.softmax(rng.normal(0, 2, rows.shape), axis=1).astype(np.float32)
    r = synth.rng_for(24, 0, 8)
    ua, us = synth.uniforms24(r, len(rows)), synth.uniforms24(r, len(rows))
    rej = oracle.accept_rejection(g.node_offsets, g.parents, g.draft_tokens, one_hot, q, ua, us, "f64")
    gre = oracle.accept_greedy(g.node_offsets, g.parents, g.draft_tokens, g.logits, "f32")
    assert rej == gre


def _g1_tv(mutant=None, trials=160000, V=32, m=3, seed=25):
    """Empirical law of the first emitted token at a node with m i.i.d. children, vs p."""
    r = synth.rng_for(seed, 0, 0)
    lg = r.normal(0, 1.0, V)
    p = oracle.target_probs(lg)
    q = scipy.special.softmax(r.normal(0, 1.0, V)).astype(np.float32)
    qd = q.astype(np.float64) / q.astype(np.float64).sum()
    n = m + 1
    counts = np.zeros(V)
    per = 20000
    for start in range(0, trials, per):
        B = min(per, trials - start)
        toks = np.zeros(n * B, np.int32)
        kids = r.choice(V, size=(B, m), p=qd)
        toks.reshape(B, n)[:, 1:] = kids
        par = np.tile(np.array([-1] + [0] * m, np.int32), B)
        offs = np.arange(0, n * B + 1, n, dtype=np.int32)
        ua = synth.uniforms24(r, n * B)
        us = synth.uniforms24(r, n * B)
        out = acc.accept_rejection(offs, par, toks, np.tile(lg, (n * B, 1)), np.tile(q, (n * B, 1)), ua, us,
                                   "f64", _mutant=mutant)
        for o in out:
            counts[o[2][0]] += 1
    return 0.5 * np.abs(counts / trials - p).sum()


@pytest.mark.slow
def test_rejection_g1_gate_and_mutants():
    gold = json.load(open(os.path.join(HERE, "golden", "rejection_g1.json")))
    trials, V = 160000, 32
    floor = math.sqrt(V / (2 * math.pi * trials))
    tv = _g1_tv(trials=trials, V=V)
    assert tv < gold["tv_gate"]
    assert tv < 2.5 * floor
    for mutant in ("skip_accept", "resample_p"):
        assert _g1_tv(mutant, trials=40000, V=V) > gold["tv_gate"]
