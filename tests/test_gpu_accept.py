"""GPU parity of spec_accept_greedy and spec_accept_rejection against the oracle: bit-exact accepted
counts, paths and tokens (rejection: every case whose smallest decision margin is above 1e-9, which
is all of them in practice; the count of skipped cases is asserted to be 0 here), and the G1
statistical gate for the GPU sampler."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import device as sdev
from gpu_util import dev

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


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
        g = g.cpu().numpy()
        assert np.array_equal(g, e), f"{name}:\n{g}\nvs\n{e}"


def _greedy(case, max_path):
    import long_context_tree_amd as lt
    t = sdev.greedy_tensors(case, dev())
    mn = int(np.diff(case.node_offsets).max())
    outs = lt.accept_greedy(t["node_offsets"], t["parents"], t["draft_tokens"], t["target_logits"], max_nodes=mn,
                            max_path=max_path)
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("name", ["tiny", "tiny_batch", "llama_v128k", "qwen_chains", "ties", "single_nodes",
                                  "odd_vocab"])
def test_greedy_matches_oracle(name):
    r = synth.rng_for(200, 0, 0)
    if name == "tiny":
        trees, V, dt = [synth.random_tree(r, 8, 4)], 32, "f32"
    elif name == "tiny_batch":
        trees, V, dt = [synth.random_tree(r, 8, 4) for _ in range(50)], 32, "f32"
    elif name == "llama_v128k":
        trees, V, dt = [synth.random_tree(r, 64, 8)], 128256, "bf16"
    elif name == "qwen_chains":
        trees, V, dt = [synth.chain_tree(5) for _ in range(16)], 151936, "bf16"
    elif name == "ties":
        trees, V, dt = [synth.random_tree(r, 128, 10) for _ in range(2)], 128256, "bf16"
    elif name == "odd_vocab":                  # rows off 16-byte boundaries: the entry-by-entry loads
        trees, V, dt = [synth.random_tree(r, 24, 5), synth.random_tree(r, 9, 3)], 20011, "bf16"
    else:
        trees, V, dt = [synth.chain_tree(1), synth.random_tree(r, 3, 2), synth.chain_tree(1)], 1000, "bf16"
    case = synth.greedy_case(200 + len(name), trees, V, dtype=dt, tie_frac=0.5 if name == "ties" else 0.25)
    print(f"case={name}", flush=True)
    max_path = 12
    outs = _greedy(case, max_path)
    ref = oracle.accept_greedy(case.node_offsets, case.parents, case.draft_tokens, case.logits, dt)
    _check(outs, _expected(ref, len(trees), max_path))


def test_greedy_path_longer_than_max_path_is_reported():
    trees = [synth.chain_tree(9)]
    case = synth.greedy_case(210, trees, 500, dtype="f32", plant_frac=1.0, tie_frac=0.0, alpha=1.0)
    ref = oracle.accept_greedy(case.node_offsets, case.parents, case.draft_tokens, case.logits, "f32")
    assert ref[0][0] == 8
    outs = _greedy(case, 5)
    _check(outs, _expected(ref, 1, 5))     # n = -1, rows of -1


def _rejection(case, max_path, max_children):
    import long_context_tree_amd as lt
    t = sdev.rejection_tensors(case, dev())
    mn = int(np.diff(case.node_offsets).max())
    outs = lt.accept_rejection(t["node_offsets"], t["parents"], t["draft_tokens"], t["target_logits"],
                               t["draft_probs"], t["u_accept"], t["u_sample"], max_nodes=mn, max_path=max_path,
                               max_children=max_children)
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("name", ["tiny", "tiny_close", "tiny_batch", "llama_v128k", "llama_v128k_close", "chains"])
def test_rejection_matches_oracle(name):
    r = synth.rng_for(220, 0, 0)
    draft = "close" if name.endswith("close") else "independent"
    if name.startswith("tiny_batch"):
        trees, V, dt = [synth.random_tree(r, 8, 4) for _ in range(64)], 32, "f32"
        draft = "close"
    elif name.startswith("tiny"):
        trees, V, dt = [synth.random_tree(r, 8, 4)], 32, "f32"
    elif name.startswith("llama"):
        trees, V, dt = [synth.random_tree(r, 64, 8)], 128256, "bf16"
    else:
        trees, V, dt = [synth.chain_tree(5) for _ in range(16)], 151936, "bf16"
        draft = "close"
    case = synth.rejection_case(220 + len(name), trees, V, dtype=dt, draft=draft, draft_noise=0.3)
    print(f"case={name}", flush=True)
    max_children = max(max(len(c) for c in synth.children_lists(t)) for t in trees)
    max_path = 12
    outs = _rejection(case, max_path, max(1, max_children))
    ref = oracle.accept_rejection(case.node_offsets, case.parents, case.draft_tokens, case.logits, case.draft_probs,
                                  case.u_accept, case.u_sample, dt, return_margins=True)
    skipped = [b for b, x in enumerate(ref) if x[3] < 1e-9]
    assert not skipped, f"decisions within the tie band: {skipped}"
    _check(outs, _expected([x[:3] for x in ref], len(trees), max_path))


def test_rejection_gpu_g1_gate():
    """G1 of the Adaptive Speculative Decoding page, run on the GPU sampler: the first emitted token at
    a node with 3 i.i.d. children, over 1.6e5 seeded trials at V=32, has TV <= 0.02 from p."""
    gold = json.load(open(os.path.join(HERE, "golden", "rejection_g1.json")))
    import long_context_tree_amd as lt
    V, m, trials = 32, 3, 160000
    n = m + 1
    rg = synth.rng_for(230, 0, 0)
    lg = rg.normal(0, 1.0, V).astype(np.float32)
    p = oracle.target_probs(lg.astype(np.float64))
    ql = rg.normal(0, 1.0, V)
    q = np.exp(ql - ql.max())
    q = (q / q.sum()).astype(np.float32)
    qd = q.astype(np.float64) / q.astype(np.float64).sum()
    counts = np.zeros(V)
    B = 16000                                  # batch * max_nodes stays <= 65535
    for start in range(0, trials, B):
        toks = np.zeros((B, n), np.int32)
        toks[:, 1:] = rg.choice(V, size=(B, m), p=qd)
        par = np.tile(np.array([-1] + [0] * m, np.int32), B)
        offs = np.arange(0, n * B + 1, n, dtype=np.int32)
        ua = synth.uniforms24(rg, n * B)
        us = synth.uniforms24(rg, n * B)
        d = dev()
        outs = lt.accept_rejection(torch.from_numpy(offs).to(d), torch.from_numpy(par).to(d),
                                   torch.from_numpy(toks.reshape(-1)).to(d),
                                   torch.from_numpy(np.tile(lg, (n * B, 1))).to(d),
                                   torch.from_numpy(np.tile(q, (n * B, 1))).to(d), torch.from_numpy(ua).to(d),
                                   torch.from_numpy(us).to(d), max_nodes=n, max_path=3, max_children=m)
        first = outs[2][:, 0].cpu().numpy()
        counts += np.bincount(first, minlength=V)
    tv = 0.5 * np.abs(counts / trials - p).sum()
    floor = math.sqrt(V / (2 * math.pi * trials))
    print(f"TV={tv:.4f} floor={floor:.4f}")
    assert tv < gold["tv_gate"] and tv < 2.5 * floor


@pytest.mark.parametrize("K", [12, 20])
def test_rejection_many_siblings(K):
    """A root with K i.i.d. children (plus one grandchild) where every child is rejected: the bonus token is
    drawn from the root's residual after K levels, past the 9 levels held in registers; bit-exact with the
    oracle, and the case is outside the tie band."""
    t = np.array([-1] + [0] * K + [1], dtype=np.int32)
    case = synth.rejection_case(263, [t], 64, dtype="bf16", draft="independent")
    ref = oracle.accept_rejection(case.node_offsets, case.parents, case.draft_tokens, case.logits, case.draft_probs,
                                  case.u_accept, case.u_sample, "bf16", return_margins=True)
    assert ref[0][0] == 0 and ref[0][3] > 1e-6
    outs = _rejection(case, 3, K)
    _check(outs, _expected([x[:3] for x in ref], 1, 3))


@pytest.mark.parametrize("dt,V", [("bf16", 5003), ("f32", 5003), ("bf16", 128256)])
def test_rejection_odd_vocab_and_masked_segments(dt, V):
    """Rows whose length is not a multiple of 8 (most rows then start off a 16-byte boundary, so their
    runs take the entry-by-entry loads, and the last segment is ragged), and target logits of -inf over
    the whole second 2048-entry segment plus 5% of the other entries (p = 0 there; a segment with no
    finite logit has no mass at any level): bit-exact with the oracle, every decision outside the tie
    band."""
    r = synth.rng_for(270, 0, 0)
    trees = [synth.random_tree(r, 24, 5), synth.random_tree(r, 9, 3)]
    case = synth.rejection_case(270 + V % 97, trees, V, dtype=dt, draft="independent")
    neg = np.uint16(0xFF80) if dt == "bf16" else np.float32(-np.inf)
    lg = case.logits.copy()
    lg[:, 2048:4096] = neg
    hit = synth.rng_for(271, 0, 0).random(lg.shape) < 0.05
    lg[hit] = neg
    case.logits = lg
    rows = oracle.acceptance._rows_f64(lg, dt)
    assert np.isfinite(rows.max(axis=1)).all()
    print(f"case={dt} V={V}", flush=True)
    max_children = max(max(len(c) for c in synth.children_lists(t)) for t in trees)
    ref = oracle.accept_rejection(case.node_offsets, case.parents, case.draft_tokens, case.logits, case.draft_probs,
                                  case.u_accept, case.u_sample, dt, return_margins=True)
    assert all(x[3] > 1e-9 for x in ref)
    outs = _rejection(case, 12, max(1, max_children))
    _check(outs, _expected([x[:3] for x in ref], len(trees), 12))


def test_rejection_single_node_trees():
    """Every tree is its root alone (max_nodes = 1, so max_children = 0: no residual level beyond p): each
    sequence accepts nothing and draws its bonus token from p, bit-exact with the oracle."""
    trees = [synth.chain_tree(1) for _ in range(5)]
    case = synth.rejection_case(275, trees, 3001, dtype="bf16", draft="independent")
    ref = oracle.accept_rejection(case.node_offsets, case.parents, case.draft_tokens, case.logits, case.draft_probs,
                                  case.u_accept, case.u_sample, "bf16", return_margins=True)
    assert all(x[0] == 0 and x[3] > 1e-9 for x in ref)
    outs = _rejection(case, 2, 0)
    _check(outs, _expected([x[:3] for x in ref], len(trees), 2))
