"""GPU parity at the full sizes of the measured workloads, with the seeds and the launch plan that
bench.py uses (the default split plan), against the oracle on every KV head of the layer:

* the Llama-3.1-8B-shaped layer at 131072 tokens of context with the 128-node tree of depth 10, in both
  V layouts: outputs and LSEs of all 32 query heads, all 2048 chunk masses, the top-256 chunks;
* the same layer shape at 65536 tokens with a 64-node tree of depth 8;
* the ragged Qwen3-8B-shaped batch: 16 sequences with contexts uniform in [4096, 65536], chains of
  4 drafts, outputs of every sequence and head and every sequence's chunk masses;
* greedy acceptance of the 128-node tree at vocabulary 128256 and rejection acceptance of the 64-node
  tree at vocabulary 128256 on the benchmark's own inputs (bit-exact).

Unused pool pages hold NaN, so a read outside the sequences' pages would show.  The oracle runs one
KV head (or one sequence) per worker thread; numpy's BLAS releases the GIL."""

import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import bits_of, compare_mass, compare_out, dev, topk_valid
from synth import device as sdev

pytestmark = pytest.mark.gpu

HQ, HKV, D, CHUNK = 32, 8, 128, 64


def _workers():
    return max(1, min(8, len(os.sched_getaffinity(0))))


def _poison_unused_pages(k, v, bt):
    used = torch.zeros(k.shape[0], dtype=torch.bool, device=k.device)
    ids = bt[bt >= 0].long()
    used[ids] = True
    k[~used] = float("nan")
    v[~used] = float("nan")


def _oracle_heads(qb, kb, vb, btn, ctx, offs, parents, v_layout, seqs=None):
    """oracle.tree_attention over every KV head, one head per task; the chunk masses of the heads are
    averaged (each task's mass is its own heads' mean)."""
    def one(g):
        return oracle.tree_attention(qb, kb, vb, btn, ctx, offs, parents, 1 / np.sqrt(D), HKV, 16, CHUNK,
                                     kv_heads=[g], seqs=seqs, v_layout=v_layout)
    with cf.ThreadPoolExecutor(_workers()) as ex:
        res = list(ex.map(one, range(HKV)))
    out = np.where(np.isnan(res[0][0]), 0.0, res[0][0])
    lse = np.where(np.isnan(res[0][1]), 0.0, res[0][1])
    for o, l, _ in res[1:]:
        out += np.where(np.isnan(o), 0.0, o)
        lse += np.where(np.isnan(l), 0.0, l)
    masses = [sum(r[2][b] for r in res) / HKV for b in range(len(res[0][2]))]
    return out, lse, masses


def _attention_full(case, L, N, depth, v_layout, top_k):
    import long_context_tree_amd as lt
    tree = synth.random_tree(synth.rng_for(case, 0, synth.S_TREE), N, depth)
    k, v, bt = sdev.paged_kv_device(case, 0, [L + N], HKV, D, dev(), v_layout=v_layout)
    _poison_unused_pages(k, v, bt)
    q = sdev.queries_device(case, 0, N, HQ, D, dev())
    cl = torch.tensor([L], dtype=torch.int32, device=dev())
    no = torch.tensor([0, N], dtype=torch.int32, device=dev())
    par = torch.from_numpy(tree).to(dev())
    print(f"full-size attention L={L} N={N} v_layout={v_layout}", flush=True)
    out, lse, h = lt.tree_attention(q, k, v, bt, cl, no, par, max_nodes=N, max_ctx_len=L, chunk_size=CHUNK,
                                    v_layout=v_layout)
    mass = torch.zeros((1, L // CHUNK), dtype=torch.float32, device=dev())
    _, ti, tm = lt.chunk_salience(h, mass, top_k=top_k)
    torch.cuda.synchronize()
    o_ref, l_ref, m_ref = _oracle_heads(bits_of(q), bits_of(k), bits_of(v), bt.cpu().numpy(), np.array([L]),
                                        np.array([0, N]), tree, v_layout)
    stats = compare_out(out, lse, o_ref, l_ref)
    mg = mass.cpu().numpy()[0].astype(np.float64)
    mstats = compare_mass(mg, m_ref[0])
    print(f"  out {stats}  mass {mstats}", flush=True)
    if top_k:
        idx = ti.cpu().numpy()[0]
        topk_valid(idx, m_ref[0], top_k)
        got = mass.cpu().numpy()[0]
        order = sorted(range(len(got)), key=lambda c: (-got[c], c))[:top_k]
        assert idx.tolist() == order
        np.testing.assert_array_equal(tm.cpu().numpy()[0], got[idx])


@pytest.mark.parametrize("v_layout", [0, 1])
def test_llama8b_128k_n128_every_head(v_layout):
    _attention_full(4, 131072, 128, 10, v_layout, 256)


def test_llama8b_64k_n64_every_head():
    _attention_full(3, 65536, 64, 8, 0, 0)


def test_qwen3_8b_ragged_chains_every_sequence():
    """16 sequences, contexts uniform in [4096, 65536] (the benchmark's seed), chains of 4 drafts."""
    import long_context_tree_amd as lt
    case, n, B = 5, 5, 16
    lens = synth.ragged_ctx_lens(case, B, 4096, 65536)
    k, v, bt = sdev.paged_kv_device(case, 0, [int(x) + n for x in lens], HKV, D, dev())
    _poison_unused_pages(k, v, bt)
    par = np.concatenate([synth.chain_tree(n)] * B).astype(np.int32)
    offs = np.arange(0, B * n + 1, n, dtype=np.int32)
    q = sdev.queries_device(case, 0, B * n, HQ, D, dev())
    print(f"ragged batch lens={lens.tolist()}", flush=True)
    out, lse, h = lt.tree_attention(q, k, v, bt, torch.from_numpy(lens).to(dev()), torch.from_numpy(offs).to(dev()),
                                    torch.from_numpy(par).to(dev()), max_nodes=n, max_ctx_len=int(lens.max()),
                                    chunk_size=CHUNK)
    n_ch = -(-int(lens.max()) // CHUNK)
    mass = torch.zeros((B, n_ch), dtype=torch.float32, device=dev())
    lt.chunk_salience(h, mass)
    torch.cuda.synchronize()
    qb, kb, vb, btn = bits_of(q), bits_of(k), bits_of(v), bt.cpu().numpy()

    def one(b):
        return oracle.tree_attention(qb, kb, vb, btn, lens, offs, par, 1 / np.sqrt(D), HKV, 16, CHUNK, seqs=[b])

    with cf.ThreadPoolExecutor(_workers()) as ex:
        res = list(ex.map(one, range(B)))
    o_ref = np.zeros((B * n, HQ, D))
    l_ref = np.zeros((B * n, HQ))
    for b, (o, l, m) in enumerate(res):
        o_ref[b * n:(b + 1) * n] = o[b * n:(b + 1) * n]
        l_ref[b * n:(b + 1) * n] = l[b * n:(b + 1) * n]
    stats = compare_out(out, lse, o_ref, l_ref)
    mg = mass.cpu().numpy().astype(np.float64)
    for b, (_, _, m) in enumerate(res):
        mr = m[0]
        compare_mass(mg[b, :len(mr)], mr)
        assert (mg[b, len(mr):] == 0).all()
    print(f"  out {stats}", flush=True)


def test_benchmark_greedy_and_rejection_cases():
    """The acceptance calls the benchmark times, on its own inputs: greedy over the 128-node tree
    (depth 10) at vocabulary 128256, rejection over the 64-node tree (depth 8, <= 4 children) with
    independent draft probabilities at vocabulary 128256; both bit-exact with the oracle."""
    import long_context_tree_amd as lt
    V = 128256
    tree = synth.random_tree(synth.rng_for(4, 0, synth.S_TREE), 128, 10)
    g = synth.greedy_case(4, [tree], V, dtype="bf16")
    gt = sdev.greedy_tensors(g, dev())
    n_acc, path, toks = lt.accept_greedy(gt["node_offsets"], gt["parents"], gt["draft_tokens"], gt["target_logits"],
                                         max_nodes=128, max_path=11)
    torch.cuda.synchronize()
    (ref_n, ref_path, ref_toks), = oracle.accept_greedy(g.node_offsets, g.parents, g.draft_tokens, g.logits, "bf16")
    assert int(n_acc[0]) == ref_n
    assert path.cpu().numpy()[0, :ref_n + 1].tolist() == ref_path
    assert toks.cpu().numpy()[0, :ref_n + 1].tolist() == ref_toks

    rtree = synth.random_tree(synth.rng_for(3, 0, synth.S_TREE), 64, 8)
    rc = synth.rejection_case(3, [rtree], V, dtype="bf16", draft="independent")
    rt = sdev.rejection_tensors(rc, dev())
    n_acc, path, toks = lt.accept_rejection(rt["node_offsets"], rt["parents"], rt["draft_tokens"], rt["target_logits"],
                                            rt["draft_probs"], rt["u_accept"], rt["u_sample"], max_nodes=64,
                                            max_path=9, max_children=4)
    torch.cuda.synchronize()
    (ref_n, ref_path, ref_toks, margin), = oracle.accept_rejection(
        rc.node_offsets, rc.parents, rc.draft_tokens, rc.logits, rc.draft_probs, rc.u_accept, rc.u_sample, "bf16",
        return_margins=True)
    assert margin > 1e-9, margin
    assert int(n_acc[0]) == ref_n
    assert path.cpu().numpy()[0, :ref_n + 1].tolist() == ref_path
    assert toks.cpu().numpy()[0, :ref_n + 1].tolist() == ref_toks
