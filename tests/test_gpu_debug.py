"""The SPEC_DEBUG build (libspec_verify_debug.so) on the GPU, called through the C ABI.

* On valid inputs its debug record says nothing is wrong, its outputs are the release build's bits,
  and the acceptance witnesses count every row reduction and every draft test of the call.
* On inputs that break a documented device precondition (a parent that is not an earlier node, a
  block-table id past the pool, a context length past max_ctx_len, a draft token past the vocabulary,
  a uniform outside [0, 1), a negative draft probability, a NaN logit) the call still completes (the
  kernels clamp what they read) and the record names the broken precondition."""

import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_util import dev
from synth import device as sdev

pytestmark = pytest.mark.gpu


def _spec():
    from long_context_tree_amd import spec
    return spec


def _attention(L, case, t, max_nodes, max_ctx, chunk=64):
    spec = _spec()
    T, Hq, D = t["q"].shape
    out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=dev())
    lse = torch.empty((T, Hq), dtype=torch.float32, device=dev())
    a = spec.tree_attention_args(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["ctx_lens"],
                                 t["node_offsets"], t["parents"], max_nodes=max_nodes, max_ctx_len=max_ctx,
                                 chunk_size=chunk, out=out, lse=lse)
    need = L.spec_tree_attention_workspace_size(ctypes.byref(a))
    ws = spec._workspace(need, dev(), None)
    ws.fill_(0xAB)                                  # the record must be written, not left over
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    st = L.spec_tree_attention(ctypes.byref(a), torch.cuda.current_stream().cuda_stream)
    assert st == 0, L.spec_last_error()
    torch.cuda.synchronize()
    return out, lse, spec.debug_record(ws, need)


def _attn_case():
    r = synth.rng_for(250, 0, 0)
    case = synth.attention_case(250, ctx_lens=[2000, 333], trees=[synth.random_tree(r, 40, 6), synth.chain_tree(5)],
                                num_q_heads=8, num_kv_heads=2, head_dim=128)
    return case, sdev.attention_tensors(case, dev())


def test_debug_attention_valid_inputs_match_release():
    spec = _spec()
    case, t = _attn_case()
    print("debug attention: valid", flush=True)
    o_rel, l_rel, _ = _attention(spec.lib(), case, t, 40, 2000)
    o_dbg, l_dbg, rec = _attention(spec.debug_lib(), case, t, 40, 2000)
    assert rec == [0, 0, 0, 0], rec
    assert torch.equal(o_rel.view(torch.int16), o_dbg.view(torch.int16)) and torch.equal(l_rel, l_dbg)


@pytest.mark.parametrize("kind", ["parents", "block_table", "ctx_lens", "node_offsets"])
def test_debug_attention_flags_broken_preconditions(kind):
    spec = _spec()
    case, t = _attn_case()
    max_ctx = 2000
    if kind == "parents":
        par = case.parents.copy()
        par[7] = 30                                 # node 7's parent is a later node: not topological
        t["parents"] = torch.from_numpy(par).to(dev())
    elif kind == "block_table":
        bt = case.kv.block_table.copy()
        bt[1, 3] = case.kv.k_pool.shape[0] + 5      # a page past the pool, inside sequence 1's slots
        t["block_table"] = torch.from_numpy(bt).to(dev())
    elif kind == "ctx_lens":
        max_ctx = 1500                              # sequence 0 holds 2000 > max_ctx_len committed tokens
    else:
        off = case.node_offsets.copy()
        off[1] = 41                                 # the first tree now has 41 > max_nodes nodes (the second's
        t["node_offsets"] = torch.from_numpy(off).to(dev())   # start is clamped back to node 40, its root)
    want = [kind]
    print(f"debug attention: {kind}", flush=True)
    out, lse, rec = _attention(spec.debug_lib(), case, t, 40, max_ctx)
    assert spec.debug_bits_names(rec[0]) == want, (rec, spec.debug_bits_names(rec[0]))
    assert rec[1:] == [0, 0, 0]


def _greedy(L, g, gt, max_nodes, max_path):
    spec = _spec()
    B = len(g.node_offsets) - 1
    outs = spec._outs(B, max_path, dev())
    a = spec._greedy_args(gt["node_offsets"], gt["parents"], gt["draft_tokens"], gt["target_logits"], max_nodes,
                          max_path, outs)
    need = L.spec_accept_greedy_workspace_size(ctypes.byref(a))
    ws = spec._workspace(need, dev(), None)
    ws.fill_(0xAB)
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    assert L.spec_accept_greedy(ctypes.byref(a), torch.cuda.current_stream().cuda_stream) == 0, L.spec_last_error()
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs], spec.debug_record(ws, need)


def _rejection(L, rc, rt, max_nodes, max_path, max_children):
    spec = _spec()
    B = len(rc.node_offsets) - 1
    outs = spec._outs(B, max_path, dev())
    r = spec.AcceptRejectionArgs()
    r.base = spec._greedy_args(rt["node_offsets"], rt["parents"], rt["draft_tokens"], rt["target_logits"], max_nodes,
                               max_path, outs)
    r.max_children = max_children
    r.draft_probs, r.u_accept, r.u_sample = (rt["draft_probs"].data_ptr(), rt["u_accept"].data_ptr(),
                                             rt["u_sample"].data_ptr())
    need = L.spec_accept_rejection_workspace_size(ctypes.byref(r))
    ws = spec._workspace(need, dev(), None)
    ws.fill_(0xAB)
    r.base.workspace, r.base.workspace_bytes = ws.data_ptr(), ws.numel()
    assert L.spec_accept_rejection(ctypes.byref(r), torch.cuda.current_stream().cuda_stream) == 0, \
        L.spec_last_error()
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs], spec.debug_record(ws, need)


def test_debug_greedy_witnesses_and_flags():
    """Witnesses: every row's argmax reduced in this call (sum of N), every draft tested (sum of N - 1)."""
    spec = _spec()
    r = synth.rng_for(251, 0, 0)
    trees = [synth.random_tree(r, 64, 8), synth.chain_tree(5), synth.random_tree(r, 17, 4)]
    g = synth.greedy_case(251, trees, 20011, dtype="bf16")
    gt = sdev.greedy_tensors(g, dev())
    print("debug greedy: valid", flush=True)
    rel, _ = _greedy(spec.lib(), g, gt, 64, 9)
    dbg, rec = _greedy(spec.debug_lib(), g, gt, 64, 9)
    for x, y in zip(rel, dbg):
        assert np.array_equal(x, y)
    n = [len(t) for t in trees]
    assert rec == [0, sum(n), sum(n) - len(n), 0], rec
    # a draft token past the vocabulary, and a NaN logit in a row that keeps a finite maximum
    tok = g.draft_tokens.copy()
    tok[3] = 20011 + 7
    gt2 = dict(gt, draft_tokens=torch.from_numpy(tok).to(dev()))
    lg = gt["target_logits"].clone()
    lg[10, 5] = float("nan")
    gt2["target_logits"] = lg
    print("debug greedy: tokens + logits", flush=True)
    _, rec = _greedy(spec.debug_lib(), g, gt2, 64, 9)
    assert spec.debug_bits_names(rec[0]) == ["logits", "tokens"], rec
    # a parent that is not an earlier node: the walk refuses that sequence (-1) and tests none of its drafts
    par = g.parents.copy()
    par[int(g.node_offsets[2]) + 4] = 9
    gt3 = dict(gt, parents=torch.from_numpy(par).to(dev()))
    print("debug greedy: parents", flush=True)
    out, rec = _greedy(spec.debug_lib(), g, gt3, 64, 9)
    assert spec.debug_bits_names(rec[0]) == ["parents"], rec
    assert out[0][2] == -1 and rec[1:] == [n[0] + n[1], n[0] + n[1] - 2, 0], rec


def test_debug_rejection_witnesses_and_flags():
    spec = _spec()
    r = synth.rng_for(252, 0, 0)
    trees = [synth.random_tree(r, 30, 6), synth.chain_tree(5)]
    rc = synth.rejection_case(252, trees, 5003, dtype="bf16", draft="close", draft_noise=0.3)
    rt = sdev.rejection_tensors(rc, dev())
    mc = max(max(len(c) for c in synth.children_lists(t)) for t in trees)
    print("debug rejection: valid", flush=True)
    rel, _ = _rejection(spec.lib(), rc, rt, 30, 12, mc)
    dbg, rec = _rejection(spec.debug_lib(), rc, rt, 30, 12, mc)
    for x, y in zip(rel, dbg):
        assert np.array_equal(x, y)
    n = [len(t) for t in trees]
    assert rec == [0, sum(n), sum(n) - len(n), 0], rec
    ua = rt["u_accept"].clone()
    ua[4] = 1.5
    q = rt["draft_probs"].clone()
    q[2, 17] = -0.25
    print("debug rejection: uniforms + draft probs", flush=True)
    _, rec = _rejection(spec.debug_lib(), rc, dict(rt, u_accept=ua, draft_probs=q), 30, 12, mc)
    assert spec.debug_bits_names(rec[0]) == ["draft_probs", "uniforms"], rec
    if mc > 1:
        print("debug rejection: children", flush=True)
        _, rec = _rejection(spec.debug_lib(), rc, rt, 30, 12, mc - 1)
        assert spec.debug_bits_names(rec[0]) == ["children"], rec
