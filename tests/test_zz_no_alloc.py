"""spec_accept_greedy_noalloc (the library's per-GPU device array in place of a workspace) against
spec_accept_greedy with a caller workspace, both called through the C ABI: two calls in a row, the
second on a smaller input, so that keys left in the array by the first call must not leak into the
second; every output element is compared (bit-exact, integer outputs), and the oracle confirms both."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import dev
from synth import device as sdev

pytestmark = pytest.mark.gpu


def _call(name, g, max_nodes, max_path):
    from long_context_tree_amd import spec
    L = spec.lib()
    gt = sdev.greedy_tensors(g, dev())
    B = len(g.node_offsets) - 1
    outs = (torch.full((B,), 77, dtype=torch.int32, device=dev()),
            torch.full((B, max_path), 77, dtype=torch.int32, device=dev()),
            torch.full((B, max_path), 77, dtype=torch.int32, device=dev()))
    a = spec._greedy_args(gt["node_offsets"], gt["parents"], gt["draft_tokens"], gt["target_logits"], max_nodes,
                          max_path, outs)
    ws = None
    if name == "spec_accept_greedy":
        need = L.spec_accept_greedy_workspace_size(ctypes.byref(a))
        ws = torch.empty(need, dtype=torch.uint8, device=dev())
        a.workspace, a.workspace_bytes = ws.data_ptr(), need
    else:
        a.workspace, a.workspace_bytes = None, 0          # ignored by the no-allocation entry point
    st = getattr(L, name)(ctypes.byref(a), torch.cuda.current_stream().cuda_stream)
    assert st == 0, (name, spec.last_error())
    torch.cuda.synchronize()
    del ws
    return [o.cpu().numpy() for o in outs]


def _cases():
    r = synth.rng_for(240, 0, 0)
    big = synth.greedy_case(240, [synth.random_tree(r, 128, 10), synth.random_tree(r, 64, 8)], 128256, dtype="bf16")
    small = synth.greedy_case(241, [synth.random_tree(r, 16, 5)], 5003, dtype="f32")
    return [(big, 128, 11), (small, 16, 6)]


def test_noalloc_greedy_matches_workspace_call_twice_second_smaller():
    for g, max_nodes, max_path in _cases():
        print(f"noalloc greedy: batch {len(g.node_offsets) - 1}, max_nodes {max_nodes}, vocab {g.logits.shape[1]}",
              flush=True)
        ref = _call("spec_accept_greedy", g, max_nodes, max_path)
        got = _call("spec_accept_greedy_noalloc", g, max_nodes, max_path)
        for x, y in zip(ref, got):
            assert np.array_equal(x, y)
        for b, (n, path, toks) in enumerate(oracle.accept_greedy(g.node_offsets, g.parents, g.draft_tokens,
                                                                 g.logits, g.dtype)):
            assert got[0][b] == n
            assert got[1][b, :n + 1].tolist() == path and (got[1][b, n + 1:] == -1).all()
            assert got[2][b, :n + 1].tolist() == toks and (got[2][b, n + 1:] == -1).all()


def test_noalloc_refuses_more_than_its_array():
    from long_context_tree_amd import spec
    r = synth.rng_for(242, 0, 0)
    g = synth.greedy_case(242, [synth.chain_tree(3)], 64, dtype="f32")
    gt = sdev.greedy_tensors(g, dev())
    outs = spec._outs(1, 4, dev())
    a = spec._greedy_args(gt["node_offsets"], gt["parents"], gt["draft_tokens"], gt["target_logits"], 3, 4, outs)
    a.batch, a.max_nodes, a.vocab = 1, 2048, 1 << 24            # 2048 x 2048 segment keys: 32 MiB
    assert spec.lib().spec_accept_greedy_noalloc(ctypes.byref(a), torch.cuda.current_stream().cuda_stream) == 2
    assert "device array" in spec.last_error()
