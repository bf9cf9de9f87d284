"""The calls allocate nothing and never synchronise, so a whole verification step can be captured into a
HIP graph: two layers of spec_tree_attention + spec_chunk_salience (the second with top-k), greedy and
rejection acceptance, the commit of the greedy path and the compact draft KV.  Every replay, with the
outputs cleared and other eager work on the device in between, must give the same bits as the eager
step, and the eager step must match the oracle."""

import ctypes

import pytest
import torch

import long_context_tree_amd as lt
from long_context_tree_amd import spec
import oracle
import synth
from synth import device as sdev
from gpu_util import compare_mass, compare_out, dev

pytestmark = pytest.mark.gpu


def _bits(x: torch.Tensor) -> torch.Tensor:
    # compare bit patterns (the caches hold NaN in unused pages, and NaN != NaN as values)
    return x.view({2: torch.int16, 4: torch.int32}[x.element_size()])


def test_captured_step_replays_bitwise_equal_to_eager():
    d = dev()
    L, N, Hq, Hkv, D, chunk, k, V = 3000, 24, 8, 2, 128, 64, 8, 512
    print(f"graph step: L={L} N={N} Hq={Hq} Hkv={Hkv} D={D} chunk={chunk} top_k={k} V={V}", flush=True)
    tree = synth.random_tree(synth.rng_for(41, 0, synth.S_TREE), N, 5)
    cases = [synth.attention_case(410 + l, ctx_lens=[L], trees=[tree], num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D)
             for l in range(2)]
    ts = [sdev.attention_tensors(c, d) for c in cases]
    nch = (L + chunk - 1) // chunk
    outs = [torch.empty((N, Hq, D), dtype=torch.bfloat16, device=d) for _ in range(2)]
    lses = [torch.empty((N, Hq), dtype=torch.float32, device=d) for _ in range(2)]
    attn = [spec.tree_attention_args(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["ctx_lens"],
                                     t["node_offsets"], t["parents"], max_nodes=N, max_ctx_len=L, chunk_size=chunk,
                                     split_tiles=0, out=outs[l], lse=lses[l]) for l, t in enumerate(ts)]
    wss = [spec._workspace(lt.lib().spec_tree_attention_workspace_size(ctypes.byref(a)), d, None) for a in attn]
    for a, w in zip(attn, wss):
        a.workspace, a.workspace_bytes = w.data_ptr(), w.numel()
    mass = torch.empty((1, nch), dtype=torch.float32, device=d)
    topi = torch.empty((1, k), dtype=torch.int32, device=d)
    topm = torch.empty((1, k), dtype=torch.float32, device=d)
    sal = []
    for l in range(2):
        s = spec.ChunkSalienceArgs()
        s.attn = ctypes.pointer(attn[l])
        s.chunk_mass, s.max_chunks, s.accumulate = mass.data_ptr(), nch, int(l > 0)
        s.top_k = k if l == 1 else 0
        s.topk_index, s.topk_mass = topi.data_ptr(), topm.data_ptr()
        sal.append(s)
    g = synth.greedy_case(42, [tree], V, dtype="bf16")
    gt = sdev.greedy_tensors(g, d)
    max_path = 6
    gouts = (torch.empty(1, dtype=torch.int32, device=d), torch.empty((1, max_path), dtype=torch.int32, device=d),
             torch.empty((1, max_path), dtype=torch.int32, device=d))
    ga = spec._greedy_args(gt["node_offsets"], gt["parents"], gt["draft_tokens"], gt["target_logits"], N, max_path,
                           gouts)
    gws = spec._workspace(lt.lib().spec_accept_greedy_workspace_size(ctypes.byref(ga)), d, None)
    ga.workspace, ga.workspace_bytes = gws.data_ptr(), gws.numel()
    rc = synth.rejection_case(43, [tree], V, dtype="bf16")
    rt = sdev.rejection_tensors(rc, d)
    routs = (torch.empty(1, dtype=torch.int32, device=d), torch.empty((1, max_path), dtype=torch.int32, device=d),
             torch.empty((1, max_path), dtype=torch.int32, device=d))
    ra = spec.AcceptRejectionArgs()
    ra.base = spec._greedy_args(rt["node_offsets"], rt["parents"], rt["draft_tokens"], rt["target_logits"], N,
                                max_path, routs)
    ra.max_children = 4
    ra.draft_probs, ra.u_accept, ra.u_sample = (rt["draft_probs"].data_ptr(), rt["u_accept"].data_ptr(),
                                                rt["u_sample"].data_ptr())
    rws = spec._workspace(lt.lib().spec_accept_rejection_workspace_size(ctypes.byref(ra)), d, None)
    ra.base.workspace, ra.base.workspace_bytes = rws.data_ptr(), rws.numel()
    # the commit of the greedy path into a copy of layer 0's cache, then the compact draft KV of the top-k
    # chunks plus a window from the uncommitted cache
    kc = [ts[0]["k_cache"].clone()]
    vc = [ts[0]["v_cache"].clone()]
    new_len = torch.empty(1, dtype=torch.int32, device=d)
    ca, ckeep = spec.kv_commit_args(kc, vc, ts[0]["block_table"], ts[0]["ctx_lens"], gouts[0], gouts[1],
                                    max_nodes=N, new_ctx_lens=new_len)
    cap = k * chunk + 128
    dk = torch.empty((1, cap, Hkv, D), dtype=torch.bfloat16, device=d)
    dv = torch.empty((1, cap, Hkv, D), dtype=torch.bfloat16, device=d)
    dpos = torch.empty((1, cap), dtype=torch.int32, device=d)
    dlen = torch.empty(1, dtype=torch.int32, device=d)
    inv_freq = torch.from_numpy(synth.rope_inv_freq(D)).to(d)
    da = spec.draft_gather_args(ts[0]["k_cache"], ts[0]["v_cache"], ts[0]["block_table"], ts[0]["ctx_lens"], topi,
                                max_ctx_len=L, chunk_size=chunk, window=128, capacity=cap, num_select=k,
                                rope=spec.ROPE_HALF, inv_freq=inv_freq, out_k=dk, out_v=dv, out_pos=dpos,
                                out_len=dlen)
    L_ = lt.lib()
    results = [outs[0], outs[1], lses[0], lses[1], mass, topi, topm, *gouts, *routs, new_len, dk, dv, dpos, dlen]

    def step(sh):
        for l in range(2):
            assert L_.spec_tree_attention(ctypes.byref(attn[l]), sh) == 0, lt.last_error()
            assert L_.spec_chunk_salience(ctypes.byref(sal[l]), sh) == 0, lt.last_error()
        assert L_.spec_accept_greedy(ctypes.byref(ga), sh) == 0, lt.last_error()
        assert L_.spec_accept_rejection(ctypes.byref(ra), sh) == 0, lt.last_error()
        assert L_.spec_kv_commit(ctypes.byref(ca), sh) == 0, lt.last_error()
        assert L_.spec_draft_gather(ctypes.byref(da), sh) == 0, lt.last_error()

    def clear():
        for x in results:
            x.fill_(-3 if x.dtype == torch.int32 else 7)
        kc[0].copy_(ts[0]["k_cache"])
        vc[0].copy_(ts[0]["v_cache"])

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        clear()
        step(stream.cuda_stream)
        torch.cuda.synchronize()
        ref = [x.clone() for x in results] + [kc[0].clone(), vc[0].clone()]

        # the eager step against the oracle (layer 1's outputs and the summed chunk masses)
        o_ref, l_ref, m1 = oracle.tree_attention(cases[1].q, cases[1].kv.k_pool, cases[1].kv.v_pool,
                                                 cases[1].kv.block_table, cases[1].ctx_lens, cases[1].node_offsets,
                                                 cases[1].parents, cases[1].scale, Hkv, 16, chunk)
        compare_out(outs[1], lses[1], o_ref, l_ref)
        _, _, m0 = oracle.tree_attention(cases[0].q, cases[0].kv.k_pool, cases[0].kv.v_pool,
                                         cases[0].kv.block_table, cases[0].ctx_lens, cases[0].node_offsets,
                                         cases[0].parents, cases[0].scale, Hkv, 16, chunk)
        compare_mass(mass.cpu().numpy()[0], m0[0] + m1[0])
        n, path, toks = oracle.accept_greedy(g.node_offsets, g.parents, g.draft_tokens, g.logits, "bf16")[0]
        assert int(gouts[0][0]) == n and gouts[1][0, :len(path)].tolist() == path

        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step(stream.cuda_stream)
        torch.cuda.synchronize()
        for rep in range(4):
            clear()
            scratch = torch.randn(1 << 20, device=d).sum()       # other eager work between the replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = results + [kc[0], vc[0]]
            for i, (a, b) in enumerate(zip(ref, got)):
                assert torch.equal(_bits(a), _bits(b)), f"replay {rep}: output {i} differs from the eager step"
            del scratch
