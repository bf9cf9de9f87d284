"""GPU parity of spec_kv_commit with the oracle: bit-exact caches (every page of every layer) and new
lengths, for both V layouts and several page sizes; and the commit of a path chosen by the GPU's own
greedy acceptance."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import dev
from synth import device as sdev

pytestmark = pytest.mark.gpu


def _root_path(parents, f):
    path = [f]
    while parents[path[-1]] >= 0:
        path.append(int(parents[path[-1]]))
    return path[::-1]


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("v_layout", [0, 1])
@pytest.mark.parametrize("page_size,head_dim", [(16, 128), (8, 64), (64, 128)])
def test_commit_matches_oracle(v_layout, page_size, head_dim):
    import long_context_tree_amd as lt
    seed = 200 + page_size + head_dim + v_layout
    r = synth.rng_for(seed, 0, 0)
    trees = [synth.random_tree(r, 40, 9), synth.chain_tree(5), synth.random_tree(r, 12, 4), synth.chain_tree(3)]
    ctx = np.array([900, 33, 0, 70], dtype=np.int32)
    slots = ctx + np.array([len(t) for t in trees], dtype=np.int32)
    layers = 3
    ks, vs = [], []
    bt = None
    for layer in range(layers):
        kv = synth.paged_kv(seed, layer, slots, 4, head_dim, page_size=page_size)
        bt = kv.block_table if bt is None else bt
        ks.append(kv.k_pool)
        vs.append(synth.dim_major(kv.v_pool) if v_layout else kv.v_pool)
    max_path = 12
    paths = np.full((4, max_path), -1, dtype=np.int32)
    nacc = np.zeros(4, dtype=np.int32)
    for b, t in enumerate(trees):
        f = int(np.argmax(synth.tree_depths(t))) if b != 2 else int(r.integers(len(t)))
        p = _root_path(t, f)
        paths[b, :len(p)] = p
        nacc[b] = len(p) - 1
    nacc[3] = -1                                # flagged: untouched
    print(f"page_size={page_size} head_dim={head_dim} v_layout={v_layout} nacc={nacc.tolist()}", flush=True)
    k_ref, v_ref, lens_ref = oracle.kv_commit(ks, vs, bt, ctx, nacc, paths, page_size, v_layout, max_nodes=40)
    kd = [sdev.bf16_tensor(k, dev()) for k in ks]
    vd = [sdev.bf16_tensor(v, dev()) for v in vs]
    lens = lt.kv_commit(kd, vd, torch.from_numpy(bt).to(dev()), torch.from_numpy(ctx).to(dev()),
                        torch.from_numpy(nacc).to(dev()), torch.from_numpy(paths).to(dev()), max_nodes=40,
                        v_layout=v_layout)
    torch.cuda.synchronize()
    assert lens.cpu().numpy().tolist() == lens_ref.tolist()
    for layer in range(layers):
        assert np.array_equal(_bits(kd[layer]), k_ref[layer])
        assert np.array_equal(_bits(vd[layer]), v_ref[layer])


def test_commit_of_the_greedy_path_in_place():
    """Greedy acceptance on the GPU, then the commit of its path with new_ctx_lens = ctx_lens."""
    import long_context_tree_amd as lt
    r = synth.rng_for(230, 0, 0)
    trees = [synth.random_tree(r, 64, 8), synth.random_tree(r, 30, 5)]
    g = synth.greedy_case(230, trees, 5000, dtype="bf16")
    gt = sdev.greedy_tensors(g, dev())
    n_acc, path, _ = lt.accept_greedy(gt["node_offsets"], gt["parents"], gt["draft_tokens"], gt["target_logits"],
                                      max_nodes=64, max_path=9)
    ctx = np.array([3000, 517], dtype=np.int32)
    slots = ctx + np.array([64, 30], dtype=np.int32)
    kv = synth.paged_kv(230, 0, slots, 8, 128)
    kd, vd = [sdev.bf16_tensor(kv.k_pool, dev())], [sdev.bf16_tensor(kv.v_pool, dev())]
    cl = torch.from_numpy(ctx).to(dev())
    lt.kv_commit(kd, vd, torch.from_numpy(kv.block_table).to(dev()), cl, n_acc, path, max_nodes=64, new_ctx_lens=cl)
    torch.cuda.synchronize()
    na, pa = n_acc.cpu().numpy(), path.cpu().numpy()
    assert (na >= 0).all()
    k_ref, v_ref, lens_ref = oracle.kv_commit([kv.k_pool], [kv.v_pool], kv.block_table, ctx, na, pa, 16)
    assert cl.cpu().numpy().tolist() == lens_ref.tolist()
    assert np.array_equal(_bits(kd[0]), k_ref[0]) and np.array_equal(_bits(vd[0]), v_ref[0])


def test_commit_with_new_lengths_over_num_accepted():
    """new_ctx_lens written over num_accepted (the same buffer): every layer and KV head still moves the
    accepted count it was given, and the buffer ends up holding the new lengths."""
    import long_context_tree_amd as lt
    r = synth.rng_for(231, 0, 0)
    trees = [synth.random_tree(r, 40, 9), synth.chain_tree(5), synth.random_tree(r, 12, 4)]
    ctx = np.array([900, 33, 70], dtype=np.int32)
    slots = ctx + np.array([len(t) for t in trees], dtype=np.int32)
    layers = 4
    ks, vs, bt = [], [], None
    for layer in range(layers):
        kv = synth.paged_kv(231, layer, slots, 8, 128)
        bt = kv.block_table if bt is None else bt
        ks.append(kv.k_pool)
        vs.append(kv.v_pool)
    max_path = 12
    paths = np.full((3, max_path), -1, dtype=np.int32)
    nacc = np.zeros(3, dtype=np.int32)
    for b, t in enumerate(trees):
        p = _root_path(t, int(np.argmax(synth.tree_depths(t))))
        paths[b, :len(p)] = p
        nacc[b] = len(p) - 1
    k_ref, v_ref, lens_ref = oracle.kv_commit(ks, vs, bt, ctx, nacc, paths, 16, 0, max_nodes=40)
    kd = [sdev.bf16_tensor(k, dev()) for k in ks]
    vd = [sdev.bf16_tensor(v, dev()) for v in vs]
    na = torch.from_numpy(nacc).to(dev())
    lt.kv_commit(kd, vd, torch.from_numpy(bt).to(dev()), torch.from_numpy(ctx).to(dev()), na,
                 torch.from_numpy(paths).to(dev()), max_nodes=40, new_ctx_lens=na)
    torch.cuda.synchronize()
    assert na.cpu().numpy().tolist() == lens_ref.tolist()
    for layer in range(layers):
        assert np.array_equal(_bits(kd[layer]), k_ref[layer])
        assert np.array_equal(_bits(vd[layer]), v_ref[layer])


def test_read_probe_xor_of_the_buffer():
    """The streaming-read probe reads every byte: its result is the XOR of all 32-bit words (checked on a
    ragged size that leaves a tail for the non-unrolled loop)."""
    import long_context_tree_amd as lt
    rng = np.random.default_rng(7)
    for n_words in (4, 4 * 1000003, 4 * (1 << 22)):
        host = rng.integers(0, 1 << 32, size=n_words, dtype=np.uint64).astype(np.uint32)
        dev_buf = torch.from_numpy(host.view(np.int32)).to(dev())
        sink = lt.read_probe(dev_buf)
        torch.cuda.synchronize()
        assert int(sink[0].item()) & 0xFFFFFFFF == int(np.bitwise_xor.reduce(host)), n_words
