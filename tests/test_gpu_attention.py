"""GPU parity of spec_tree_attention and spec_chunk_salience against the oracle (same seeded inputs),
plus determinism and block-table invariance.  Tolerances: out max-abs 1e-2, mean-abs 1e-3, relative L2
1e-2, lse max-abs 1e-3; chunk mass the same absolute bounds plus sum|d| / sum(mass) <= 1e-3."""

import numpy as np
import pytest
import torch

import synth
from gpu_util import (bits_of, compare_mass, compare_out, dev, oracle_attention, run_attention, topk_valid)

pytestmark = pytest.mark.gpu


def _case(name):
    r = synth.rng_for(100, 0, 0)
    if name == "tiny":         # 1 layer, 512 context, 4 q / 2 kv heads, D=64, 8-node tree depth <= 4
        return synth.attention_case(101, ctx_lens=[512], trees=[synth.random_tree(r, 8, 4)], num_q_heads=4,
                                    num_kv_heads=2, head_dim=64)
    if name == "llama64":      # Llama-3.1-8B layer shape, 64-node tree depth 8, ragged context
        return synth.attention_case(102, ctx_lens=[2000], trees=[synth.random_tree(r, 64, 8)], num_q_heads=32,
                                    num_kv_heads=8, head_dim=128)
    if name == "llama128":     # 128-node tree depth 10: two row groups per KV head
        return synth.attention_case(103, ctx_lens=[1500], trees=[synth.random_tree(r, 128, 10)], num_q_heads=32,
                                    num_kv_heads=8, head_dim=128)
    if name == "ragged":       # Qwen3-8B shape, ragged batch of chains (k=4 drafts) and a lone root
        return synth.attention_case(104, ctx_lens=[0, 1, 100, 777, 3000, 64],
                                    trees=[synth.chain_tree(5)] * 5 + [synth.chain_tree(1)], num_q_heads=32,
                                    num_kv_heads=8, head_dim=128)
    if name == "gqa1_d64":     # no GQA sharing, D=64, bushy tree, several sequences
        return synth.attention_case(105, ctx_lens=[300, 1000], trees=[synth.random_tree(r, 30, 3),
                                                                      synth.random_tree(r, 17, 6)],
                                    num_q_heads=6, num_kv_heads=6, head_dim=64)
    raise KeyError(name)


@pytest.mark.parametrize("v_layout", [0, 1])
@pytest.mark.parametrize("name,chunk,split", [("tiny", 64, 0), ("tiny", 16, 1), ("llama64", 64, 0),
                                              ("llama64", 32, 3), ("llama64", 128, 4), ("llama128", 64, 0),
                                              ("llama128", 64, 2), ("ragged", 32, 0), ("ragged", 64, 1),
                                              ("gqa1_d64", 64, 0), ("gqa1_d64", 16, 5)])
def test_attention_and_mass_match_oracle(name, chunk, split, v_layout):
    case = _case(name)
    print(f"case={name} chunk={chunk} split={split} v_layout={v_layout}", flush=True)
    out, lse, h, t = run_attention(case, chunk_size=chunk, split_tiles=split, v_layout=v_layout)
    import long_context_tree_amd as lt
    n_ch = max(1, -(-int(case.ctx_lens.max()) // chunk))
    mass = torch.full((len(case.ctx_lens), n_ch), 7.0, dtype=torch.float32, device=dev())
    lt.chunk_salience(h, mass)
    torch.cuda.synchronize()
    o_ref, l_ref, m_ref = oracle_attention(case, chunk)
    compare_out(out, lse, o_ref, l_ref)
    mg = mass.cpu().numpy().astype(np.float64)
    for b, mr in enumerate(m_ref):
        compare_mass(mg[b, :len(mr)], mr)
        assert (mg[b, len(mr):] == 0).all()


def test_mass_accumulates_over_layers_and_topk():
    """Three layers summed with accumulate=1, then top-k by (mass desc, index asc)."""
    import long_context_tree_amd as lt
    r = synth.rng_for(110, 0, 0)
    tree = synth.random_tree(r, 16, 4)
    L, chunk, k = 3000, 64, 20
    total = np.zeros(-(-L // chunk))
    mass = torch.zeros((1, len(total)), dtype=torch.float32, device=dev())
    for layer in range(3):
        case = synth.attention_case(110, layer=layer, ctx_lens=[L], trees=[tree], num_q_heads=8, num_kv_heads=2,
                                    head_dim=128)
        out, lse, h, _ = run_attention(case, chunk_size=chunk)
        _, ti, tm = lt.chunk_salience(h, mass, accumulate=layer > 0, top_k=k if layer == 2 else 0)
        total += oracle_attention(case, chunk)[2][0]
    torch.cuda.synchronize()
    compare_mass(mass.cpu().numpy()[0].astype(np.float64), total)
    idx = ti.cpu().numpy()[0]
    topk_valid(idx, total, k)
    got = mass.cpu().numpy()[0]
    # the top-k values are the GPU's own masses at those indices, in (desc, asc) order
    np.testing.assert_array_equal(tm.cpu().numpy()[0], got[idx])
    order = sorted(range(len(got)), key=lambda c: (-got[c], c))[:k]
    assert idx.tolist() == order


def test_needle_chunks_selected():
    """Planted keys make 32 chunks salient: top-32 must be exactly those chunks."""
    import long_context_tree_amd as lt
    r = synth.rng_for(111, 0, 0)
    case = synth.attention_case(111, ctx_lens=[8192], trees=[synth.random_tree(r, 16, 4)], num_q_heads=32,
                                num_kv_heads=8, head_dim=128, needle={"count": 32, "chunk": 64, "score": 6.0})
    out, lse, h, _ = run_attention(case, chunk_size=64)
    mass = torch.zeros((1, 128), dtype=torch.float32, device=dev())
    _, ti, _ = lt.chunk_salience(h, mass, top_k=32)
    torch.cuda.synchronize()
    o_ref, l_ref, m_ref = oracle_attention(case, 64)
    compare_out(out, lse, o_ref, l_ref)
    compare_mass(mass.cpu().numpy()[0].astype(np.float64), m_ref[0])
    assert sorted(ti.cpu().numpy()[0].tolist()) == sorted(case.needle_chunks[0].tolist())
    topk_valid(ti.cpu().numpy()[0], m_ref[0], 32)


def test_deterministic_and_block_table_invariant():
    r = synth.rng_for(112, 0, 0)
    trees = [synth.random_tree(r, 64, 8)]
    a = synth.attention_case(112, ctx_lens=[5000], trees=trees, num_q_heads=32, num_kv_heads=8, head_dim=128)
    b = synth.attention_case(112, ctx_lens=[5000], trees=trees, num_q_heads=32, num_kv_heads=8, head_dim=128,
                             perm_stream=60)
    import long_context_tree_amd as lt
    res = []
    for case in (a, a, b):
        out, lse, h, _ = run_attention(case, chunk_size=64)
        mass = torch.zeros((1, 79), dtype=torch.float32, device=dev())
        lt.chunk_salience(h, mass)
        torch.cuda.synchronize()
        res.append((bits_of(out), lse.cpu().numpy(), mass.cpu().numpy()))
    for x, y in zip(res[0], res[1]):
        assert np.array_equal(x, y)
    for x, y in zip(res[0], res[2]):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_v_layouts_agree(chunk):
    """Token-row and dim-major V give the same scores for every key (page sizes below, equal to and above
    a 64-slot tile).  Both layouts are checked against the oracle.  Where both run the same kernel (16- and
    32-slot chunks), only the order in which the keys of a tile are contracted differs, so outputs, LSEs and
    masses must also agree with each other to fp32 rounding.  With 64-slot chunks the wide tree's token-row
    V runs the software-pipelined kernel, which rounds P per half-tile, so there the oracle decides."""
    import long_context_tree_amd as lt
    r = synth.rng_for(113, chunk, 0)
    for ps in (8, 16, 64, 128):
        case = synth.attention_case(113, ctx_lens=[1000, 333], trees=[synth.random_tree(r, 40, 6),
                                                                       synth.chain_tree(5)],
                                    num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=ps)
        o_ref, l_ref, m_ref = oracle_attention(case, chunk)
        res = []
        for vl in (0, 1):
            print(f"chunk={chunk} page_size={ps} v_layout={vl}", flush=True)
            out, lse, h, _ = run_attention(case, chunk_size=chunk, split_tiles=4, v_layout=vl)
            mass = torch.zeros((2, -(-1000 // chunk)), dtype=torch.float32, device=dev())
            lt.chunk_salience(h, mass)
            torch.cuda.synchronize()
            compare_out(out, lse, o_ref, l_ref)
            mg = mass.cpu().numpy().astype(np.float64)
            for b, mr in enumerate(m_ref):
                compare_mass(mg[b, :len(mr)], mr)
            res.append((out.float().cpu().numpy(), lse.cpu().numpy(), mass.cpu().numpy()))
        if chunk == 64:
            continue
        (o0, l0, m0), (o1, l1, m1) = res
        assert np.abs(o0 - o1).max() <= 1e-3            # a bf16 rounding flip of |out| < 0.25 at most
        assert np.abs(l0 - l1).max() <= 1e-5
        assert np.abs(m0 - m1).sum() <= 1e-5 * m0.sum()


def test_split_count_invariance_within_tolerance():
    case = _case("llama64")
    outs = [run_attention(case, split_tiles=s)[:2] for s in (1, 5, 33)]
    torch.cuda.synchronize()
    base = outs[0][0].float()
    for o, l in outs[1:]:
        assert (o.float() - base).abs().max().item() <= 2e-3
        assert (l - outs[0][1]).abs().max().item() <= 1e-4


def test_full_size_llama_32k_sampled_heads():
    """The Llama-3.1-8B-shaped layer at 32K context (64-node tree depth 8, chunk 64), in the launch
    configuration the benchmark uses; the oracle checks two KV heads' rows and every chunk mass."""
    import long_context_tree_amd as lt
    from synth import device as sdev
    import oracle
    L, N = 32768, 64
    tree = synth.random_tree(synth.rng_for(120, 0, 4), N, 8)
    k, v, bt = sdev.paged_kv_device(120, 0, [L + N], 8, 128, dev())
    q = sdev.queries_device(120, 0, N, 32, 128, dev())
    cl = torch.tensor([L], dtype=torch.int32, device=dev())
    no = torch.tensor([0, N], dtype=torch.int32, device=dev())
    par = torch.from_numpy(tree).to(dev())
    out, lse, h = lt.tree_attention(q, k, v, bt, cl, no, par, max_nodes=N, max_ctx_len=L, chunk_size=64)
    mass = torch.zeros((1, L // 64), dtype=torch.float32, device=dev())
    lt.chunk_salience(h, mass)
    torch.cuda.synchronize()
    kp, vp, qb = bits_of(k), bits_of(v), bits_of(q)
    btn = bt.cpu().numpy()
    o_ref, l_ref, m_ref = oracle.tree_attention(qb, kp, vp, btn, np.array([L]), np.array([0, N]), tree,
                                                1 / np.sqrt(128), 8, 16, 64)
    compare_out(out, lse, o_ref, l_ref)
    compare_mass(mass.cpu().numpy()[0].astype(np.float64), m_ref[0])
    s = mass.sum().item()
    assert 0.0 < s <= 1.0


@pytest.mark.parametrize("v_layout", [0, 1])
@pytest.mark.parametrize("page_size", [8, 32, 64, 128, 256])
def test_page_sizes(page_size, v_layout):
    """Pages smaller than, equal to and larger than a 64-slot tile (the last spans several tiles)."""
    r = synth.rng_for(130, page_size, 0)
    case = synth.attention_case(130 + page_size, ctx_lens=[700, 1300], trees=[synth.random_tree(r, 20, 5),
                                                                              synth.chain_tree(4)],
                                num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=page_size)
    print(f"page_size={page_size} v_layout={v_layout}", flush=True)
    out, lse, h, _ = run_attention(case, chunk_size=64, split_tiles=3, v_layout=v_layout)
    import long_context_tree_amd as lt
    mass = torch.zeros((2, 21), dtype=torch.float32, device=dev())
    lt.chunk_salience(h, mass)
    torch.cuda.synchronize()
    o_ref, l_ref, m_ref = oracle_attention(case, 64)
    compare_out(out, lse, o_ref, l_ref)
    for b, mr in enumerate(m_ref):
        compare_mass(mass.cpu().numpy()[b, :len(mr)].astype(np.float64), mr)


def test_batch_invariance():
    """Ragged batch of chains (the Qwen3-8B shape, 4 drafts): each sequence's outputs and LSE are the same
    bytes whether it runs alone or inside the batch (with the split size fixed, the plan is the same)."""
    ctx = [4096, 9001, 6000, 12345]
    trees = [synth.chain_tree(5) for _ in ctx]
    case = synth.attention_case(140, ctx_lens=ctx, trees=trees, num_q_heads=32, num_kv_heads=8, head_dim=128)
    out, lse, _, _ = run_attention(case, chunk_size=64, split_tiles=16, max_ctx=12345)
    for b in range(len(ctx)):
        one = synth.attention_case(140, ctx_lens=ctx, trees=trees, num_q_heads=32, num_kv_heads=8, head_dim=128)
        sel = slice(int(one.node_offsets[b]), int(one.node_offsets[b + 1]))
        one.ctx_lens = one.ctx_lens[b:b + 1].copy()
        one.q = one.q[sel].copy()
        one.parents = one.parents[sel].copy()
        one.node_offsets = np.array([0, 5], dtype=np.int32)
        one.kv.block_table = one.kv.block_table[b:b + 1].copy()
        o1, l1, _, _ = run_attention(one, chunk_size=64, split_tiles=16, max_ctx=12345, max_nodes=5)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), out[sel].view(torch.int16)), b
        assert torch.equal(l1, lse[sel]), b


def test_chain_equals_causal_decode():
    """A chain of drafts is ordinary causal decode: node i's output equals a one-token decode of its query
    over the L + i committed slots plus its own (the same cache, the same physical pages)."""
    L, n = 3000, 6
    case = synth.attention_case(141, ctx_lens=[L], trees=[synth.chain_tree(n)], num_q_heads=32, num_kv_heads=8,
                                head_dim=128)
    out, lse, _, _ = run_attention(case)
    for i in range(n):
        dec = synth.attention_case(141, ctx_lens=[L], trees=[synth.chain_tree(n)], num_q_heads=32, num_kv_heads=8,
                                   head_dim=128)
        dec.ctx_lens = np.array([L + i], dtype=np.int32)
        dec.q = dec.q[i:i + 1].copy()
        dec.parents = np.array([-1], dtype=np.int32)
        dec.node_offsets = np.array([0, 1], dtype=np.int32)
        o1, l1, _, _ = run_attention(dec, max_ctx=L + n, max_nodes=1)
        torch.cuda.synchronize()
        d = (o1.float() - out[i:i + 1].float()).abs().max().item()
        assert d <= 2 ** -8 * max(out[i].float().abs().max().item(), 1e-3) + 1e-3, (i, d)
        assert (l1 - lse[i:i + 1]).abs().max().item() <= 1e-4


@pytest.mark.parametrize("v_layout", [0, 1])
@pytest.mark.parametrize("chunk,split,nodes", [(64, 4, 16), (128, 4, 16), (32, 3, 16), (16, 5, 16), (64, 4, 40),
                                               (128, 5, 40), (0, 7, 40)])
def test_rising_scores_rescale_mid_split(chunk, split, nodes, v_layout):
    """Keys whose magnitude grows along the context make later tiles' score maxima jump past the running
    max by far more than the lazy-rescale headroom, several times inside each split: the exps are redone
    against a moved max, and O, the row sums and the chunk accumulators are rescaled mid-split (with
    128-slot chunks, between the two tiles of one chunk).  40 nodes give 160 rows per KV head, the
    8-wave work-groups (with token-row V, the software-pipelined kernel, whose half-tiles rescale on
    their own)."""
    r = synth.rng_for(106, 0, 0)
    case = synth.attention_case(106, ctx_lens=[1000], trees=[synth.random_tree(r, nodes, 4)], num_q_heads=8,
                                num_kv_heads=2, head_dim=128)
    kv = case.kv
    k = synth.bf16_to_f32(kv.k_pool).astype(np.float64)
    for tkn in range(int(kv.slots[0])):
        pg, slot = kv.block_table[0, tkn // kv.page_size], tkn % kv.page_size
        k[pg, :, slot, :] *= 1.0 + 0.02 * tkn             # many rows see their tile max jump by > 8 (log2) inside a split
    kv.k_pool[...] = synth.bf16_bits(k.astype(np.float32))
    # the softmax is now nearly one-hot, so the outputs are V-sized; V / 8 (exact in bf16) keeps them in the
    # range the output tolerance is set for, and leaves the scores (the rescale path) unchanged
    kv.v_pool[...] = synth.bf16_bits((synth.bf16_to_f32(kv.v_pool) * 0.125).astype(np.float32))
    print(f"case=rising chunk={chunk} split={split} nodes={nodes} v_layout={v_layout}", flush=True)
    out, lse, h, t = run_attention(case, chunk_size=chunk, split_tiles=split, v_layout=v_layout)
    import long_context_tree_amd as lt
    o_ref, l_ref, m_ref = oracle_attention(case, chunk)
    if chunk:
        n_ch = -(-int(case.ctx_lens.max()) // chunk)
        mass = torch.full((1, n_ch), 7.0, dtype=torch.float32, device=dev())
        lt.chunk_salience(h, mass)
    torch.cuda.synchronize()
    compare_out(out, lse, o_ref, l_ref)
    if chunk:
        compare_mass(mass.cpu().numpy().astype(np.float64)[0, :len(m_ref[0])], m_ref[0])


@pytest.mark.parametrize("case_name,split", [("n32_g4", 64), ("chain_g3", 160), ("ragged_g2", 150), ("n32_g4", 0)])
def test_chunk_ring_write_outs(case_name, split):
    """Narrow trees (4-wave work-groups, token-row V, 64-slot chunks) collect a split's chunk values in an
    LDS ring of 2048 values, [chunk end][row], and write it out whenever it fills: splits longer than
    2048 / rows chunk ends.  n32_g4: 128 rows per KV head, 16 chunk ends per write-out, several inside each
    64-tile split (16-byte stores).  chain_g3: G = 3, 15 rows (4-byte stores: rows not a multiple of 4),
    136 chunk ends per write-out.  ragged_g2: max_nodes 8 with a 5-node tree, 16 rows per chunk end in the
    layout but 10 of the sequence's own (4-byte stores, rows past the sequence's not written)."""
    r = synth.rng_for(107, 0, 0)
    if case_name == "n32_g4":
        case = synth.attention_case(107, ctx_lens=[6000], trees=[synth.random_tree(r, 32, 6)], num_q_heads=32,
                                    num_kv_heads=8, head_dim=128)
    elif case_name == "chain_g3":
        case = synth.attention_case(108, ctx_lens=[12000], trees=[synth.chain_tree(5)], num_q_heads=6,
                                    num_kv_heads=2, head_dim=64)
    else:
        case = synth.attention_case(109, ctx_lens=[9000, 7000], trees=[synth.random_tree(r, 8, 3),
                                                                       synth.random_tree(r, 5, 3)],
                                    num_q_heads=4, num_kv_heads=2, head_dim=128)
    print(f"case=ring {case_name} split={split}", flush=True)
    out, lse, h, t = run_attention(case, chunk_size=64, split_tiles=split)
    import long_context_tree_amd as lt
    n_ch = -(-int(case.ctx_lens.max()) // 64)
    mass = torch.full((len(case.ctx_lens), n_ch), 7.0, dtype=torch.float32, device=dev())
    lt.chunk_salience(h, mass)
    torch.cuda.synchronize()
    o_ref, l_ref, m_ref = oracle_attention(case, 64)
    compare_out(out, lse, o_ref, l_ref)
    mg = mass.cpu().numpy().astype(np.float64)
    for b, mr in enumerate(m_ref):
        compare_mass(mg[b, :len(mr)], mr)
        assert (mg[b, len(mr):] == 0).all()


@pytest.mark.parametrize("ctx,k,kind,width", [
    (32768, 256, "ties", 0), (32768, 1, "ties", 0), (32768, 256, "equal", 0), (1600, 256, "ties", 0),
    (32768, 256, "zeros", 0), (32768, 200, "distinct", 0),
    # more than 2048 chunks (the sort through LDS, strides of 64 and more cross waves)
    (65536, 256, "ties", 0), (131072, 256, "ties", 0), (131072, 300, "distinct", 0), (131072, 256, "equal", 0),
    (98304, 1000, "ties", 0),
    # a mass row wider than 2048 while the sequence has fewer chunks
    (20000, 256, "ties", 3000), (40000, 64, "distinct", 8192)])
def test_topk_order_ties_and_padding(ctx, k, kind, width):
    """Exact top-k: (mass desc, index asc) with planted ties, equal and zero masses, and -1 / 0 padding
    when there are fewer chunks than k, up to 8192 chunks, and mass rows wider than the sequence's
    chunks.  The masses are planted as large fp32 values in the accumulator, so one layer's attention
    mass (~1e-4 per chunk) leaves them unchanged when it is accumulated."""
    import long_context_tree_amd as lt
    import oracle
    r = synth.rng_for(107, 0, 0)
    case = synth.attention_case(107, ctx_lens=[ctx], trees=[synth.random_tree(r, 4, 2)], num_q_heads=4,
                                num_kv_heads=1, head_dim=64)
    chunk = 16
    n_ch = -(-ctx // chunk)
    rng = np.random.default_rng(ctx + k)
    base = np.float32(1 << 27)                      # fp32 spacing 16 here: the added mass rounds away
    if kind == "ties":
        planted = base + 16 * rng.integers(0, 64, n_ch)
    elif kind == "equal":
        planted = np.full(n_ch, base)
    elif kind == "zeros":
        planted = np.where(rng.random(n_ch) < 0.95, 0.0, base + 16 * rng.integers(0, 8, n_ch))
    else:
        planted = base + 16 * rng.permutation(n_ch)
    planted = planted.astype(np.float32)
    print(f"topk ctx={ctx} k={k} kind={kind} width={width}", flush=True)
    out, lse, h, t = run_attention(case, chunk_size=chunk)
    width = max(n_ch, k, width)                     # the row may be wider than the sequence's chunks (top_k <= width)
    row = np.zeros(width, dtype=np.float32)
    row[:n_ch] = planted
    mass = torch.from_numpy(row[None, :].copy()).to(dev())
    before = mass.clone()
    _, ti, tm = lt.chunk_salience(h, mass, accumulate=True, top_k=k)
    torch.cuda.synchronize()
    m = mass.cpu().numpy()[0, :n_ch].astype(np.float64)
    if kind != "zeros":
        assert np.array_equal(m, before.cpu().numpy()[0, :n_ch].astype(np.float64)), "the planted masses moved"
    idx_ref, val_ref = oracle.topk_chunks(m, k)
    assert np.array_equal(ti.cpu().numpy()[0].astype(np.int64), idx_ref)
    assert np.array_equal(tm.cpu().numpy()[0].astype(np.float64), val_ref.astype(np.float32).astype(np.float64))
