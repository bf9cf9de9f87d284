"""GPU parity of spec_draft_gather with the oracle.

Checked bit-exactly: positions, lengths, V rows, and K rows without rotation.
Rotated K rows are bf16 values of magnitude up to ~5, where one bf16 ulp (up to 2^-5) is above the
absolute 1e-2 used for attention outputs.  So each element is held to one bf16 ulp of the exact
(fp64) rotation plus the fp32 rotation error, 4e-7 (|x| + |y|) for the pair (x, y).  At most 0.1% of
the elements may round to the other neighbour than the exact value does.
Also covered:
  - both rotation forms, both V layouts, head dims 64 and 128, several page and chunk sizes;
  - ragged and empty contexts, windows longer than the context, repeated / padded / out-of-range
    chunk ids, a chunk cut by the window, a partial last chunk;
  - slots past the length left untouched, an invalid page read as zeros;
  - the benchmark shape (128K context, 24 chunks + a 512-token window in a 2048-slot budget);
  - the chain attention -> chunk salience top-k -> gather, against the oracle's own chain."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import dev, oracle_attention, run_attention
from oracle import draft_kv as odk
from synth import device as sdev

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1          # a NaN pattern the kernel never writes


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _pair_mag(k_pre, style):
    """|x| + |y| of each element's rotation pair (pre-RoPE values, [..][D])."""
    D = k_pre.shape[-1]
    if style == 1:
        return np.abs(k_pre) + np.abs(np.roll(k_pre, D // 2, axis=-1))
    idx = np.arange(D) ^ 1
    return np.abs(k_pre) + np.abs(k_pre[..., idx])


def _compare(got, ref, ref_pre_k, style):
    ok_, ov_, op_, ol_ = got
    rk, rv, rp, rl = ref
    ol = ol_.cpu().numpy()
    op = op_.cpu().numpy()
    np.testing.assert_array_equal(ol, rl)
    np.testing.assert_array_equal(op, rp)
    kb, vb = _bits(ok_), _bits(ov_)
    n_round = 0
    for b in range(len(rl)):
        n = int(rl[b])
        if n == 0:
            continue
        v_got = oracle.bf16_to_f64(vb[b, :n])
        np.testing.assert_array_equal(v_got, rv[b, :n])
        k_got = oracle.bf16_to_f64(kb[b, :n])
        if style == 0:
            np.testing.assert_array_equal(k_got, rk[b, :n])
            continue
        ref_k = rk[b, :n]
        ulp = np.spacing(np.abs(ref_k).astype(np.float32)).astype(np.float64) * 65536.0
        bound = ulp + 4e-7 * _pair_mag(ref_pre_k[b, :n], style)
        err = np.abs(k_got - ref_k)
        assert (err <= bound).all(), (b, float(err.max()), float((err - bound).max()))
        flips = int((synth.bf16_to_f32(synth.bf16_bits(ref_k.astype(np.float32))) != k_got).sum())
        # the fp32 rotation error is ~2^-14 of a bf16 ulp, so few elements may round the other way
        assert flips <= max(2, 1e-3 * ref_k.size), (b, flips, ref_k.size)
        n_round += flips
    return n_round


def _run_case(seed, ctx, H, D, ps, cs, W, num_select, style, v_layout, *, cap_extra=0, max_ctx=None,
              pad=0.2, dup=0.2, bad=0.1, theta=500000.0):
    import long_context_tree_amd as lt
    ctx = np.asarray(ctx, dtype=np.int32)
    mc = int(ctx.max(initial=0)) if max_ctx is None else max_ctx
    kv = synth.paged_kv(seed, 0, ctx, H, D, page_size=ps, max_blocks=max(1, -(-mc // ps)))
    nch = -(-ctx // cs)
    ids = synth.chunk_selection(seed, nch, num_select, pad_frac=pad, dup_frac=dup, bad_frac=bad)
    inv = synth.rope_inv_freq(D, theta)
    cap = num_select * cs + W + cap_extra
    vpool = synth.dim_major(kv.v_pool) if v_layout else kv.v_pool
    k_t, v_t = sdev.bf16_tensor(kv.k_pool, dev()), sdev.bf16_tensor(vpool, dev())
    bt_t = torch.from_numpy(kv.block_table).to(dev())
    lens_t = torch.from_numpy(ctx).to(dev())
    ids_t = torch.from_numpy(ids).to(dev()) if num_select else None
    inv_t = torch.from_numpy(inv).to(dev())
    B = len(ctx)
    out_k = torch.full((B, cap, H, D), 0, dtype=torch.int16, device=dev())
    out_k.fill_(SENTINEL)
    out_v = out_k.clone()
    got = lt.draft_gather(k_t, v_t, bt_t, lens_t, ids_t, max_ctx_len=mc, chunk_size=cs, window=W, capacity=cap,
                          rope=style, inv_freq=inv_t if style else None, out_k=out_k.view(torch.bfloat16),
                          out_v=out_v.view(torch.bfloat16), v_layout=v_layout)
    torch.cuda.synchronize()
    ids_np = ids if num_select else np.zeros((B, 0), dtype=np.int32)
    ref = odk.draft_gather(kv.k_pool, vpool, kv.block_table, ctx, ids_np, ps, cs, W, cap, inv, style, v_layout)
    pre = odk.draft_gather(kv.k_pool, vpool, kv.block_table, ctx, ids_np, ps, cs, W, cap, inv, 0, v_layout)[0]
    n_round = _compare(got, ref, pre, style)
    # slots past each length were not written
    kb, vb = _bits(got[0]), _bits(got[1])
    for b in range(B):
        n = int(ref[3][b])
        assert (kb[b, n:] == SENTINEL).all() and (vb[b, n:] == SENTINEL).all()
    return got, ref, n_round


@pytest.mark.parametrize("v_layout", [0, 1])
@pytest.mark.parametrize("style", [0, 1, 2])
@pytest.mark.parametrize("H,D,ps,cs", [(2, 64, 16, 32), (8, 128, 16, 64), (4, 128, 8, 48)])
def test_gather_matches_oracle(H, D, ps, cs, style, v_layout):
    seed = 300 + H + D + ps + cs + 10 * style + v_layout
    ctx = [1000, 0, 77, 2 * cs, 531]
    _, ref, n_round = _run_case(seed, ctx, H, D, ps, cs, 100, 6, style, v_layout, cap_extra=13)
    assert ref[3].max() > 0
    print(f"rounded differently: {n_round} elements")


def test_gather_edge_cases():
    # window longer than every context, chunk size 1, no selection at all
    _run_case(321, [5, 64, 300], 2, 64, 16, 1, 1000, 0, 1, 0, cap_extra=3)
    _run_case(322, [5, 64, 300, 1], 2, 64, 16, 1, 7, 20, 2, 0, pad=0.0, dup=0.3, bad=0.2)
    # a selection that covers the whole context, no window
    _run_case(323, [640, 600], 2, 128, 16, 64, 0, 10, 1, 1, pad=0.0, dup=0.0, bad=0.0)
    # every id invalid or padding
    _run_case(324, [900], 8, 128, 16, 64, 50, 8, 1, 0, pad=0.5, dup=0.0, bad=0.5)
    # max_ctx_len above every length (a larger bitmap than needed)
    _run_case(325, [300, 1000], 2, 64, 16, 16, 33, 12, 1, 0, max_ctx=50000)


def test_gather_reads_only_num_select_columns_and_zeroes_invalid_pages():
    import long_context_tree_amd as lt
    H, D, ps, cs, W = 2, 64, 16, 32, 20
    ctx = np.array([700], dtype=np.int32)
    kv = synth.paged_kv(330, 0, ctx, H, D, page_size=ps)
    ids = np.array([[3, 9, 0, 15, 20, 2, 4, 6]], dtype=np.int32)     # only the first 4 are read
    inv = synth.rope_inv_freq(D)
    bt = kv.block_table.copy()
    bt[0, 2] = kv.k_pool.shape[0] + 3                                 # page 2 (tokens 32..47, chunk 1) invalid
    bt[0, 18] = -5                                                    # page 18 (tokens 288..303, chunk 9) invalid
    got = lt.draft_gather(sdev.bf16_tensor(kv.k_pool, dev()), sdev.bf16_tensor(kv.v_pool, dev()),
                          torch.from_numpy(bt).to(dev()), torch.from_numpy(ctx).to(dev()),
                          torch.from_numpy(ids).to(dev()), max_ctx_len=700, chunk_size=cs, window=W,
                          capacity=4 * cs + W, num_select=4, rope=1, inv_freq=torch.from_numpy(inv).to(dev()))
    torch.cuda.synchronize()
    ref = odk.draft_gather(kv.k_pool, kv.v_pool, kv.block_table, ctx, ids[:, :4], ps, cs, W, 4 * cs + W, inv, 1)
    pos = ref[2][0, :ref[3][0]]
    bad = (pos // ps == 18)
    assert bad.any()
    kb, vb = _bits(got[0])[0], _bits(got[1])[0]
    # zero rows (a zero K row rotates to signed zeros)
    assert (oracle.bf16_to_f64(kb[:len(pos)][bad]) == 0).all() and (vb[:len(pos)][bad] == 0).all()
    rk, rv = ref[0].copy(), ref[1].copy()
    rk[0, :len(pos)][bad] = 0.0
    rv[0, :len(pos)][bad] = 0.0
    pre = odk.draft_gather(kv.k_pool, kv.v_pool, kv.block_table, ctx, ids[:, :4], ps, cs, W, 4 * cs + W, inv, 0)[0]
    _compare(got, (rk, rv, ref[2], ref[3]), pre, 1)


def test_gather_at_benchmark_shape():
    """128K context, 8 KV heads x 128, chunk 64, the 24 heaviest of a 256-entry top-k list plus a 512-token
    window in a 2048-slot budget; the same call twice gives the same bytes."""
    import long_context_tree_amd as lt
    L, H, D, cs, W, sel, cap = 131072, 8, 128, 64, 512, 24, 2048
    k, v, bt = sdev.paged_kv_device(340, 0, [L], H, D, dev())
    ids = synth.chunk_selection(340, [L // cs], 256)
    inv = synth.rope_inv_freq(D)
    args = dict(max_ctx_len=L, chunk_size=cs, window=W, capacity=cap, num_select=sel, rope=1,
                inv_freq=torch.from_numpy(inv).to(dev()))
    lens = torch.tensor([L], dtype=torch.int32, device=dev())
    ids_t = torch.from_numpy(ids).to(dev())
    got = lt.draft_gather(k, v, bt, lens, ids_t, **args)
    again = lt.draft_gather(k, v, bt, lens, ids_t, **args)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(got[0]), _bits(again[0])) and np.array_equal(_bits(got[1]), _bits(again[1]))
    kp, vp, btn = _bits(k), _bits(v), bt.cpu().numpy()
    ref = odk.draft_gather(kp, vp, btn, [L], ids[:, :sel], 16, cs, W, cap, inv, 1)
    pre = odk.draft_gather(kp, vp, btn, [L], ids[:, :sel], 16, cs, W, cap, inv, 0)[0]
    n_round = _compare(got, ref, pre, 1)
    win_chunks = {c for c in ids[0, :sel] if c * cs >= L - W}
    assert ref[3][0] == (sel - len(win_chunks)) * cs + W
    print(f"len {ref[3][0]}, rounded differently: {n_round} of {ref[3][0] * H * D}")


def test_chain_salience_topk_then_gather():
    """Attention with chunk partials, chunk salience with top-32 on a needle workload, then the gather of the
    selected chunks; the oracle runs the same chain on the same inputs."""
    import long_context_tree_amd as lt
    r = synth.rng_for(350, 0, 0)
    L, cs, W, k = 8192, 64, 256, 32
    case = synth.attention_case(350, ctx_lens=[L], trees=[synth.random_tree(r, 16, 4)], num_q_heads=32,
                                num_kv_heads=8, head_dim=128, needle={"count": 32, "chunk": cs, "score": 6.0})
    out, lse, h, t = run_attention(case, chunk_size=cs)
    mass = torch.zeros((1, L // cs), dtype=torch.float32, device=dev())
    _, ti, _ = lt.chunk_salience(h, mass, top_k=k)
    draft = synth.paged_kv(350, 7, [L], 8, 128)                       # the draft layer's canonical cache
    inv = synth.rope_inv_freq(128)
    got = lt.draft_gather(sdev.bf16_tensor(draft.k_pool, dev()), sdev.bf16_tensor(draft.v_pool, dev()),
                          torch.from_numpy(draft.block_table).to(dev()), t["ctx_lens"], ti, max_ctx_len=L,
                          chunk_size=cs, window=W, capacity=k * cs + W, rope=1,
                          inv_freq=torch.from_numpy(inv).to(dev()))
    torch.cuda.synchronize()
    m_ref = oracle_attention(case, cs)[2]
    ids_ref = np.array([oracle.topk_chunks(m_ref[0], k)[0]], dtype=np.int32)
    assert sorted(ti.cpu().numpy()[0].tolist()) == sorted(ids_ref[0].tolist())
    ref = odk.draft_gather(draft.k_pool, draft.v_pool, draft.block_table, [L], ids_ref, 16, cs, W, k * cs + W, inv, 1)
    pre = odk.draft_gather(draft.k_pool, draft.v_pool, draft.block_table, [L], ids_ref, 16, cs, W, k * cs + W,
                           inv, 0)[0]
    _compare(got, ref, pre, 1)
