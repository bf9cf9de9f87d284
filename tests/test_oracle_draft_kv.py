"""Pins for the compact-draft-KV oracle.  The selection is checked against a mask painted over the
context and against closed-form counts.  The rotation is checked against the rotary helpers of the
transformers library (Llama's rotate-half form, GPT-J's adjacent-pair form) and against the
relative-position property that justifies local positions.  The gather through the block table is
checked against logical arrays built by the test itself."""

import numpy as np
import pytest

import oracle
import synth
from oracle import draft_kv as odk


def _mask_positions(L, ids, cs, W):
    m = np.zeros(L, dtype=bool)
    m[max(0, L - W):] = True
    for c in ids:
        if 0 <= c < -(-L // cs):
            m[c * cs:(c + 1) * cs] = True
    return np.flatnonzero(m)


@pytest.mark.parametrize("seed", range(6))
def test_selection_equals_painted_mask(seed):
    rng = np.random.default_rng(seed)
    for _ in range(40):
        cs = int(rng.choice([16, 32, 64, 48]))
        L = int(rng.integers(0, 700))
        W = int(rng.integers(0, 300))
        ids = rng.integers(-2, L // cs + 3, size=int(rng.integers(0, 12)))
        got = odk.selected_positions(L, ids, cs, W)
        assert np.array_equal(got, _mask_positions(L, ids, cs, W))


def test_selection_closed_forms():
    cs, W, L = 64, 100, 1000                     # window [900, 1000); chunk 14 = [896, 960) straddles it
    assert len(odk.selected_positions(L, [0, 3, 7], cs, W)) == 3 * cs + W
    assert len(odk.selected_positions(L, [0, 3, 7, 3, 3, -1, 99], cs, W)) == 3 * cs + W
    assert len(odk.selected_positions(L, [14], cs, W)) == (900 - 896) + W
    assert len(odk.selected_positions(L, [15], cs, W)) == W      # inside the window
    assert np.array_equal(odk.selected_positions(L, [], cs, W), np.arange(900, 1000))
    assert np.array_equal(odk.selected_positions(L, range(16), cs, 0), np.arange(L))
    assert np.array_equal(odk.selected_positions(50, [], cs, 100), np.arange(50))
    assert len(odk.selected_positions(0, [0, 1], cs, 10)) == 0
    last = odk.selected_positions(L, [15], cs, 0)              # partial last chunk [960, 1000)
    assert np.array_equal(last, np.arange(960, 1000))


def _hf_rope(x, pos, inv_freq, style):
    import torch
    xt = torch.from_numpy(x)                                    # [n][H][D]
    freqs = torch.from_numpy(np.outer(pos.astype(np.float64), inv_freq.astype(np.float64)))   # [n][D/2]
    if style == 1:
        from transformers.models.llama.modeling_llama import apply_rotary_pos_emb
        emb = torch.cat([freqs, freqs], dim=-1)[None]           # [1][n][D]
        q = xt.permute(1, 0, 2)[None]                           # [1][H][n][D]
        out, _ = apply_rotary_pos_emb(q, q, emb.cos(), emb.sin(), unsqueeze_dim=1)
        return out[0].permute(1, 0, 2).numpy()
    from transformers.models.gptj.modeling_gptj import apply_rotary_pos_emb
    out = apply_rotary_pos_emb(xt[None], freqs.sin()[None], freqs.cos()[None])   # [1][n][H][D]
    return out[0].numpy()


@pytest.mark.parametrize("style", [1, 2])
@pytest.mark.parametrize("D", [64, 128])
def test_rope_matches_library(style, D):
    rng = np.random.default_rng(D + style)
    x = rng.standard_normal((37, 3, D))
    pos = rng.integers(0, 4096, size=37)
    inv = synth.rope_inv_freq(D)
    got = odk.rope(x, pos, inv, style)
    assert np.abs(got - _hf_rope(x, pos, inv, style)).max() < 1e-12
    # a rotation keeps every pair's norm, and position 0 is the identity
    if style == 1:
        n0 = x[..., :D // 2] ** 2 + x[..., D // 2:] ** 2
        n1 = got[..., :D // 2] ** 2 + got[..., D // 2:] ** 2
    else:
        n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
        n1 = got[..., 0::2] ** 2 + got[..., 1::2] ** 2
    assert np.abs(n0 - n1).max() < 1e-12
    assert np.array_equal(odk.rope(x, np.zeros(37, dtype=np.int64), inv, style), x)


@pytest.mark.parametrize("style", [1, 2])
def test_local_positions_keep_relative_scores(style):
    """A window kept whole: a query rotated at the next local position scores the compact keys exactly as
    a query at the next absolute position scores the keys at their absolute positions."""
    rng = np.random.default_rng(3)
    D, L, W = 64, 900, 300
    inv = synth.rope_inv_freq(D, 10000.0)
    k = rng.standard_normal((L, 1, D))
    q = rng.standard_normal((1, 1, D))
    pos = odk.selected_positions(L, [], 64, W)
    local = odk.rope(k[pos], np.arange(len(pos)), inv, style)
    absolute = odk.rope(k[pos], pos, inv, style)
    s_local = local[:, 0] @ odk.rope(q, np.array([len(pos)]), inv, style)[0, 0]
    s_abs = absolute[:, 0] @ odk.rope(q, np.array([L]), inv, style)[0, 0]
    assert np.abs(s_local - s_abs).max() < 1e-9


def _pools_from_logical(k_log, v_log, page_size, rng):
    """Page pools holding the logical [B][slots][H][D] arrays through a shuffled block table."""
    B, S, H, D = k_log.shape
    npg = -(-S // page_size)
    pool = B * npg + 3
    perm = rng.permutation(pool)[:B * npg].reshape(B, npg).astype(np.int32)
    kp = np.full((pool, H, page_size, D), synth.BF16_QNAN, dtype=np.uint16)
    vp = kp.copy()
    for b in range(B):
        for t in range(S):
            kp[perm[b, t // page_size], :, t % page_size] = k_log[b, t]
            vp[perm[b, t // page_size], :, t % page_size] = v_log[b, t]
    return kp, vp, perm


@pytest.mark.parametrize("v_layout", [0, 1])
@pytest.mark.parametrize("style", [0, 1, 2])
def test_gather_reads_the_logical_rows(v_layout, style):
    rng = np.random.default_rng(7 + style)
    B, S, H, D, ps, cs, W, sel = 3, 300, 2, 64, 16, 32, 40, 4
    k_log = synth.bf16_bits(rng.standard_normal((B, S, H, D)))
    v_log = synth.bf16_bits(rng.standard_normal((B, S, H, D)))
    kp, vp, bt = _pools_from_logical(k_log, v_log, ps, rng)
    if v_layout:
        vp = synth.dim_major(vp)
    lens = np.array([300, 0, 77], dtype=np.int32)
    ids = synth.chunk_selection(5, -(-lens // cs), sel, pad_frac=0.2, dup_frac=0.2, bad_frac=0.1)
    inv = synth.rope_inv_freq(D)
    cap = sel * cs + W + 5
    ok, ov, opos, olen = odk.draft_gather(kp, vp, bt, lens, ids, ps, cs, W, cap, inv, style, v_layout)
    for b in range(B):
        pos = _mask_positions(int(lens[b]), ids[b], cs, W)
        n = len(pos)
        assert olen[b] == n and np.array_equal(opos[b, :n], pos) and (opos[b, n:] == -1).all()
        assert np.array_equal(ov[b, :n], oracle.bf16_to_f64(v_log[b, pos]))
        kk = oracle.bf16_to_f64(k_log[b, pos])
        want = kk if style == 0 else _hf_rope(kk, np.arange(n), inv, style)
        assert np.abs(ok[b, :n] - want).max(initial=0) < 1e-12
        assert np.isnan(ok[b, n:]).all() and np.isnan(ov[b, n:]).all()


def test_gather_refuses_overflow():
    kp = np.zeros((4, 1, 16, 64), dtype=np.uint16)
    with pytest.raises(ValueError, match="capacity"):
        odk.draft_gather(kp, kp, np.arange(4)[None], [64], [[0]], 16, 16, 8, 16, None, 0)
