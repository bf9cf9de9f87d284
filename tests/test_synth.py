"""The seeded input generators: bf16 rounding agrees with torch's float32 -> bfloat16 cast, trees are
topological with the requested depth and fan-out, page pools hold each logical slot once, uniforms
are exact on the 2^-24 grid, and draws are reproducible from their seeds."""

import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(1)
    x = np.concatenate([r.normal(0, 3, 100000), r.normal(0, 1e-30, 1000), [0.0, -0.0, 1e38, -1e38]]).astype(np.float32)
    ours = synth.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    np.testing.assert_array_equal(synth.bf16_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_trees():
    rng = synth.rng_for(30, 0, 0)
    for n, d in [(1, 0), (5, 4), (8, 4), (64, 8), (128, 10), (256, 12)]:
        par = synth.random_tree(rng, n, d)
        assert par[0] == -1 and all(0 <= par[i] < i for i in range(1, n))
        dep = synth.tree_depths(par)
        assert dep.max() == min(d, n - 1)
        assert max(len(c) for c in synth.children_lists(par)) <= 4
    assert synth.chain_tree(4).tolist() == [-1, 0, 1, 2]


def test_paged_kv_layout():
    kv = synth.paged_kv(31, 0, [40, 17, 16], 2, 64)
    used = kv.block_table[kv.block_table >= 0]
    assert len(np.unique(used)) == len(used) == 3 + 2 + 1
    assert kv.k_pool.shape[0] >= int(np.ceil(1.25 * 6))
    # tail slots of the last page are poisoned, live slots are finite
    k = synth.bf16_to_f32(kv.k_pool)
    assert np.isnan(k[kv.block_table[0, 2], :, 8:]).all() and np.isfinite(k[kv.block_table[0, 2], :, :8]).all()
    assert np.isfinite(k[kv.block_table[2, 0]]).all()
    again = synth.paged_kv(31, 0, [40, 17, 16], 2, 64)
    assert np.array_equal(kv.k_pool, again.k_pool) and np.array_equal(kv.block_table, again.block_table)


def test_uniforms_and_cases_reproducible():
    u = synth.uniforms24(synth.rng_for(32, 0, 8), 1000)
    assert u.dtype == np.float32 and (u >= 0).all() and (u < 1).all()
    assert np.array_equal((u.astype(np.float64) * 2 ** 24) % 1, np.zeros(1000))
    trees = [synth.random_tree(synth.rng_for(32, 0, 4), 16, 4)]
    a = synth.rejection_case(32, trees, 64)
    b = synth.rejection_case(32, trees, 64)
    assert np.array_equal(a.draft_tokens, b.draft_tokens) and np.array_equal(a.logits, b.logits)
    np.testing.assert_allclose(a.draft_probs.sum(1), 1.0, atol=1e-5)
