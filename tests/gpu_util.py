"""Helpers shared by the GPU parity tests: run the HIP path through the binding, run the oracle on
the same seeded inputs, compare at the stated tolerances."""

import numpy as np
import torch

import oracle
import synth
from synth import device as sdev

# tolerances for floating-point outputs (fp32 accumulation of bf16 products, bf16 output)
OUT_MAX_ABS = 1e-2
OUT_MEAN_ABS = 1e-3
OUT_REL_L2 = 1e-2
LSE_MAX_ABS = 1e-3
MASS_REL_L1 = 1e-3


def dev():
    return torch.device("cuda:0")


def bits_of(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run_attention(case: synth.AttentionCase, chunk_size=0, split_tiles=0, max_nodes=None, max_ctx=None, v_layout=0,
                  subtree_end=None):
    """subtree_end: sequence-local int32 [T] (trees in preorder) to take the ancestors from index ranges."""
    import long_context_tree_amd as lt
    t = sdev.attention_tensors(case, dev(), v_layout)
    sizes = np.diff(case.node_offsets)
    mn = int(max_nodes or max(1, sizes.max(initial=1)))
    mc = int(max_ctx if max_ctx is not None else case.ctx_lens.max(initial=0))
    se = None if subtree_end is None else torch.from_numpy(np.asarray(subtree_end, dtype=np.int32)).to(dev())
    out, lse, h = lt.tree_attention(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["ctx_lens"],
                                    t["node_offsets"], t["parents"], max_nodes=mn, max_ctx_len=mc,
                                    scale=case.scale, chunk_size=chunk_size, split_tiles=split_tiles,
                                    v_layout=v_layout, subtree_end=se)
    return out, lse, h, t


def oracle_attention(case: synth.AttentionCase, chunk_size=0, **kw):
    return oracle.tree_attention(case.q, case.kv.k_pool, case.kv.v_pool, case.kv.block_table, case.ctx_lens,
                                 case.node_offsets, case.parents, case.scale, case.num_kv_heads, case.kv.page_size,
                                 chunk_size, **kw)


def compare_out(out_gpu: torch.Tensor, lse_gpu: torch.Tensor, out_ref: np.ndarray, lse_ref: np.ndarray, mask=None):
    o = out_gpu.float().cpu().numpy().astype(np.float64)
    l = lse_gpu.float().cpu().numpy().astype(np.float64)
    if mask is not None:
        o, out_ref, l, lse_ref = o[mask], out_ref[mask], l[mask], lse_ref[mask]
    assert np.isfinite(o).all() and np.isfinite(l).all()
    d = np.abs(o - out_ref)
    rel = np.linalg.norm(o - out_ref) / max(np.linalg.norm(out_ref), 1e-30)
    stats = dict(max_abs=float(d.max()), mean_abs=float(d.mean()), rel_l2=float(rel),
                 lse_max_abs=float(np.abs(l - lse_ref).max()))
    assert stats["max_abs"] <= OUT_MAX_ABS, stats
    assert stats["mean_abs"] <= OUT_MEAN_ABS, stats
    assert stats["rel_l2"] <= OUT_REL_L2, stats
    assert stats["lse_max_abs"] <= LSE_MAX_ABS, stats
    return stats


def compare_mass(mass_gpu: np.ndarray, mass_ref: np.ndarray):
    if len(mass_ref) == 0:
        return {}
    d = np.abs(mass_gpu - mass_ref)
    stats = dict(max_abs=float(d.max(initial=0)), rel_l1=float(d.sum() / max(mass_ref.sum(), 1e-30)))
    assert stats["max_abs"] <= OUT_MAX_ABS and d.mean() <= OUT_MEAN_ABS, stats
    assert stats["rel_l1"] <= MASS_REL_L1, stats
    return stats


def topk_valid(idx_gpu, mass_ref, k, tau_rel=1e-4):
    """The GPU's top-k set S is valid iff min_{c in S} m_ref >= max_{c not in S} m_ref - tau."""
    n = len(mass_ref)
    sel = [int(i) for i in idx_gpu[:min(k, n)]]
    assert len(set(sel)) == len(sel) and all(0 <= i < n for i in sel)
    assert all(int(i) == -1 for i in idx_gpu[min(k, n):])
    if len(sel) == n:
        return
    tau = tau_rel * mass_ref.max()
    rest = np.ones(n, dtype=bool)
    rest[sel] = False
    assert mass_ref[sel].min() >= mass_ref[rest].max() - tau
