"""Move synthetic cases to a torch device, and draw full-size workloads directly on the GPU.

Full-size KV (hundreds of MiB per layer) is drawn with torch's seeded device generator instead of
numpy, so that a 32-layer 128K-context workload is generated in seconds.  Values are N(0, 1) rounded
to bf16, as in ``synth.inputs``; only the generator differs.
"""

from __future__ import annotations

import math

import numpy as np
import torch

from .inputs import PAGE_SIZE, AttentionCase, GreedyCase, RejectionCase, dim_major


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def attention_tensors(case: AttentionCase, device, v_layout: int = 0) -> dict:
    """``v_layout`` 1 hands V over dim-major ([pages][kv_heads][head_dim][page_size])."""
    return dict(
        q=bf16_tensor(case.q, device),
        k_cache=bf16_tensor(case.kv.k_pool, device),
        v_cache=bf16_tensor(dim_major(case.kv.v_pool) if v_layout else case.kv.v_pool, device),
        block_table=torch.from_numpy(case.kv.block_table).to(device),
        ctx_lens=torch.from_numpy(case.ctx_lens).to(device),
        node_offsets=torch.from_numpy(case.node_offsets).to(device),
        parents=torch.from_numpy(case.parents).to(device),
    )


def greedy_tensors(case: GreedyCase, device) -> dict:
    logits = bf16_tensor(case.logits, device) if case.dtype == "bf16" else torch.from_numpy(case.logits).to(device)
    return dict(node_offsets=torch.from_numpy(case.node_offsets).to(device),
                parents=torch.from_numpy(case.parents).to(device),
                draft_tokens=torch.from_numpy(case.draft_tokens).to(device),
                target_logits=logits)


def rejection_tensors(case: RejectionCase, device) -> dict:
    logits = bf16_tensor(case.logits, device) if case.dtype == "bf16" else torch.from_numpy(case.logits).to(device)
    return dict(node_offsets=torch.from_numpy(case.node_offsets).to(device),
                parents=torch.from_numpy(case.parents).to(device),
                draft_tokens=torch.from_numpy(case.draft_tokens).to(device),
                target_logits=logits,
                draft_probs=torch.from_numpy(case.draft_probs).to(device),
                u_accept=torch.from_numpy(case.u_accept).to(device),
                u_sample=torch.from_numpy(case.u_sample).to(device))


def _gen(device, *seed_parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([int(s) for s in seed_parts]).generate_state(1, dtype=np.uint64)[0]
                      & 0x7FFFFFFFFFFFFFFF))
    return g


def paged_kv_device(case: int, layer: int, slots, num_kv_heads: int, head_dim: int, device, *,
                    page_size: int = PAGE_SIZE, pool_factor: float = 1.25, v_layout: int = 0):
    """K/V pools bf16 [pool][Hkv][page_size][D] ~ N(0,1) drawn on the device, a seeded permutation block
    table (int32 [B][max_blocks], -1 padded).  Returns (k_pool, v_pool, block_table); with ``v_layout`` 1
    the same V values are returned dim-major, [pool][Hkv][D][page_size]."""
    slots = [int(s) for s in slots]
    npages = [(s + page_size - 1) // page_size for s in slots]
    total = sum(npages)
    pool = max(total, int(math.ceil(pool_factor * total)))
    perm = np.random.Generator(np.random.PCG64(np.random.SeedSequence([case, layer, 3]))).permutation(pool)[:total]
    bt = np.full((len(slots), max(npages)), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(npages):
        bt[b, :n] = perm[off:off + n]
        off += n
    shape = (pool, num_kv_heads, page_size, head_dim)
    k = torch.randn(shape, generator=_gen(device, case, layer, 1), device=device, dtype=torch.bfloat16)
    v = torch.randn(shape, generator=_gen(device, case, layer, 2), device=device, dtype=torch.bfloat16)
    if v_layout:
        v = v.transpose(2, 3).contiguous()
    return k, v, torch.from_numpy(bt).to(device)


def queries_device(case: int, layer: int, total_nodes: int, num_q_heads: int, head_dim: int, device):
    return torch.randn((total_nodes, num_q_heads, head_dim), generator=_gen(device, case, layer, 0), device=device,
                       dtype=torch.bfloat16)


def logits_device(case: int, layer: int, rows: int, vocab: int, device, std: float = 2.0, dtype=torch.bfloat16,
                  stream: int = 5):
    x = torch.randn((rows, vocab), generator=_gen(device, case, layer, stream), device=device, dtype=torch.float32)
    return (x * std).to(dtype)
