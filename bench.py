#!/usr/bin/env python3
"""Benchmark of the tree-verification step on one MI355X.

One step = the verification of one 128-node draft tree (depth 10) of a Llama-3.1-8B-shaped target at
131072 tokens of context: for each of the 32 layers, spec_tree_attention (32 q / 8 KV heads,
head_dim 128, bf16 KV in 16-token pages through a shuffled block table) and spec_chunk_salience
(64-token chunks, accumulated over the layers, top-256 chunks after the last layer), then
spec_accept_greedy over a 128256-token vocabulary.  Every layer has its own seeded KV (17.2 GB of
KV per step), so no cache level can serve a repeated layer.

Prints one JSON line: KV GB/s over the whole step (the metric), steps/s, the roofline of the
dominant call (spec_tree_attention, timed per call with HIP events on its stream inside the timed
region), the step's KV rate against a measured streaming-read rate (spec_read_probe over 4 GiB) beside
the 8 TB/s spec, and the CPU oracle's rate on a bounded sample of the same workload.  After the timed
region, the other calls of the path are timed alone ("kernels"), and spec_tree_attention alone for the
HBM-bound shapes ("attention_widths": 64-node trees at 32K, 64K and 128K, a 4-draft chain at 128K, and
a ragged batch of 16 Qwen3-8B-shaped chains).

    python bench.py [--steps K] [--warmup W] [--nodes N] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tree-verify KV GB/s & % HBM roofline at 128K ctx; verify steps/sec"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--context", type=int, default=131072)
    ap.add_argument("--nodes", type=int, default=128)
    ap.add_argument("--depth", type=int, default=10)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--split-tiles", type=int, default=0)
    ap.add_argument("--v-layout", choices=["token-rows", "dim-major"], default="token-rows",
                    help="V cache layout inside a page (token-rows: like K; dim-major: each dim's 16 tokens "
                         "contiguous)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device-to-device copy 3 times (reference for HBM byte counters)")
    return ap.parse_args()


def host_cores() -> int:
    return len(os.sched_getaffinity(0))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_heads(qb, kb, vb, btn, ctx, offs, tree, head_dim, kv_heads, heads, v_layout, chunk=64):
    """oracle.tree_attention over the listed KV heads, one head per worker thread (numpy releases the GIL in
    its array and BLAS work); returns the seconds taken."""
    import concurrent.futures as cf
    import numpy as np
    import oracle
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max(1, min(len(heads), host_cores()))) as ex:
        list(ex.map(lambda g: oracle.tree_attention(qb, kb, vb, btn, ctx, offs, tree, 1 / math.sqrt(head_dim),
                                                    kv_heads, 16, chunk, kv_heads=[g], v_layout=v_layout), heads))
    return time.perf_counter() - t0


def host_bits(t):
    import numpy as np
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def cpu_baseline(pools, qs, bt, tree, L, N, kv_heads, head_dim, v_layout, budget_s=12.0):
    """The oracle (numpy float64) on whole layers of the step (all KV heads of a layer in parallel, one per
    host thread), layer after layer until ~budget_s of oracle time; the rate is KV bytes of the heads done
    per second, the unit of the benchmark's value."""
    import numpy as np
    btn = bt.cpu().numpy()
    done, layers_used, dt = 0, 0, 0.0               # dt: oracle time only (device-to-host copies excluded)
    for (k_pool, v_pool), q in zip(pools, qs):
        if dt >= budget_s:
            break
        kb, vb, qb = host_bits(k_pool), host_bits(v_pool), host_bits(q)
        dt += oracle_heads(qb, kb, vb, btn, np.array([L]), np.array([0, N]), tree, head_dim, kv_heads,
                           list(range(kv_heads)), v_layout)
        done += kv_heads
        layers_used += 1
    kv_bytes = done * (L + N) * head_dim * 2 * 2
    return {"value": kv_bytes / dt / 1e9, "unit": "GB/s", "cores": host_cores(), "cpu_model": cpu_model(),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"oracle.tree_attention (numpy float64) on {layers_used} whole layers of the step "
                      f"({done} KV heads, one per worker thread on {host_cores()} host cores), {L} context + "
                      f"{N}-node tree each, chunk masses included, {dt:.1f} s; rate = KV bytes of those heads / time"}


def traffic_record(kernel_src: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE counters, if they were taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_tree_attention_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    sha = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    if rec.get("kernel_sha256") != sha:
        return None
    return rec.get("bytes_per_launch")


def read_ceiling(torch, lt, dev, gib: int = 4, reps: int = 5) -> float:
    """Measured streaming-read rate of this GPU in GB/s: the median time of spec_read_probe (every byte read
    once with 16-byte loads) over a gib-GiB buffer, the practical ceiling beside the 8 TB/s spec."""
    import numpy as np
    x = torch.zeros((gib << 30,), dtype=torch.uint8, device=dev)
    sink = lt.read_probe(x)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        lt.read_probe(x, sink)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    del x
    return (gib << 30) / float(np.median(ts)) / 1e9


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the verification step runs on a single MI355X and this build has no "
              "multi-GPU path; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import long_context_tree_amd as lt
    from long_context_tree_amd import spec
    import synth
    from synth import device as sdev

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.int16, device=dev)      # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ceiling = read_ceiling(torch, lt, dev)
    print(f"[bench] measured streaming read: {ceiling:.0f} GB/s", file=sys.stderr, flush=True)
    L, N, depth, layers = args.context, args.nodes, args.depth, args.layers
    Hq, Hkv, D, chunk, top_k, V = 32, 8, 128, 64, 256, 128256
    workload = f"llama8b-{L // 1024}k-n{N}"
    v_layout = spec.V_DIM_MAJOR if args.v_layout == "dim-major" else spec.V_TOKEN_ROWS
    case = 4
    tree = synth.random_tree(synth.rng_for(case, 0, synth.S_TREE), N, depth)
    par = torch.from_numpy(tree).to(dev)
    cl = torch.tensor([L], dtype=torch.int32, device=dev)
    no = torch.tensor([0, N], dtype=torch.int32, device=dev)

    pools, qs = [], []
    bt = None
    for layer in range(layers):
        k, v, b = sdev.paged_kv_device(case, layer, [L + N], Hkv, D, dev, v_layout=v_layout)
        bt = b if bt is None else bt                  # one page mapping shared by all layers
        pools.append((k, v))
        qs.append(sdev.queries_device(case, layer, N, Hq, D, dev))
    outs = [torch.empty((N, Hq, D), dtype=torch.bfloat16, device=dev) for _ in range(layers)]
    lses = [torch.empty((N, Hq), dtype=torch.float32, device=dev) for _ in range(layers)]

    attn = [spec.tree_attention_args(qs[l], pools[l][0], pools[l][1], bt, cl, no, par, max_nodes=N, max_ctx_len=L,
                                     chunk_size=chunk, split_tiles=args.split_tiles, out=outs[l], lse=lses[l],
                                     v_layout=v_layout)
            for l in range(layers)]
    need = lt.lib().spec_tree_attention_workspace_size(ctypes.byref(attn[0]))
    ws = spec._workspace(need, dev, None)
    for a in attn:
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    n_chunks = L // chunk
    mass = torch.zeros((1, n_chunks), dtype=torch.float32, device=dev)
    topi = torch.empty((1, top_k), dtype=torch.int32, device=dev)
    topm = torch.empty((1, top_k), dtype=torch.float32, device=dev)
    sal = []
    for l in range(layers):
        s = spec.ChunkSalienceArgs()
        s.attn = ctypes.pointer(attn[l])
        s.chunk_mass, s.max_chunks, s.accumulate = mass.data_ptr(), n_chunks, int(l > 0)
        s.top_k = top_k if l == layers - 1 else 0
        s.topk_index, s.topk_mass = topi.data_ptr(), topm.data_ptr()
        sal.append(s)
    g = synth.greedy_case(case, [tree], V, dtype="bf16")
    gt = sdev.greedy_tensors(g, dev)
    max_path = depth + 1
    gouts = (torch.empty(1, dtype=torch.int32, device=dev), torch.empty((1, max_path), dtype=torch.int32, device=dev),
             torch.empty((1, max_path), dtype=torch.int32, device=dev))
    ga = spec._greedy_args(gt["node_offsets"], gt["parents"], gt["draft_tokens"], gt["target_logits"], N, max_path,
                           gouts)
    gneed = lt.lib().spec_accept_greedy_workspace_size(ctypes.byref(ga))
    gws = spec._workspace(gneed, dev, None)
    ga.workspace, ga.workspace_bytes = gws.data_ptr(), gws.numel()

    L_ = lt.lib()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    def events():
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(layers)]

    def step(ev):
        for l in range(layers):
            if ev is not None:
                ev[l][0].record(stream)
            st = L_.spec_tree_attention(ctypes.byref(attn[l]), sh)
            if ev is not None:
                ev[l][1].record(stream)
            st |= L_.spec_chunk_salience(ctypes.byref(sal[l]), sh)
            if st:
                raise RuntimeError(lt.last_error())
        if L_.spec_accept_greedy(ctypes.byref(ga), sh):
            raise RuntimeError(lt.last_error())

    print(f"[bench] workload {workload}: {layers} layers, KV {layers * (L + N) * 4096 / 1e9:.2f} GB/step; "
          f"warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()

    # timed region 1 (the value): K whole steps between two events on the stream, nothing else inside
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        step(None)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / args.steps
    print(f"[bench] {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)

    # timed region 2 (the roofline): the same K steps again, every spec_tree_attention call bracketed by its
    # own pair of events on the stream it is launched on (read after the region ends).  The events add
    # their own gaps, so this region's step time is reported beside the value, not as it.
    step_events = [events() for _ in range(args.steps)]
    t2 = torch.cuda.Event(enable_timing=True)
    t3 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t2.record(stream)
    for k in range(args.steps):
        step(step_events[k])
    t3.record(stream)
    torch.cuda.synchronize()
    ms_per_step_events = t2.elapsed_time(t3) / args.steps
    attn_ms = [e0.elapsed_time(e1) for ev in step_events for e0, e1 in ev]

    # correctness guard: outputs finite, greedy produced a path
    assert torch.isfinite(outs[-1].float()).all().item() and int(gouts[0][0]) >= 0

    kv_bytes_layer = (L + N) * Hkv * D * 2 * 2
    alg_bytes = kv_bytes_layer + 2 * N * Hq * D * 2 + N * Hq * 4          # KV + Q + out + lse
    depths = synth.tree_depths(tree)
    alg_flops = 4.0 * D * Hq * float(np.sum(L + depths + 1))               # QK^T and PV over visible keys
    t_attn = float(np.median(attn_ms)) * 1e-3
    hbm_gbs = alg_bytes / t_attn / 1e9
    tflops = alg_flops / t_attn / 1e12
    mfma_bound = alg_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > alg_bytes / (HBM_PEAK_GBS * 1e9)
    kernel_src = os.path.join(ROOT, "long_context_tree_amd", "csrc", "tree_attention.hip")
    traffic = traffic_record(kernel_src, workload)
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(hbm_gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    roof.update({"kernel": "spec_tree_attention (tree_attn_pipe_kernel + attn_merge_kernel)",
                 "alg_bytes_per_launch": alg_bytes, "alg_flops_per_launch": alg_flops,
                 "launch_us_median": round(t_attn * 1e6, 2),
                 "launch_us_p10_p90": [round(float(np.percentile(attn_ms, 10)) * 1e3, 2),
                                       round(float(np.percentile(attn_ms, 90)) * 1e3, 2)],
                 "hbm_gbs": round(hbm_gbs, 1), "hbm_frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
                 "mfma_tflops": round(tflops, 2), "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)})
    kv_gbs_step = layers * kv_bytes_layer / (ms_per_step * 1e-3) / 1e9

    # the other calls of the path, each timed alone with events on the same stream after the timed region
    # (not part of the step's value): the salience reduction of one layer, greedy acceptance of the step,
    # and rejection acceptance on a 64-node tree (depth 8) at the same vocabulary
    def time_call(fn, reps=30):
        for _ in range(3):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3

    def call(st):
        if st:
            raise RuntimeError(lt.last_error())

    do_cpu = not args.no_cpu_baseline

    def oracle_time(fn):
        """Seconds of one oracle call on the host (the oracle as it stands, numpy float64)."""
        t = time.perf_counter()
        fn()
        return time.perf_counter() - t

    kernels = {}
    rows = N * Hq
    sal_bytes = rows * n_chunks * 4 + rows * 4 + 2 * n_chunks * 4
    us = time_call(lambda: call(L_.spec_chunk_salience(ctypes.byref(sal[1]), sh)))
    kernels["spec_chunk_salience"] = {"median_us": round(us, 2), "alg_bytes": sal_bytes,
                                      "gbs": round(sal_bytes / us / 1e3, 1), "bound": "hbm",
                                      "note": "one layer, accumulate, no top-k"}
    us = time_call(lambda: call(L_.spec_chunk_salience(ctypes.byref(sal[-1]), sh)))
    kernels["spec_chunk_salience_topk"] = {"median_us": round(us, 2), "alg_bytes": sal_bytes,
                                           "gbs": round(sal_bytes / us / 1e3, 1), "bound": "hbm",
                                           "note": f"last layer, accumulate, top-{top_k}"}
    if do_cpu:
        import oracle
        m_host = mass.cpu().numpy()[0].astype(np.float64)
        kernels["spec_chunk_salience_topk"].update(
            oracle_ms=round(oracle_time(lambda: oracle.topk_chunks(m_host, top_k)) * 1e3, 2),
            oracle_sample=f"oracle.topk_chunks over the step's {n_chunks} masses (one host thread); the masses "
                          "themselves come out of oracle.tree_attention, timed in cpu_baseline")
    g_bytes = N * V * 2
    us = time_call(lambda: call(L_.spec_accept_greedy(ctypes.byref(ga), sh)))
    kernels["spec_accept_greedy"] = {"median_us": round(us, 2), "alg_bytes": g_bytes,
                                     "gbs": round(g_bytes / us / 1e3, 1), "bound": "hbm",
                                     "note": f"{N} nodes, vocab {V}, bf16 logits"}
    if do_cpu:
        import oracle
        kernels["spec_accept_greedy"].update(
            oracle_ms=round(oracle_time(lambda: oracle.accept_greedy(g.node_offsets, g.parents, g.draft_tokens,
                                                                      g.logits, "bf16")) * 1e3, 2),
            oracle_sample="oracle.accept_greedy on the same inputs (one host thread)")
    # the commit of the step's greedy path into all 32 layers' caches (new lengths to a scratch buffer)
    ca, ckeep = spec.kv_commit_args([pl[0] for pl in pools], [pl[1] for pl in pools], bt, cl, gouts[0], gouts[1],
                                    max_nodes=N, new_ctx_lens=torch.empty_like(cl), v_layout=v_layout)
    n_acc = int(gouts[0][0])
    c_bytes = max(n_acc, 0) * layers * Hkv * D * 2 * 2 * 2
    us = time_call(lambda: call(L_.spec_kv_commit(ctypes.byref(ca), sh)))
    kernels["spec_kv_commit"] = {"median_us": round(us, 2), "alg_bytes": c_bytes,
                                 "gbs": round(c_bytes / us / 1e3, 1), "bound": "latency",
                                 "note": f"{n_acc} accepted drafts moved in {layers} layers x {Hkv} KV heads "
                                         "(K and V, read and write)"}
    # the compact draft KV from the step's top-k list: its 24 heaviest chunks plus a 512-token window in a
    # 2048-token budget, K rotated at local positions (layer 0's pool stands in for the draft layer's
    # canonical cache: same shape, 8 KV heads x 128)
    g_sel, g_win, g_cap = 24, 512, 2048
    g_out = (torch.empty((1, g_cap, Hkv, D), dtype=torch.bfloat16, device=dev),
             torch.empty((1, g_cap, Hkv, D), dtype=torch.bfloat16, device=dev),
             torch.empty((1, g_cap), dtype=torch.int32, device=dev), torch.empty(1, dtype=torch.int32, device=dev))
    inv_freq = torch.from_numpy(synth.rope_inv_freq(D)).to(dev)
    da = spec.draft_gather_args(pools[0][0], pools[0][1], bt, cl, topi, max_ctx_len=L, chunk_size=chunk,
                                window=g_win, capacity=g_cap, num_select=g_sel, rope=spec.ROPE_HALF,
                                inv_freq=inv_freq, out_k=g_out[0], out_v=g_out[1], out_pos=g_out[2],
                                out_len=g_out[3], v_layout=v_layout)
    us = time_call(lambda: call(L_.spec_draft_gather(ctypes.byref(da), sh)))
    g_len = int(g_out[3][0])
    d_bytes = g_len * Hkv * D * 2 * 2 * 2 + g_cap * 4
    kernels["spec_draft_gather"] = {"median_us": round(us, 2), "alg_bytes": d_bytes,
                                    "gbs": round(d_bytes / us / 1e3, 1), "bound": "hbm",
                                    "note": f"{g_len} kept tokens ({g_sel} top chunks + {g_win}-token window), "
                                            f"{Hkv} KV heads x {D}, K rotated; K and V read and written"}
    rtree = synth.random_tree(synth.rng_for(3, 0, synth.S_TREE), 64, 8)
    rc = synth.rejection_case(3, [rtree], V, dtype="bf16", draft="independent")
    rt = sdev.rejection_tensors(rc, dev)
    r_outs = (torch.empty(1, dtype=torch.int32, device=dev), torch.empty((1, 9), dtype=torch.int32, device=dev),
              torch.empty((1, 9), dtype=torch.int32, device=dev))
    ra = spec.AcceptRejectionArgs()
    ra.base = spec._greedy_args(rt["node_offsets"], rt["parents"], rt["draft_tokens"], rt["target_logits"], 64, 9,
                                r_outs)
    ra.max_children = 4
    ra.draft_probs, ra.u_accept, ra.u_sample = (rt["draft_probs"].data_ptr(), rt["u_accept"].data_ptr(),
                                                rt["u_sample"].data_ptr())
    rneed = lt.lib().spec_accept_rejection_workspace_size(ctypes.byref(ra))
    rws = spec._workspace(rneed, dev, None)
    ra.base.workspace, ra.base.workspace_bytes = rws.data_ptr(), rws.numel()
    r_bytes = 64 * V * (2 + 4)
    us = time_call(lambda: call(L_.spec_accept_rejection(ctypes.byref(ra), sh)))
    kernels["spec_accept_rejection"] = {"median_us": round(us, 2), "alg_bytes": r_bytes,
                                        "gbs": round(r_bytes / us / 1e3, 1), "bound": "hbm",
                                        "note": f"64 nodes (depth 8, <= 4 children), vocab {V}, bf16 logits + "
                                                "fp32 draft probabilities read once"}
    if do_cpu:
        import oracle
        kernels["spec_accept_rejection"].update(
            oracle_ms=round(oracle_time(lambda: oracle.accept_rejection(
                rc.node_offsets, rc.parents, rc.draft_tokens, rc.logits, rc.draft_probs, rc.u_accept, rc.u_sample,
                "bf16")) * 1e3, 2),
            oracle_sample="oracle.accept_rejection on the same inputs (one host thread)")

    # spec_tree_attention alone for narrower trees at the same context, and for the ragged Qwen3-8B-shaped
    # batch of 4-draft chains: these are HBM-bound (<= 256 query rows per KV head), so the KV rate against
    # 8 TB/s is their roofline.  Calls rotate over layers with independent KV, so no cache level serves a
    # repeated layer; medians of 64 calls after 8 warm-up calls.
    def attention_widths():
        out = {}

        def timed(arg_list, reps=64):
            for i in range(8):
                call(L_.spec_tree_attention(ctypes.byref(arg_list[i % len(arg_list)]), sh))
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for i, (e0, e1) in enumerate(ev):
                e0.record(stream)
                call(L_.spec_tree_attention(ctypes.byref(arg_list[i % len(arg_list)]), sh))
                e1.record(stream)
            torch.cuda.synchronize()
            return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3

        def entry(us, kv_bytes, flops, note, oracle_s=None, oracle_note=None):
            gbs = kv_bytes / us / 1e3
            tf = flops / us / 1e6
            bound = "mfma" if flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > kv_bytes / (HBM_PEAK_GBS * 1e9) else "hbm"
            e = {"median_us": round(us, 2), "kv_bytes": kv_bytes, "kv_gbs": round(gbs, 1),
                 "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "hbm_frac_of_read_ceiling": round(gbs / ceiling, 4),
                 "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "bound": bound, "note": note}
            if oracle_s is not None:
                e.update(oracle_s=round(oracle_s, 3), oracle_kv_gbs=round(kv_bytes / oracle_s / 1e9, 4),
                         oracle_cores=host_cores(), oracle_note=oracle_note)
            return e

        def oracle_one_layer(q, k_pool, v_pool, btab, ctx, offs, par, hkv, hd, seqs=None):
            """The oracle on the same call (first layer): KV heads (one sequence) or sequences (a batch) in
            parallel, one per host thread."""
            if not do_cpu:
                return None, None
            import concurrent.futures as cf
            import oracle
            qb, kb, vb, btn = host_bits(q), host_bits(k_pool), host_bits(v_pool), btab.cpu().numpy()
            if seqs is None:
                return oracle_heads(qb, kb, vb, btn, ctx, offs, par, hd, hkv, list(range(hkv)), v_layout, chunk), \
                    f"oracle.tree_attention on the first layer, {hkv} KV heads in parallel"
            t = time.perf_counter()
            with cf.ThreadPoolExecutor(max(1, min(seqs, host_cores()))) as ex:
                list(ex.map(lambda b: oracle.tree_attention(qb, kb, vb, btn, ctx, offs, par, 1 / math.sqrt(hd), hkv,
                                                            16, chunk, seqs=[b], v_layout=v_layout), range(seqs)))
            return time.perf_counter() - t, f"oracle.tree_attention on the first layer, {seqs} sequences in parallel"

        # the tiny parity workload: 512 committed tokens, 4 q / 2 KV heads, head_dim 64, an 8-node tree of
        # depth <= 4 (launch-latency bound; timed like the others)
        tiny = synth.attention_case(1, ctx_lens=[512], trees=[synth.random_tree(synth.rng_for(1, 0, synth.S_TREE),
                                                                                  8, 4)],
                                    num_q_heads=4, num_kv_heads=2, head_dim=64)
        tt = sdev.attention_tensors(tiny, dev, v_layout)
        to = torch.empty((8, 4, 64), dtype=torch.bfloat16, device=dev)
        tl = torch.empty((8, 4), dtype=torch.float32, device=dev)
        ta = [spec.tree_attention_args(tt["q"], tt["k_cache"], tt["v_cache"], tt["block_table"], tt["ctx_lens"],
                                       tt["node_offsets"], tt["parents"], max_nodes=8, max_ctx_len=512,
                                       chunk_size=chunk, out=to, lse=tl, v_layout=v_layout)]
        tws = spec._workspace(lt.lib().spec_tree_attention_workspace_size(ctypes.byref(ta[0])), dev, None)
        ta[0].workspace, ta[0].workspace_bytes = tws.data_ptr(), tws.numel()
        t_kvb = (512 + 8) * 2 * 64 * 2 * 2
        t_fl = 4.0 * 64 * 4 * float(np.sum(512 + synth.tree_depths(tiny.parents) + 1))
        os_, on_ = oracle_one_layer(tt["q"], tt["k_cache"], tt["v_cache"], tt["block_table"], tiny.ctx_lens,
                                    tiny.node_offsets, tiny.parents, 2, 64)
        out["tiny-512-n8"] = entry(timed(ta), t_kvb, t_fl, "512 context, 8-node tree, 4 q / 2 KV heads, head_dim 64",
                                   os_, on_)
        del ta, tws

        # (the 32K and 64K contexts use the first slots of the same pools: a shorter committed length)
        for name, wn, wd, wl in (("n64-depth8", 64, 8, L), ("chain-k4", 5, 4, L), ("n64-depth8", 64, 8, 32768),
                                 ("n64-depth8", 64, 8, 65536)):
            if wl > L:
                continue
            wtree = (synth.chain_tree(wn) if name.startswith("chain") else
                     synth.random_tree(synth.rng_for(case, 1, synth.S_TREE), wn, wd))
            wpar = torch.from_numpy(wtree).to(dev)
            wno = torch.tensor([0, wn], dtype=torch.int32, device=dev)
            wcl = torch.tensor([wl], dtype=torch.int32, device=dev)
            wq = [sdev.queries_device(case, 100 + l, wn, Hq, D, dev) for l in range(layers)]
            wo = [torch.empty((wn, Hq, D), dtype=torch.bfloat16, device=dev) for _ in range(layers)]
            wlse = [torch.empty((wn, Hq), dtype=torch.float32, device=dev) for _ in range(layers)]
            wa = [spec.tree_attention_args(wq[l], pools[l][0], pools[l][1], bt, wcl, wno, wpar, max_nodes=wn,
                                           max_ctx_len=wl, chunk_size=chunk, split_tiles=0, out=wo[l], lse=wlse[l],
                                           v_layout=v_layout) for l in range(layers)]
            wws = spec._workspace(lt.lib().spec_tree_attention_workspace_size(ctypes.byref(wa[0])), dev, None)
            for x in wa:
                x.workspace, x.workspace_bytes = wws.data_ptr(), wws.numel()
            kvb = (wl + wn) * Hkv * D * 2 * 2
            fl = 4.0 * D * Hq * float(np.sum(wl + synth.tree_depths(wtree) + 1))
            us_w = timed(wa)
            # the oracle reads the same slots: a shorter context is the first wl slots of the same pages
            os_, on_ = oracle_one_layer(wq[0], pools[0][0], pools[0][1], bt, np.array([wl]), np.array([0, wn]), wtree,
                                        Hkv, D)
            out[f"llama8b-{wl // 1024}k-{name}"] = entry(us_w, kvb, fl,
                                                       f"{wn}-node tree, chunk partials ({chunk}-token chunks)",
                                                       os_, on_)
            del wa, wws, wq, wo, wlse
        # ragged batch: 16 sequences, contexts uniform in [4096, 65536], 4-draft chains, Qwen3-8B layer shape
        rb_case, rb_n, rb_layers = 5, 5, 4
        rlens = synth.ragged_ctx_lens(rb_case, 16, 4096, 65536)
        rpools = [sdev.paged_kv_device(rb_case, l, [int(x) + rb_n for x in rlens], Hkv, D, dev, v_layout=v_layout)
                  for l in range(rb_layers)]
        rpar = torch.from_numpy(np.concatenate([synth.chain_tree(rb_n)] * 16).astype(np.int32)).to(dev)
        rno = torch.arange(0, 16 * rb_n + 1, rb_n, dtype=torch.int32, device=dev)
        rcl = torch.from_numpy(rlens).to(dev)
        rq = [sdev.queries_device(rb_case, l, 16 * rb_n, Hq, D, dev) for l in range(rb_layers)]
        ro = [torch.empty((16 * rb_n, Hq, D), dtype=torch.bfloat16, device=dev) for _ in range(rb_layers)]
        rlse = [torch.empty((16 * rb_n, Hq), dtype=torch.float32, device=dev) for _ in range(rb_layers)]
        kvb = int(np.sum(rlens.astype(np.int64) + rb_n)) * Hkv * D * 2 * 2
        fl = 4.0 * D * Hq * float(np.sum([np.sum(int(x) + np.arange(rb_n) + 1) for x in rlens]))
        for cs in (chunk, 0):
            ra_ = [spec.tree_attention_args(rq[l], rpools[l][0], rpools[l][1], rpools[l][2], rcl, rno, rpar,
                                            max_nodes=rb_n, max_ctx_len=int(rlens.max()), chunk_size=cs,
                                            split_tiles=0, out=ro[l], lse=rlse[l], v_layout=v_layout)
                   for l in range(rb_layers)]
            rws = spec._workspace(lt.lib().spec_tree_attention_workspace_size(ctypes.byref(ra_[0])), dev, None)
            for x in ra_:
                x.workspace, x.workspace_bytes = rws.data_ptr(), rws.numel()
            tag = "with chunk partials" if cs else "without chunk partials"
            us_r = timed(ra_)
            os_, on_ = (oracle_one_layer(rq[0], rpools[0][0], rpools[0][1], rpools[0][2], rlens,
                                         np.arange(0, 16 * rb_n + 1, rb_n), rpar.cpu().numpy(), Hkv, D, seqs=16)
                        if cs else (None, None))
            out[f"qwen3-8b-ragged16-chain-k4-{'chunks' if cs else 'nochunks'}"] = entry(
                us_r, kvb, fl, f"16 sequences, contexts {int(rlens.min())}..{int(rlens.max())} "
                               f"(sum {int(rlens.sum())}), {tag}", os_, on_)
            del ra_, rws
        del rpools
        return out

    widths = attention_widths()
    torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(pools, qs, bt, tree, L, N, Hkv, D, v_layout)

    line = {
        "metric": METRIC, "value": round(kv_gbs_step, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": workload, "context": L, "tree_nodes": N, "tree_depth": depth, "layers": layers,
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "page_size": 16, "v_layout": args.v_layout,
                   "chunk_size": chunk,
                   "top_k": top_k, "vocab": V, "acceptance": "greedy", "kv_bytes_per_step": layers * kv_bytes_layer},
        "verify_steps_per_s": round(1000.0 / ms_per_step, 2),
        "ms_per_step_with_call_events": round(ms_per_step_events, 4),
        "hbm_frac_step": round(kv_gbs_step / HBM_PEAK_GBS, 4),
        "hbm_read_ceiling_gbs": round(ceiling, 1),
        "hbm_frac_step_of_read_ceiling": round(kv_gbs_step / ceiling, 4),
        "roofline": roof,
        "kernels": kernels,
        "attention_widths": widths,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
