"""The C-ABI library without a GPU: it loads, exports every function include/spec_verify.h declares,
reports its ABI version, and refuses bad host arguments by name with the documented status, before
any HIP call."""

import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")


def _lib():
    from long_context_tree_amd import spec
    if not os.path.exists(spec.LIB_PATH):
        pytest.skip("libspec_verify.so not built (python -m long_context_tree_amd.build)")
    return spec


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(spec_[a-z_]+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    spec = _lib()
    names = declared_functions()
    assert {"spec_tree_attention", "spec_chunk_salience", "spec_accept_greedy", "spec_accept_rejection"} <= set(names)
    assert len(names) == 20, names
    for path in (spec.LIB_PATH, spec.DEBUG_LIB_PATH):
        L = ctypes.CDLL(path)
        for n in names:
            assert hasattr(L, n), (path, n)
    assert spec.lib().spec_abi_version() == 5 and spec.debug_lib().spec_abi_version() == 5
    assert spec.lib().spec_debug_build() == 0 and spec.debug_lib().spec_debug_build() == 1
    assert spec.status_string(3) == "SPEC_ERR_WORKSPACE"


def _attn_args(spec, **over):
    q = torch.zeros(8, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(40, 2, 16, 64, dtype=torch.bfloat16)
    bt = torch.zeros(1, 40, dtype=torch.int32)
    cl = torch.tensor([512], dtype=torch.int32)
    no = torch.tensor([0, 8], dtype=torch.int32)
    par = torch.tensor([-1, 0, 1, 2, 3, 0, 1, 2], dtype=torch.int32)
    out = torch.zeros_like(q)
    keep = (q, k, bt, cl, no, par, out)
    a = spec.tree_attention_args(q, k, k, bt, cl, no, par, max_nodes=8, max_ctx_len=512, chunk_size=64, out=out)
    for key, v in over.items():
        if key.startswith("kv_"):
            setattr(a.kv, key[3:], v)
        else:
            setattr(a, key, v)
    return a, keep


@pytest.mark.parametrize("field,value,status,text", [
    ("batch", 0, 1, "batch"),
    ("num_q_heads", 3, 1, "num_q_heads"),
    ("head_dim", 96, 2, "head_dim"),
    ("max_nodes", 300, 2, "max_nodes"),
    ("max_nodes", 0, 1, "max_nodes"),
    ("q", None, 1, "q:"),
    ("q", 8, 1, "16-byte"),
    ("kv_page_size", 12, 2, "page_size"),
    ("kv_page_size", 4, 2, "page_size"),
    ("kv_block_table_stride", 10, 1, "block_table_stride"),
    ("kv_token_stride", 60, 1, "token_stride"),
    ("kv_v_layout", 2, 1, "v_layout"),
    ("kv_v_layout", -1, 1, "v_layout"),
    ("parents", None, 1, "parents"),
    ("scale", float("nan"), 1, "scale"),
    ("scale", -1.0, 1, "scale"),
    ("chunk_size", 48, 2, "chunk_size"),
    ("split_tiles", -1, 1, "split_tiles"),
])
def test_attention_refuses_bad_arguments(field, value, status, text):
    spec = _lib()
    a, keep = _attn_args(spec, **{field: value})
    st = spec.lib().spec_tree_attention(ctypes.byref(a), None)
    assert st == status and text in spec.last_error(), (st, spec.last_error())
    assert spec.lib().spec_tree_attention_workspace_size(ctypes.byref(a)) == 0


def test_attention_workspace_checks_and_hip_error_without_gpu():
    spec = _lib()
    a, keep = _attn_args(spec)
    need = spec.lib().spec_tree_attention_workspace_size(ctypes.byref(a))
    assert need > 0 and spec.last_error() == ""
    assert spec.lib().spec_tree_attention(ctypes.byref(a), None) == 3        # no workspace
    ws = torch.zeros(need + 512, dtype=torch.uint8)
    base = ws.data_ptr() + (-ws.data_ptr()) % 256
    a.workspace, a.workspace_bytes = base + 8, need                        # misaligned
    assert spec.lib().spec_tree_attention(ctypes.byref(a), None) == 3 and "aligned" in spec.last_error()
    a.workspace, a.workspace_bytes = base, need - 1                        # too small
    assert spec.lib().spec_tree_attention(ctypes.byref(a), None) == 3
    if not torch.cuda.is_available():
        a.workspace_bytes = need                                           # valid: fails only at the launch
        assert spec.lib().spec_tree_attention(ctypes.byref(a), None) == 4
        assert "HIP error" in spec.last_error()


def test_salience_state_and_argument_checks():
    spec = _lib()
    a, keep = _attn_args(spec, chunk_size=0)
    mass = torch.zeros(1, 8)
    s = spec.ChunkSalienceArgs()
    s.attn = ctypes.pointer(a)
    s.chunk_mass = mass.data_ptr()
    s.max_chunks = 8
    assert spec.lib().spec_chunk_salience(ctypes.byref(s), None) == 5          # no partials: SPEC_ERR_STATE
    a.chunk_size = 64
    need = spec.lib().spec_tree_attention_workspace_size(ctypes.byref(a))
    ws = torch.zeros(need + 256, dtype=torch.uint8)
    a.workspace, a.workspace_bytes = ws.data_ptr() + (-ws.data_ptr()) % 256, need
    s.max_chunks = 7
    assert spec.lib().spec_chunk_salience(ctypes.byref(s), None) == 1 and "max_chunks" in spec.last_error()
    s.max_chunks, s.top_k = 8, 4
    assert spec.lib().spec_chunk_salience(ctypes.byref(s), None) == 1 and "topk_index" in spec.last_error()
    s.top_k, s.accumulate = 0, 2
    assert spec.lib().spec_chunk_salience(ctypes.byref(s), None) == 1 and "accumulate" in spec.last_error()


def _greedy_args(spec, **over):
    no = torch.tensor([0, 8], dtype=torch.int32)
    par = torch.tensor([-1, 0, 1, 2, 3, 0, 1, 2], dtype=torch.int32)
    tok = torch.zeros(8, dtype=torch.int32)
    lg = torch.zeros(8, 32)
    outs = (torch.zeros(1, dtype=torch.int32), torch.zeros(1, 5, dtype=torch.int32), torch.zeros(1, 5, dtype=torch.int32))
    a = spec._greedy_args(no, par, tok, lg, 8, 5, outs)
    for k, v in over.items():
        setattr(a, k, v)
    return a, (no, par, tok, lg, outs)


@pytest.mark.parametrize("field,value,status,text", [
    ("vocab", 0, 1, "vocab"), ("max_nodes", 2049, 2, "max_nodes"), ("max_path", 0, 1, "max_path"),
    ("logits_dtype", 7, 2, "logits_dtype"), ("draft_tokens", None, 1, "draft_tokens"),
    ("batch", 10000, 2, "batch * max_nodes"),
])
def test_greedy_refuses_bad_arguments(field, value, status, text):
    spec = _lib()
    a, keep = _greedy_args(spec, **{field: value})
    assert spec.lib().spec_accept_greedy(ctypes.byref(a), None) == status
    assert text in spec.last_error()


def test_rejection_refuses_bad_arguments():
    spec = _lib()
    g, keep = _greedy_args(spec)
    r = spec.AcceptRejectionArgs()
    r.base = g
    r.max_children = 9
    assert spec.lib().spec_accept_rejection(ctypes.byref(r), None) == 1 and "max_children" in spec.last_error()
    r.max_children = 2
    assert spec.lib().spec_accept_rejection(ctypes.byref(r), None) == 1 and "draft_probs" in spec.last_error()
    r.base.vocab = -1
    assert spec.lib().spec_accept_rejection(ctypes.byref(r), None) == 1 and "base.vocab" in spec.last_error()


def _commit_args(spec, **over):
    k = [torch.zeros(40, 2, 16, 64, dtype=torch.bfloat16) for _ in range(2)]
    bt = torch.zeros(1, 40, dtype=torch.int32)
    cl = torch.tensor([100], dtype=torch.int32)
    na = torch.tensor([2], dtype=torch.int32)
    pn = torch.tensor([[0, 1, 3, -1]], dtype=torch.int32)
    out = torch.empty_like(cl)
    a, keep = spec.kv_commit_args(k, k, bt, cl, na, pn, max_nodes=8, new_ctx_lens=out)
    for key, v in over.items():
        setattr(a, key, v)
    return a, (keep, k, bt, cl, na, pn, out)


@pytest.mark.parametrize("field,value,status,text", [
    ("batch", 0, 1, "batch"),
    ("num_layers", 0, 2, "num_layers"),
    ("num_layers", 129, 2, "num_layers"),
    ("head_dim", 96, 2, "head_dim"),
    ("max_nodes", 2049, 2, "max_nodes"),
    ("max_path", 0, 1, "max_path"),
    ("page_size", 12, 2, "page_size"),
    ("token_stride", 60, 1, "token_stride"),
    ("v_layout", 2, 1, "v_layout"),
    ("ctx_lens", None, 1, "ctx_lens"),
    ("new_ctx_lens", None, 1, "new_ctx_lens"),
])
def test_kv_commit_refuses_bad_arguments(field, value, status, text):
    spec = _lib()
    a, keep = _commit_args(spec, **{field: value})
    st = spec.lib().spec_kv_commit(ctypes.byref(a), None)
    assert st == status and text in spec.last_error(), (st, spec.last_error())


def _gather_args(spec, **over):
    k = torch.zeros(40, 2, 16, 64, dtype=torch.bfloat16)
    bt = torch.zeros(1, 40, dtype=torch.int32)
    cl = torch.tensor([600], dtype=torch.int32)
    ids = torch.zeros(1, 8, dtype=torch.int32)
    inv = torch.ones(32)
    ok = torch.zeros(1, 8 * 64 + 32, 2, 64, dtype=torch.bfloat16)
    pos = torch.zeros(1, 8 * 64 + 32, dtype=torch.int32)
    ln = torch.zeros(1, dtype=torch.int32)
    a = spec.draft_gather_args(k, k, bt, cl, ids, max_ctx_len=640, chunk_size=64, window=32, capacity=8 * 64 + 32,
                               inv_freq=inv, out_k=ok, out_v=ok, out_pos=pos, out_len=ln)
    for key, v in over.items():
        if key.startswith("kv_"):
            setattr(a.kv, key[3:], v)
        else:
            setattr(a, key, v)
    return a, (k, bt, cl, ids, inv, ok, pos, ln)


@pytest.mark.parametrize("field,value,status,text", [
    ("batch", 0, 1, "batch"),
    ("num_kv_heads", 0, 1, "num_kv_heads"),
    ("head_dim", 96, 2, "head_dim"),
    ("max_ctx_len", -1, 1, "max_ctx_len"),
    ("chunk_size", 0, 1, "chunk_size"),
    ("chunk_size", 70000, 1, "chunk_size"),
    ("max_ctx_len", 1 << 25, 2, "chunks"),
    ("kv_page_size", 12, 2, "page_size"),
    ("kv_block_table_stride", 39, 1, "block_table_stride"),
    ("kv_v_layout", 3, 1, "v_layout"),
    ("window", -1, 1, "window"),
    ("num_select", 8193, 1, "num_select"),
    ("chunk_index", None, 1, "chunk_index"),
    ("chunk_index_stride", 7, 1, "chunk_index_stride"),
    ("capacity", 8 * 64 + 31, 1, "capacity"),
    ("rope", 3, 1, "rope"),
    ("inv_freq", None, 1, "inv_freq"),
    ("out_k", None, 1, "out_k"),
    ("out_v", 8, 1, "out_v"),
    ("out_pos", None, 1, "out_pos"),
    ("out_len", None, 1, "out_len"),
])
def test_draft_gather_refuses_bad_arguments(field, value, status, text):
    spec = _lib()
    a, keep = _gather_args(spec, **{field: value})
    st = spec.lib().spec_draft_gather(ctypes.byref(a), None)
    assert st == status and text in spec.last_error(), (st, spec.last_error())


def test_draft_gather_accepts_valid_arguments_until_the_launch():
    spec = _lib()
    a, keep = _gather_args(spec)
    a.rope, a.inv_freq = 0, None                       # no frequencies needed without rotation
    a.num_select, a.chunk_index = 0, None              # no selection: the window alone
    if not torch.cuda.is_available():
        assert spec.lib().spec_draft_gather(ctypes.byref(a), None) == 4 and "HIP error" in spec.last_error()


def test_attention_node_limits_depend_on_the_mask():
    """Up to 256 nodes with ancestor bit masks; up to SPEC_MAX_TREE_NODES with subtree ends."""
    spec = _lib()
    se = torch.arange(1, 9, dtype=torch.int32)
    for mn, with_end, status in ((256, False, None), (257, False, 2), (2048, True, None), (2049, True, 2)):
        a, keep = _attn_args(spec, max_nodes=mn, kv_block_table_stride=200)
        if with_end:
            a.subtree_end, a.parents = se.data_ptr(), None
        need = spec.lib().spec_tree_attention_workspace_size(ctypes.byref(a))
        if status is None:
            assert need > 0, spec.last_error()
        else:
            assert need == 0 and "max_nodes" in spec.last_error()


def test_read_probe_refuses_bad_arguments():
    spec = _lib()
    buf = torch.zeros(64, dtype=torch.uint8)
    sink = torch.zeros(spec.READ_PROBE_SINK_WORDS, dtype=torch.int32)
    L = spec.lib()
    assert L.spec_read_probe(None, 64, sink.data_ptr(), None) == 1 and "data" in spec.last_error()
    base = buf.data_ptr() + (-buf.data_ptr()) % 16
    assert L.spec_read_probe(base, 40, sink.data_ptr(), None) == 1 and "bytes" in spec.last_error()
    assert L.spec_read_probe(base, 32, None, None) == 1 and "sink" in spec.last_error()


def test_greedy_noalloc_refuses_inputs_beyond_its_device_array():
    """The no-allocation greedy call refuses, before any HIP call, an input whose segment keys need more
    than its fixed device array, and says which call to use instead."""
    spec = _lib()
    no = torch.tensor([0, 3], dtype=torch.int32)
    par = torch.tensor([-1, 0, 1], dtype=torch.int32)
    tok = torch.zeros(3, dtype=torch.int32)
    logits = torch.zeros(3, 64, dtype=torch.float32)
    outs = spec._outs(1, 4, "cpu")
    a = spec._greedy_args(no, par, tok, logits, 3, 4, outs)
    a.max_nodes, a.vocab = 2048, 1 << 24                      # 2048 x 2048 segment keys: 32 MiB
    assert spec.lib().spec_accept_greedy_noalloc(ctypes.byref(a), None) == 2
    assert "device array" in spec.last_error() and "spec_accept_greedy" in spec.last_error()
    assert spec.GREEDY_NOALLOC_SCRATCH_BYTES == 4 << 20


def test_workspaces_end_with_the_debug_record():
    """Every workspace size includes the 256-byte debug record at its end, in both builds (the same size)."""
    spec = _lib()
    a, keep = _attn_args(spec)
    n1 = spec.lib().spec_tree_attention_workspace_size(ctypes.byref(a))
    n2 = spec.debug_lib().spec_tree_attention_workspace_size(ctypes.byref(a))
    assert n1 == n2 and n1 % 256 == 0 and n1 > spec.DEBUG_RECORD_BYTES
    no = torch.tensor([0, 3], dtype=torch.int32)
    par = torch.tensor([-1, 0, 1], dtype=torch.int32)
    outs = spec._outs(1, 4, "cpu")
    g = spec._greedy_args(no, par, torch.zeros(3, dtype=torch.int32), torch.zeros(3, 64), 3, 4, outs)
    # 3 rows x 1 segment key (8 bytes each), padded to 256, then the record
    assert spec.lib().spec_accept_greedy_workspace_size(ctypes.byref(g)) == 256 + spec.DEBUG_RECORD_BYTES
    assert spec.debug_lib().spec_accept_greedy_workspace_size(ctypes.byref(g)) == 256 + spec.DEBUG_RECORD_BYTES
