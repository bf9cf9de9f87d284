"""Python binding of libspec_verify (include/spec_verify.h), argument marshalling only.

torch supplies device memory and the current HIP stream; every step of the verification path runs
in the library's HIP kernels.  If the library is missing the calls raise: there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspec_verify.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libspec_verify_debug.so")   # the SPEC_DEBUG build

SPEC_OK = 0
SPEC_DTYPE_BF16 = 0
SPEC_DTYPE_F32 = 1
ABI_VERSION = 5
MAX_TREE_NODES = 2048
GREEDY_NOALLOC_SCRATCH_BYTES = 4 << 20   # SPEC_GREEDY_NOALLOC_SCRATCH_BYTES
V_TOKEN_ROWS = 0   # spec_v_layout: V pages like K, [pages][kv_heads][page_size][head_dim]
V_DIM_MAJOR = 1    # V pages [pages][kv_heads][head_dim][page_size]
ROPE_NONE = 0      # spec_rope: K copied as stored
ROPE_HALF = 1      # pairs (i, i + head_dim/2)
ROPE_PAIRS = 2     # pairs (2i, 2i + 1)
DEBUG_RECORD_BYTES = 256   # SPEC_DEBUG_RECORD_BYTES: the last bytes of every workspace
DBG_BITS = {"parents": 1 << 0, "block_table": 1 << 1, "node_offsets": 1 << 2, "ctx_lens": 1 << 3,
            "subtree_end": 1 << 4, "tokens": 1 << 5, "uniforms": 1 << 6, "draft_probs": 1 << 7,
            "children": 1 << 8, "logits": 1 << 9}   # SPEC_DBG_*

_lib = None
_debug_lib = None


class SpecError(RuntimeError):
    def __init__(self, status: int, func: str, text: str):
        super().__init__(f"{func}: {status_string(status)}: {text}")
        self.status = status


def _load(path: str):
    """Load one build of the library and declare its functions' argument and result types."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m long_context_tree_amd.build`")
    L = ctypes.CDLL(path)
    L.spec_abi_version.restype = ctypes.c_int
    L.spec_status_string.restype = ctypes.c_char_p
    L.spec_status_string.argtypes = [ctypes.c_int]
    L.spec_last_error.restype = ctypes.c_char_p
    for name, argt in (("spec_tree_attention", TreeAttentionArgs), ("spec_chunk_salience", ChunkSalienceArgs),
                       ("spec_accept_greedy", AcceptGreedyArgs), ("spec_accept_greedy_noalloc", AcceptGreedyArgs),
                       ("spec_accept_rejection", AcceptRejectionArgs),
                       ("spec_kv_commit", KvCommitArgs), ("spec_draft_gather", DraftGatherArgs)):
        f = getattr(L, name)
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.POINTER(argt), ctypes.c_void_p]
    for name, argt in (("spec_tree_attention_workspace_size", TreeAttentionArgs),
                       ("spec_accept_greedy_workspace_size", AcceptGreedyArgs),
                       ("spec_accept_rejection_workspace_size", AcceptRejectionArgs)):
        f = getattr(L, name)
        f.restype = ctypes.c_size_t
        f.argtypes = [ctypes.POINTER(argt)]
    L.spec_read_probe.restype = ctypes.c_int
    L.spec_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    L.spec_tree_bundle_order.restype = ctypes.c_int
    L.spec_tree_bundle_order.argtypes = [ctypes.c_void_p, ctypes.c_int32] + [ctypes.c_void_p] * 4
    L.spec_controller_speedup.restype = ctypes.c_double
    L.spec_controller_speedup.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_int32]
    L.spec_controller_choose.restype = ctypes.c_int32
    L.spec_controller_choose.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_int32]
    L.spec_controller_init.restype = ctypes.c_int
    L.spec_controller_init.argtypes = [ctypes.POINTER(DepthControllerState), ctypes.c_int32, ctypes.c_double,
                                       ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int32]
    L.spec_controller_update.restype = ctypes.c_int
    L.spec_controller_update.argtypes = [ctypes.POINTER(DepthControllerState), ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_double, ctypes.c_double]
    L.spec_debug_build.restype = ctypes.c_int
    if L.spec_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libspec_verify ABI {L.spec_abi_version()} != binding ABI {ABI_VERSION}")
    return L


def lib():
    """The loaded library; raises if it has not been built (python -m long_context_tree_amd.build)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def debug_lib():
    """The SPEC_DEBUG build (device-side precondition checks and acceptance witnesses in the debug record
    at the end of each workspace); the same argument structs as lib()."""
    global _debug_lib
    if _debug_lib is None:
        _debug_lib = _load(DEBUG_LIB_PATH)
    return _debug_lib


def debug_record(workspace: torch.Tensor, workspace_size: int):
    """The four uint32 words of the debug record of a call whose workspace (uint8 tensor) had
    workspace_size bytes required: (error bits, rows witnessed, drafts tested, 0)."""
    w = workspace[workspace_size - DEBUG_RECORD_BYTES:workspace_size - DEBUG_RECORD_BYTES + 16]
    return [int(x) & 0xFFFFFFFF for x in w.view(torch.int32).cpu().tolist()]


def debug_bits_names(bits: int):
    return sorted(k for k, v in DBG_BITS.items() if bits & v)



def status_string(status: int) -> str:
    return lib().spec_status_string(status).decode()


def last_error() -> str:
    return lib().spec_last_error().decode()


# ---------------------------------------------------------------------------------------------
# C structs (field order and types follow include/spec_verify.h)
# ---------------------------------------------------------------------------------------------

class PagedKV(ctypes.Structure):
    _fields_ = [("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("page_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64), ("token_stride", ctypes.c_int64),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("block_table_stride", ctypes.c_int32),
                ("v_layout", ctypes.c_int32)]


class TreeAttentionArgs(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_nodes", ctypes.c_int32), ("max_ctx_len", ctypes.c_int32),
                ("ctx_lens", ctypes.c_void_p), ("node_offsets", ctypes.c_void_p), ("parents", ctypes.c_void_p),
                ("subtree_end", ctypes.c_void_p),
                ("q", ctypes.c_void_p), ("kv", PagedKV), ("scale", ctypes.c_float), ("out", ctypes.c_void_p),
                ("lse", ctypes.c_void_p), ("chunk_size", ctypes.c_int32), ("split_tiles", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class ChunkSalienceArgs(ctypes.Structure):
    _fields_ = [("attn", ctypes.POINTER(TreeAttentionArgs)), ("chunk_mass", ctypes.c_void_p),
                ("max_chunks", ctypes.c_int32), ("accumulate", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("topk_index", ctypes.c_void_p), ("topk_mass", ctypes.c_void_p)]


class AcceptGreedyArgs(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("vocab", ctypes.c_int32), ("max_nodes", ctypes.c_int32),
                ("max_path", ctypes.c_int32), ("node_offsets", ctypes.c_void_p), ("parents", ctypes.c_void_p),
                ("draft_tokens", ctypes.c_void_p), ("target_logits", ctypes.c_void_p),
                ("logits_dtype", ctypes.c_int32), ("out_num_accepted", ctypes.c_void_p),
                ("out_path_nodes", ctypes.c_void_p), ("out_tokens", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class KvCommitArgs(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_layers", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_nodes", ctypes.c_int32), ("max_path", ctypes.c_int32),
                ("k_caches", ctypes.POINTER(ctypes.c_void_p)), ("v_caches", ctypes.POINTER(ctypes.c_void_p)),
                ("page_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64), ("token_stride", ctypes.c_int64),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("block_table_stride", ctypes.c_int32),
                ("v_layout", ctypes.c_int32),
                ("ctx_lens", ctypes.c_void_p), ("num_accepted", ctypes.c_void_p), ("path_nodes", ctypes.c_void_p),
                ("new_ctx_lens", ctypes.c_void_p)]


class DraftGatherArgs(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_ctx_len", ctypes.c_int32), ("ctx_lens", ctypes.c_void_p), ("kv", PagedKV),
                ("chunk_size", ctypes.c_int32), ("window", ctypes.c_int32), ("num_select", ctypes.c_int32),
                ("chunk_index", ctypes.c_void_p), ("chunk_index_stride", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("rope", ctypes.c_int32), ("inv_freq", ctypes.c_void_p),
                ("out_k", ctypes.c_void_p), ("out_v", ctypes.c_void_p), ("out_pos", ctypes.c_void_p),
                ("out_len", ctypes.c_void_p)]


class DepthControllerState(ctypes.Structure):
    _fields_ = [("alpha", ctypes.c_double), ("cost_ratio", ctypes.c_double), ("alpha_decay", ctypes.c_double),
                ("cost_decay", ctypes.c_double), ("k_max", ctypes.c_int32), ("k", ctypes.c_int32),
                ("rounds", ctypes.c_int64)]


class AcceptRejectionArgs(ctypes.Structure):
    _fields_ = [("base", AcceptGreedyArgs), ("max_children", ctypes.c_int32), ("draft_probs", ctypes.c_void_p),
                ("u_accept", ctypes.c_void_p), ("u_sample", ctypes.c_void_p)]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int, func: str):
    if status != SPEC_OK:
        raise SpecError(status, func, last_error())


def _need(t: torch.Tensor, name: str, dtype, contiguous=True):
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    if workspace is not None and workspace.numel() * workspace.element_size() >= nbytes:
        return workspace
    # 256 extra bytes so the start can be aligned to 256 bytes
    buf = torch.empty(max(nbytes, 1) + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + max(nbytes, 1)]


# ---------------------------------------------------------------------------------------------
# spec_tree_attention
# ---------------------------------------------------------------------------------------------

class AttentionHandle:
    """The argument struct (and the workspace it points to) of one spec_tree_attention call, as
    spec_chunk_salience needs it."""

    def __init__(self, args: TreeAttentionArgs, keep):
        self.args = args
        self._keep = keep


def _check_kv_layout(k_cache, v_cache, v_layout):
    _need(k_cache, "k_cache", torch.bfloat16, contiguous=False)
    _need(v_cache, "v_cache", torch.bfloat16, contiguous=False)
    if k_cache.stride(3) != 1:
        raise ValueError("k_cache: the head_dim stride must be 1")
    if v_layout == V_TOKEN_ROWS:
        if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
            raise ValueError("k_cache and v_cache must have the same shape and strides")
    elif v_layout == V_DIM_MAJOR:
        P, H, S, D_ = k_cache.shape
        if tuple(v_cache.shape) != (P, H, D_, S) or v_cache.stride()[:2] != k_cache.stride()[:2] \
                or v_cache.stride(2) != S or v_cache.stride(3) != 1:
            raise ValueError("dim-major v_cache must be [pages][kv_heads][head_dim][page_size] with k_cache's page "
                             "and head strides and contiguous pages")
    else:
        raise ValueError(f"v_layout {v_layout}: expected V_TOKEN_ROWS or V_DIM_MAJOR")


def _fill_kv(kv: PagedKV, k_cache, v_cache, block_table, v_layout):
    kv.k_cache, kv.v_cache = _ptr(k_cache), _ptr(v_cache)
    kv.page_stride, kv.head_stride, kv.token_stride = k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)
    kv.page_size = k_cache.shape[2]
    kv.num_pages = k_cache.shape[0]
    kv.block_table = _ptr(block_table)
    kv.block_table_stride = block_table.shape[1]
    kv.v_layout = v_layout


def tree_attention_args(q, k_cache, v_cache, block_table, ctx_lens, node_offsets, parents, *, max_nodes: int,
                        max_ctx_len: int, scale: Optional[float] = None, chunk_size: int = 0, split_tiles: int = 0,
                        out=None, lse=None, workspace=None, v_layout: int = V_TOKEN_ROWS,
                        subtree_end=None) -> TreeAttentionArgs:
    """Fill the C argument struct from tensors (no launch).  k_cache is bf16 [pages][kv_heads][page_size]
    [head_dim] with unit stride in the last dimension; v_cache has the same shape and strides
    (V_TOKEN_ROWS) or is [pages][kv_heads][head_dim][page_size] with K's page and head strides
    (V_DIM_MAJOR)."""
    a = TreeAttentionArgs()
    T, Hq, D = q.shape
    a.batch = ctx_lens.numel()
    a.num_q_heads = Hq
    a.num_kv_heads = k_cache.shape[1]
    a.head_dim = D
    a.max_nodes = max_nodes
    a.max_ctx_len = max_ctx_len
    a.ctx_lens, a.node_offsets, a.parents = _ptr(ctx_lens), _ptr(node_offsets), _ptr(parents)
    a.subtree_end = _ptr(subtree_end)
    a.q = _ptr(q)
    _fill_kv(a.kv, k_cache, v_cache, block_table, v_layout)
    a.scale = (1.0 / math.sqrt(D)) if scale is None else scale
    a.out = _ptr(out)
    a.lse = _ptr(lse)
    a.chunk_size = chunk_size
    a.split_tiles = split_tiles
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return a


def tree_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                   ctx_lens: torch.Tensor, node_offsets: torch.Tensor, parents: torch.Tensor, *, max_nodes: int,
                   max_ctx_len: int, scale: Optional[float] = None, chunk_size: int = 0, split_tiles: int = 0,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                   workspace: Optional[torch.Tensor] = None, stream=None, v_layout: int = V_TOKEN_ROWS,
                   subtree_end: Optional[torch.Tensor] = None):
    """Tree-masked attention of every draft-tree node over the paged KV cache.  With subtree_end
    (int32 [T], sequence-local; trees in preorder, e.g. from tree_bundle_order) the ancestors come
    from index ranges and trees may have up to MAX_TREE_NODES nodes; parents may then be None.

    Returns (out bf16 [T][Hq][D], lse fp32 [T][Hq] or None, handle for spec_chunk_salience)."""
    _need(q, "q", torch.bfloat16)
    for name, t in (("ctx_lens", ctx_lens), ("node_offsets", node_offsets), ("parents", parents),
                    ("block_table", block_table), ("subtree_end", subtree_end)):
        if t is not None or name not in ("parents", "subtree_end"):
            _need(t, name, torch.int32)
    _check_kv_layout(k_cache, v_cache, v_layout)
    T, Hq, D = q.shape
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    a = tree_attention_args(q, k_cache, v_cache, block_table, ctx_lens, node_offsets, parents, max_nodes=max_nodes,
                            max_ctx_len=max_ctx_len, scale=scale, chunk_size=chunk_size, split_tiles=split_tiles,
                            out=out, lse=lse, v_layout=v_layout, subtree_end=subtree_end)
    need = lib().spec_tree_attention_workspace_size(ctypes.byref(a))
    if need == 0:
        _check(lib().spec_tree_attention(ctypes.byref(a), None), "spec_tree_attention")
    ws = _workspace(need, q.device, workspace)
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    _check(lib().spec_tree_attention(ctypes.byref(a), _stream(stream)), "spec_tree_attention")
    return out, lse, AttentionHandle(a, (q, k_cache, v_cache, block_table, ctx_lens, node_offsets, parents, out, lse,
                                         ws, subtree_end))


def tree_attention_workspace_size(**kw) -> int:
    """Workspace bytes for the given host bounds (fields of spec_tree_attention_args)."""
    a = TreeAttentionArgs()
    for k, v in kw.items():
        if k.startswith("kv_"):
            setattr(a.kv, k[3:], v)
        else:
            setattr(a, k, v)
    return lib().spec_tree_attention_workspace_size(ctypes.byref(a))


# ---------------------------------------------------------------------------------------------
# spec_chunk_salience
# ---------------------------------------------------------------------------------------------

def chunk_salience(handle: AttentionHandle, chunk_mass: torch.Tensor, *, accumulate: bool = False, top_k: int = 0,
                   topk_index: Optional[torch.Tensor] = None, topk_mass: Optional[torch.Tensor] = None, stream=None):
    """Per-chunk attention mass of the attention call behind ``handle`` (fp32 [batch][max_chunks],
    written or accumulated in place), and optionally the top_k chunks.  Returns (chunk_mass,
    topk_index, topk_mass)."""
    _need(chunk_mass, "chunk_mass", torch.float32)
    B = handle.args.batch
    if top_k > 0:
        if topk_index is None:
            topk_index = torch.empty((B, top_k), dtype=torch.int32, device=chunk_mass.device)
        if topk_mass is None:
            topk_mass = torch.empty((B, top_k), dtype=torch.float32, device=chunk_mass.device)
    s = ChunkSalienceArgs()
    s.attn = ctypes.pointer(handle.args)
    s.chunk_mass = _ptr(chunk_mass)
    s.max_chunks = chunk_mass.shape[1]
    s.accumulate = int(accumulate)
    s.top_k = top_k
    s.topk_index = _ptr(topk_index)
    s.topk_mass = _ptr(topk_mass)
    _check(lib().spec_chunk_salience(ctypes.byref(s), _stream(stream)), "spec_chunk_salience")
    return chunk_mass, topk_index, topk_mass


# ---------------------------------------------------------------------------------------------
# spec_accept_greedy / spec_accept_rejection
# ---------------------------------------------------------------------------------------------

def _greedy_args(node_offsets, parents, draft_tokens, logits, max_nodes, max_path, outs) -> AcceptGreedyArgs:
    for name, t in (("node_offsets", node_offsets), ("parents", parents), ("draft_tokens", draft_tokens)):
        _need(t, name, torch.int32)
    if logits.dtype not in (torch.bfloat16, torch.float32) or not logits.is_contiguous():
        raise TypeError("target_logits: contiguous bf16 or fp32 [total_nodes][vocab]")
    a = AcceptGreedyArgs()
    a.batch = node_offsets.numel() - 1
    a.vocab = logits.shape[1]
    a.max_nodes = max_nodes
    a.max_path = max_path
    a.node_offsets, a.parents, a.draft_tokens = _ptr(node_offsets), _ptr(parents), _ptr(draft_tokens)
    a.target_logits = _ptr(logits)
    a.logits_dtype = SPEC_DTYPE_BF16 if logits.dtype == torch.bfloat16 else SPEC_DTYPE_F32
    a.out_num_accepted, a.out_path_nodes, a.out_tokens = (_ptr(t) for t in outs)
    return a


def _outs(batch, max_path, device):
    return (torch.empty(batch, dtype=torch.int32, device=device),
            torch.empty((batch, max_path), dtype=torch.int32, device=device),
            torch.empty((batch, max_path), dtype=torch.int32, device=device))


def accept_greedy(node_offsets, parents, draft_tokens, target_logits, *, max_nodes: int, max_path: int,
                  workspace=None, outs=None, stream=None):
    """Greedy longest-accepted-path acceptance.  Returns (num_accepted [B], path_nodes [B][max_path],
    tokens [B][max_path])."""
    B = node_offsets.numel() - 1
    outs = outs or _outs(B, max_path, target_logits.device)
    a = _greedy_args(node_offsets, parents, draft_tokens, target_logits, max_nodes, max_path, outs)
    need = lib().spec_accept_greedy_workspace_size(ctypes.byref(a))
    if need == 0:
        _check(lib().spec_accept_greedy(ctypes.byref(a), None), "spec_accept_greedy")
    ws = _workspace(need, target_logits.device, workspace)
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    _check(lib().spec_accept_greedy(ctypes.byref(a), _stream(stream)), "spec_accept_greedy")
    return outs


def accept_greedy_noalloc(node_offsets, parents, draft_tokens, target_logits, *, max_nodes: int, max_path: int,
                          outs=None, stream=None):
    """accept_greedy with the library's own per-GPU device array in place of a workspace (no allocation in
    the call; refused when the keys need more than GREEDY_NOALLOC_SCRATCH_BYTES).  Returns as accept_greedy."""
    B = node_offsets.numel() - 1
    outs = outs or _outs(B, max_path, target_logits.device)
    a = _greedy_args(node_offsets, parents, draft_tokens, target_logits, max_nodes, max_path, outs)
    _check(lib().spec_accept_greedy_noalloc(ctypes.byref(a), _stream(stream)), "spec_accept_greedy_noalloc")
    return outs


def accept_rejection(node_offsets, parents, draft_tokens, target_logits, draft_probs, u_accept, u_sample, *,
                     max_nodes: int, max_path: int, max_children: int, workspace=None, outs=None, stream=None):
    """Rejection-sampling acceptance (recursive residual over siblings).  Returns as accept_greedy."""
    for name, t in (("draft_probs", draft_probs), ("u_accept", u_accept), ("u_sample", u_sample)):
        _need(t, name, torch.float32)
    B = node_offsets.numel() - 1
    outs = outs or _outs(B, max_path, target_logits.device)
    r = AcceptRejectionArgs()
    r.base = _greedy_args(node_offsets, parents, draft_tokens, target_logits, max_nodes, max_path, outs)
    r.max_children = max_children
    r.draft_probs, r.u_accept, r.u_sample = _ptr(draft_probs), _ptr(u_accept), _ptr(u_sample)
    need = lib().spec_accept_rejection_workspace_size(ctypes.byref(r))
    if need == 0:
        _check(lib().spec_accept_rejection(ctypes.byref(r), None), "spec_accept_rejection")
    ws = _workspace(need, target_logits.device, workspace)
    r.base.workspace, r.base.workspace_bytes = ws.data_ptr(), ws.numel()
    _check(lib().spec_accept_rejection(ctypes.byref(r), _stream(stream)), "spec_accept_rejection")
    return outs


def kv_commit_args(k_caches, v_caches, block_table, ctx_lens, num_accepted, path_nodes, *, max_nodes: int,
                   new_ctx_lens, v_layout: int = V_TOKEN_ROWS):
    """Fill the C argument struct (no launch).  k_caches / v_caches: one tensor per layer, laid out as
    for tree_attention (all layers share the strides).  Returns (args, objects to keep alive)."""
    n_layers = len(k_caches)
    kp = (ctypes.c_void_p * n_layers)(*[t.data_ptr() for t in k_caches])
    vp = (ctypes.c_void_p * n_layers)(*[t.data_ptr() for t in v_caches])
    k0 = k_caches[0]
    a = KvCommitArgs()
    a.batch = ctx_lens.numel()
    a.num_layers = n_layers
    a.num_kv_heads = k0.shape[1]
    a.head_dim = k0.shape[3]
    a.max_nodes = max_nodes
    a.max_path = path_nodes.shape[1]
    a.k_caches = ctypes.cast(kp, ctypes.POINTER(ctypes.c_void_p))
    a.v_caches = ctypes.cast(vp, ctypes.POINTER(ctypes.c_void_p))
    a.page_stride, a.head_stride, a.token_stride = k0.stride(0), k0.stride(1), k0.stride(2)
    a.page_size = k0.shape[2]
    a.num_pages = k0.shape[0]
    a.block_table = _ptr(block_table)
    a.block_table_stride = block_table.shape[1]
    a.v_layout = v_layout
    a.ctx_lens, a.num_accepted, a.path_nodes = _ptr(ctx_lens), _ptr(num_accepted), _ptr(path_nodes)
    a.new_ctx_lens = _ptr(new_ctx_lens)
    return a, (kp, vp)


def kv_commit(k_caches, v_caches, block_table, ctx_lens, num_accepted, path_nodes, *, max_nodes: int,
              v_layout: int = V_TOKEN_ROWS, new_ctx_lens=None, stream=None):
    """Move each sequence's accepted path (path_nodes / num_accepted from accept_greedy or
    accept_rejection) next to its committed context in every layer's cache, in place, and return the
    new lengths (int32 [batch]; pass new_ctx_lens=ctx_lens to update in place)."""
    for name, t in (("block_table", block_table), ("ctx_lens", ctx_lens), ("num_accepted", num_accepted),
                    ("path_nodes", path_nodes)):
        _need(t, name, torch.int32)
    if len(k_caches) != len(v_caches) or not k_caches:
        raise ValueError("k_caches and v_caches: one tensor per layer, the same number of each")
    for t in list(k_caches) + list(v_caches):
        _need(t, "k_caches / v_caches", torch.bfloat16, contiguous=False)
    k0 = k_caches[0]
    for t in k_caches:
        if t.shape != k0.shape or t.stride() != k0.stride():
            raise ValueError("every layer's k cache must have the same shape and strides")
    for t in v_caches:
        if v_layout == V_TOKEN_ROWS and (t.shape != k0.shape or t.stride() != k0.stride()):
            raise ValueError("token-row v caches must have k's shape and strides")
        if v_layout == V_DIM_MAJOR:
            P, H, S, D_ = k0.shape
            if tuple(t.shape) != (P, H, D_, S) or t.stride()[:2] != k0.stride()[:2] or t.stride(2) != S \
                    or t.stride(3) != 1:
                raise ValueError("dim-major v caches must be [pages][kv_heads][head_dim][page_size] with k's page "
                                 "and head strides")
    if new_ctx_lens is None:
        new_ctx_lens = torch.empty_like(ctx_lens)
    a, keep = kv_commit_args(k_caches, v_caches, block_table, ctx_lens, num_accepted, path_nodes,
                             max_nodes=max_nodes, new_ctx_lens=new_ctx_lens, v_layout=v_layout)
    _check(lib().spec_kv_commit(ctypes.byref(a), _stream(stream)), "spec_kv_commit")
    del keep
    return new_ctx_lens


class DepthController:
    """The host-side draft-depth controller of the library (spec_controller_*): keeps the online
    acceptance rate and cost ratio and proposes the next depth ``k``."""

    def __init__(self, k_max: int, alpha0: float = 0.7, cost_ratio0: float = 0.1, alpha_decay: float = 0.02,
                 cost_decay: float = 0.1, ctx_len: int = 0, long_ctx_threshold: int = 0, long_ctx_depth: int = 2):
        self.state = DepthControllerState()
        _check(lib().spec_controller_init(ctypes.byref(self.state), k_max, alpha0, cost_ratio0, alpha_decay,
                                          cost_decay, ctx_len, long_ctx_threshold, long_ctx_depth),
               "spec_controller_init")

    @property
    def k(self) -> int:
        return self.state.k

    @property
    def alpha(self) -> float:
        return self.state.alpha

    @property
    def cost_ratio(self) -> float:
        return self.state.cost_ratio

    def update(self, drafted: int, accepted: int, t_draft: float, t_target: float) -> int:
        _check(lib().spec_controller_update(ctypes.byref(self.state), drafted, accepted, t_draft, t_target),
               "spec_controller_update")
        return self.state.k


def controller_speedup(alpha: float, cost_ratio: float, k: int) -> float:
    return lib().spec_controller_speedup(alpha, cost_ratio, k)


def controller_choose(alpha: float, cost_ratio: float, k_max: int) -> int:
    return lib().spec_controller_choose(alpha, cost_ratio, k_max)


def draft_gather_args(k_cache, v_cache, block_table, ctx_lens, chunk_index, *, max_ctx_len: int, chunk_size: int,
                      window: int, capacity: int, num_select: Optional[int] = None, rope: int = ROPE_HALF,
                      inv_freq=None, out_k=None, out_v=None, out_pos=None, out_len=None,
                      v_layout: int = V_TOKEN_ROWS) -> DraftGatherArgs:
    """Fill the C argument struct (no launch).  chunk_index: int32 [batch][stride] (or None); its first
    num_select columns are read (all of them by default)."""
    a = DraftGatherArgs()
    a.batch = ctx_lens.numel()
    a.num_kv_heads = k_cache.shape[1]
    a.head_dim = k_cache.shape[3]
    a.max_ctx_len = max_ctx_len
    a.ctx_lens = _ptr(ctx_lens)
    _fill_kv(a.kv, k_cache, v_cache, block_table, v_layout)
    a.chunk_size, a.window, a.capacity, a.rope = chunk_size, window, capacity, rope
    if chunk_index is None:
        a.num_select, a.chunk_index, a.chunk_index_stride = 0, None, 0
    else:
        a.num_select = chunk_index.shape[1] if num_select is None else num_select
        a.chunk_index, a.chunk_index_stride = _ptr(chunk_index), chunk_index.stride(0)
    a.inv_freq = _ptr(inv_freq)
    a.out_k, a.out_v, a.out_pos, a.out_len = _ptr(out_k), _ptr(out_v), _ptr(out_pos), _ptr(out_len)
    return a


def draft_gather(k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor, ctx_lens: torch.Tensor,
                 chunk_index: Optional[torch.Tensor], *, max_ctx_len: int, chunk_size: int, window: int,
                 capacity: int, num_select: Optional[int] = None, rope: int = ROPE_HALF,
                 inv_freq: Optional[torch.Tensor] = None, out_k=None, out_v=None, out_pos=None, out_len=None,
                 v_layout: int = V_TOKEN_ROWS, stream=None):
    """The compact draft KV of each sequence: its selected chunks (chunk_index rows, e.g. the top-k
    output of chunk_salience) and its last ``window`` tokens, in context order, K rotated at local
    positions.  k_cache / v_cache: the canonical pre-RoPE draft cache, laid out as for tree_attention.

    Returns (out_k, out_v bf16 [batch][capacity][kv_heads][head_dim], out_pos int32 [batch][capacity],
    out_len int32 [batch]); K/V slots at or past out_len are not written."""
    _check_kv_layout(k_cache, v_cache, v_layout)
    _need(block_table, "block_table", torch.int32)
    _need(ctx_lens, "ctx_lens", torch.int32)
    if chunk_index is not None:
        _need(chunk_index, "chunk_index", torch.int32, contiguous=False)
        if chunk_index.dim() != 2 or chunk_index.stride(1) != 1:
            raise ValueError("chunk_index: int32 [batch][stride] with unit column stride")
    if inv_freq is not None:
        _need(inv_freq, "inv_freq", torch.float32)
    B, H, D = ctx_lens.numel(), k_cache.shape[1], k_cache.shape[3]
    dev = k_cache.device
    if out_k is None:
        out_k = torch.empty((B, capacity, H, D), dtype=torch.bfloat16, device=dev)
    if out_v is None:
        out_v = torch.empty((B, capacity, H, D), dtype=torch.bfloat16, device=dev)
    if out_pos is None:
        out_pos = torch.empty((B, capacity), dtype=torch.int32, device=dev)
    if out_len is None:
        out_len = torch.empty((B,), dtype=torch.int32, device=dev)
    for name, t, dt in (("out_k", out_k, torch.bfloat16), ("out_v", out_v, torch.bfloat16),
                        ("out_pos", out_pos, torch.int32), ("out_len", out_len, torch.int32)):
        _need(t, name, dt)
    if tuple(out_k.shape) != (B, capacity, H, D) or tuple(out_v.shape) != (B, capacity, H, D):
        raise ValueError("out_k / out_v: bf16 [batch][capacity][kv_heads][head_dim]")
    a = draft_gather_args(k_cache, v_cache, block_table, ctx_lens, chunk_index, max_ctx_len=max_ctx_len,
                          chunk_size=chunk_size, window=window, capacity=capacity, num_select=num_select, rope=rope,
                          inv_freq=inv_freq, out_k=out_k, out_v=out_v, out_pos=out_pos, out_len=out_len,
                          v_layout=v_layout)
    _check(lib().spec_draft_gather(ctypes.byref(a), _stream(stream)), "spec_draft_gather")
    return out_k, out_v, out_pos, out_len


def tree_bundle_order(parents):
    """Bundle (preorder) order of one draft tree, computed by the library on the host.

    parents: sequence-local int array (parents[0] = -1, 0 <= parents[i] < i).  Returns numpy int32
    arrays (order, new_parents, subtree_end, bundle) in the new numbering; see spec_tree_bundle_order."""
    import numpy as np
    par = np.ascontiguousarray(np.asarray(parents, dtype=np.int32))
    n = len(par)
    outs = [np.empty(n, dtype=np.int32) for _ in range(4)]
    st = lib().spec_tree_bundle_order(par.ctypes.data, n, *[o.ctypes.data for o in outs])
    _check(st, "spec_tree_bundle_order")
    return tuple(outs)


READ_PROBE_SINK_WORDS = 2049


def read_probe(data: torch.Tensor, sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Streaming-read probe (a measurement helper): reads every byte of ``data`` (contiguous, 16-byte aligned,
    a multiple of 16 bytes) with 16-byte loads; returns the int32 sink whose element 0 is the XOR of all the
    buffer's 32-bit words."""
    if not data.is_contiguous():
        raise ValueError("data: must be contiguous")
    if sink is None:
        sink = torch.empty(READ_PROBE_SINK_WORDS, dtype=torch.int32, device=data.device)
    _check(lib().spec_read_probe(data.data_ptr(), data.numel() * data.element_size(), sink.data_ptr(),
                                 _stream(stream)), "spec_read_probe")
    return sink
