"""CPU oracle for the verification step of tree speculative decoding.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or run anything in this package; the
library never does, and it shares no code, table or helper with the GPU path.

It is plain numpy in float64, written from the defining passages of the pages
and kept slow and obvious on purpose: masked softmax attention of every
draft-tree node over the paged context plus its own ancestors, the per-chunk
attention mass, greedy longest-accepted-path acceptance, the
recursive-residual rejection walk, the commit of the accepted path into
the paged cache, the compact draft KV built from the selected chunks and the
recent window, the bundle (preorder) order of a draft tree, and the
closed-form draft-depth controller.  Each function cites the passage it follows.

Every function here is pinned by tests against something other than itself
(closed forms, library routines, brute force on tiny inputs, exact
enumeration of the sampler's output law).  None is "parity unpinned".
"""

from .attention import bf16_to_f64, ancestor_matrix, gather_kv, tree_attention, topk_chunks
from .acceptance import argmax_lowest, accept_greedy, target_probs, accept_rejection
from .kvcache import kv_commit
from .draft_kv import draft_gather
from .bundle import bundle_order
from . import controller, draft_kv

__all__ = ["bf16_to_f64", "ancestor_matrix", "gather_kv", "tree_attention", "topk_chunks", "argmax_lowest",
           "accept_greedy", "target_probs", "accept_rejection", "kv_commit", "draft_gather", "draft_kv",
           "bundle_order", "controller"]
