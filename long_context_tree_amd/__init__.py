"""Tree verification for speculative decoding on AMD Instinct MI355X (gfx950).

A thin Python binding over libspec_verify (include/spec_verify.h): tree-masked paged attention,
per-chunk attention mass with top-k selection, greedy / rejection-sampling acceptance, the commit of
the accepted path into the paged cache, the compact draft KV gathered from the selected chunks, the
bundle (preorder) order of a draft tree, and the draft-depth controller.
"""

from .spec import (ROPE_HALF, ROPE_NONE, ROPE_PAIRS, V_DIM_MAJOR, V_TOKEN_ROWS, AttentionHandle, DepthController,
                   SpecError, accept_greedy, accept_greedy_noalloc, accept_rejection, chunk_salience, controller_choose, controller_speedup,
                   draft_gather, kv_commit, last_error, lib, read_probe, status_string, tree_attention,
                   tree_attention_args, tree_bundle_order)

__all__ = ["ROPE_HALF", "ROPE_NONE", "ROPE_PAIRS", "V_DIM_MAJOR", "V_TOKEN_ROWS", "AttentionHandle",
           "DepthController", "SpecError", "accept_greedy", "accept_greedy_noalloc", "accept_rejection", "chunk_salience", "controller_choose",
           "controller_speedup", "draft_gather", "kv_commit", "last_error", "lib", "read_probe", "status_string",
           "tree_attention", "tree_attention_args", "tree_bundle_order"]
