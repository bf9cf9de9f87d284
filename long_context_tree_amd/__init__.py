"""Tree verification for speculative decoding on AMD Instinct MI355X (gfx950).

A thin Python binding over libspec_verify (include/spec_verify.h): tree-masked paged attention,
per-chunk attention mass with top-k selection, and greedy / rejection-sampling acceptance.
"""

from .spec import (V_DIM_MAJOR, V_TOKEN_ROWS, AttentionHandle, DepthController, SpecError, accept_greedy,
                   accept_rejection, chunk_salience, controller_choose, controller_speedup, kv_commit, last_error, lib,
                   status_string, tree_attention, tree_attention_args)

__all__ = ["V_DIM_MAJOR", "V_TOKEN_ROWS", "AttentionHandle", "DepthController", "SpecError", "accept_greedy",
           "accept_rejection", "chunk_salience", "controller_choose", "controller_speedup", "kv_commit", "last_error",
           "lib", "status_string", "tree_attention", "tree_attention_args"]
