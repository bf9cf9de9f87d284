"""Seeded synthetic inputs for tree verification.

This package only draws random inputs and lays them out (bf16 bit patterns,
paged KV pools, block tables, draft trees, logits, uniforms).  It holds none of
the verification arithmetic: no attention, no softmax of target logits, no
argmax, no acceptance walk.  Both the CPU oracle (through the tests) and the
GPU path (through the tests and the benchmark) consume what it produces.
"""

from .inputs import *  # noqa: F401,F403
