"""Oracle: the draft-depth controller.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Adaptive Speculative Decoding", section "The controller": with per-token acceptance rate a,
a round that drafts k tokens yields (1 - a^(k+1)) / (1 - a) tokens in expectation and costs
(k + 1) * c + 1 target forwards (c = t_draft / t_target; the extra draft forward commits the last
draft into the draft cache); the controller maximises the ratio over k in [1, k_max], with a and c
measured online, the acceptance estimate decayed per token.  The DiffSpec plugin's "Configuration"
(long-context threshold, initial depth) and "Architecture" (adaptive verification starts long
contexts shallow) give the starting depth of long sequences.
Readings: ties go to the smaller k; a round contributes its accepted drafts as 1s and its first
rejected draft as a 0 (the drafts after it were never tested); c is a per-round weighted mean.
"""

from __future__ import annotations


def expected_tokens(alpha: float, k: int) -> float:
    """(1 - a^(k+1)) / (1 - a); k + 1 at a = 1."""
    if alpha == 1.0:
        return float(k + 1)
    return (1.0 - alpha ** (k + 1)) / (1.0 - alpha)


def speedup(alpha: float, cost_ratio: float, k: int) -> float:
    return expected_tokens(alpha, k) / ((k + 1) * cost_ratio + 1.0)


def choose(alpha: float, cost_ratio: float, k_max: int) -> int:
    best, best_v = 1, speedup(alpha, cost_ratio, 1)
    for k in range(2, k_max + 1):
        v = speedup(alpha, cost_ratio, k)
        if v > best_v:
            best, best_v = k, v
    return best


class Controller:
    def __init__(self, k_max, alpha0, cost_ratio0, alpha_decay, cost_decay, ctx_len=0, long_ctx_threshold=0,
                 long_ctx_depth=2):
        self.k_max, self.alpha, self.cost_ratio = k_max, alpha0, cost_ratio0
        self.alpha_decay, self.cost_decay = alpha_decay, cost_decay
        if long_ctx_threshold > 0 and ctx_len >= long_ctx_threshold:
            self.k = min(long_ctx_depth, k_max)
        else:
            self.k = choose(alpha0, cost_ratio0, k_max)

    def update(self, drafted, accepted, t_draft, t_target):
        w = self.alpha_decay
        for _ in range(accepted):
            self.alpha = (1.0 - w) * self.alpha + w * 1.0
        if accepted < drafted:
            self.alpha = (1.0 - w) * self.alpha
        if t_draft > 0.0:
            self.cost_ratio = (1.0 - self.cost_decay) * self.cost_ratio + self.cost_decay * (t_draft / t_target)
        self.k = choose(self.alpha, self.cost_ratio, self.k_max)
        return self.k
