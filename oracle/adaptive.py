"""CPU oracle for the adaptive draft-length (gamma) controller.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or load
this module: only the tests, the smoke check and the benchmark's CPU-baseline leg
use it. It shares no code with the HIP library.

What it computes, from the pages:
  [P4] "투기적 디코딩 — 초안 모델을 무엇으로 세울 것인가", ailab.paldyn.com, "도입할 때
       순서대로 확인할 것" (second point): do not fix the draft length; look at the
       acceptance results of the last few steps and move it up or down; after
       rejections in a row bring it down to 1, raise it again while acceptances
       continue.
  [P1] "Speculative Decoding", atonlee.tistory.com/330, ch.4 (after the speedup table):
       the best gamma depends on the acceptance rate, which is why implementations
       adjust it as they go.

Readings where the pages leave the rule open (also listed in the design notes):
  * The unit is a round (a step) of one sequence. A round "accepts" when every draft
    was accepted (n_b == gamma_b, the bonus round: a run of gamma_b acceptances) and
    "rejects" when its first draft was rejected (n_b == 0). A round that accepted some
    drafts and then rejected one is neither: it breaks both runs.
  * State per sequence: gamma_b in [0, gamma_max] and a streak s_b: s_b > 0 counts the
    fully accepted rounds in a row, s_b < 0 minus the rejecting rounds in a row.
  * After a fully accepted round: s = max(s, 0) + 1; once s reaches up_after, gamma
    goes up by one (at most gamma_max) and s restarts at 0.
  * After a rejecting round: s = min(s, 0) - 1; once -s reaches down_after, gamma is
    cut to 1 and s restarts at 0.
  * After a partly accepted round: s = 0.
  * A round that "rejects" whenever it ends at a rejection would count most rounds of
    long drafts as rejections and cut gamma to 1 even where acceptance is high; that
    loses to a fixed gamma, whereas the page says the simple rule beats a fixed value.
  * A sequence whose round was not run (accepted count -1, a flagged input) keeps its
    state. A gamma outside [0, gamma_max] or a streak outside [-down_after, up_after]
    in the state is first clamped into that range.
  * The next round's packed layout is the exclusive prefix of the new gamma_b.
"""
from __future__ import annotations

import numpy as np

__all__ = ["adapt_gamma", "adapt_gamma_batch"]


def adapt_gamma(gamma: int, streak: int, accepted: int, gamma_max: int, up_after: int,
                down_after: int):
    """One sequence, one round: returns the new (gamma, streak)."""
    g = min(max(int(gamma), 0), gamma_max)
    s = min(max(int(streak), -down_after), up_after)
    n = int(accepted)
    if n < 0:
        return g, s
    if n >= g:     # every draft accepted
        s = max(s, 0) + 1
        if s >= up_after:
            g = min(g + 1, gamma_max)
            s = 0
    elif n == 0:   # the first draft was rejected
        s = min(s, 0) - 1
        if -s >= down_after:
            g = 1
            s = 0
    else:          # some accepted, then a rejection
        s = 0
    return g, s


def adapt_gamma_batch(gammas, streaks, accepted, gamma_max: int, up_after: int, down_after: int):
    """Every sequence of a batch. Returns (gamma int32 [B], streak int32 [B],
    cu_gamma int32 [B+1], the exclusive prefix of the new gammas)."""
    B = len(gammas)
    g = np.empty(B, dtype=np.int32)
    s = np.empty(B, dtype=np.int32)
    for b in range(B):
        g[b], s[b] = adapt_gamma(gammas[b], streaks[b], accepted[b], gamma_max, up_after, down_after)
    cu = np.zeros(B + 1, dtype=np.int64)
    np.cumsum(g, out=cu[1:])
    return g, s, cu.astype(np.int32)
