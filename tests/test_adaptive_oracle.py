"""Pins of the adaptive draft-length controller's oracle (no GPU).

The controller is pinned to a hand-worked trace of the rule (tests/golden/
adaptive_trace.txt, with the citation) and to the behaviour the pages ask of it
(always accepting climbs to the cap, always rejecting falls to 1). Rounds driven by
it are pinned to the expected tokens per round of the pages, E = (1 - a^(g+1)) / (1 - a),
taken at each round's own draft length: whatever the controller does, a round with
g drafts and per-position acceptance a yields E tokens on average.
"""
import math
import os

import numpy as np
import pytest

import oracle as O
import synth
from _pool import pmap

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "adaptive_trace.txt")


def test_hand_worked_trace():
    g, s = 3, 0
    n_lines = 0
    for line in open(GOLDEN, encoding="utf-8"):
        if line.startswith("#") or not line.strip():
            continue
        left, right = line.split("->")
        eg, es = map(int, right.split())
        g, s = O.adapt_gamma(g, s, int(left), 5, 2, 2)
        assert (g, s) == (eg, es), line
        n_lines += 1
    assert n_lines >= 20


@pytest.mark.parametrize("up,down,gmax", [(1, 1, 8), (2, 2, 8), (3, 2, 4)])
def test_always_accepting_climbs_always_rejecting_falls(up, down, gmax):
    g, s = 1, 0
    for k in range(up * (gmax - 1)):
        assert g == 1 + k // up
        g, s = O.adapt_gamma(g, s, g, gmax, up, down)
    assert g == gmax
    for _ in range(5):
        g, s = O.adapt_gamma(g, s, g, gmax, up, down)
        assert g == gmax
    for k in range(down):
        assert g == gmax
        g, s = O.adapt_gamma(g, s, 0, gmax, up, down)
    assert (g, s) == (1, 0)


def test_partial_rounds_break_both_runs():
    assert O.adapt_gamma(4, 0, 3, 8, 2, 2) == (4, 0)
    assert O.adapt_gamma(4, -1, 3, 8, 2, 2) == (4, 0)   # no cut: the run of rejections broke
    assert O.adapt_gamma(4, 1, 2, 8, 2, 2) == (4, 0)    # no raise: the run of acceptances broke
    assert O.adapt_gamma(4, 1, 0, 8, 2, 2) == (4, -1)   # a rejection after an accepting round
    assert O.adapt_gamma(4, -1, 0, 8, 2, 2) == (1, 0)


def test_edges():
    assert O.adapt_gamma(5, -1, -1, 8, 2, 2) == (5, -1)      # round not run: unchanged
    assert O.adapt_gamma(0, 0, 0, 8, 1, 1) == (1, 0)          # no drafts counts as accepted
    assert O.adapt_gamma(12, 0, 0, 8, 2, 1) == (1, 0)         # clamped, then cut
    assert O.adapt_gamma(-3, 1, 0, 8, 2, 1) == (1, 0)         # clamped to 0, accepted, raised
    assert O.adapt_gamma(1, 0, 1, 1, 1, 1) == (1, 0)          # cap of 1
    assert O.adapt_gamma(3, 2**31 - 1, -1, 8, 2, 3) == (3, 2)  # streak clamped to [-3, 2]
    assert O.adapt_gamma(3, -2**31, 3, 8, 2, 3) == (3, 1)
    assert O.adapt_gamma(3, -2**31, 0, 8, 2, 3) == (1, 0)
    g, s, cu = O.adapt_gamma_batch([1, 4, 0], [0, 1, 0], [1, 4, -1], 8, 2, 2)
    assert list(g) == [1, 5, 0] and list(s) == [1, 0, 0] and list(cu) == [0, 1, 6, 6]


def _rounds(alpha, rounds, seed, gmax=8, up=1, down=2, V=8):
    """Rounds of one sequence with fixed p, q of overlap alpha under the controller;
    returns arrays (gamma used, tokens emitted)."""
    L, Q = synth.controlled_alpha_rows([alpha], V)
    Lr, Qr = L[0].astype(np.float64), Q[0]
    cq = np.cumsum(Qr.astype(np.float64))
    rng = np.random.default_rng(seed)
    g, s = 4, 0
    gs, toks = [], []
    for _ in range(rounds):
        ids = [min(int(np.searchsorted(cq, rng.random() * cq[-1], side="right")), V - 1) for _ in range(g)]
        res = O.verify_sequence(np.tile(Lr, (g + 1, 1)), np.tile(Qr, (g, 1)), ids, rng.random(g + 1), 1.0,
                                all_p=False)
        gs.append(g)
        toks.append(res.n + 1)
        g, s = O.adapt_gamma(g, s, res.n, gmax, up, down)
    return np.array(gs), np.array(toks)


def test_rounds_under_the_controller_follow_E():
    alphas = [0.2, 0.5, 0.8, 0.95]

    def job(k):
        a = alphas[k % len(alphas)]
        gs, toks = _rounds(a, 4000, seed=[40, k])
        E = np.array([O.expected_tokens_per_round(a, int(g)) for g in gs])
        return a, gs, toks, E

    res = pmap(job, range(16))
    d = np.concatenate([t - E for _, _, t, E in res])
    se = d.std() / math.sqrt(d.size)
    assert abs(d.mean()) < 5 * se, (d.mean(), se)
    mean_g = {a: np.mean(np.concatenate([g for aa, g, _, _ in res if aa == a])) for a in alphas}
    assert mean_g[0.2] < mean_g[0.5] < mean_g[0.8] < mean_g[0.95]
    assert mean_g[0.2] < 1.6 and mean_g[0.95] > 6.0


def test_planted_mistake_fails_the_trace(monkeypatch):
    """A controller that cuts gamma by one instead of to 1 must fail the golden trace."""
    import oracle.adaptive as OA

    def step_down(gamma, streak, accepted, gamma_max, up_after, down_after):
        g, s = min(max(int(gamma), 0), gamma_max), int(streak)
        if accepted < 0:
            return g, s
        if accepted >= g:
            s = max(s, 0) + 1
            if s >= up_after:
                return min(g + 1, gamma_max), 0
            return g, s
        s = min(s, 0) - 1
        if -s >= down_after:
            return max(g - 1, 1), 0
        return g, s

    monkeypatch.setattr(O, "adapt_gamma", step_down)
    monkeypatch.setattr(OA, "adapt_gamma", step_down)
    with pytest.raises(AssertionError):
        test_hand_worked_trace()
