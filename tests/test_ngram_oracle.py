"""Pins of the n-gram (prompt-lookup) proposer oracle (no GPU).

The oracle compares the suffix with every window through NumPy. It is pinned to
hand-worked cases of the rule (tests/golden/ngram_cases.txt, with the citation),
to an independent formulation on tiny alphabets (Python's own substring search,
str.rfind, over the context written as text), and to properties any proposal must
have. A planted mistake (the earliest occurrence instead of the latest) must fail
the brute-force pin.
"""
import os

import numpy as np
import pytest

import oracle as O
import oracle.ngram as ON
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ngram_cases.txt")


def _cases():
    out = []
    for line in open(GOLDEN, encoding="utf-8"):
        if line.startswith("#") or not line.strip():
            continue
        name, nn, ctx, exp = (x.strip() for x in line.split("|"))
        n_min, n_max, gamma = map(int, nn.split())
        out.append((name, n_min, n_max, gamma, [int(t) for t in ctx.split()],
                    [] if exp == "-" else [int(t) for t in exp.split()]))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c[0])
def test_hand_worked_cases(case):
    _, n_min, n_max, gamma, ctx, expected = case
    assert list(O.ngram_propose(ctx, n_min, n_max, gamma)) == expected


def _by_rfind(ctx, n_min, n_max, gamma):
    """The rule through str.rfind: tokens as characters, the haystack is the context
    without its last token (an occurrence must end before it)."""
    s = "".join(chr(0x4E00 + int(t)) for t in ctx)
    L = len(s)
    if gamma <= 0 or L < 2:
        return []
    for n in range(min(n_max, L - 1), n_min - 1, -1):
        j = s[:L - 1].rfind(s[L - n:])
        if j >= 0:
            return [ord(ch) - 0x4E00 for ch in s[j + n:j + n + gamma]]
    return []


def test_matches_substring_search_on_small_alphabets():
    rng = np.random.default_rng(11)
    n = 0
    for _ in range(3000):
        L = int(rng.integers(0, 40))
        alpha = int(rng.integers(1, 6))
        ctx = rng.integers(0, alpha, L)
        n_min = int(rng.integers(1, 4))
        n_max = n_min + int(rng.integers(0, 5))
        gamma = int(rng.integers(0, 7))
        got = list(O.ngram_propose(ctx, n_min, n_max, gamma))
        assert got == _by_rfind(ctx, n_min, n_max, gamma), (ctx.tolist(), n_min, n_max, gamma)
        n += bool(got)
    assert n > 1000  # most cases propose something


def test_properties_on_copy_heavy_contexts():
    """A proposal continues an earlier occurrence of the longest matching suffix, and no
    longer suffix within n_max occurs earlier."""
    ctx = synth.make_ngram_contexts(24, (50, 3000), 5000, seed=3)
    for b in range(ctx.B):
        c = ctx.context(b)
        L = c.size
        p = O.ngram_propose(c, 2, 6, 5)
        if p.size == 0:
            continue
        assert 1 <= p.size <= 5
        # the winning n: the largest n with an earlier occurrence whose continuation is p
        found = False
        for n in range(min(6, L - 1), 1, -1):
            wins = np.lib.stride_tricks.sliding_window_view(c[:L - 1], n)
            hits = np.flatnonzero(np.all(wins == c[L - n:], axis=1))
            if hits.size:
                j = hits[-1]
                assert np.array_equal(c[j + n:j + n + p.size], p)
                assert p.size == min(5, L - j - n)
                found = True
                break
        assert found


def test_batch_layout():
    ctx = synth.make_ngram_contexts(9, (0, 200), 50, seed=4)
    ids, lens = O.ngram_propose_batch(ctx.tokens, ctx.cu_ctx, 1, 4, 3)
    assert ids.shape == (9, 3) and lens.shape == (9,)
    for b in range(9):
        p = O.ngram_propose(ctx.context(b), 1, 4, 3)
        assert lens[b] == p.size and list(ids[b, :p.size]) == list(p)
        assert np.all(ids[b, p.size:] == -1)


def test_planted_mistake_is_caught(monkeypatch):
    """The earliest occurrence instead of the latest must fail the substring pin."""
    def earliest(context, n_min, n_max, gamma):
        c = np.asarray(context, dtype=np.int64).reshape(-1)
        L = c.size
        if gamma <= 0 or L < 2:
            return np.zeros(0, dtype=np.int64)
        for n in range(min(n_max, L - 1), n_min - 1, -1):
            w = np.lib.stride_tricks.sliding_window_view(c[:L - 1], n)
            hits = np.flatnonzero(np.all(w == c[L - n:], axis=1))
            if hits.size:
                j = int(hits[0])
                return c[j + n:j + n + gamma].copy()
        return np.zeros(0, dtype=np.int64)

    monkeypatch.setattr(ON, "ngram_propose", earliest)
    rng = np.random.default_rng(12)
    diffs = 0
    for _ in range(300):
        ctx = rng.integers(0, 3, int(rng.integers(5, 40)))
        diffs += list(ON.ngram_propose(ctx, 1, 3, 4)) != _by_rfind(ctx, 1, 3, 4)
    assert diffs > 30
