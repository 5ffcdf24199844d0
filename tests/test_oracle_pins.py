"""Pins of the CPU oracle to what the pages and the mathematics fix (no GPU).

Each test ties the oracle to something other than itself: numbers the pages
print (tests/golden, each with its citation), closed forms, the distribution
theorem (chi-square), exact enumeration on tiny inputs, and special cases that
reduce to a library routine. Negative controls plant a mistake in the oracle (on
the CPU) and check that the statistical pins then fail.
"""
import math

import numpy as np
import pytest
from scipy import stats

import oracle as O
import oracle.verify as OV
import synth
from _pool import pmap
from conftest import read_table


# --------------------------------------------------------------------------
# Numbers printed on the pages
# --------------------------------------------------------------------------

def test_expected_tokens_table_matches_pages():
    rows = read_table("expected_tokens_table.txt")
    gammas = (2, 4, 7, 10)
    assert len(rows) == 5
    for row in rows:
        a = float(row[0])
        for g, printed in zip(gammas, row[1:]):
            assert abs(O.expected_tokens_per_round(a, g) - float(printed)) <= 0.005 + 1e-12, (a, g)


def test_speedup_table_matches_pages():
    rows = read_table("speedup_table.txt")
    for row in rows:
        a = float(row[0])
        for g, printed in zip((2, 4, 7, 10), row[1:]):
            assert abs(O.speedup_factor(a, g, 0.05) - float(printed)) <= 0.005 + 1e-12, (a, g)


def test_worked_numbers():
    vals = {r[0]: (float(r[1]), float(r[2])) for r in read_table("worked_numbers.txt")}

    def chk(key, got):
        want, tol = vals[key]
        assert abs(got - want) <= tol, (key, got, want)

    chk("accept_ratio_q0.4_p0.1", O.acceptance_threshold(0.1, 0.4))
    chk("emit_prob_q0.4_p0.1", 0.4 * O.acceptance_threshold(0.1, 0.4))
    chk("E_a0.8_g4", O.expected_tokens_per_round(0.8, 4))
    chk("speedup_a0.8_g4_c0.05", O.speedup_factor(0.8, 4, 0.05))
    chk("E_a0.5_g2", O.expected_tokens_per_round(0.5, 2))
    chk("E_a0.5_g7", O.expected_tokens_per_round(0.5, 7))
    chk("E_a0.9_g7", O.expected_tokens_per_round(0.9, 7))
    chk("denominator_c0.1_k5", 5 * 0.1 + 1)
    chk("speedup_E3.0_c0.1_k5", 3.0 / (5 * 0.1 + 1))
    chk("five_in_a_row_a0.8", 0.8 ** 5)
    # ceiling: E -> 1/(1-alpha) as gamma grows
    chk("ceiling_a0.8", O.expected_tokens_per_round(0.8, 400))
    # exact value behind "about 3.4"
    assert abs(O.expected_tokens_per_round(0.8, 4) - 3.3616) < 1e-12


def test_expected_tokens_closed_form_is_geometric_sum():
    # E = sum_{k=0..gamma} alpha^k (tokens per round = accepted + 1)
    for a in (0.0, 0.3, 0.77, 0.99):
        for g in range(0, 12):
            assert abs(O.expected_tokens_per_round(a, g) - sum(a ** k for k in range(g + 1))) < 1e-12
    assert O.expected_tokens_per_round(1.0, 6) == 7.0


# --------------------------------------------------------------------------
# The worked example, through the oracle's own round
# --------------------------------------------------------------------------

def _worked_inputs():
    p = np.array([0.1, 0.9])
    q = np.array([0.4, 0.6])
    L = np.log(np.vstack([p, p]))  # gamma = 1: judged row + bonus row
    return p, q, L


def test_worked_example_exact_grid():
    p, q, L = _worked_inputs()
    N = 10000
    emit0 = 0.0
    acc0 = 0
    for x, wx in ((0, 0.4), (1, 0.6)):
        for k in range(N):
            r = O.verify_sequence(L, q[None], [x], [(k + 0.5) / N, 0.5], 1.0)
            if x == 0:
                assert abs(r.thresholds[0] - 0.25) < 1e-15
                acc0 += r.n
                if r.n == 0:
                    # residual max(0, p - q) = [0, 0.3]: a rejection always emits 1
                    assert r.tokens == [1] and r.mode == "residual"
                    assert abs(r.S - 0.3) < 1e-15
            else:
                assert r.thresholds[0] == 1.0 and r.n == 1
            emit0 += wx * (r.tokens[0] == 0) / N
    assert acc0 == N // 4
    assert abs(emit0 - 0.1) < 1e-12


def test_worked_example_random_trials():
    p, q, L = _worked_inputs()

    def chunk(seed):
        rng = np.random.default_rng(seed)
        acc = emit0 = n = 0
        for _ in range(25000):
            x = int(rng.random() >= 0.4)
            r = O.verify_sequence(L, q[None], [x], rng.random(2), 1.0, all_p=False)
            if x == 0:
                n += 1
                acc += r.n
            emit0 += r.tokens[0] == 0
        return acc, n, emit0

    res = pmap(chunk, range(100, 108))
    acc = sum(r[0] for r in res)
    n = sum(r[1] for r in res)
    emit0 = sum(r[2] for r in res)
    N = 25000 * 8
    assert stats.binomtest(acc, n, 0.25).pvalue > 1e-4
    assert stats.binomtest(emit0, N, 0.1).pvalue > 1e-4


# --------------------------------------------------------------------------
# Target distribution and inverse CDF: closed forms and library reductions
# --------------------------------------------------------------------------

def test_target_distribution_closed_forms():
    rng = np.random.default_rng(1)
    for V in (2, 7, 64, 1000):
        p = rng.dirichlet(np.ones(V))
        p = np.maximum(p, 1e-300)
        p /= p.sum()
        np.testing.assert_allclose(O.target_distribution(np.log(p), 1.0), p, rtol=1e-12, atol=0)
        for T in (0.5, 0.8, 2.0):
            want = p ** (1.0 / T)
            want /= want.sum()
            # softmax(l / T) = p^(1/T) / sum p^(1/T) for l = log p
            np.testing.assert_allclose(O.target_distribution(np.log(p), T), want, rtol=1e-10)
            # dividing by T undoes a logit scale of T
            np.testing.assert_allclose(O.target_distribution(T * np.log(p), T), p, rtol=1e-10)
        # shift invariance
        np.testing.assert_allclose(O.target_distribution(np.log(p) + 37.0, 1.0), p, rtol=1e-12)


def test_inverse_cdf_reduces_to_searchsorted():
    rng = np.random.default_rng(2)
    for _ in range(300):
        V = int(rng.integers(1, 50))
        w = rng.random(V) * (rng.random(V) < 0.6)
        if w.sum() == 0:
            w[int(rng.integers(V))] = 1.0
        u = rng.random()
        tok, t, C = O.inverse_cdf(w, u)
        assert tok == int(np.searchsorted(np.cumsum(w), u * w.sum(), side="right"))
        assert w[tok] > 0
    # u = 0 picks the first positive-mass token; zero-mass tokens are never chosen
    assert O.inverse_cdf(np.array([0.0, 0.0, 0.2, 0.0, 0.8]), 0.0)[0] == 2
    # u = 1 (no crossing): last positive-mass token
    assert O.inverse_cdf(np.array([0.3, 0.7, 0.0]), 1.0)[0] == 1


# --------------------------------------------------------------------------
# Special cases
# --------------------------------------------------------------------------

def test_q_equal_p_always_accepts_and_bonus_is_searchsorted():
    rng = np.random.default_rng(3)
    for _ in range(200):
        V, g = int(rng.integers(2, 40)), int(rng.integers(1, 6))
        T = float(rng.choice([0.7, 1.0, 1.5]))
        L = rng.normal(0, 2, (g + 1, V))
        Q = np.array([O.target_distribution(L[i], T) for i in range(g)])
        ids = [int(rng.integers(V)) for _ in range(g)]
        u = rng.random(g + 1)
        r = O.verify_sequence(L, Q, ids, u, T)
        assert r.n == g and r.mode == "bonus" and r.S == 0.0
        pg = O.target_distribution(L[g], T)
        assert r.tokens == ids + [int(np.searchsorted(np.cumsum(pg), u[g] * pg.sum(), side="right"))]


def test_greedy_is_numpy_argmax_with_lowest_index_ties():
    rng = np.random.default_rng(4)
    for _ in range(300):
        V, g = int(rng.integers(2, 30)), int(rng.integers(0, 6))
        L = np.round(rng.normal(0, 1, (g + 1, V)))  # coarse values: many ties
        ids = [int(np.argmax(L[i])) if rng.random() < 0.7 else int(rng.integers(V)) for i in range(g)]
        r = O.verify_sequence(L, None, ids, None, 0.0)
        n = next((i for i in range(g) if ids[i] != int(np.argmax(L[i]))), g)
        assert r.n == n and r.tokens == ids[:n] + [int(np.argmax(L[n]))]
    row = np.array([[0.0, 1.5, -2.0, 3.0, 1.0, 3.0, 3.0]])
    assert O.verify_sequence(row, None, [], None, 0.0).tokens == [3]


def test_zero_target_mass_always_rejects_and_residual_is_p():
    rng = np.random.default_rng(5)
    V = 12
    for _ in range(100):
        L = rng.normal(0, 1, (2, V))
        x = int(rng.integers(V))
        L[0, x] = -np.inf               # p(x) = 0
        q = np.zeros((1, V))
        q[0, x] = 1.0                   # one-hot draft
        u = rng.random(2)
        r = O.verify_sequence(L, q, [x], u, 1.0)
        p = O.target_distribution(L[0], 1.0)
        assert r.n == 0 and r.mode == "residual"
        assert abs(r.S - 1.0) < 1e-15
        assert r.tokens == [int(np.searchsorted(np.cumsum(p), u[1] * p.sum(), side="right"))]


def test_p_at_least_q_accepts_for_every_u():
    p = np.array([0.5, 0.35, 0.15])
    q = np.array([0.2, 0.3, 0.5])
    L = np.log(np.vstack([p, p]))
    for x in (0, 1):  # p >= q
        for u in np.linspace(0.0, 1.0, 1001, endpoint=False).tolist() + [np.nextafter(1.0, 0.0)]:
            assert O.verify_sequence(L, q[None], [x], [u, 0.3], 1.0).n == 1


def test_round_structure_matches_page_example():
    g_row = {r[0]: int(r[1]) for r in read_table("round_example.txt")}
    gamma = g_row["gamma"]
    V = 8
    rng = np.random.default_rng(6)
    L = rng.normal(0, 1, (gamma + 1, V))
    ids = [1, 2, 3, 4, 5]
    Q = np.array([O.target_distribution(L[i], 1.0) for i in range(gamma)])
    for i in range(3):          # positions 1-3: p(x) >= q(x) -> accepted
        Q[i] = np.full(V, 1.0 / V)
        L[i, ids[i]] = 10.0
    L[3, ids[3]] = -np.inf      # position 4: p(x) = 0 -> rejected
    Q[3] = np.full(V, 1.0 / V)
    cu = np.array([0, gamma], dtype=np.int32)
    res = O.verify_batch(L, Q, np.array(ids, np.int32), np.full(gamma + 1, 0.5, np.float32), cu, 1.0)
    assert res.accepted_count[0] == g_row["accepted"]
    emitted = res.emitted_tokens
    assert (emitted >= 0).sum() == g_row["emitted"]
    assert list(emitted[:3]) == ids[:3] and emitted[3] != ids[3]
    assert list(emitted[4:]) == [-1] * (gamma + 1 - g_row["emitted"])
    assert g_row["discarded"] == gamma - g_row["accepted"] - 1
    assert res.seq[0].mode == "residual"


# --------------------------------------------------------------------------
# Exact enumeration on tiny inputs (V = 3, gamma = 1, 2) over uniform grids
# --------------------------------------------------------------------------

def _tiny_case(seed, gamma):
    rng = np.random.default_rng(seed)
    P = rng.dirichlet(np.ones(3) * 2, size=gamma + 1)
    Qd = rng.dirichlet(np.ones(3) * 2, size=gamma)
    return P, Qd


def _exact_outcomes(P, Qd):
    """Outcome probabilities written from the rule: accept x w.p. min(1, p/q),
    first rejection draws from max(0, p - q)/S, all accepted draws from p_gamma."""
    gamma = len(Qd)
    out = {}

    def rec(i, prefix, w):
        if i == gamma:
            for y in range(3):
                key = (gamma, tuple(prefix) + (y,))
                out[key] = out.get(key, 0.0) + w * P[gamma][y]
            return
        for x in range(3):
            a = min(1.0, P[i][x] / Qd[i][x])
            rec(i + 1, prefix + [x], w * Qd[i][x] * a)
            r = np.maximum(0.0, P[i] - Qd[i])
            for y in range(3):
                key = (i, tuple(prefix) + (y,))
                out[key] = out.get(key, 0.0) + w * Qd[i][x] * (1 - a) * r[y] / r.sum()
    rec(0, [], 1.0)
    return out


@pytest.mark.parametrize("gamma,N,seed", [(1, 160, 11), (2, 22, 12)])
def test_tiny_exact_enumeration(gamma, N, seed):
    P, Qd = _tiny_case(seed, gamma)
    L = np.log(P)
    exact = _exact_outcomes(P, Qd)
    grid = (np.arange(N) + 0.5) / N
    draws = [tuple(d) for d in np.array(np.meshgrid(*[range(3)] * gamma, indexing="ij")).reshape(gamma, -1).T]

    def part(d):
        w = np.prod([Qd[i][d[i]] for i in range(gamma)])
        freq = {}
        for us in np.array(np.meshgrid(*[grid] * (gamma + 1), indexing="ij")).reshape(gamma + 1, -1).T:
            r = O.verify_sequence(L, Qd, list(d), us, 1.0, all_p=False)
            key = (r.n, tuple(r.tokens))
            freq[key] = freq.get(key, 0.0) + w / N ** (gamma + 1)
        return freq

    freq = {}
    for f in pmap(part, draws):
        for k, v in f.items():
            freq[k] = freq.get(k, 0.0) + v
    assert abs(sum(freq.values()) - 1.0) < 1e-9
    for key in set(exact) | set(freq):
        assert abs(freq.get(key, 0.0) - exact.get(key, 0.0)) <= (gamma + 1) / N, key


# --------------------------------------------------------------------------
# The distribution theorem: chi-square on V <= 16, plus negative controls
# --------------------------------------------------------------------------

V_CHI, G_CHI = 16, 4


def _theorem_case():
    rng = np.random.default_rng(20)
    P = rng.dirichlet(np.ones(V_CHI) * 3, size=G_CHI + 1)
    P = np.maximum(P, 1e-3)
    P /= P.sum(axis=1, keepdims=True)
    Qd = rng.dirichlet(np.ones(V_CHI) * 3, size=G_CHI)
    return P, Qd


def _run_rounds(P, Qd, rounds, seed, nchunks=16):
    L = np.log(P)
    gamma = len(Qd)

    def chunk(k):
        rng = np.random.default_rng([seed, k])
        counts = np.zeros((gamma + 1, V_CHI), dtype=np.int64)
        reach_acc = np.zeros((gamma, 2), dtype=np.int64)
        s_err = 0.0
        cdfs = [np.cumsum(Qd[i]) for i in range(gamma)]
        for _ in range(rounds // nchunks):
            ids = [min(int(np.searchsorted(cdfs[i], rng.random() * cdfs[i][-1], side="right")), V_CHI - 1)
                   for i in range(gamma)]
            r = O.verify_sequence(L, Qd, ids, rng.random(gamma + 1), 1.0, all_p=False)
            for i, tok in enumerate(r.tokens):
                counts[i, tok] += 1
            for i in range(min(r.n + 1, gamma)):
                reach_acc[i, 0] += 1
                reach_acc[i, 1] += r.n > i
            if r.mode == "residual":
                s_err = max(s_err, abs(r.S - (1.0 - O.acceptance_rate(P[r.n], Qd[r.n]))))
        return counts, reach_acc, s_err

    res = pmap(chunk, range(nchunks))
    return (sum(r[0] for r in res), sum(r[1] for r in res), max(r[2] for r in res))


def _slot_pvalues(P, counts):
    pv = []
    for i in range(counts.shape[0]):
        n = counts[i].sum()
        pv.append(stats.chisquare(counts[i], n * P[i]).pvalue)
    return pv


def test_theorem_emitted_tokens_follow_p():
    P, Qd = _theorem_case()
    counts, reach_acc, s_err = _run_rounds(P, Qd, 10 ** 6, seed=21)
    pv = _slot_pvalues(P, counts)
    # Bonferroni over the gamma + 1 slots
    assert min(pv) * len(pv) > 1e-4, pv
    # every slot was reached often enough to mean something
    assert counts[G_CHI].sum() > 10000
    # S = sum max(0, p - q) = 1 - sum min(p, q) on every rejected row
    assert s_err < 1e-12
    # per-position acceptance frequency = sum min(p_i, q_i)
    for i in range(G_CHI):
        a = O.acceptance_rate(P[i], Qd[i])
        assert stats.binomtest(int(reach_acc[i, 1]), int(reach_acc[i, 0]), a).pvalue * G_CHI > 1e-4


@pytest.mark.parametrize("mistake", ["resample_from_p", "drop_clamp", "accept_all", "inverted_ratio"])
def test_theorem_negative_controls_fail(monkeypatch, mistake):
    if mistake == "resample_from_p":
        monkeypatch.setattr(OV, "residual_weights", lambda p, q: np.array(p, copy=True))
    elif mistake == "drop_clamp":
        monkeypatch.setattr(OV, "residual_weights", lambda p, q: p - q)
    elif mistake == "accept_all":
        monkeypatch.setattr(OV, "acceptance_threshold", lambda px, qx: 1.0)
    elif mistake == "inverted_ratio":
        monkeypatch.setattr(OV, "acceptance_threshold", lambda px, qx: 1.0 if qx >= px else qx / px)
    P, Qd = _theorem_case()
    counts, _, _ = _run_rounds(P, Qd, 10 ** 5, seed=22, nchunks=8)
    assert min(_slot_pvalues(P, counts)) < 1e-8


# --------------------------------------------------------------------------
# Expected tokens per round with a controlled alpha
# --------------------------------------------------------------------------

def _controlled_pair(alpha, V=8):
    """p = alpha*s + (1-alpha)*u, q = alpha*s + (1-alpha)*w with s uniform on all
    ids, u uniform on the first half, w on the second: sum min(p, q) = alpha."""
    s = np.full(V, 1.0 / V)
    u = np.r_[np.full(V // 2, 2.0 / V), np.zeros(V // 2)]
    w = u[::-1].copy()
    return alpha * s + (1 - alpha) * u, alpha * s + (1 - alpha) * w


@pytest.mark.parametrize("alpha,gamma", [(0.5, 2), (0.8, 4), (0.9, 7)])
def test_expected_tokens_controlled_alpha(alpha, gamma):
    p, q = _controlled_pair(alpha)
    assert abs(O.acceptance_rate(p, q) - alpha) < 1e-15
    P = np.tile(p, (gamma + 1, 1))
    Qd = np.tile(q, (gamma, 1))
    L = np.log(np.maximum(P, 1e-300))
    rounds, nch = 160000, 16

    def chunk(k):
        rng = np.random.default_rng([30, k])
        cq = np.cumsum(q)
        out = []
        for _ in range(rounds // nch):
            ids = [min(int(np.searchsorted(cq, rng.random(), side="right")), len(q) - 1) for _ in range(gamma)]
            out.append(O.verify_sequence(L, Qd, ids, rng.random(gamma + 1), 1.0, all_p=False).n + 1)
        return out

    toks = np.concatenate(pmap(chunk, range(nch)))
    E = O.expected_tokens_per_round(alpha, gamma)
    se = toks.std() / math.sqrt(len(toks))
    assert abs(toks.mean() - E) < 5 * se, (toks.mean(), E, se)


def test_greedy_controlled_agreement_follows_E():
    V, gamma = 50, 8
    w = synth.make_greedy("greedy-small", np.full(20000, gamma), V, "bf16", 4.0, 0.8, seed=40)
    res = O.verify_batch(w.logits_f64(), None, w.draft_ids, None, w.cu_gamma, 0.0)
    L = w.logits_f64()
    for b in range(0, w.B, 97):  # accepted drafts and the emitted token are target argmaxes
        n = res.accepted_count[b]
        base = int(w.cu_gamma[b])
        for i in range(n + 1):
            assert res.emitted_tokens[base + b + i] == int(np.argmax(L[base + b + i]))
    alpha = 0.8 + 0.2 / V
    toks = res.accepted_count.astype(np.float64) + 1
    E = O.expected_tokens_per_round(alpha, gamma)
    assert abs(toks.mean() - E) < 5 * toks.std() / math.sqrt(len(toks))


def test_first_argmax_ties_and_inf():
    """The greedy token over finite logits (-inf allowed) is the largest logit, lowest
    index on ties: checked against a plain scan that keeps the first strict maximum, on
    hand cases and on small random rows with many ties (values from a grid of 4)."""
    assert O.first_argmax([1.0, 3.0, 2.0, 3.0]) == 1
    assert O.first_argmax([-np.inf, -np.inf]) == 0
    assert O.first_argmax([-np.inf, -5.0, -np.inf, -5.0]) == 1
    assert O.first_argmax([7.0]) == 0

    def scan(row):
        best, at = -np.inf, 0
        for v, x in enumerate(row):
            if x > best:
                best, at = x, v
        return at

    rng = np.random.default_rng(71)
    for _ in range(2000):
        V = int(rng.integers(1, 12))
        row = rng.integers(-2, 2, V).astype(np.float64)
        row[rng.random(V) < 0.2] = -np.inf
        assert O.first_argmax(row) == scan(row)
