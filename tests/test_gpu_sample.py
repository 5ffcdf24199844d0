"""GPU parity of spec_sample_run (one token per row from a given distribution) against
the oracle's inverse CDF, through the C ABI.

Rows come from the seeded generator in `synth` (target logits, draft distributions q);
expected tokens come from `oracle` only.
"""
import sys

import numpy as np
import pytest
from scipy import stats

import oracle as O
import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

FLAG_WINDOW = 1e-6


def _say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import speculative_sampling_verification_03_amd as sv
    sv.load_library()
    return sv


def compare_tokens(weights_rows, uniforms, got):
    """Exact match, except rows whose oracle t lies within 1e-6 relative of a prefix
    boundary between the two tokens (flagged). Returns (mismatches, flagged)."""
    bad, flagged = [], 0
    for r, (w, u) in enumerate(zip(weights_rows, uniforms)):
        tok, t, C = O.inverse_cdf(w, float(u))
        g = int(got[r])
        if g == tok:
            continue
        lo, hi = min(g, tok), max(g, tok)
        if 0 <= lo and hi <= len(C) and t > 0 and np.any(np.abs(t - C[lo:hi]) <= FLAG_WINDOW * t):
            flagged += 1
        else:
            bad.append((r, tok, g))
    return bad, flagged


def _logits_tensor(w, rows):
    if w.dtype == "bf16":
        return torch.from_numpy(w.logits[rows].view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(w.logits[rows]).cuda()


@pytest.mark.parametrize("cfg,T,batch", [("C3", 1.0, 40), ("C2", 0.8, 40), ("C3", 0.6, 40),
                                         ("C3", 1.0, 150), ("C2", 0.8, 80)])
def test_sample_logits_parity(lib, cfg, T, batch):
    """Rows from the configurations' target rows (batch 150 / 80: more rows than compute
    units, which the one-launch plan draws with one workgroup per compute unit)."""
    T = synth.fp32_temperature(T)  # the value the library receives
    w = synth.make_config(cfg, seed=21, batch=batch)
    rows = slice(0, w.target_rows)
    L = _logits_tensor(w, rows)
    nrows = w.target_rows
    u = np.random.default_rng(70).random(nrows, dtype=np.float32)
    _say("sample logits", cfg, f"rows={nrows} V={w.V} T={T}")
    code = lib.SV_BF16 if w.dtype == "bf16" else lib.SV_F32
    for plan in (lib.SV_PATH_TWO_LAUNCH, lib.SV_PATH_ONE_LAUNCH):
        v = lib.Verifier(w.V, code, nrows, 1, 1)
        v.set_path(plan)
        tok = v.sample(L, uniforms=torch.from_numpy(u).cuda(), temperature=T).cpu().numpy()
        assert v.status() == lib.SV_OK, v.last_error()
        P = [O.target_distribution(w.logits_f64(slice(r, r + 1))[0], T) for r in range(nrows)]
        bad, flagged = compare_tokens(P, u, tok)
        _say("sample logits", cfg, f"plan={plan} mismatches={len(bad)} flagged={flagged}")
        assert not bad and flagged == 0, bad[:5]
        v.close()


def test_sample_logits_rows_outside_table(lib):
    """More rows than compute units (one workgroup per compute unit draws row after row),
    with rows holding a logit beyond the value table's window (|l k2| > 990 at T = 1):
    those rows are drawn on the exp2 path, the others through the table; all must match
    the oracle."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nrows = 3 * cus + 11
    w = synth.make_config("C3", seed=23, batch=(nrows + 4) // 5, vocab=32000)
    L = w.logits_f32()[:nrows].copy()
    rng = np.random.default_rng(71)
    hot = rng.choice(nrows, 40, replace=False)
    for r in hot[:20]:
        L[r, rng.integers(0, w.V)] = 2000.0  # far outside: the row is one-hot
    for r in hot[20:]:
        L[r, rng.integers(0, w.V, 3)] = 700.0  # just outside (700 k2 > 990): three equal peaks
    bits = synth.bf16_round(L)
    L = synth.bf16_widen(bits)  # the values the GPU reads (2000 and 700 are exact in bf16)
    Lt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    u = np.random.default_rng(72).random(nrows, dtype=np.float32)
    v = lib.Verifier(w.V, lib.SV_BF16, nrows, 1, 1)
    v.set_path(lib.SV_PATH_ONE_LAUNCH)
    _say("sample logits outside table", f"rows={nrows} V={w.V}")
    tok = v.sample(Lt, uniforms=torch.from_numpy(u).cuda(), temperature=1.0).cpu().numpy()
    assert v.status() == lib.SV_OK, v.last_error()
    P = [O.target_distribution(L[r].astype(np.float64), 1.0) for r in range(nrows)]
    bad, flagged = compare_tokens(P, u, tok)
    assert not bad and flagged == 0, bad[:5]
    for r in hot[:20]:
        assert L[r, tok[r]] == 2000.0
    v.close()


def test_sample_logits_greedy(lib):
    w = synth.make_config("C4", seed=22, batch=24, vocab=8192)
    L = _logits_tensor(w, slice(0, w.target_rows))
    v = lib.Verifier(w.V, lib.SV_BF16, w.target_rows, 1, 1)
    tok = v.sample(L, temperature=0.0).cpu().numpy()
    assert v.status() == lib.SV_OK
    ref = [O.first_argmax(w.logits_f64(slice(r, r + 1))[0]) for r in range(w.target_rows)]
    assert np.array_equal(tok, ref)
    v.close()


@pytest.mark.parametrize("vocab", [128256, 32000, 1001])
def test_sample_weights_parity(lib, vocab):
    w = synth.make_config("C3", seed=23, batch=32, vocab=vocab)
    Q = w.q  # fp32 draft distributions [rows, V]
    u = np.random.default_rng(71).random(Q.shape[0], dtype=np.float32)
    _say("sample weights", f"rows={Q.shape[0]} V={vocab}")
    v = lib.Verifier(vocab, lib.SV_BF16, Q.shape[0], 1, 1)
    tok = v.sample_weights(torch.from_numpy(Q).cuda(), uniforms=torch.from_numpy(u).cuda()).cpu().numpy()
    assert v.status() == lib.SV_OK, v.last_error()
    bad, flagged = compare_tokens([q.astype(np.float64) for q in Q], u, tok)
    _say("sample weights", f"V={vocab} mismatches={len(bad)} flagged={flagged}")
    assert not bad and flagged == 0, bad[:5]
    v.close()


def test_sample_weights_unnormalised_and_edges(lib):
    rng = np.random.default_rng(72)
    V, rows = 5000, 12
    W = (rng.random((rows, V)) ** 4 * 1000.0).astype(np.float32)
    W[1, :] = 0.0
    W[1, 4321] = 3.0                 # a single positive weight
    W[2, ::2] = 0.0                  # zero-weight ids are never drawn
    u = rng.random(rows, dtype=np.float32)
    u[3] = 0.0                       # first positive weight
    v = lib.Verifier(V, lib.SV_F32, rows, 1, 1)
    Wt = torch.from_numpy(W).cuda()
    tok = v.sample_weights(Wt, uniforms=torch.from_numpy(u).cuda()).cpu().numpy()
    assert v.status() == lib.SV_OK
    bad, flagged = compare_tokens([x.astype(np.float64) for x in W], u, tok)
    assert not bad and flagged == 0, bad
    assert tok[1] == 4321 and tok[2] % 2 == 1
    assert tok[3] == int(np.nonzero(W[3] > 0)[0][0])
    # misaligned start (the element-wise path) gives the same tokens
    big = torch.empty(W.size + 1, dtype=torch.float32, device="cuda")
    big[1:].copy_(Wt.reshape(-1))
    tok2 = v.sample_weights(big[1:], uniforms=torch.from_numpy(u).cuda()).cpu().numpy()
    assert np.array_equal(tok, tok2)
    # negative, NaN and all-zero rows: counted as 0, flagged
    W2 = W.copy()
    W2[0, 17] = -1.0
    W2[5, 100] = np.nan
    W2[6, :] = 0.0
    tok3 = v.sample_weights(torch.from_numpy(W2).cuda(), uniforms=torch.from_numpy(u).cuda()).cpu().numpy()
    assert v.status() == lib.SV_EDATA and "non-finite" in v.last_error()
    clean = np.where(np.isfinite(W2) & (W2 > 0), W2, 0.0).astype(np.float64)
    for r in (0, 5):
        assert tok3[r] == O.inverse_cdf(clean[r], float(u[r]))[0]
    assert tok3[6] == V - 1
    v.close()


def test_sample_distribution_chi_square(lib):
    """10^5 rows of one distribution at V = 24: the GPU's tokens follow it (both modes)."""
    rng = np.random.default_rng(73)
    V, rows = 24, 100_000
    p = rng.dirichlet(np.ones(V) * 2.0)
    logit = np.log(p).astype(np.float32)
    u = torch.from_numpy(rng.random(rows, dtype=np.float32)).cuda()
    v = lib.Verifier(V, lib.SV_F32, rows, 1, 1)
    L = torch.from_numpy(logit).cuda().repeat(rows, 1)
    Wt = torch.from_numpy(p.astype(np.float32)).cuda().repeat(rows, 1)
    for name, tok in (("logits", v.sample(L, uniforms=u, temperature=1.0)),
                      ("weights", v.sample_weights(Wt, uniforms=u))):
        cnt = np.bincount(tok.cpu().numpy(), minlength=V)
        p_exp = np.exp(logit.astype(np.float64)) if name == "logits" else p.astype(np.float32).astype(np.float64)
        p_exp /= p_exp.sum()
        pv = stats.chisquare(cnt, rows * p_exp).pvalue
        _say("chi-square", name, f"p={pv:.3g}")
        assert pv > 1e-4
    assert v.status() == lib.SV_OK
    v.close()
