"""Seeded synthetic inputs for the batched speculative-sampling verification step.

This module builds inputs only. It holds none of the verification arithmetic
(no accept test, no residual, no target sampling). Both the CPU oracle's tests
and the GPU path's tests and benchmark draw their inputs from here.

What it constructs, per sequence b with gamma_b draft positions:
  * target logits for gamma_b + 1 positions (row-major, packed back to back);
  * the draft distribution q for gamma_b positions. It stands in for the draft
    model: q = softmax(stored logits + sigma_b * noise), built in fp64 from the
    logit values exactly as stored, then cast to fp32;
  * draft ids drawn from that fp32 q by an fp64 inverse CDF of the draft's own
    uniform stream (so q(x) > 0 for every draft), or, in greedy workloads, the
    target argmax with probability `agree` and a uniform random id otherwise;
  * one fp32 uniform in [0, 1) per target row, drawn directly in fp32.

Packing: `cu_gamma[b]` is the exclusive prefix of gamma_b. The logits row of
(b, i) is cu_gamma[b] + b + i (i <= gamma_b); the q / draft-id row of (b, i) is
cu_gamma[b] + i (i < gamma_b); the uniform of (b, i) shares the logits index.

bf16 logits are held as uint16 bit patterns, rounded once from fp32 with
round-to-nearest-even. Both sides read the same bits.

Seeding: numpy PCG64. The base seed is 0x5EED0000 + config number + 1000*seed.
Separate spawned streams serve logits, noise, drafts, uniforms, gamma_b and
sigma_b; logits and noise are further split into fixed 64-row blocks, each
with its own spawned stream, so the result does not depend on thread count.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "CONFIGS", "make_config", "make_sampling", "make_greedy",
    "pack", "fp32_temperature", "bf16_round", "bf16_widen", "config_number", "make_onehot", "boost_drafts", "controlled_alpha_rows",
    "Contexts", "make_ngram_contexts",
]

_BLOCK = 64  # rows per independently seeded block
_THREADS = max(1, min(16, os.cpu_count() or 1))


def bf16_round(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even. Inputs are finite."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exactly equal fp32 values."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Workload:
    """One batch of verification inputs (host arrays)."""
    name: str
    B: int
    V: int
    dtype: str                    # "f32" or "bf16"
    T: float
    gammas: np.ndarray            # int32 [B]
    cu_gamma: np.ndarray          # int32 [B+1]
    uniform_gamma: Optional[int]  # gamma if every gamma_b is equal, else None
    logits: np.ndarray            # [sum(gamma_b+1), V]: float32, or uint16 bf16 bits
    q: Optional[np.ndarray]       # float32 [sum gamma_b, V]; None in greedy workloads
    draft_ids: np.ndarray         # int32 [sum gamma_b]
    uniforms: Optional[np.ndarray]  # float32 [sum(gamma_b+1)]; None in greedy workloads

    @property
    def draft_rows(self) -> int:
        return int(self.cu_gamma[-1])

    @property
    def target_rows(self) -> int:
        return int(self.cu_gamma[-1]) + self.B

    def logits_f32(self, rows=slice(None)) -> np.ndarray:
        x = self.logits[rows]
        return bf16_widen(x) if self.dtype == "bf16" else np.asarray(x, dtype=np.float32)

    def logits_f64(self, rows=slice(None)) -> np.ndarray:
        return self.logits_f32(rows).astype(np.float64)

    def logit_row(self, b: int, i: int) -> int:
        return int(self.cu_gamma[b]) + b + i

    def draft_row(self, b: int, i: int) -> int:
        return int(self.cu_gamma[b]) + i

    def nbytes(self) -> int:
        n = self.logits.nbytes + self.draft_ids.nbytes + self.cu_gamma.nbytes
        if self.q is not None:
            n += self.q.nbytes
        if self.uniforms is not None:
            n += self.uniforms.nbytes
        return n


def fp32_temperature(T) -> float:
    """The temperature as the verification step receives it: a 32-bit float (0.8 becomes
    0.800000011920929). Workloads carry that value, so every side computes with it."""
    return float(np.float32(T))


def pack(gammas) -> np.ndarray:
    """Exclusive prefix of gamma_b, int32 [B+1]."""
    g = np.asarray(gammas, dtype=np.int64)
    cu = np.zeros(len(g) + 1, dtype=np.int64)
    np.cumsum(g, out=cu[1:])
    return cu.astype(np.int32)


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    names = ("logits", "noise", "drafts", "uniforms", "gammas", "sigmas")
    return dict(zip(names, ss.spawn(len(names))))


def _blockwise(ss: np.random.SeedSequence, rows: int, V: int, fn):
    """Run fn(rng, r0, r1) over fixed 64-row blocks, each with its own spawned stream."""
    nblk = (rows + _BLOCK - 1) // _BLOCK
    kids = ss.spawn(nblk)

    def work(k):
        r0, r1 = k * _BLOCK, min(rows, (k + 1) * _BLOCK)
        fn(np.random.Generator(np.random.PCG64(kids[k])), r0, r1)

    if nblk <= 1:
        for k in range(nblk):
            work(k)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(work, range(nblk)))


def _normal_logits(ss, rows, V, sigma, dtype):
    out = np.empty((rows, V), dtype=np.uint16 if dtype == "bf16" else np.float32)

    def fn(rng, r0, r1):
        z = rng.standard_normal((r1 - r0, V), dtype=np.float32)
        z *= np.float32(sigma)
        out[r0:r1] = bf16_round(z) if dtype == "bf16" else z

    _blockwise(ss, rows, V, fn)
    return out


def _draft_q(ss, logits_f32_rows, sigmas_per_row):
    """q = softmax(l + sigma * N(0,1)) in fp64 from the stored logit values, cast to fp32.

    This is the draft model's stand-in, an input to verification.
    logits_f32_rows(r0, r1) returns the stored logits of draft rows r0..r1 as fp32.
    """
    rows = len(sigmas_per_row)
    V = logits_f32_rows(0, min(1, rows)).shape[1] if rows else 0
    out = np.empty((rows, V), dtype=np.float32)

    def fn(rng, r0, r1):
        z = rng.standard_normal((r1 - r0, V), dtype=np.float32).astype(np.float64)
        x = logits_f32_rows(r0, r1).astype(np.float64) + sigmas_per_row[r0:r1, None] * z
        x -= x.max(axis=1, keepdims=True)
        np.exp(x, out=x)
        x /= x.sum(axis=1, keepdims=True)
        out[r0:r1] = x

    _blockwise(ss, rows, V, fn)
    return out


def _draws_from(q32: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Draft ids: fp64 inverse CDF of the fp32 draft rows q32 at draft uniforms w."""
    ids = np.empty(q32.shape[0], dtype=np.int32)
    for r0 in range(0, q32.shape[0], 256):
        c = np.cumsum(q32[r0:r0 + 256].astype(np.float64), axis=1)
        t = w[r0:r0 + 256] * c[:, -1]
        k = (c <= t[:, None]).sum(axis=1)
        ids[r0:r0 + 256] = np.minimum(k, q32.shape[1] - 1)
    return ids


def _row_maps(cu: np.ndarray):
    """For each draft row: its logits row. Returns int64 [sum gamma_b]."""
    B = len(cu) - 1
    g = np.diff(cu.astype(np.int64))
    seq = np.repeat(np.arange(B, dtype=np.int64), g)
    return np.arange(int(cu[-1]), dtype=np.int64) + seq


def make_sampling(name, gammas, V, dtype, T, sigma_logit, sigma_noise, seed,
                  replicate_first=False) -> Workload:
    """Sampling-mode workload (T > 0).

    gammas: int array [B]. sigma_noise: scalar or per-sequence array [B].
    replicate_first: every sequence reuses sequence 0's logits and q (fixed p and
    q, fresh draft ids and uniforms per round).
    """
    st = _streams(seed)
    gammas = np.asarray(gammas, dtype=np.int32)
    B = len(gammas)
    cu = pack(gammas)
    R = int(cu[-1])
    sig = np.broadcast_to(np.asarray(sigma_noise, dtype=np.float64), (B,))
    if replicate_first:
        g0 = int(gammas[0])
        assert np.all(gammas == g0)
        one = _normal_logits(st["logits"], g0 + 1, V, sigma_logit, dtype)
        logits = np.tile(one, (B, 1))
        w0 = bf16_widen(one) if dtype == "bf16" else one
        q0 = _draft_q(st["noise"], lambda a, b: w0[a:b], np.full(g0, sig[0]))
        q = np.tile(q0, (B, 1))
    else:
        logits = _normal_logits(st["logits"], R + B, V, sigma_logit, dtype)
        lrow = _row_maps(cu)
        wid = (lambda a, b: bf16_widen(logits[lrow[a:b]])) if dtype == "bf16" else \
              (lambda a, b: logits[lrow[a:b]])
        sig_rows = np.repeat(sig, gammas.astype(np.int64))
        q = _draft_q(st["noise"], wid, sig_rows)
    rd = np.random.Generator(np.random.PCG64(st["drafts"]))
    draft_ids = _draws_from(q, rd.random(R))
    ru = np.random.Generator(np.random.PCG64(st["uniforms"]))
    uniforms = ru.random(R + B, dtype=np.float32)
    ug = int(gammas[0]) if B and np.all(gammas == gammas[0]) else None
    return Workload(name, B, V, dtype, fp32_temperature(T), gammas, cu, ug, logits, q, draft_ids, uniforms)


def make_greedy(name, gammas, V, dtype, sigma_logit, agree, seed) -> Workload:
    """Greedy workload (T = 0): draft = target argmax (lowest index) with prob `agree`,
    else a uniform random id. No q, no uniforms."""
    st = _streams(seed)
    gammas = np.asarray(gammas, dtype=np.int32)
    B = len(gammas)
    cu = pack(gammas)
    R = int(cu[-1])
    logits = _normal_logits(st["logits"], R + B, V, sigma_logit, dtype)
    lrow = _row_maps(cu)
    top = np.empty(R, dtype=np.int64)
    for r0 in range(0, R, 256):
        rows = lrow[r0:r0 + 256]
        x = bf16_widen(logits[rows]) if dtype == "bf16" else logits[rows]
        top[r0:r0 + 256] = np.argmax(x, axis=1)  # first maximum
    rd = np.random.Generator(np.random.PCG64(st["drafts"]))
    coin = rd.random(R)
    other = rd.integers(0, V, size=R)
    draft_ids = np.where(coin < agree, top, other).astype(np.int32)
    ug = int(gammas[0]) if B and np.all(gammas == gammas[0]) else None
    return Workload(name, B, V, dtype, 0.0, gammas, cu, ug, logits, None, draft_ids, None)


def make_onehot(name, gammas, V, dtype, T, sigma_logit, agree, seed) -> Workload:
    """Workload with deterministic drafts (an n-gram style proposer): draft = target argmax
    (lowest index) with prob `agree`, else a uniform random id; q is left None (the
    draft distribution is one-hot at the draft). Uniforms drawn as fp32 in [0, 1)."""
    w = make_greedy(name, gammas, V, dtype, sigma_logit, agree, seed)
    st = _streams(seed)
    ru = np.random.Generator(np.random.PCG64(st["uniforms"]))
    u = ru.random(w.target_rows, dtype=np.float32)
    return Workload(name, w.B, V, dtype, fp32_temperature(T), w.gammas, w.cu_gamma, w.uniform_gamma, w.logits, None,
                    w.draft_ids, u)


def boost_drafts(w: Workload, frac: float, margin: float, seed: int) -> Workload:
    """Make the target confident about some drafts, as in copy-heavy text: in a fraction
    `frac` of the draft rows with a valid id, that id's target logit is set to the row's
    maximum plus `margin` (then stored in the workload's dtype). Changes w.logits in place."""
    rg = np.random.Generator(np.random.PCG64(_streams(seed)["noise"]))
    coin = rg.random(w.draft_rows)
    lrow = _row_maps(w.cu_gamma)
    for r in np.flatnonzero((coin < frac) & (w.draft_ids >= 0) & (w.draft_ids < w.V)):
        row = w.logits_f32(slice(int(lrow[r]), int(lrow[r]) + 1))[0].copy()
        row[w.draft_ids[r]] = row.max() + np.float32(margin)
        w.logits[lrow[r]] = bf16_round(row) if w.dtype == "bf16" else row
    return w


def controlled_alpha_rows(alphas, V: int):
    """Per-sequence target logits and draft distributions with a known overlap alpha_b:
    p = a*s + (1-a)*u, q = a*s + (1-a)*w, s uniform on all V ids, u uniform on the first
    half, w on the second half (V even), so sum_v min(p, q) = a. Returns (logits = log p
    as fp32 [B, V], q fp32 [B, V]). Needs every alpha_b > 0 (p > 0 everywhere)."""
    a = np.asarray(alphas, dtype=np.float64)[:, None]
    assert V % 2 == 0 and np.all(a > 0)
    s = np.full(V, 1.0 / V)
    u = np.r_[np.full(V // 2, 2.0 / V), np.zeros(V // 2)]
    w = u[::-1]
    p = a * s + (1 - a) * u
    q = a * s + (1 - a) * w
    return np.log(p).astype(np.float32), q.astype(np.float32)


@dataclasses.dataclass
class Contexts:
    """A packed batch of token contexts (host arrays)."""
    B: int
    tokens: np.ndarray   # int32 [sum L_b]
    cu_ctx: np.ndarray   # int32 [B+1] exclusive prefix of L_b

    def context(self, b: int) -> np.ndarray:
        return self.tokens[self.cu_ctx[b]:self.cu_ctx[b + 1]]


def make_ngram_contexts(B, lengths, V, seed, copy_prob=0.7, prompt_frac=0.6) -> Contexts:
    """Copy-heavy contexts (summaries, edits, retrieval answers that repeat their input).

    lengths: (L_min, L_max), each L_b uniform in it (inclusive). The first prompt_frac of
    a context are ids uniform in [0, V); the rest is built piece by piece: with
    probability copy_prob a span of 4..32 tokens copied from a uniform earlier place,
    else 1..4 fresh uniform ids; the last piece is cut at L_b."""
    st = _streams(seed)
    rg = np.random.Generator(np.random.PCG64(st["drafts"]))
    lo, hi = lengths
    L = rg.integers(lo, hi + 1, B)
    cu = pack(L)
    out = np.empty(int(cu[-1]), dtype=np.int32)
    for b in range(B):
        n = int(L[b])
        c = np.empty(n, dtype=np.int32)
        k = min(n, max(1, int(prompt_frac * n))) if n else 0
        c[:k] = rg.integers(0, V, k)
        while k < n:
            if rg.random() < copy_prob and k >= 4:
                m = min(int(rg.integers(4, 33)), n - k)
                j = int(rg.integers(0, k))
                if j + m <= k:
                    c[k:k + m] = c[j:j + m]
                else:
                    for t in range(m):  # element by element: the copy overlaps itself
                        c[k + t] = c[j + t]
            else:
                m = min(int(rg.integers(1, 5)), n - k)
                c[k:k + m] = rg.integers(0, V, m)
            k += m
        out[cu[b]:cu[b + 1]] = c
    return Contexts(B, out, cu)


# The five workloads the verification step is measured and checked on.
CONFIGS = {
    "C1": dict(B=1, gamma=4, V=32, dtype="f32", T=1.0, sigma_logit=2.0, sigma_noise=0.5,
               note="fixed p and q, fresh drafts and uniforms per round"),
    "C2": dict(B=64, gamma=5, V=32000, dtype="f32", T=0.8, sigma_logit=3.0, sigma_noise=1.0),
    "C3": dict(B=256, gamma=4, V=128256, dtype="bf16", T=1.0, sigma_logit=3.0, sigma_noise=0.7),
    "C4": dict(B=512, gamma=8, V=152064, dtype="bf16", T=0.0, sigma_logit=4.0, agree=0.8),
    "C5": dict(B=1024, gamma=(1, 8), V=128256, dtype="bf16", T=1.0, sigma_logit=3.0,
               sigma_noise=(0.2, 2.0)),
}


def config_number(name: str) -> int:
    return int(name[1:])


def make_config(name: str, seed: int = 0, batch: Optional[int] = None,
                vocab: Optional[int] = None, gamma: Optional[int] = None) -> Workload:
    """Build workload `name` (C1..C5). batch / vocab override B / V, gamma the draft
    length of the uniform-gamma configurations (same recipe)."""
    c = CONFIGS[name]
    B = int(batch if batch is not None else c["B"])
    V = int(vocab if vocab is not None else c["V"])
    if gamma is not None:
        if name == "C5":
            raise ValueError("C5 draws its per-sequence draft lengths; gamma applies to C1..C4")
        c = dict(c, gamma=int(gamma))
    base = 0x5EED0000 + config_number(name) + 1000 * int(seed)
    if name == "C4":
        return make_greedy(name, np.full(B, c["gamma"]), V, c["dtype"], c["sigma_logit"],
                           c["agree"], base)
    if name == "C5":
        st = _streams(base)
        rg = np.random.Generator(np.random.PCG64(st["gammas"]))
        rs = np.random.Generator(np.random.PCG64(st["sigmas"]))
        lo, hi = c["gamma"]
        gammas = rg.integers(lo, hi + 1, size=B)
        sig = rs.uniform(c["sigma_noise"][0], c["sigma_noise"][1], size=B)
        return make_sampling(name, gammas, V, c["dtype"], c["T"], c["sigma_logit"], sig,
                             base + 0x100000)
    return make_sampling(name, np.full(B, c["gamma"]), V, c["dtype"], c["T"],
                         c["sigma_logit"], c["sigma_noise"], base,
                         replicate_first=(name == "C1"))
