"""CPU oracle for the batched speculative-sampling verification step.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or load
this module: only the tests, the smoke check and the benchmark's CPU-baseline
leg use it. It shares no code with the HIP library.

It is the plain, slow definition of what the verification step computes,
written out in float64 with NumPy, one sequence at a time. Sources:

  [P1] "Speculative Decoding", atonlee.tistory.com/330
       ch.2 "propose와 verify가 한 round를 만드는 방식" (round structure, k+1 tokens,
       bonus token, discard after the first rejection);
       ch.3 "target distribution을 보존하는 acceptance rule" (accept test
       r < min(1, p/q), residual norm(max(0, p-q)), greedy rule at T = 0);
       ch.4 "acceptance만으로 속도를 설명할 수 없는 이유" (E per round, table).
  [P2] "Speculative Decoding으로 LLM 추론 속도 높이기", donmain.dev
       "미리 그려놓고 한 번에 검증한다" (1 .. gamma+1 tokens per iteration);
       "품질은 rejection sampling이 지킨다" (worked example q=0.4, p=0.1; E; p >= q
       accepts outright).
  [P3] "Fast Inference from Transformers via Speculative Decoding" (notes),
       방법론 상세: 단계 1-3 (drafts, gamma+1 target distributions, accept
       probability alpha_i, residual at the first rejection, bonus from
       p(. | x_{1:n+gamma})); 이론적 동등성 증명; 예상 수용 길이 (E, alpha).
  [P4] "투기적 디코딩 — 초안 모델을 무엇으로 세울 것인가", ailab.paldyn.com
       "출력이 변하지 않는다는 것이 핵심이다" (rule; greedy = argmax equality);
       "이득의 크기는 두 숫자가 정한다" (E, the +1 in gamma+1).

Readings where the pages leave a step open (each is also listed in the design
notes):
  * p = softmax(logits / T). The pages never write the temperature step; this is
    the standard reading, with T = 0 meaning greedy ([P1] ch.3, greedy paragraph).
  * Uniforms: gamma_b + 1 per sequence. Slot i < gamma_b is the accept test of
    draft position i; slot gamma_b drives the single final draw (residual or
    bonus). A rejecting uniform is never reused.
  * Accept iff u < thr (strict, [P1] ch.3 step 2), thr = 1 when p(x) >= q(x)
    ([P2], [P4]); otherwise thr = p(x) / q(x).
  * Inverse CDF over ascending token ids with an inclusive prefix sum C: the draw
    is the first v with C[v] > t, t = u * sum(weights). If rounding leaves no such
    v, the last v with positive weight.
  * A rejection whose residual mass S = sum max(0, p - q) is not positive (only
    through rounding, or a uniform >= 1) draws from p instead (degenerate row).
  * Greedy ties: lowest index wins. The greedy bonus is the argmax of row gamma_b.
  * S reported for a rejected row is sum max(0, p - q); 0.0 when every draft is
    accepted and in greedy mode.
  * A draft id outside [0, V) is treated as rejected at that position.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

__all__ = [
    "target_distribution", "acceptance_threshold", "residual_weights",
    "inverse_cdf", "first_argmax", "verify_sequence", "verify_batch",
    "SequenceResult", "BatchResult", "expected_tokens_per_round",
    "acceptance_rate", "speedup_factor",
]


def target_distribution(logits_row, T: float) -> np.ndarray:
    """p = softmax(l / T) in float64 (the temperature reading above)."""
    x = np.asarray(logits_row, dtype=np.float64) / float(T)
    m = np.max(x)
    e = np.exp(x - m)
    return e / np.sum(e)


def acceptance_threshold(p_x: float, q_x: float) -> float:
    """min(1, p(x)/q(x)); p >= q accepts outright, so no division there.

    [P1] ch.3 (modified rejection sampling, steps 1-2); [P2] "품질은 rejection
    sampling이 지킨다" (p >= q always accepted); [P3] 단계 3 (alpha_i).
    """
    if p_x >= q_x:
        return 1.0
    return p_x / q_x


def residual_weights(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Unnormalised residual max(0, p - q); its sum is the normaliser S.

    [P1] ch.3 (잔차 분포 = normalize(max(0, p - q))); [P3] 단계 3 (x' ~ norm(max(0, p - q)));
    [P3] 이론적 동등성 증명 (S = sum max(0, p - q) = 1 - sum min(p, q)).
    """
    return np.maximum(0.0, p - np.asarray(q, dtype=np.float64))


def inverse_cdf(weights: np.ndarray, u: float):
    """Draw from weights / sum(weights) with the uniform u.

    Returns (token, t, C): t = u * sum(weights), C the inclusive prefix sum; the
    token is the first v with C[v] > t, else the last v with positive weight.
    """
    C = np.cumsum(weights)
    t = float(u) * C[-1]
    above = np.nonzero(C > t)[0]
    if above.size:
        return int(above[0]), t, C
    pos = np.nonzero(weights > 0)[0]
    return (int(pos[-1]) if pos.size else len(weights) - 1), t, C


def first_argmax(row) -> int:
    """Greedy target token: the most likely target token, argmax of the logits with the
    lowest index on ties ([P1] ch.3 greedy paragraph; [P4] "출력이 변하지 않는다는 것이
    핵심이다"). Defined for the input domain of finite logits (-inf allowed); a row of
    -inf gives index 0. A NaN logit is outside the domain: the library reports it as a
    data error and its outputs for that sequence are unspecified, so the oracle gives
    no answer of its own for such rows."""
    return int(np.argmax(np.asarray(row, dtype=np.float64)))


@dataclasses.dataclass
class SequenceResult:
    n: int                       # accepted draft count
    tokens: List[int]            # the n + 1 emitted tokens
    S: float                     # residual mass (0.0 if none drawn from a residual)
    thresholds: List[float]      # thr_i for every judged position i <= min(n, gamma-1)
    p_draft: List[float]         # p(x_i) for every draft position (sampling mode)
    mode: str                    # "residual", "bonus", "degenerate", "greedy"
    t: float = 0.0               # u * sum(weights) of the final draw
    C: Optional[np.ndarray] = None  # inclusive prefix of the final draw (keep_cdf)


def verify_sequence(logits_rows, q_rows, draft_ids, uniforms, T: float,
                    keep_cdf: bool = False, all_p: bool = True) -> SequenceResult:
    """One round's verification for one sequence.

    logits_rows: [gamma+1, V] target logits; q_rows: [gamma, V] draft
    distributions (unused when T == 0); draft_ids: [gamma]; uniforms: [gamma+1]
    (unused when T == 0).

    Left-to-right judging, stop at the first rejection, discard every later
    draft ([P1] ch.2 round example; [P2] "미리 그려놓고 한 번에 검증한다"; [P3] 단계 3).
    A round emits the n accepted drafts plus one token: the residual draw at the
    first rejection, or the bonus draw from p at position gamma + 1 when all
    gamma are accepted ([P1] ch.2; [P3] 단계 3; [P4] "이득의 크기는 두 숫자가 정한다").
    """
    L = np.asarray(logits_rows)
    gamma = L.shape[0] - 1
    V = L.shape[1]
    ids = [int(x) for x in np.asarray(draft_ids).reshape(-1)[:gamma]]

    if T == 0.0:
        # Greedy: accept iff the draft equals the target argmax; on a mismatch
        # emit the target argmax. No uniforms, no residual ([P1] ch.3 greedy
        # paragraph; [P4] "출력이 변하지 않는다는 것이 핵심이다").
        for i in range(gamma):
            a = first_argmax(L[i])
            if ids[i] != a:
                return SequenceResult(i, ids[:i] + [a], 0.0, [], [], "greedy")
        return SequenceResult(gamma, ids + [first_argmax(L[gamma])], 0.0, [], [], "greedy")

    Q = np.asarray(q_rows, dtype=np.float64)
    U = np.asarray(uniforms, dtype=np.float64).reshape(-1)
    thresholds: List[float] = []
    p_draft: List[float] = []
    n = gamma
    p_rej = None
    for i in range(gamma):
        if n < gamma and not all_p:
            break
        # Rows past the first rejection are only evaluated for the p(x_i)
        # diagnostic (all_p); they never influence n, the tokens or S.
        p = target_distribution(L[i], T)
        x = ids[i]
        valid = 0 <= x < V
        px = float(p[x]) if valid else float("nan")
        p_draft.append(px)
        if n == gamma:  # still judging, left to right
            thr = acceptance_threshold(px, float(Q[i, x])) if valid else float("nan")
            thresholds.append(thr)
            if not (valid and U[i] < thr):
                n = i
                p_rej = p

    if n < gamma:
        r = residual_weights(p_rej, Q[n])
        S = float(np.sum(r))
        mode = "residual"
        if not S > 0.0:
            r, mode = p_rej, "degenerate"
    else:
        r = target_distribution(L[gamma], T)
        S, mode = 0.0, "bonus"
    tok, t, C = inverse_cdf(r, U[gamma])
    return SequenceResult(n, ids[:n] + [tok], S, thresholds, p_draft, mode, t,
                          C if keep_cdf else None)


@dataclasses.dataclass
class BatchResult:
    accepted_count: np.ndarray   # int32 [B]
    emitted_tokens: np.ndarray   # int32 [sum(gamma_b+1)]: n_b + 1 tokens, then -1
    residual_sum: np.ndarray     # float64 [B]
    p_draft: np.ndarray          # float64 [sum gamma_b] (NaN in greedy mode / invalid ids)
    seq: List[SequenceResult]


def verify_batch(logits_f64, q, draft_ids, uniforms, cu_gamma, T: float,
                 keep_cdf: bool = False, only=None) -> BatchResult:
    """Apply verify_sequence to every sequence of a packed batch.

    logits_f64: [sum(gamma_b+1), V] (any float dtype; read as float64), or a
    callable rows -> float64 array, so huge batches need not be widened whole.
    Packing: logits row of (b, i) = cu_gamma[b] + b + i; q / id row = cu_gamma[b] + i.
    only: optional iterable of sequence indices to verify (others left at -1 / NaN).
    """
    cu = np.asarray(cu_gamma, dtype=np.int64)
    B = len(cu) - 1
    R = int(cu[-1])
    get = logits_f64 if callable(logits_f64) else (lambda rows: np.asarray(logits_f64[rows], dtype=np.float64))
    acc = np.full(B, -1, dtype=np.int32)
    emitted = np.full(R + B, -1, dtype=np.int32)
    S = np.full(B, np.nan)
    pd = np.full(R, np.nan)
    seqs: List[Optional[SequenceResult]] = [None] * B
    for b in (range(B) if only is None else only):
        g = int(cu[b + 1] - cu[b])
        base = int(cu[b])
        rows = slice(base + b, base + b + g + 1)
        res = verify_sequence(get(rows),
                              None if T == 0.0 else q[base:base + g],
                              draft_ids[base:base + g],
                              None if T == 0.0 else uniforms[base + b:base + b + g + 1],
                              T, keep_cdf=keep_cdf)
        acc[b] = res.n
        emitted[base + b:base + b + res.n + 1] = res.tokens
        S[b] = res.S
        if res.p_draft:
            pd[base:base + len(res.p_draft)] = res.p_draft
        seqs[b] = res
    return BatchResult(acc, emitted, S, pd, seqs)


def acceptance_rate(p, q) -> float:
    """alpha = E_{x~q}[min(1, p(x)/q(x))] = sum_v min(p, q).

    [P3] 예상 수용 길이 (alpha as the expected acceptance); [P1] ch.3 proof
    (total rejection probability 1 - sum min(q, p)).
    """
    return float(np.sum(np.minimum(np.asarray(p, np.float64), np.asarray(q, np.float64))))


def expected_tokens_per_round(alpha: float, gamma: int) -> float:
    """E = (1 - alpha^(gamma+1)) / (1 - alpha), tokens per round (accepted + 1).

    [P1] ch.4 (formula and table); [P2] "품질은 rejection sampling이 지킨다";
    [P3] 예상 수용 길이; [P4] "이득의 크기는 두 숫자가 정한다" (the +1).
    At alpha = 1 every draft is accepted: gamma + 1.
    """
    if alpha == 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def speedup_factor(alpha: float, gamma: int, c: float) -> float:
    """Wall-time factor E / (gamma * c + 1), c = draft cost / target cost.

    [P1] ch.4 (second table); [P2] (3.4 / 1.2); [P4] "이득의 크기는 두 숫자가 정한다".
    Only checked against the pages' numbers; it needs model costs otherwise.
    """
    return expected_tokens_per_round(alpha, gamma) / (gamma * c + 1.0)
