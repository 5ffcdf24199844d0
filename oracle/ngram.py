"""CPU oracle for the n-gram (prompt-lookup) draft proposer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or load
this module: only the tests, the smoke check and the benchmark's CPU-baseline leg
use it. It shares no code with the HIP library.

What it computes, from the pages:
  [P1] "Speculative Decoding", atonlee.tistory.com/330, ch.5 "draft model에서
       EAGLE·MTP·n-gram까지" (prompt lookup): with no model at all, look in the
       context so far for the string the current suffix forms and take the tokens
       that followed it there as the drafts.
  [P2] "Speculative Decoding으로 LLM 추론 속도 높이기", donmain.dev, "draft를 어디서
       구하는가": the last few generated tokens are searched for in the prompt and
       the tokens after the matched place become the draft.
  [P4] "투기적 디코딩 — 초안 모델을 무엇으로 세울 것인가", ailab.paldyn.com, "네 가지
       방식" (n-gram lookup: match the most recent tokens against the earlier
       context, copy what came after).

Readings where the pages leave a step open (also listed in the design notes):
  * The suffix length n is tried from n_max down to n_min; the first n whose
    suffix occurs earlier wins (a longer match is the more specific evidence).
  * "Earlier" means an occurrence that ends before the last token of the context:
    it starts at some j <= L - n - 1, so at least one token follows it. It may
    overlap the suffix itself (periodic text).
  * Among the occurrences of that suffix the most recent one (largest j) is used.
  * The proposal is the tokens that follow the occurrence, at most gamma of them;
    it is shorter when the context ends first, and empty when no n in
    [n_min, n_max] matches.
"""
from __future__ import annotations

import numpy as np

__all__ = ["ngram_propose", "ngram_propose_batch"]


def ngram_propose(context, n_min: int, n_max: int, gamma: int) -> np.ndarray:
    """Drafts proposed for one context (int64 array, length 0..gamma).

    context: 1-D sequence of token ids. For n = n_max .. n_min: the suffix
    s = context[L-n:] is compared with every window context[j:j+n] for
    j = 0 .. L-n-1 (a library comparison over all windows); the largest matching
    j gives context[j+n : j+n+gamma].
    """
    c = np.asarray(context, dtype=np.int64).reshape(-1)
    L = c.size
    if gamma <= 0 or L < 2:
        return np.zeros(0, dtype=np.int64)
    for n in range(min(n_max, L - 1), n_min - 1, -1):
        if n < 1:
            break
        suffix = c[L - n:]
        windows = np.lib.stride_tricks.sliding_window_view(c[:L - 1], n)  # starts j = 0 .. L-n-1
        hits = np.flatnonzero(np.all(windows == suffix, axis=1))
        if hits.size:
            j = int(hits[-1])
            return c[j + n: j + n + gamma].copy()
    return np.zeros(0, dtype=np.int64)


def ngram_propose_batch(tokens, cu_ctx, n_min: int, n_max: int, gamma: int):
    """Every context of a packed batch (tokens[cu_ctx[b]:cu_ctx[b+1]]).

    Returns (draft_ids int32 [B, gamma] with -1 after each proposal, draft_len int32 [B]).
    """
    cu = np.asarray(cu_ctx, dtype=np.int64)
    B = cu.size - 1
    ids = np.full((B, max(gamma, 0)), -1, dtype=np.int32)
    lens = np.zeros(B, dtype=np.int32)
    t = np.asarray(tokens)
    for b in range(B):
        p = ngram_propose(t[cu[b]:cu[b + 1]], n_min, n_max, gamma)
        ids[b, :p.size] = p
        lens[b] = p.size
    return ids, lens
