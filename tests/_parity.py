"""Parity harness: run the HIP library through its C ABI and compare with the oracle.

Comparison rule (the bar):
  * accepted counts and token ids must match exactly, except a FLAGGED case: a
    sequence where the two differ and the oracle's uniform at the first
    differing decision lies within 1e-6 relative of a threshold that separates
    the two answers. For an accept decision that is |u_i - thr_i| <= 1e-6 thr_i;
    for a drawn token it is some prefix boundary C[k], k between the two tokens,
    with |t - C[k]| <= 1e-6 t.
  * unflagged mismatches must be 0 and flagged cases < 1e-5 of sequences;
  * greedy mode has no thresholds: any mismatch fails;
  * p(x_i) (p_draft) and the residual sum S must match within 1e-5 relative for
    fp32 logits and 2e-3 for bf16 logits (S below 1e-3 is judged with an
    absolute 1e-8 instead).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

import oracle as O

FLAG_WINDOW = 1e-6
FLAGGED_RATE_MAX = 1e-5


def tolerance(dtype: str) -> float:
    return 1e-5 if dtype == "f32" else 2e-3


def to_device(w, device="cuda", with_q=True):
    """Host workload -> dict of device tensors (the layout of the C ABI)."""
    import torch
    d = {}
    if w.dtype == "bf16":
        d["logits"] = torch.from_numpy(w.logits.view(np.int16)).view(torch.bfloat16).to(device)
    else:
        d["logits"] = torch.from_numpy(w.logits).to(device)
    d["q"] = torch.from_numpy(w.q).to(device) if (w.q is not None and with_q) else None
    d["draft_ids"] = torch.from_numpy(w.draft_ids).to(device)
    d["uniforms"] = torch.from_numpy(w.uniforms).to(device) if w.uniforms is not None else None
    d["cu_gamma"] = torch.from_numpy(w.cu_gamma).to(device)
    return d


def run_gpu(verifier, w, dev=None, ragged=None, want_p_draft=True, onehot=False):
    """Run the library on workload w; returns host numpy outputs and the status code.
    onehot: the drafts are deterministic (q = one-hot(draft)) and q is not passed."""
    import torch
    dev = dev or to_device(w, with_q=not onehot)
    if ragged is None:
        ragged = w.uniform_gamma is None
    kw = dict(temperature=w.T, q=None if onehot else dev["q"], uniforms=dev["uniforms"],
              want_p_draft=want_p_draft, onehot=onehot)
    if ragged:
        out = verifier.run(dev["logits"], dev["draft_ids"], cu_gamma=dev["cu_gamma"],
                           total_draft_rows=w.draft_rows, **kw)
    else:
        out = verifier.run(dev["logits"], dev["draft_ids"], gamma=w.uniform_gamma, **kw)
    torch.cuda.synchronize()
    status = verifier.status()
    res = dict(
        accepted_count=out.accepted_count.cpu().numpy(),
        emitted_tokens=out.emitted_tokens.cpu().numpy(),
        residual_sum=out.residual_sum.cpu().numpy(),
        p_draft=out.p_draft.cpu().numpy() if out.p_draft is not None else None,
        status=status,
    )
    return res


def oracle_batch(w, only=None, keep_cdf=False):
    return O.verify_batch(lambda rows: w.logits_f64(rows), w.q, w.draft_ids, w.uniforms,
                          w.cu_gamma, w.T, keep_cdf=keep_cdf, only=only)


@dataclasses.dataclass
class ParityReport:
    sequences: int = 0
    exact: int = 0
    flagged: int = 0
    unflagged: list = dataclasses.field(default_factory=list)
    p_rel_max: float = 0.0
    s_rel_max: float = 0.0
    p_bad: int = 0
    s_bad: int = 0
    pad_bad: int = 0
    notes: list = dataclasses.field(default_factory=list)

    def ok(self) -> bool:
        return (not self.unflagged and self.p_bad == 0 and self.s_bad == 0 and self.pad_bad == 0
                and self.flagged <= math.floor(FLAGGED_RATE_MAX * self.sequences))

    def summary(self) -> str:
        return (f"sequences={self.sequences} exact={self.exact} flagged={self.flagged} "
                f"unflagged={len(self.unflagged)} p_rel_max={self.p_rel_max:.3g} "
                f"S_rel_max={self.s_rel_max:.3g} p_bad={self.p_bad} S_bad={self.s_bad} pad_bad={self.pad_bad}"
                + (f" first_unflagged={self.unflagged[:5]}" if self.unflagged else ""))


def compare(w, gpu, ora: "O.BatchResult", check_p_draft=True) -> ParityReport:
    rep = ParityReport(sequences=w.B)
    tol = tolerance(w.dtype)
    cu = w.cu_gamma.astype(np.int64)
    for b in range(w.B):
        g = int(cu[b + 1] - cu[b])
        base = int(cu[b])
        s0 = base + b
        n_o, n_g = int(ora.accepted_count[b]), int(gpu["accepted_count"][b])
        em_o = ora.emitted_tokens[s0:s0 + g + 1]
        em_g = gpu["emitted_tokens"][s0:s0 + g + 1]
        seq = ora.seq[b]
        if n_o == n_g and np.array_equal(em_o, em_g):
            rep.exact += 1
            if w.T > 0 and seq.mode in ("residual", "degenerate"):
                S_o, S_g = float(ora.residual_sum[b]), float(gpu["residual_sum"][b])
                err = abs(S_g - S_o)
                rel = err / abs(S_o) if S_o != 0 else err
                rep.s_rel_max = max(rep.s_rel_max, rel if abs(S_o) >= 1e-3 else 0.0)
                if (abs(S_o) >= 1e-3 and rel > tol) or (abs(S_o) < 1e-3 and err > 1e-8):
                    rep.s_bad += 1
            elif float(gpu["residual_sum"][b]) != 0.0:
                rep.s_bad += 1
            continue
        if w.T == 0.0:
            rep.unflagged.append((b, "greedy", n_o, n_g))
            continue
        if np.any(em_g[n_g + 1:] != -1):
            rep.pad_bad += 1
        if n_o != n_g:
            i = min(n_o, n_g)
            if i >= len(seq.thresholds) or not np.isfinite(seq.thresholds[i]):
                rep.unflagged.append((b, "accept-noinfo", n_o, n_g))
                continue
            thr = seq.thresholds[i]
            u = float(w.uniforms[s0 + i])
            if abs(u - thr) <= FLAG_WINDOW * thr:
                rep.flagged += 1
                rep.notes.append((b, "accept", u, thr))
            else:
                rep.unflagged.append((b, "accept", n_o, n_g, u, thr))
            continue
        # same n: accepted drafts must agree; only the drawn token may differ
        if not np.array_equal(em_o[:n_o], em_g[:n_g]):
            rep.unflagged.append((b, "prefix"))
            continue
        tok_o, tok_g = int(em_o[n_o]), int(em_g[n_g])
        full = oracle_batch(w, only=[b], keep_cdf=True).seq[b]
        C, t = full.C, full.t
        lo, hi = min(tok_o, tok_g), max(tok_o, tok_g)
        if 0 <= lo < len(C) and hi <= len(C) and t > 0 and np.any(np.abs(t - C[lo:hi]) <= FLAG_WINDOW * t):
            rep.flagged += 1
            rep.notes.append((b, "draw", tok_o, tok_g))
        else:
            rep.unflagged.append((b, "draw", tok_o, tok_g, full.mode))
    if check_p_draft and w.T > 0 and gpu.get("p_draft") is not None:
        po, pg = ora.p_draft, gpu["p_draft"].astype(np.float64)
        fin = np.isfinite(po)
        if np.any(np.isfinite(pg[~fin])):
            rep.p_bad += int(np.sum(np.isfinite(pg[~fin])))
        denom = np.where(po[fin] > 0, po[fin], 1.0)
        rel = np.abs(pg[fin] - po[fin]) / denom
        small = po[fin] < 1e-30
        rel = np.where(small, np.abs(pg[fin] - po[fin]), rel)
        if rel.size:
            rep.p_rel_max = float(rel.max())
            rep.p_bad += int(np.sum(rel > tol))
    return rep
