"""Torch-facing wrapper over the C ABI: checks tensors, allocates outputs, passes the stream.

Torch supplies device memory and the current HIP stream only; the computation
is the library's.
"""
from __future__ import annotations

from typing import NamedTuple, Optional

from .binding import (SV_BF16, SV_EDATA, SV_F32, spec_verify_create, spec_verify_destroy,
                      spec_verify_kernel_times, spec_verify_last_error, spec_verify_last_path,
                      spec_verify_run, spec_verify_run_bound, spec_verify_set_path, spec_verify_set_timing,
                      spec_verify_set_timing_stride, spec_verify_status, spec_sample_run,
                      spec_verify_run_onehot, spec_ngram_propose, spec_adapt_gamma,
                      SV_SAMPLE_LOGITS, SV_SAMPLE_WEIGHTS, spec_vshard_rows, spec_vshard_decide,
                      spec_vshard_finish, vshard_desc, VSHARD_LOCAL_DOUBLES, VSHARD_PART_DOUBLES)


class VerifyOutputs(NamedTuple):
    accepted_count: "torch.Tensor"   # int32 [B]
    emitted_tokens: "torch.Tensor"   # int32 [sum(gamma_b + 1)]
    residual_sum: "torch.Tensor"     # float32 [B]
    p_draft: Optional["torch.Tensor"]  # float32 [sum gamma_b] or None


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


class Verifier:
    """One library context on one device, sized by the max_* arguments."""

    def __init__(self, vocab: int, logits_dtype, max_batch: int, max_draft_rows: int,
                 max_gamma: int, device: int = 0):
        import torch
        self.device = torch.device("cuda", device)
        code = logits_dtype if isinstance(logits_dtype, int) else (
            SV_BF16 if logits_dtype == torch.bfloat16 else SV_F32)
        self.vocab, self.dtype_code = vocab, code
        self.max_batch, self.max_draft_rows, self.max_gamma = max_batch, max_draft_rows, max_gamma
        self.ctx = spec_verify_create(device, vocab, code, max_batch, max_draft_rows, max_gamma)

    # ------------------------------------------------------------------
    def _check(self, name, t, dtype, numel=None):
        import torch
        if t is None:
            return
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
        if t.device != self.device:
            raise ValueError(f"{name} is on {t.device}, expected {self.device}")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if numel is not None and t.numel() != numel:
            raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")

    def run(self, logits, draft_ids, *, temperature: float, q=None, uniforms=None,
            gamma: Optional[int] = None, cu_gamma=None, total_draft_rows: Optional[int] = None,
            out: Optional[VerifyOutputs] = None, want_p_draft: bool = True,
            stream=None, onehot: bool = False) -> VerifyOutputs:
        """Enqueue one verification step on `stream` (default: torch's current stream).

        Uniform gamma: pass `gamma`. Ragged: pass `cu_gamma` (int32 [B+1] on the device)
        and the host value `total_draft_rows` (defaults to draft_ids.numel()).
        onehot=True: deterministic drafts, q = one-hot(draft); `q` is not passed.
        """
        import torch
        if _dtype_code(logits) != self.dtype_code:
            raise TypeError("logits dtype differs from the context's")
        V = self.vocab
        if cu_gamma is not None:
            self._check("cu_gamma", cu_gamma, torch.int32)
            B = cu_gamma.numel() - 1
            R = int(total_draft_rows if total_draft_rows is not None else draft_ids.numel())
            g_arg = -1
        else:
            if gamma is None:
                raise ValueError("pass gamma or cu_gamma")
            B = logits.numel() // ((gamma + 1) * V)
            R = B * gamma
            g_arg = gamma
        self._check("logits", logits, None, (R + B) * V)
        self._check("draft_ids", draft_ids, torch.int32, R)
        greedy = float(temperature) == 0.0
        if not greedy and not onehot:
            self._check("q", q, torch.float32, R * V)
        if not greedy:
            self._check("uniforms", uniforms, torch.float32, R + B)
        if out is None:
            dev = self.device
            out = VerifyOutputs(
                torch.empty(B, dtype=torch.int32, device=dev),
                torch.empty(R + B, dtype=torch.int32, device=dev),
                torch.empty(B, dtype=torch.float32, device=dev),
                torch.empty(R, dtype=torch.float32, device=dev) if (want_p_draft and not greedy) else None)
        self._check("accepted_count", out.accepted_count, torch.int32, B)
        self._check("emitted_tokens", out.emitted_tokens, torch.int32, R + B)
        self._check("residual_sum", out.residual_sum, torch.float32, B)
        self._check("p_draft", out.p_draft, torch.float32, R)
        st = stream if stream is not None else torch.cuda.current_stream(self.device)
        if onehot:
            spec_verify_run_onehot(self.ctx, st, B, g_arg, cu_gamma, R, float(temperature), logits, draft_ids,
                                   None if greedy else uniforms, out.accepted_count, out.emitted_tokens,
                                   out.residual_sum, out.p_draft)
        else:
            spec_verify_run(self.ctx, st, B, g_arg, cu_gamma, R, float(temperature), logits,
                            None if greedy else q, draft_ids, None if greedy else uniforms,
                            out.accepted_count, out.emitted_tokens, out.residual_sum, out.p_draft)
        return out

    def bind(self, logits, draft_ids, *, temperature: float, q=None, uniforms=None,
             gamma: Optional[int] = None, cu_gamma=None, total_draft_rows: Optional[int] = None,
             out: VerifyOutputs, stream=None):
        """The checks of run() once, then a function of no arguments that enqueues that
        same step (same tensors, same stream) each time it is called. The tensors must stay
        alive and in place while the function is used."""
        import torch
        self.run(logits, draft_ids, temperature=temperature, q=q, uniforms=uniforms, gamma=gamma,
                 cu_gamma=cu_gamma, total_draft_rows=total_draft_rows, out=out, stream=stream)
        st = stream if stream is not None else torch.cuda.current_stream(self.device)
        greedy = float(temperature) == 0.0
        if cu_gamma is not None:
            B = cu_gamma.numel() - 1
            R = int(total_draft_rows if total_draft_rows is not None else draft_ids.numel())
            g_arg = -1
        else:
            B = logits.numel() // ((gamma + 1) * self.vocab)
            R, g_arg = B * gamma, gamma
        return spec_verify_run_bound(self.ctx, st, B, g_arg, cu_gamma, R, float(temperature), logits,
                                     None if greedy else q, draft_ids, None if greedy else uniforms,
                                     out.accepted_count, out.emitted_tokens, out.residual_sum, out.p_draft)

    def sample(self, x, *, uniforms=None, temperature: float = 1.0, tokens=None, stream=None):
        """One token per row of logits `x` ([rows, V], the context's dtype): p = softmax(l / T),
        T = 0 takes the argmax. Returns the int32 tokens tensor."""
        import torch
        if _dtype_code(x) != self.dtype_code:
            raise TypeError("logits dtype differs from the context's")
        return self._sample(x, SV_SAMPLE_LOGITS, uniforms, temperature, tokens, stream)

    def sample_weights(self, w, *, uniforms, tokens=None, stream=None):
        """One token per row of fp32 weights `w` ([rows, V], >= 0, not necessarily normalised)."""
        import torch
        self._check("weights", w, torch.float32)
        return self._sample(w, SV_SAMPLE_WEIGHTS, uniforms, 1.0, tokens, stream)

    def _sample(self, x, mode, uniforms, temperature, tokens, stream):
        import torch
        if not x.is_contiguous() or x.numel() % self.vocab:
            raise ValueError("x must be a contiguous [rows, V] tensor")
        rows = x.numel() // self.vocab
        if mode == SV_SAMPLE_WEIGHTS or float(temperature) != 0.0:
            self._check("uniforms", uniforms, torch.float32, rows)
        if tokens is None:
            tokens = torch.empty(rows, dtype=torch.int32, device=self.device)
        self._check("tokens", tokens, torch.int32, rows)
        st = stream if stream is not None else torch.cuda.current_stream(self.device)
        spec_sample_run(self.ctx, st, rows, mode, float(temperature), x,
                        None if (mode == SV_SAMPLE_LOGITS and float(temperature) == 0.0) else uniforms, tokens)
        return tokens

    def propose_ngram(self, tokens, cu_ctx, *, gamma: int, n_min: int = 1, n_max: int = 4,
                      total_tokens: Optional[int] = None, draft_ids=None, draft_len=None, stream=None):
        """Prompt-lookup drafts for B packed contexts (tokens int32, cu_ctx int32 [B+1] on the
        device; total_tokens defaults to tokens.numel()). Returns (draft_ids int32 [B, gamma]
        with -1 after each proposal, draft_len int32 [B]); the ids feed run(..., onehot=True)."""
        import torch
        self._check("tokens", tokens, torch.int32)
        self._check("cu_ctx", cu_ctx, torch.int32)
        B = cu_ctx.numel() - 1
        total = int(tokens.numel() if total_tokens is None else total_tokens)
        if draft_ids is None:
            draft_ids = torch.empty((B, gamma), dtype=torch.int32, device=self.device)
        if draft_len is None:
            draft_len = torch.empty(B, dtype=torch.int32, device=self.device)
        self._check("draft_ids", draft_ids, torch.int32, B * gamma)
        self._check("draft_len", draft_len, torch.int32, B)
        st = stream if stream is not None else torch.cuda.current_stream(self.device)
        spec_ngram_propose(self.ctx, st, B, tokens, cu_ctx, total, n_min, n_max, gamma, draft_ids, draft_len)
        return draft_ids, draft_len

    def adapt_gamma(self, accepted_count, gamma, streak, *, gamma_max: int, up_after: int = 1,
                    down_after: int = 2, cu_gamma_next=None, stream=None):
        """Next round's draft lengths from this round's accepted counts: `gamma` and `streak`
        (int32 [B] on the device) are updated in place; returns cu_gamma_next (int32 [B+1])."""
        import torch
        B = gamma.numel()
        self._check("accepted_count", accepted_count, torch.int32, B)
        self._check("gamma", gamma, torch.int32, B)
        self._check("streak", streak, torch.int32, B)
        if cu_gamma_next is None:
            cu_gamma_next = torch.empty(B + 1, dtype=torch.int32, device=self.device)
        self._check("cu_gamma_next", cu_gamma_next, torch.int32, B + 1)
        st = stream if stream is not None else torch.cuda.current_stream(self.device)
        spec_adapt_gamma(self.ctx, st, B, accepted_count, gamma, streak, gamma_max, up_after, down_after,
                         cu_gamma_next)
        return cu_gamma_next

    def status(self) -> int:
        """SV_OK, or SV_EDATA when the device flagged a data error (see last_error)."""
        return spec_verify_status(self.ctx)

    def data_error(self) -> Optional[str]:
        return spec_verify_last_error(self.ctx) if self.status() == SV_EDATA else None

    def last_error(self) -> str:
        return spec_verify_last_error(self.ctx)

    def set_timing(self, runs: int, stride: int = 1):
        """Record per-kernel events for `runs` of the next runs, one in every `stride` (0 runs: off)."""
        spec_verify_set_timing(self.ctx, runs)
        spec_verify_set_timing_stride(self.ctx, stride)

    def kernel_times(self):
        """([(kernel, mean ms), ...], runs) over the recorded runs."""
        return spec_verify_kernel_times(self.ctx)

    def set_path(self, mode: int):
        """Launch plan for the next runs: SV_PATH_AUTO, SV_PATH_TWO_LAUNCH or SV_PATH_ONE_LAUNCH."""
        spec_verify_set_path(self.ctx, mode)

    def last_path(self) -> int:
        return spec_verify_last_path(self.ctx)

    def close(self):
        if getattr(self, "ctx", None):
            spec_verify_destroy(self.ctx)
            self.ctx = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class VocabShard:
    """One shard of vocabulary-parallel verification (spec_vshard_* in spec_verify.h):
    a context for this shard's columns [bounds[k], bounds[k + 1]) and the three steps of
    a round. Between the steps the caller gathers every shard's records in shard order
    (over RCCL across devices, or by concatenation when the shards share one device)."""

    def __init__(self, bounds, shard: int, logits_dtype, max_batch: int, max_draft_rows: int,
                 max_gamma: int, device: int = 0):
        self.bounds = [int(x) for x in bounds]
        self.shard = int(shard)
        self.width = self.bounds[self.shard + 1] - self.bounds[self.shard]
        self.ver = Verifier(self.width, logits_dtype, max_batch, max_draft_rows, max_gamma, device)
        self.desc, self._bounds_arr = vshard_desc(self.bounds, self.shard)

    def _geom(self, logits, draft_ids, gamma, cu_gamma, total_draft_rows):
        import torch
        v = self.ver
        if _dtype_code(logits) != v.dtype_code:
            raise TypeError("logits dtype differs from the context's")
        if cu_gamma is not None:
            v._check("cu_gamma", cu_gamma, torch.int32)
            B = cu_gamma.numel() - 1
            R = int(total_draft_rows if total_draft_rows is not None else draft_ids.numel())
            g_arg = -1
        else:
            if gamma is None:
                raise ValueError("pass gamma or cu_gamma")
            B = logits.numel() // ((gamma + 1) * self.width)
            R = B * gamma
            g_arg = gamma
        v._check("logits", logits, None, (R + B) * self.width)
        v._check("draft_ids", draft_ids, torch.int32, R)
        return B, R, g_arg

    def rows(self, logits, draft_ids, *, temperature: float, q=None, gamma=None, cu_gamma=None,
             total_draft_rows=None, rec=None, stream=None):
        """Step 1: this shard's 16-byte record per judged row, as float32 [records, 4]."""
        import torch
        B, R, g_arg = self._geom(logits, draft_ids, gamma, cu_gamma, total_draft_rows)
        greedy = float(temperature) == 0.0
        if not greedy:
            self.ver._check("q", q, torch.float32, R * self.width)
        n = R + (B if greedy else 0)
        if rec is None:
            rec = torch.empty((n, 4), dtype=torch.float32, device=self.ver.device)
        self.ver._check("rec", rec, torch.float32, n * 4)
        st = stream if stream is not None else torch.cuda.current_stream(self.ver.device)
        spec_vshard_rows(self.ver.ctx, st, self.desc, B, g_arg, cu_gamma, R, float(temperature), logits,
                         None if greedy else q, draft_ids, rec)
        return rec

    def decide(self, logits, draft_ids, rec_all, *, temperature: float, q=None, uniforms=None, gamma=None,
               cu_gamma=None, total_draft_rows=None, out: Optional[VerifyOutputs] = None,
               want_p_draft: bool = True, stream=None):
        """Step 2: the decisions from every shard's records (rec_all: the gathered
        records, shard by shard) and this shard's sums of each drawn row. Returns
        (outputs, part, local): part (fp64 [B, 3]) is exchanged, local (fp64 [B, 52])
        stays for step 3. At T = 0 every output is final here."""
        import torch
        B, R, g_arg = self._geom(logits, draft_ids, gamma, cu_gamma, total_draft_rows)
        greedy = float(temperature) == 0.0
        G = len(self.bounds) - 1
        self.ver._check("rec_all", rec_all, torch.float32, G * (R + (B if greedy else 0)) * 4)
        if not greedy:
            self.ver._check("q", q, torch.float32, R * self.width)
            self.ver._check("uniforms", uniforms, torch.float32, R + B)
        dev = self.ver.device
        if out is None:
            out = VerifyOutputs(
                torch.empty(B, dtype=torch.int32, device=dev),
                torch.empty(R + B, dtype=torch.int32, device=dev),
                torch.empty(B, dtype=torch.float32, device=dev),
                torch.empty(R, dtype=torch.float32, device=dev) if (want_p_draft and not greedy) else None)
        part = local = None
        if not greedy:
            part = torch.empty((B, VSHARD_PART_DOUBLES), dtype=torch.float64, device=dev)
            local = torch.empty((B, VSHARD_LOCAL_DOUBLES), dtype=torch.float64, device=dev)
        st = stream if stream is not None else torch.cuda.current_stream(dev)
        spec_vshard_decide(self.ver.ctx, st, self.desc, B, g_arg, cu_gamma, R, float(temperature), logits,
                           None if greedy else q, draft_ids, None if greedy else uniforms, rec_all,
                           out.accepted_count, out.emitted_tokens, out.residual_sum, out.p_draft, part, local)
        return out, part, local

    def finish(self, logits, part_all, local, out: VerifyOutputs, *, temperature: float, q=None, uniforms=None,
               gamma=None, cu_gamma=None, total_draft_rows=None, stream=None):
        """Step 3: the shard that owns a sequence's drawn token writes it, the -1 padding
        and S into `out`; other shards leave those entries as they are."""
        import torch
        if float(temperature) == 0.0:
            return out
        if cu_gamma is None:
            B = logits.numel() // ((gamma + 1) * self.width)
            R, g_arg = B * gamma, gamma
        else:
            B, R, g_arg = cu_gamma.numel() - 1, int(total_draft_rows), -1
        G = len(self.bounds) - 1
        self.ver._check("part_all", part_all, torch.float64, G * B * VSHARD_PART_DOUBLES)
        self.ver._check("local", local, torch.float64, B * VSHARD_LOCAL_DOUBLES)
        self.ver._check("q", q, torch.float32, R * self.width)
        self.ver._check("uniforms", uniforms, torch.float32, R + B)
        st = stream if stream is not None else torch.cuda.current_stream(self.ver.device)
        spec_vshard_finish(self.ver.ctx, st, self.desc, B, g_arg, cu_gamma, R, float(temperature), logits, q,
                           uniforms, part_all, local, out.emitted_tokens, out.residual_sum)
        return out

    def status(self) -> int:
        return self.ver.status()

    def last_error(self) -> str:
        return self.ver.last_error()

    def close(self):
        self.ver.close()

