"""ctypes binding of libspecverify.so (argument marshalling only).

The functions here carry the C ABI's names and arguments (include/spec_verify.h).
Device buffers may be given as torch tensors (their data_ptr is passed) or as
raw integer device addresses. Every step of the verification runs in the HIP
kernels of the library; there is no other code path. If the library is missing
the calls raise: build it with `python -m speculative_sampling_verification_03_amd.build`.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libspecverify.so")

SV_OK, SV_EINVAL, SV_ENOMEM, SV_EHIP, SV_EDATA = 0, 1, 2, 3, 4
SV_F32, SV_BF16 = 0, 1
SV_DATA_DRAFT_ID, SV_DATA_NONFINITE, SV_DATA_UNIFORM, SV_DATA_CU_GAMMA, SV_DATA_CONTEXT, SV_DATA_STATE = \
    1, 2, 4, 8, 16, 32
SV_DATA_STALL = 64
SV_NGRAM_MAX_N = 64
SV_PATH_AUTO, SV_PATH_TWO_LAUNCH, SV_PATH_ONE_LAUNCH, SV_PATH_POOLED = 0, 1, 2, 3
SV_SAMPLE_LOGITS, SV_SAMPLE_WEIGHTS = 0, 1
_CODE_NAMES = {SV_OK: "SV_OK", SV_EINVAL: "SV_EINVAL", SV_ENOMEM: "SV_ENOMEM",
               SV_EHIP: "SV_EHIP", SV_EDATA: "SV_EDATA"}

EXPORTED = (
    "spec_verify_create", "spec_verify_run", "spec_verify_status",
    "spec_verify_last_error", "spec_verify_destroy", "spec_verify_set_timing",
    "spec_verify_kernel_times", "spec_verify_check_args", "spec_verify_set_path", "spec_verify_set_timing_stride",
    "spec_verify_last_path", "spec_sample_run", "spec_verify_run_onehot", "spec_ngram_propose",
    "spec_adapt_gamma", "spec_vshard_rows", "spec_vshard_decide", "spec_vshard_finish",
    "spec_verify_run_static",
)
SV_STATIC_MAX_BATCH, SV_STATIC_MAX_ROWS, SV_STATIC_MAX_GAMMA = 1024, 16384, 64


class SpecVerifyError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_CODE_NAMES.get(code, code)}: {msg}")
        self.code = code


_lib = None

# Sizes of the vocabulary-shard exchange records (include/spec_verify.h).
VSHARD_REC_BYTES = 16      # per judged row
VSHARD_PART_DOUBLES = 3    # per sequence, exchanged
VSHARD_LOCAL_DOUBLES = 52  # per sequence, kept on the shard's device


class VShardDesc(ctypes.Structure):
    """struct spec_vshard: vocab_total, shards, shard, bounds (host int32 [shards + 1])."""
    _fields_ = [("vocab_total", ctypes.c_int), ("shards", ctypes.c_int), ("shard", ctypes.c_int),
                ("bounds", ctypes.POINTER(ctypes.c_int32))]


def vshard_desc(bounds, shard: int):
    """A spec_vshard for shard `shard` of the column bounds `bounds` (a sequence of ints);
    returns the struct and the array it points to (keep both alive)."""
    arr = (ctypes.c_int32 * len(bounds))(*[int(x) for x in bounds])
    return VShardDesc(int(bounds[-1]), len(bounds) - 1, int(shard), arr), arr


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libspecverify.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(
            f"{p} is missing: build it with `python -m speculative_sampling_verification_03_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.spec_verify_create.argtypes = [ctypes.POINTER(vp), i32, i32, i32, i32, i32, i32]
    lib.spec_verify_create.restype = i32
    lib.spec_verify_run.argtypes = [vp, vp, i32, i32, vp, i32, f32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.spec_verify_run.restype = i32
    lib.spec_verify_status.argtypes = [vp]
    lib.spec_verify_status.restype = i32
    lib.spec_verify_last_error.argtypes = [vp]
    lib.spec_verify_last_error.restype = ctypes.c_char_p
    lib.spec_verify_destroy.argtypes = [vp]
    lib.spec_verify_destroy.restype = None
    lib.spec_verify_set_timing.argtypes = [vp, i32]
    lib.spec_verify_set_timing.restype = i32
    lib.spec_verify_kernel_times.argtypes = [vp, ctypes.POINTER(f32), ctypes.POINTER(ctypes.c_char_p), i32,
                                             ctypes.POINTER(i32)]
    lib.spec_verify_kernel_times.restype = i32
    lib.spec_verify_check_args.argtypes = [i32] * 9 + [f32] + [i32] * 7 + [ctypes.c_char_p, i32]
    lib.spec_verify_check_args.restype = i32
    lib.spec_verify_run_static.argtypes = [i32, vp, i32, i32, i32, i32, vp, i32, f32, vp, vp, vp, vp, vp, vp, vp,
                                           vp, vp]
    lib.spec_verify_run_static.restype = i32
    lib.spec_verify_run_onehot.argtypes = [vp, vp, i32, i32, vp, i32, f32, vp, vp, vp, vp, vp, vp, vp]
    lib.spec_verify_run_onehot.restype = i32
    lib.spec_ngram_propose.argtypes = [vp, vp, i32, vp, vp, i32, i32, i32, i32, vp, vp]
    lib.spec_ngram_propose.restype = i32
    lib.spec_adapt_gamma.argtypes = [vp, vp, i32, vp, vp, vp, i32, i32, i32, vp]
    lib.spec_adapt_gamma.restype = i32
    lib.spec_vshard_rows.argtypes = [vp, vp, ctypes.POINTER(VShardDesc), i32, i32, vp, i32, f32, vp, vp, vp, vp]
    lib.spec_vshard_rows.restype = i32
    lib.spec_vshard_decide.argtypes = [vp, vp, ctypes.POINTER(VShardDesc), i32, i32, vp, i32, f32, vp, vp, vp,
                                       vp, vp, vp, vp, vp, vp, vp, vp]
    lib.spec_vshard_decide.restype = i32
    lib.spec_vshard_finish.argtypes = [vp, vp, ctypes.POINTER(VShardDesc), i32, i32, vp, i32, f32, vp, vp, vp,
                                       vp, vp, vp, vp]
    lib.spec_vshard_finish.restype = i32
    lib.spec_sample_run.argtypes = [vp, vp, i32, i32, f32, vp, vp, vp]
    lib.spec_sample_run.restype = i32
    lib.spec_verify_set_timing_stride.argtypes = [vp, i32]
    lib.spec_verify_set_timing_stride.restype = i32
    lib.spec_verify_set_path.argtypes = [vp, i32]
    lib.spec_verify_set_path.restype = i32
    lib.spec_verify_last_path.argtypes = [vp]
    lib.spec_verify_last_path.restype = i32
    if path is None:
        _lib = lib
    return lib


def _ptr(x) -> Optional[int]:
    """Device address of a torch tensor / integer address / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x or None
    return int(x.data_ptr()) or None


def _stream(s) -> Optional[int]:
    if s is None:
        return None
    if isinstance(s, int):
        return s or None
    return int(s.cuda_stream) or None


def _msg(ctx) -> str:
    return (load_library().spec_verify_last_error(ctx) or b"").decode()


def spec_verify_create(device: int, vocab: int, logits_dtype: int, max_batch: int,
                       max_draft_rows: int, max_gamma: int) -> int:
    """Returns the context handle (an integer); raises SpecVerifyError."""
    lib = load_library()
    out = ctypes.c_void_p()
    rc = lib.spec_verify_create(ctypes.byref(out), device, vocab, logits_dtype, max_batch,
                                max_draft_rows, max_gamma)
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_create failed")
    return out.value


def spec_verify_run(ctx: int, stream, batch: int, gamma: int, cu_gamma, total_draft_rows: int,
                    temperature: float, logits, q, draft_ids, uniforms, accepted_count,
                    emitted_tokens, residual_sum, p_draft=None) -> None:
    """Enqueue one verification step; raises SpecVerifyError on a non-OK code."""
    rc = load_library().spec_verify_run(
        ctx, _stream(stream), batch, gamma, _ptr(cu_gamma), total_draft_rows, float(temperature),
        _ptr(logits), _ptr(q), _ptr(draft_ids), _ptr(uniforms), _ptr(accepted_count),
        _ptr(emitted_tokens), _ptr(residual_sum), _ptr(p_draft))
    if rc != SV_OK:
        raise SpecVerifyError(rc, _msg(ctx))


def spec_verify_run_static(device: int, stream, vocab: int, logits_dtype: int, batch: int, gamma: int, cu_gamma,
                           total_draft_rows: int, temperature: float, logits, q, draft_ids, uniforms,
                           accepted_count, emitted_tokens, residual_sum, p_draft, data_flags) -> None:
    """Enqueue one verification step with no context and no allocation (the library's
    static workspace); data-error bits are OR-ed into data_flags. Raises SpecVerifyError."""
    lib = load_library()
    rc = lib.spec_verify_run_static(
        device, _stream(stream), vocab, logits_dtype, batch, gamma, _ptr(cu_gamma), total_draft_rows,
        float(temperature), _ptr(logits), _ptr(q), _ptr(draft_ids), _ptr(uniforms), _ptr(accepted_count),
        _ptr(emitted_tokens), _ptr(residual_sum), _ptr(p_draft), _ptr(data_flags))
    if rc != SV_OK:
        raise SpecVerifyError(rc, (lib.spec_verify_last_error(None) or b"").decode())


def spec_verify_run_bound(ctx: int, stream, batch: int, gamma: int, cu_gamma, total_draft_rows: int,
                          temperature: float, logits, q, draft_ids, uniforms, accepted_count,
                          emitted_tokens, residual_sum, p_draft=None):
    """spec_verify_run with its arguments marshalled once. Returns a function of no
    arguments that enqueues the same step (same buffers, same stream) each time it is
    called, so a loop of steps pays one foreign call per step and no conversions."""
    fn = load_library().spec_verify_run
    args = (ctx, _stream(stream), batch, gamma, _ptr(cu_gamma), total_draft_rows, float(temperature),
            _ptr(logits), _ptr(q), _ptr(draft_ids), _ptr(uniforms), _ptr(accepted_count),
            _ptr(emitted_tokens), _ptr(residual_sum), _ptr(p_draft))

    def go():
        rc = fn(*args)
        if rc != SV_OK:
            raise SpecVerifyError(rc, _msg(ctx))
    return go


def spec_verify_run_onehot(ctx: int, stream, batch: int, gamma: int, cu_gamma, total_draft_rows: int,
                           temperature: float, logits, draft_ids, uniforms, accepted_count,
                           emitted_tokens, residual_sum, p_draft=None) -> None:
    """Enqueue one verification step of deterministic drafts (q = one-hot(draft))."""
    rc = load_library().spec_verify_run_onehot(
        ctx, _stream(stream), batch, gamma, _ptr(cu_gamma), total_draft_rows, float(temperature),
        _ptr(logits), _ptr(draft_ids), _ptr(uniforms), _ptr(accepted_count), _ptr(emitted_tokens),
        _ptr(residual_sum), _ptr(p_draft))
    if rc != SV_OK:
        raise SpecVerifyError(rc, _msg(ctx))


def spec_vshard_rows(ctx: int, stream, desc, batch: int, gamma: int, cu_gamma, total_draft_rows: int,
                     temperature: float, logits, q, draft_ids, rec) -> None:
    """Step 1 of vocabulary-parallel verification on one shard (records of its columns)."""
    rc = load_library().spec_vshard_rows(ctx, _stream(stream), ctypes.byref(desc), batch, gamma, _ptr(cu_gamma),
                                         total_draft_rows, float(temperature), _ptr(logits), _ptr(q),
                                         _ptr(draft_ids), _ptr(rec))
    if rc != SV_OK:
        raise SpecVerifyError(rc, _msg(ctx))


def spec_vshard_decide(ctx: int, stream, desc, batch: int, gamma: int, cu_gamma, total_draft_rows: int,
                       temperature: float, logits, q, draft_ids, uniforms, rec_all, accepted_count,
                       emitted_tokens, residual_sum, p_draft, part, local) -> None:
    """Step 2: the decisions from every shard's records, and this shard's draw sums."""
    rc = load_library().spec_vshard_decide(
        ctx, _stream(stream), ctypes.byref(desc), batch, gamma, _ptr(cu_gamma), total_draft_rows,
        float(temperature), _ptr(logits), _ptr(q), _ptr(draft_ids), _ptr(uniforms), _ptr(rec_all),
        _ptr(accepted_count), _ptr(emitted_tokens), _ptr(residual_sum), _ptr(p_draft), _ptr(part), _ptr(local))
    if rc != SV_OK:
        raise SpecVerifyError(rc, _msg(ctx))


def spec_vshard_finish(ctx: int, stream, desc, batch: int, gamma: int, cu_gamma, total_draft_rows: int,
                       temperature: float, logits, q, uniforms, part_all, local, emitted_tokens,
                       residual_sum) -> None:
    """Step 3: the drawn token, written by the shard that owns it."""
    rc = load_library().spec_vshard_finish(
        ctx, _stream(stream), ctypes.byref(desc), batch, gamma, _ptr(cu_gamma), total_draft_rows,
        float(temperature), _ptr(logits), _ptr(q), _ptr(uniforms), _ptr(part_all), _ptr(local),
        _ptr(emitted_tokens), _ptr(residual_sum))
    if rc != SV_OK:
        raise SpecVerifyError(rc, _msg(ctx))


def spec_sample_run(ctx: int, stream, rows: int, mode: int, temperature: float, x, uniforms, tokens) -> None:
    """Enqueue one token per row drawn from logits (SV_SAMPLE_LOGITS) or fp32 weights
    (SV_SAMPLE_WEIGHTS); raises SpecVerifyError on a non-OK code."""
    rc = load_library().spec_sample_run(ctx, _stream(stream), rows, mode, float(temperature), _ptr(x),
                                        _ptr(uniforms), _ptr(tokens))
    if rc != SV_OK:
        raise SpecVerifyError(rc, _msg(ctx))


def spec_ngram_propose(ctx: int, stream, batch: int, tokens, cu_ctx, total_tokens: int, n_min: int,
                       n_max: int, gamma: int, draft_ids, draft_len) -> None:
    """Enqueue the prompt-lookup proposer; raises SpecVerifyError on a non-OK code."""
    rc = load_library().spec_ngram_propose(ctx, _stream(stream), batch, _ptr(tokens), _ptr(cu_ctx),
                                           total_tokens, n_min, n_max, gamma, _ptr(draft_ids),
                                           _ptr(draft_len))
    if rc != SV_OK:
        raise SpecVerifyError(rc, _msg(ctx))


def spec_adapt_gamma(ctx: int, stream, batch: int, accepted_count, gamma, streak, gamma_max: int,
                     up_after: int, down_after: int, cu_gamma_next) -> None:
    """Enqueue the adaptive draft-length update; raises SpecVerifyError on a non-OK code."""
    rc = load_library().spec_adapt_gamma(ctx, _stream(stream), batch, _ptr(accepted_count), _ptr(gamma),
                                         _ptr(streak), gamma_max, up_after, down_after, _ptr(cu_gamma_next))
    if rc != SV_OK:
        raise SpecVerifyError(rc, _msg(ctx))


def spec_verify_status(ctx: int) -> int:
    """Sync and read/clear the device data flag. Returns SV_OK or SV_EDATA; raises on others."""
    rc = load_library().spec_verify_status(ctx)
    if rc not in (SV_OK, SV_EDATA):
        raise SpecVerifyError(rc, _msg(ctx))
    return rc


def spec_verify_last_error(ctx: int) -> str:
    return _msg(ctx)


def spec_verify_destroy(ctx: Optional[int]) -> None:
    load_library().spec_verify_destroy(ctx)


def spec_verify_set_timing(ctx: int, runs: int) -> None:
    """Record per-kernel events for the next `runs` runs (0 switches recording off)."""
    rc = load_library().spec_verify_set_timing(ctx, int(runs))
    if rc != SV_OK:
        raise SpecVerifyError(rc, _msg(ctx))


def spec_verify_set_timing_stride(ctx: int, stride: int) -> None:
    """Record one run in every `stride` of the following runs."""
    rc = load_library().spec_verify_set_timing_stride(ctx, int(stride))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "bad stride" if ctx else "NULL context")


def spec_verify_kernel_times(ctx: int, cap: int = 8):
    """([(kernel name, mean ms), ...], recorded runs) over the runs recorded since
    spec_verify_set_timing / the previous call."""
    ms = (ctypes.c_float * cap)()
    names = (ctypes.c_char_p * cap)()
    runs = ctypes.c_int(0)
    n = load_library().spec_verify_kernel_times(ctx, ms, names, cap, ctypes.byref(runs))
    if n < 0:
        raise SpecVerifyError(-n, _msg(ctx))
    return [(names[i].decode(), float(ms[i])) for i in range(min(n, cap))], runs.value


def spec_verify_check_args(vocab, logits_dtype, max_batch, max_draft_rows, max_gamma, batch, gamma,
                           has_cu_gamma, total_draft_rows, temperature, has_logits=True, has_q=True,
                           has_draft_ids=True, has_uniforms=True, has_accepted_count=True,
                           has_emitted_tokens=True, has_residual_sum=True):
    """Host-side argument check without a device. Returns (code, message)."""
    buf = ctypes.create_string_buffer(256)
    rc = load_library().spec_verify_check_args(
        vocab, logits_dtype, max_batch, max_draft_rows, max_gamma, batch, gamma, int(bool(has_cu_gamma)),
        total_draft_rows, float(temperature), int(bool(has_logits)), int(bool(has_q)),
        int(bool(has_draft_ids)), int(bool(has_uniforms)), int(bool(has_accepted_count)),
        int(bool(has_emitted_tokens)), int(bool(has_residual_sum)), buf, len(buf))
    return rc, buf.value.decode()


def spec_verify_set_path(ctx: int, mode: int) -> None:
    """Choose the launch plan: SV_PATH_AUTO, SV_PATH_TWO_LAUNCH or SV_PATH_ONE_LAUNCH."""
    rc = load_library().spec_verify_set_path(ctx, int(mode))
    if rc != SV_OK:
        raise SpecVerifyError(rc, f"unknown path mode {mode}" if ctx else "NULL context")


def spec_verify_last_path(ctx: int) -> int:
    """The launch plan of the last successful run (SV_PATH_AUTO if none yet)."""
    rc = load_library().spec_verify_last_path(ctx)
    if rc < 0:
        raise SpecVerifyError(-rc, "NULL context")
    return rc
