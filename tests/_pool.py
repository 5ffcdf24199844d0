"""Fork-based process pool for the oracle's statistical pins (CPU only)."""
import multiprocessing as mp
import os

_NPROC = max(1, min(16, len(os.sched_getaffinity(0))))


def pmap(fn, args):
    """Map fn over args in forked workers (fn may be a closure; fork copies it)."""
    args = list(args)
    if _NPROC == 1 or len(args) == 1:
        return [fn(a) for a in args]
    global _FN
    _FN = fn
    ctx = mp.get_context("fork")
    with ctx.Pool(min(_NPROC, len(args))) as pool:
        return pool.map(_call, args)


_FN = None


def _call(a):
    return _FN(a)


def nproc():
    return _NPROC
