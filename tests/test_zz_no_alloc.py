"""spec_verify_run_static, the entry point that allocates nothing, against spec_verify_run.

Both run the same inputs; the static entry point must give the same outputs bit for bit
(the same kernels, except that greedy batches never take the helper plan, whose outputs
are the same by construction, and sampling batches never take the small-batch plan's
several workgroups per sequence: there the context runs the plan the static entry point
takes instead, one launch from 0.55 x CUs sequences up and two launches below) and pass the oracle's bar. Each case makes two static calls in a row, the
second with a smaller input, so that what the first call leaves in the static workspace
cannot leak into the second. Captured into a HIP graph, static calls replay with new
inputs and match the eager results.
"""
import sys

import numpy as np
import pytest

import synth
from _parity import compare, oracle_batch, run_gpu, to_device

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


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


def _static(sv, w, dev, flags):
    ragged = w.uniform_gamma is None
    code = sv.SV_BF16 if w.dtype == "bf16" else sv.SV_F32
    acc = torch.empty(w.B, dtype=torch.int32, device="cuda")
    em = torch.empty(w.target_rows, dtype=torch.int32, device="cuda")
    S = torch.empty(w.B, dtype=torch.float32, device="cuda")
    pd = torch.empty(w.draft_rows, dtype=torch.float32, device="cuda") if w.T > 0 else None
    greedy = w.T == 0
    sv.spec_verify_run_static(0, torch.cuda.current_stream(), w.V, code, w.B, -1 if ragged else w.uniform_gamma,
                              dev["cu_gamma"] if ragged else None, w.draft_rows, w.T, dev["logits"],
                              None if greedy else dev["q"], dev["draft_ids"], None if greedy else dev["uniforms"],
                              acc, em, S, pd, flags)
    torch.cuda.synchronize()
    return dict(accepted_count=acc.cpu().numpy(), emitted_tokens=em.cpu().numpy(), residual_sum=S.cpu().numpy(),
                p_draft=pd.cpu().numpy() if pd is not None else None)


def _static_plan(sv, w):
    """The plan the static entry point takes for a sampling batch that the context would
    give to the small-batch plan: one launch from 0.55 x CUs sequences up (the AUTO rule's
    crossover), else two launches."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return sv.SV_PATH_ONE_LAUNCH if w.B >= (11 * cus + 19) // 20 else sv.SV_PATH_TWO_LAUNCH


def _check(sv, w, label):
    _say(label, f"B={w.B} V={w.V} {w.dtype} T={w.T} rows={w.draft_rows}")
    dev = to_device(w)
    code = sv.SV_BF16 if w.dtype == "bf16" else sv.SV_F32
    with sv.Verifier(w.V, code, w.B, max(w.draft_rows, 1), 16) as v:
        ref = run_gpu(v, w, dev=dev)
        assert ref["status"] == sv.SV_OK, v.last_error()
        if v.last_path() == sv.SV_PATH_POOLED and w.V > 4096:  # not taken by the static entry point
            v.set_path(_static_plan(sv, w))
            ref = run_gpu(v, w, dev=dev)
            assert ref["status"] == sv.SV_OK, v.last_error()
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = _static(sv, w, dev, flags)
    assert int(flags.item()) == 0
    for k in ("accepted_count", "emitted_tokens", "residual_sum"):
        assert np.array_equal(got[k], ref[k]), (label, k)
    if w.T > 0:
        assert np.array_equal(got["p_draft"], ref["p_draft"], equal_nan=True), label
    rep = compare(w, dict(got, status=sv.SV_OK), oracle_batch(w))
    _say(label, rep.summary())
    assert rep.ok(), rep.summary()


@pytest.mark.parametrize("cfg,big,small", [("C3", 256, 64), ("C2", 64, 24), ("C4", 512, 100), ("C5", 1024, 200)])
def test_static_entry_point_matches_context(lib, cfg, big, small):
    """Two static calls in a row, the second smaller (C3: one launch, then the split draw
    of a small batch; C4: greedy without helpers; C5: the ordered ragged launch)."""
    _check(lib, synth.make_config(cfg, seed=40, batch=big), f"static {cfg} B={big}")
    _check(lib, synth.make_config(cfg, seed=41, batch=small), f"static {cfg} B={small}")


def test_static_data_flags_and_limits(lib):
    sv = lib
    w = synth.make_config("C3", seed=42, batch=16, vocab=4096)
    w.draft_ids = w.draft_ids.copy()
    w.draft_ids[5] = w.V + 7
    dev = to_device(w)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    _say("static data flags", f"B={w.B}")
    _static(sv, w, dev, flags)
    assert int(flags.item()) & sv.SV_DATA_DRAFT_ID
    code = sv.SV_BF16
    with pytest.raises(sv.SpecVerifyError) as e:  # beyond the static workspace: nothing launched
        sv.spec_verify_run_static(0, None, w.V, code, sv.SV_STATIC_MAX_BATCH + 1, 4, None,
                                  4 * (sv.SV_STATIC_MAX_BATCH + 1), 1.0, dev["logits"], dev["q"], dev["draft_ids"],
                                  dev["uniforms"], flags, flags, flags, None, flags)
    assert e.value.code == sv.SV_EINVAL and "SV_STATIC_MAX_BATCH" in str(e.value)
    with pytest.raises(sv.SpecVerifyError) as e:
        sv.spec_verify_run_static(0, None, w.V, code, 1000, 17, None, 17000, 1.0, dev["logits"], dev["q"],
                                  dev["draft_ids"], dev["uniforms"], flags, flags, flags, None, flags)
    assert e.value.code == sv.SV_EINVAL and "SV_STATIC_MAX_ROWS" in str(e.value)
    with pytest.raises(sv.SpecVerifyError) as e:
        sv.spec_verify_run_static(0, None, w.V, code, 16, 4, None, 64, 1.0, dev["logits"], dev["q"],
                                  dev["draft_ids"], dev["uniforms"], flags, flags, flags, None, None)
    assert e.value.code == sv.SV_EINVAL and "data_flags" in str(e.value)


@pytest.mark.parametrize("cfg,batch,vocab", [("C3", 256, 32768), ("C2", 64, None), ("C1", 8, None),
                                             ("C5", 300, 8192), ("C4", 128, 16384), ("C4", 300, 8192)])
def test_static_entry_point_graph_replays(lib, cfg, batch, vocab):
    """A static call captured into a HIP graph (one launch; the split draw of a small
    fp32 batch; short rows; the ordered ragged launch; greedy in two launches and in one)
    and replayed six times, new inputs copied into the captured buffers before each
    replay and eager work between replays: every replay gives the eager outputs of the
    inputs it saw, and no data flag is raised."""
    sv = lib
    w0 = synth.make_config(cfg, seed=50, batch=batch, vocab=vocab)
    if w0.uniform_gamma is None:  # the same gamma_b in every set, so the captured shapes hold
        ws = [w0] + [synth.make_sampling("graph ragged", w0.gammas, w0.V, w0.dtype, w0.T, 3.0, 0.7, seed=51 + k)
                     for k in range(2)]
    else:
        ws = [w0] + [synth.make_config(cfg, seed=51 + k, batch=batch, vocab=vocab) for k in range(2)]
    devs = [to_device(w) for w in ws]
    ragged = w0.uniform_gamma is None
    greedy = w0.T == 0
    code = sv.SV_BF16 if w0.dtype == "bf16" else sv.SV_F32
    # eager reference outputs of each input set (the static entry point itself)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    refs = [_static(sv, w, d, flags) for w, d in zip(ws, devs)]
    assert int(flags.item()) == 0
    _say("graph replays", cfg, f"B={w0.B} V={w0.V} {w0.dtype} T={w0.T}")
    # the captured buffers: inputs that each replay reads, outputs it writes
    buf = {k: t.clone() for k, t in devs[0].items() if t is not None}
    acc = torch.empty(w0.B, dtype=torch.int32, device="cuda")
    em = torch.empty(w0.target_rows, dtype=torch.int32, device="cuda")
    S = torch.empty(w0.B, dtype=torch.float32, device="cuda")
    pd = torch.empty(w0.draft_rows, dtype=torch.float32, device="cuda") if not greedy else None
    gflags = torch.zeros(1, dtype=torch.int32, device="cuda")

    def call():
        sv.spec_verify_run_static(0, torch.cuda.current_stream(), w0.V, code, w0.B,
                                  -1 if ragged else w0.uniform_gamma, buf["cu_gamma"] if ragged else None,
                                  w0.draft_rows, w0.T, buf["logits"], None if greedy else buf["q"],
                                  buf["draft_ids"], None if greedy else buf["uniforms"], acc, em, S, pd, gflags)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # outside the capture: the static workspace's set-up on this device is done
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for k in range(6):
        i = (k + 1) % 3
        for key, t in buf.items():
            t.copy_(devs[i][key])
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        got = dict(accepted_count=acc.cpu().numpy(), emitted_tokens=em.cpu().numpy(), residual_sum=S.cpu().numpy())
        for key in ("accepted_count", "emitted_tokens", "residual_sum"):
            assert np.array_equal(got[key], refs[i][key]), (k, i, key)
        if pd is not None:
            assert np.array_equal(pd.cpu().numpy(), refs[i]["p_draft"], equal_nan=True), (k, i)
    assert int(gflags.item()) == 0
