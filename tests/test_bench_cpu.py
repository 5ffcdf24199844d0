"""CPU checks of bench.py's accounting: the algorithmic bytes per step that the roofline
divides by the kernel time, and the lookup of rocprofv3 traffic that is reported only
while the kernel sources match the profiled ones."""
import importlib
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

bench = importlib.import_module("bench")


def _tiny(dtype, T, gammas, V=10):
    gammas = np.asarray(gammas, np.int32)
    cu = synth.pack(gammas)
    return synth.Workload("tiny", len(gammas), V, dtype, T, gammas, cu, None, None, None, None, None)


def test_method_bytes_by_hand():
    # per sequence: gamma V s_l (draft rows) + V s_l (drawn row) + [n < gamma] V 4 (q row
    # of the rejection) + gamma (4 + 4) (id, q(x)) + (gamma + 1) 4 (uniforms)
    # + 4 (count) + (gamma + 1) 4 (tokens) + 4 (S)
    w = _tiny("bf16", 1.0, [2, 3])
    n = np.array([0, 3])
    seq0 = 2 * 10 * 2 + 10 * 2 + 10 * 4 + 2 * 8 + 3 * 4 + 4 + 3 * 4 + 4
    seq1 = 3 * 10 * 2 + 10 * 2 + 0 + 3 * 8 + 4 * 4 + 4 + 4 * 4 + 4
    assert bench.method_bytes(w, n) == seq0 + seq1 == 148 + 144
    wf = _tiny("f32", 0.8, [2, 3])
    assert bench.method_bytes(wf, n) == (148 + 40 + 20) + (144 + 60 + 20)


def test_method_bytes_greedy_by_hand():
    # greedy: no q, no uniforms, no S; the bonus row only when every draft matched
    w = _tiny("bf16", 0.0, [2, 3])
    n = np.array([1, 3])
    seq0 = 2 * 10 * 2 + 0 + 2 * 4 + 4 + 3 * 4
    seq1 = 3 * 10 * 2 + 10 * 2 + 3 * 4 + 4 + 4 * 4
    assert bench.method_bytes(w, n) == seq0 + seq1


def test_needed_bytes_stop_at_rejection():
    # the one-launch plan reads rows 0..min(n, gamma - 1): here 1 and 3 rows
    w = _tiny("bf16", 1.0, [2, 3])
    n = np.array([0, 3])
    out0, out1 = 4 + 3 * 4 + 4, 4 + 4 * 4 + 4
    seq0 = 1 * 10 * 2 + 10 * 2 + 10 * 4 + 2 * 12 + 4 + out0
    seq1 = 3 * 10 * 2 + 10 * 2 + 0 + 3 * 12 + 4 + out1
    assert bench.needed_bytes(w, n, True) == seq0 + seq1
    # reading every row: the draft rows of both sequences in full
    assert bench.needed_bytes(w, n, False) == seq0 + seq1 + 1 * 10 * 2


def test_counter_traffic_needs_matching_sources(tmp_path, monkeypatch):
    csrc = tmp_path / "speculative_sampling_verification_03_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "spec_verify.hip").write_text("kernel sources A\n")
    (csrc / "sv_device.h").write_text("device helpers\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    src = bench.kernel_source_hash()
    (tmp_path / "profiles" / "k.txt").write_text(
        "summary text\n"
        f"traffic k_verify_seq C3-one 123456 {src}\n"
        f"traffic k_verify_seq C5-one 999 {src}\n"
        "traffic k_verify_seq C3-two 777 0000\n")
    assert bench.counter_traffic("k_verify_seq", "C3-one") == 123456.0
    assert bench.counter_traffic("k_verify_seq", "C5-one") == 999.0
    assert bench.counter_traffic("k_verify_seq", "C3-two") is None  # other sources
    assert bench.counter_traffic("k_greedy_seq1", "C3-one") is None
    (csrc / "spec_verify.hip").write_text("kernel sources B\n")  # the kernel changed
    assert bench.counter_traffic("k_verify_seq", "C3-one") is None


def test_rotated_inputs_exceed_the_last_level_cache():
    """Each workload rotates enough input sets that, between two uses of one set, the
    other sets' calls read over 1 GiB (four times the 256 MB last-level cache), by the
    most bytes a call can read: C3 needs 4 sets, C2's 57 MB calls 20."""
    import numpy as np
    import synth
    for cfg in ("C1", "C2", "C3", "C4", "C5"):
        w = synth.make_config(cfg, seed=0)
        n = bench.auto_sets(cfg)
        per = bench.max_call_bytes(w)
        assert (n - 1) * per >= bench.SET_BYTES_TARGET or n == bench.MAX_SETS, cfg
        assert n >= 2, cfg
        # the bound is the larger of the two extreme acceptances
        g = w.gammas.astype(np.int64)
        for acc in (np.zeros_like(g), g, g // 2):
            assert bench.method_bytes(w, acc) <= per, (cfg, acc[:4])
    assert bench.auto_sets("C3") == 4
    assert bench.auto_sets("C2") == 20
