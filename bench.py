#!/usr/bin/env python3
"""Throughput of the batched speculative-sampling verification step on one MI355X.

A step is one call of spec_verify_run over one batch: B = 256 sequences, gamma = 4
drafts each, V = 128256, bf16 target logits, fp32 draft distributions, T = 1
(the full hot path: row statistics + accept test, first-rejection scan,
residual / bonus draw). Inputs are seeded synthetic data (see synth/), resident
in HBM before timing starts; input sets rotate, as many as it takes to hold over
1 GiB, so that no step re-reads the previous steps' data from the 256 MB
last-level cache.

Prints one JSON line on stdout:
  value       verified positions/s (sum gamma_b per step / seconds per step)
  roofline    the dominant kernel against HBM peak, from its mean launch duration
              (HIP events recorded on the launch stream during the timed loop):
              frac over the method's algorithmic bytes, frac_read over the bytes this
              launch plan has to read and write, frac_traffic over the HBM bytes the
              rocprofv3 counters measured for these kernel sources (null without them)
  next_rows   the other workloads (C1, C2, C4, C5), the follow-on rows and the
              per-GPU shares, each on its own rotated inputs
  cpu_baseline the CPU oracle timed on a bounded sample of the same inputs
Diagnostics go to stderr.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified positions/s + achieved HBM GB/s (% of peak), B=256 gamma=4 V=128256"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
TIMING_STRIDE = 8       # per-kernel events on one timed step in every 8


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def method_bytes(w, n):
    """Algorithmic bytes of one step by the two-pass method's per-sequence figure, from
    this run's accepted counts n: every draft row once, the drawn row once, the rejected
    position's q row once, the per-position id and uniform reads and the outputs.
    Greedy drops q and u, and reads its bonus row only when all drafts were accepted."""
    import numpy as np
    sl = 2 if w.dtype == "bf16" else 4
    g = w.gammas.astype(np.int64)
    n = n.astype(np.int64)
    if w.T == 0.0:
        per = g * w.V * sl + (n == g) * w.V * sl + g * 4 + 4 + (g + 1) * 4
    else:
        per = (g * w.V * sl + w.V * sl + (n < g) * w.V * 4 + g * (4 + 4) + (g + 1) * 4
               + 4 + (g + 1) * 4 + 4)
    return int(per.sum())


def needed_bytes(w, n, stop_at_rejection):
    """Bytes this launch plan has to read and write: as method_bytes, except that with
    `stop_at_rejection` only rows 0..min(n, gamma - 1) of each sequence are read (the rows
    the left-to-right verification looks at) and q(x) is read for every draft."""
    import numpy as np
    sl = 2 if w.dtype == "bf16" else 4
    g = w.gammas.astype(np.int64)
    n = n.astype(np.int64)
    rows = np.minimum(n + 1, g) if stop_at_rejection else g
    outputs = 4 + (g + 1) * 4 + (4 if w.T > 0 else 0)
    if w.T == 0.0:
        per = rows * w.V * sl + (n == g) * w.V * sl + g * 4 + outputs
    else:
        per = rows * w.V * sl + w.V * sl + (n < g) * w.V * 4 + g * 12 + 4 + outputs
    return int(per.sum())


def kernel_source_hash():
    """sha256 of the kernel sources; a committed counter summary applies only to them."""
    import hashlib
    h = hashlib.sha256()
    for f in ("csrc/spec_verify.hip", "csrc/sv_device.h"):
        with open(os.path.join(ROOT, "speculative_sampling_verification_03_amd", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_traffic(kernel, workload_tag):
    """HBM bytes per launch of `kernel` on `workload_tag` from a rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary under profiles/ whose kernel sources match these ones, else None.
    A summary states it on a line: traffic <kernel> <workload> <bytes> <source sha256>."""
    import glob
    src = kernel_source_hash()
    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt"))):
        for line in open(f, encoding="utf-8"):
            parts = line.split()
            if len(parts) == 5 and parts[0] == "traffic" and parts[1] == kernel and parts[2] == workload_tag \
                    and parts[4] == src:
                return float(parts[3])
    return None


def bench_sampling(sv, torch, sets, dev, code, args, iters=100):
    """Tokens/s of spec_sample_run on the workload's target rows (softmax of the logits)
    and on its draft rows (fp32 weights q), with inputs resident in HBM."""
    import numpy as np
    res = {}
    w0, d0 = sets[0]
    sl = 2 if w0.dtype == "bf16" else 4
    for name, x, rows, per_row in (
            ("target_rows_from_logits", [d["logits"] for _, d in sets], w0.target_rows, w0.V * sl),
            ("draft_rows_from_q", [d["q"] for _, d in sets], w0.draft_rows, w0.V * 4)):
        v = sv.Verifier(w0.V, code, rows, 1, 1)
        u = torch.rand(rows, device=dev)
        tok = torch.empty(rows, dtype=torch.int32, device=dev)

        def go(k):
            if name == "target_rows_from_logits":
                v.sample(x[k % len(x)], uniforms=u, temperature=w0.T, tokens=tok)
            else:
                v.sample_weights(x[k % len(x)], uniforms=u, tokens=tok)
        for k in range(10):
            go(k)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(iters):
            go(k)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / iters
        assert v.status() == sv.SV_OK, v.last_error()
        v.close()
        nbytes = rows * (per_row + 8)
        res[name] = {"rows": rows, "us_per_call": dt * 1e6, "tokens_per_s": rows / dt,
                     "GBps": nbytes / dt / 1e9, "frac_of_peak": nbytes / dt / 1e9 / HBM_PEAK_GBPS}
        log(f"[bench] F1 sampling {name}: {rows} rows in {dt * 1e6:.1f} us, "
            f"{nbytes / dt / 1e9:.0f} GB/s")
    return res


def _timed(torch, go, iters, warm=10):
    """Seconds per call of go(k) on torch's current stream (events around the loop)."""
    for k in range(warm):
        go(k)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(iters):
        go(k)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / iters


def bench_ngram(sv, torch, dev, iters=200):
    """Deterministic drafts: the prompt-lookup proposer over copy-heavy contexts, and the
    one-hot verification of drafts the target is often confident about, at B=256 gamma=4
    V=128256 bf16, T=1."""
    import numpy as np
    import synth
    res = {}
    B, L, gamma, n_min, n_max = 256, 8192, 4, 2, 6
    ctx = synth.make_ngram_contexts(B, (L, L), 128256, seed=31)
    tok = torch.from_numpy(ctx.tokens).to(dev)
    cu = torch.from_numpy(ctx.cu_ctx).to(dev)
    ver = sv.Verifier(128256, sv.SV_BF16, B, B * gamma, gamma)
    ids = torch.empty((B, gamma), dtype=torch.int32, device=dev)
    lens = torch.empty(B, dtype=torch.int32, device=dev)
    dt = _timed(torch, lambda k: ver.propose_ngram(tok, cu, gamma=gamma, n_min=n_min, n_max=n_max,
                                                 draft_ids=ids, draft_len=lens), iters)
    assert ver.status() == sv.SV_OK, ver.last_error()
    ctx_bytes = ctx.tokens.nbytes + ctx.cu_ctx.nbytes + ids.numel() * 4 + B * 4
    ln = lens.cpu().numpy()
    res["ngram_propose"] = {
        "workload": f"B={B} contexts of {L} tokens (copy-heavy), n={n_min}..{n_max}, gamma={gamma}",
        "us_per_call": dt * 1e6, "contexts_per_s": B / dt,
        "context_GBps": ctx_bytes / dt / 1e9,
        "context_bytes_basis": "every context read once (an upper bound: the scan stops early)",
        "proposing_fraction": float((ln > 0).mean()), "mean_draft_len": float(ln.mean())}
    log(f"[bench] F3 n-gram proposer: {B} x {L} tokens in {dt * 1e6:.1f} us "
        f"({ctx_bytes / dt / 1e9:.0f} GB/s over whole contexts), mean proposal {ln.mean():.2f}")

    w = synth.make_onehot("C3-onehot", np.full(B, gamma), 128256, "bf16", 1.0, 3.0, 1.0, seed=32)
    synth.boost_drafts(w, 0.8, 4.0, seed=33)
    d = {"logits": torch.from_numpy(w.logits.view(np.int16)).view(torch.bfloat16).to(dev),
         "ids": torch.from_numpy(w.draft_ids).to(dev), "u": torch.from_numpy(w.uniforms).to(dev)}
    out = sv.VerifyOutputs(torch.empty(B, dtype=torch.int32, device=dev),
                           torch.empty(w.target_rows, dtype=torch.int32, device=dev),
                           torch.empty(B, dtype=torch.float32, device=dev), None)
    dt = _timed(torch, lambda k: ver.run(d["logits"], d["ids"], temperature=1.0, uniforms=d["u"], gamma=gamma,
                                         out=out, onehot=True), iters)
    assert ver.status() == sv.SV_OK, ver.last_error()
    n = out.accepted_count.cpu().numpy()
    res["onehot_verify"] = {
        "workload": f"B={B} gamma={gamma} V=128256 bf16 logits, T=1, one-hot drafts (no q), "
                    "target confident about 80% of the drafts",
        "plan": {sv.SV_PATH_ONE_LAUNCH: "one launch", sv.SV_PATH_TWO_LAUNCH: "two launches"}.get(ver.last_path()),
        "us_per_step": dt * 1e6, "positions_per_s": B * gamma / dt,
        "tokens_per_round": float(np.mean(n + 1))}
    log(f"[bench] F3 one-hot verification: {dt * 1e6:.1f} us/step, {B * gamma / dt / 1e6:.2f} M positions/s, "
        f"{np.mean(n + 1):.2f} tokens/round")
    ver.close()
    return res


def bench_adaptive(sv, torch, dev, warm_rounds=10, rounds=30, c=0.05):
    """Adaptive draft length against fixed ones on C5's sequences: B=1024, V=128256 bf16,
    T=1, a fixed target row p_b and draft row q_b per sequence with sigma_b ~ U[0.2, 2]
    (per-position acceptance from ~0.3 to ~0.9). Every round packs the rows for the
    current gamma_b (index_select), draws the drafts from q_b on the GPU (spec_sample_run)
    with seeded uniforms, verifies, and (adaptive) updates gamma_b on the GPU. Reports
    tokens per round and per cost unit 1 + c*gamma_b (c = draft/target cost, 0.05 as in
    the speedup table of the pages), and the GPU time of verification + controller."""
    import numpy as np
    import synth
    cfg = synth.CONFIGS["C5"]
    B, V, gmax = 1024, cfg["V"], 8
    st = np.random.Generator(np.random.PCG64(0xADA))
    sig = st.uniform(cfg["sigma_noise"][0], cfg["sigma_noise"][1], size=B)
    w = synth.make_sampling("C5-rows", np.ones(B, np.int32), V, "bf16", 1.0, cfg["sigma_logit"], sig, 0xADA1)
    base_l = torch.from_numpy(w.logits[np.arange(B) * 2].view(np.int16)).view(torch.bfloat16).to(dev)
    base_q = torch.from_numpy(w.q).to(dev)
    ver = sv.Verifier(V, sv.SV_BF16, B, B * gmax, gmax)
    drafter = sv.Verifier(V, sv.SV_BF16, B * gmax, 1, 1)  # one draw per draft row
    gen = torch.Generator(device=dev)
    res = {}
    for mode in ("fixed 4", "fixed 8", "adaptive"):
        gen.manual_seed(0xADA2)
        g0 = 4 if mode != "fixed 8" else 8
        g_dev = torch.full((B,), g0, dtype=torch.int32, device=dev)
        s_dev = torch.zeros(B, dtype=torch.int32, device=dev)
        cu_dev = torch.arange(0, (B + 1) * g0, g0, dtype=torch.int32, device=dev)
        toks, cost, pos, gpu_ms, gam = 0.0, 0.0, 0, 0.0, []
        for k in range(warm_rounds + rounds):
            g = g_dev.cpu().numpy()
            R = int(g.sum())
            seq_t = torch.from_numpy(np.repeat(np.arange(B), g + 1)).to(dev)
            seq_d = torch.from_numpy(np.repeat(np.arange(B), g)).to(dev)
            L = base_l.index_select(0, seq_t)
            Q = base_q.index_select(0, seq_d)
            ids = drafter.sample_weights(Q, uniforms=torch.rand(R, generator=gen, device=dev))
            u = torch.rand(R + B, generator=gen, device=dev)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            out = ver.run(L, ids, temperature=1.0, q=Q, uniforms=u, cu_gamma=cu_dev, total_draft_rows=R,
                          want_p_draft=False)
            if mode == "adaptive":
                cu_dev = ver.adapt_gamma(out.accepted_count, g_dev, s_dev, gamma_max=gmax)
            e1.record()
            torch.cuda.synchronize()
            n = out.accepted_count.cpu().numpy()
            if k >= warm_rounds:
                toks += float((n + 1).sum())
                cost += float((1 + c * g).sum())
                pos += R
                gpu_ms += e0.elapsed_time(e1)
                gam.append(g.mean())
        assert ver.status() == sv.SV_OK, ver.last_error()
        assert drafter.status() == sv.SV_OK, drafter.last_error()
        res[mode] = {"tokens_per_round": toks / (rounds * B), "tokens_per_cost_unit": toks / cost,
                     "mean_gamma": float(np.mean(gam)), "us_per_round": gpu_ms * 1e3 / rounds,
                     "verified_positions_per_s": pos / (gpu_ms * 1e-3)}
        log(f"[bench] F2 {mode}: {toks / (rounds * B):.3f} tokens/round, {toks / cost:.3f} per cost unit "
            f"(c={c}), mean gamma {np.mean(gam):.2f}, {gpu_ms * 1e3 / rounds:.1f} us/round")
    ver.close()
    drafter.close()
    res["workload"] = (f"C5 sequences: B={B}, V={V} bf16, T=1, fixed p_b and q_b, sigma_b ~ U[0.2, 2]; "
                       f"{rounds} rounds after {warm_rounds}; gamma_max={gmax}, up_after=1, down_after=2")
    return res


def bench_shares(sv, torch, sets, dev, code, iters=200):
    """One GPU's share when C3 is split by sequence over G GPUs (no exchange is needed:
    sequences are independent): B/G sequences per step, the plan the library picks for
    that size, wall time per step. Step k takes slice (k // sets) mod G of input set
    k mod sets, so every slice of every set is rotated through (G x sets distinct inputs)."""
    import numpy as np
    res = {}
    w0 = sets[0][0]
    g = w0.uniform_gamma
    for G in (2, 4, 8):
        b = w0.B // G
        if b < 1 or g is None:
            continue
        v = sv.Verifier(w0.V, code, b, b * g, 16)
        calls = []
        for j in range(G):
            for _, d in sets:
                L = d["logits"][j * b * (g + 1):(j + 1) * b * (g + 1)]
                Q = d["q"][j * b * g:(j + 1) * b * g]
                X = d["ids"][j * b * g:(j + 1) * b * g]
                U = d["u"][j * b * (g + 1):(j + 1) * b * (g + 1)]
                out = sv.VerifyOutputs(torch.empty(b, dtype=torch.int32, device=dev),
                                       torch.empty(b * (g + 1), dtype=torch.int32, device=dev),
                                       torch.empty(b, dtype=torch.float32, device=dev), None)
                calls.append(v.bind(L, X, temperature=w0.T, q=Q, uniforms=U, gamma=g, out=out))
        dt, kt = timed_steps(sv, torch, v, lambda k: calls[k % len(calls)](), iters, 20, 4)
        plan = plan_name(sv, v)
        v.close()
        res[f"G={G}"] = {"B": b, "us_per_step": dt * 1e6, "positions_per_s": b * g / dt, "plan": plan,
                         "kernel_us": {nm: t * 1e3 for nm, t in kt}, "distinct_inputs": len(calls)}
        log(f"[bench] share of G={G} GPUs (B={b}): {dt * 1e6:.1f} us/step ({plan}; kernels "
            + ", ".join(f"{nm} {t * 1e3:.1f}" for nm, t in kt) + f" us), {b * g / dt / 1e6:.2f} M positions/s per GPU")
    return res


def bench_vshard(sv, torch, sets, dev, code, G=8, iters=200):
    """F4: one GPU's part of the workload under vocabulary sharding over G devices. Every
    shard k holds columns [bounds[k], bounds[k + 1]) of every row and has its own context;
    round j runs the three steps of shard j mod G (so the G shards' columns, 8 x 53 MB at
    C3, rotate through the last-level cache). The records and draw totals of the other
    shards are computed once beforehand and stand in for the two all-gathers, which are
    not timed. Reports the time of one shard's round on this device, each step alone, the
    shard's column bytes per round and the bytes each exchange gathers."""
    import numpy as np
    w0, d0 = sets[0]
    g = w0.uniform_gamma
    if g is None or w0.T == 0:
        return {}
    V, B, R, T = w0.V, w0.B, w0.draft_rows, w0.T
    bounds = [round(k * V / G) for k in range(G + 1)]
    L2 = d0["logits"].view(R + B, V)
    Q2 = d0["q"].view(R, V)
    ids, u = d0["ids"], d0["u"]
    rec_all = torch.empty((G * R, 4), dtype=torch.float32, device=dev)
    part_all = torch.empty((G, B, sv.VSHARD_PART_DOUBLES), dtype=torch.float64, device=dev)
    sh, cols, outs = [], [], []
    for k in range(G):
        s_k = sv.VocabShard(bounds, k, code, B, R, 16)
        Lk = L2[:, bounds[k]:bounds[k + 1]].contiguous()
        Qk = Q2[:, bounds[k]:bounds[k + 1]].contiguous()
        s_k.rows(Lk, ids, temperature=T, q=Qk, gamma=g, rec=rec_all[k * R:(k + 1) * R])
        sh.append(s_k)
        cols.append((Lk, Qk))
    for k in range(G):
        o, part, loc = sh[k].decide(cols[k][0], ids, rec_all, temperature=T, q=cols[k][1], uniforms=u, gamma=g,
                                    want_p_draft=False)
        part_all[k].copy_(part)
        outs.append((o, loc))
    st = torch.cuda.current_stream(dev)

    def rows(j):
        k = j % G
        sv.spec_vshard_rows(sh[k].ver.ctx, st, sh[k].desc, B, g, None, R, T, cols[k][0], cols[k][1], ids,
                            rec_all[k * R:(k + 1) * R])

    def decide(j):
        k = j % G
        o, loc = outs[k]
        sv.spec_vshard_decide(sh[k].ver.ctx, st, sh[k].desc, B, g, None, R, T, cols[k][0], cols[k][1], ids, u,
                              rec_all, o.accepted_count, o.emitted_tokens, o.residual_sum, None, part_all[k], loc)

    def finish(j):
        k = j % G
        o, loc = outs[k]
        sv.spec_vshard_finish(sh[k].ver.ctx, st, sh[k].desc, B, g, None, R, T, cols[k][0], cols[k][1], u,
                              part_all, loc, o.emitted_tokens, o.residual_sum)

    def round_(j):
        rows(j)
        decide(j)
        finish(j)
    dt = _timed(torch, round_, iters)
    steps = {nm: _timed(torch, fn, iters) * 1e6 for nm, fn in
             (("k_vs_rows", rows), ("k_vs_decide", decide), ("k_vs_finish", finish))}
    for s_k in sh:
        assert s_k.status() == sv.SV_OK, s_k.last_error()
    acc = outs[0][0].accepted_count.cpu().numpy()
    for s_k in sh:
        s_k.close()
    W = float(np.mean([bounds[k + 1] - bounds[k] for k in range(G)]))
    s_l = 2 if code == sv.SV_BF16 else 4
    n_res = int((acc < g).sum())
    col_bytes = R * W * s_l + B * W * s_l + n_res * W * 4
    res = {"workload": f"C3 columns of one of {G} shards ({W:.0f} columns), the shards rotated: B={B} gamma={g} V={V}",
           "us_per_round": dt * 1e6, "step_us": steps,
           "positions_per_s_device_part": R / dt, "column_bytes_per_round": col_bytes,
           "column_GBps": col_bytes / dt / 1e9,
           "gathered_bytes": {"records": G * R * sv.VSHARD_REC_BYTES,
                              "draw_totals": G * B * sv.VSHARD_PART_DOUBLES * 8}}
    log(f"[bench] F4 vocab shard (1 of {G}, {W:.0f} columns, shards rotated): {dt * 1e6:.1f} us/round on this "
        f"device (rows {steps['k_vs_rows']:.1f}, decide {steps['k_vs_decide']:.1f}, finish "
        f"{steps['k_vs_finish']:.1f} us alone), {col_bytes / dt / 1e9:.0f} GB/s over its columns; all-gathers of "
        f"{G * R * sv.VSHARD_REC_BYTES / 1e3:.0f} KB and {G * B * 24 / 1e3:.0f} KB")
    return res


def cpu_baseline(w, seconds):
    """The oracle as it stands, single process, cycling over the sequences of one input
    set until about `seconds` of CPU work have been done."""
    import numpy as np
    import oracle as O
    cu = w.cu_gamma.astype(np.int64)
    t0 = time.perf_counter()
    done = positions = 0
    while True:
        b = done % w.B
        g = int(cu[b + 1] - cu[b])
        base = int(cu[b])
        O.verify_sequence(w.logits_f64(slice(base + b, base + b + g + 1)),
                          None if w.T == 0 else w.q[base:base + g], w.draft_ids[base:base + g],
                          None if w.T == 0 else w.uniforms[base + b:base + b + g + 1], w.T)
        done += 1
        positions += g
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return dict(value=positions / dt, unit="verified positions/s", cores=1, kind="oracle",
                sample=f"{done} sequences ({positions} positions) cycling over input set 0 "
                       f"({w.B} sequences), float64 NumPy oracle in one process, {dt:.1f} s")


SET_BYTES_TARGET = 1 << 30  # bytes read between two uses of one input set (four times the 256 MB last-level cache)
MAX_SETS = 32


def input_bytes(w):
    """Bytes of one input set of workload w (logits, q, ids, uniforms)."""
    return (w.logits.nbytes + (w.q.nbytes if w.q is not None else 0) + w.draft_ids.nbytes
            + (w.uniforms.nbytes if w.uniforms is not None else 0))


def max_call_bytes(w):
    """Bytes one call of workload w reads at most: method_bytes at the acceptance that
    reads the most (every q row for sampling, every bonus row for greedy)."""
    import numpy as np
    g = w.gammas.astype(np.int64)
    return max(method_bytes(w, np.zeros_like(g)), method_bytes(w, g))


def auto_sets(config):
    """Input sets to rotate for `config`: enough that between two uses of one set the
    other sets' calls read at least SET_BYTES_TARGET (four times the 256 MB last-level
    cache), so that no call finds its rows still cached from the last use of its set."""
    import synth
    w = synth.make_config(config, seed=0)
    per = max_call_bytes(w)
    return min(MAX_SETS, max(2, -(-SET_BYTES_TARGET // per) + 1))


def load_sets(torch, config, n, dev, batch=None):
    """n seeded input sets of `config` resident on the device: [(workload, tensors)]."""
    import numpy as np
    import synth
    sets = []
    for s in range(n):
        w = synth.make_config(config, seed=s, batch=batch)
        d = {}
        if w.dtype == "bf16":
            d["logits"] = torch.from_numpy(w.logits.view(np.int16)).view(torch.bfloat16).to(dev)
        else:
            d["logits"] = torch.from_numpy(w.logits).to(dev)
        d["q"] = torch.from_numpy(w.q).to(dev) if w.q is not None else None
        d["ids"] = torch.from_numpy(w.draft_ids).to(dev)
        d["u"] = torch.from_numpy(w.uniforms).to(dev) if w.uniforms is not None else None
        d["cu"] = torch.from_numpy(w.cu_gamma).to(dev)
        sets.append((w, d))
    return sets


class Steps:
    """Bound steps over rotated input sets on one context: step k runs set k mod n with
    its own output buffers (p(x) requested when want_p)."""

    def __init__(self, sv, torch, ver, sets, dev, want_p=False):
        self.sets, self.outs, self.calls = sets, [], []
        ragged = sets[0][0].uniform_gamma is None
        for w, d in sets:
            o = sv.VerifyOutputs(torch.empty(w.B, dtype=torch.int32, device=dev),
                                 torch.empty(w.target_rows, dtype=torch.int32, device=dev),
                                 torch.empty(w.B, dtype=torch.float32, device=dev),
                                 torch.empty(w.draft_rows, dtype=torch.float32, device=dev)
                                 if want_p and w.T > 0 else None)
            kw = (dict(cu_gamma=d["cu"], total_draft_rows=w.draft_rows) if ragged
                  else dict(gamma=w.uniform_gamma))
            self.calls.append(ver.bind(d["logits"], d["ids"], temperature=w.T, q=d["q"], uniforms=d["u"],
                                       out=o, **kw))
            self.outs.append(o)

    def __call__(self, k):
        self.calls[k % len(self.calls)]()


def timed_steps(sv, torch, ver, steps, n, warmup, stride):
    """Wall seconds per step over n steps (after warmup) and the per-kernel mean
    durations [(name, ms)] from dispatch events on one step in every `stride`."""
    for k in range(warmup):
        steps(k)
    torch.cuda.synchronize()
    ver.set_timing((n + stride - 1) // stride, stride)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(n):
        steps(k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ktimes, kruns = ver.kernel_times()
    ver.set_timing(0)
    assert ver.status() == sv.SV_OK, ver.last_error()
    assert kruns == (n + stride - 1) // stride, (kruns, n, stride)
    return (t1 - t0) / n, ktimes


def PLANS(sv):
    return {"auto": sv.SV_PATH_AUTO, "two": sv.SV_PATH_TWO_LAUNCH, "one": sv.SV_PATH_ONE_LAUNCH,
            "pooled": sv.SV_PATH_POOLED}


def plan_name(sv, ver):
    return {sv.SV_PATH_ONE_LAUNCH: "one launch", sv.SV_PATH_TWO_LAUNCH: "two launches",
            sv.SV_PATH_POOLED: "small-batch pooled launch"}.get(ver.last_path())


def plan_key(sv, ver):
    """'one', 'two' or 'pool': the plan the last call ran, as profiles name it."""
    return {sv.SV_PATH_ONE_LAUNCH: "one", sv.SV_PATH_TWO_LAUNCH: "two", sv.SV_PATH_POOLED: "pool"}[ver.last_path()]


def traffic_tag(config, key):
    return f"{config}-{key}"


def bench_config(sv, torch, dev, config, n_steps, warmup, stride, plan="auto", batch=None, n_sets=None):
    """One workload on its own rotated inputs: wall time per step, per-kernel dispatch
    times, the method's bytes and the bytes the plan reads, against the HBM peak."""
    import numpy as np
    import synth
    n_sets = n_sets or auto_sets(config)
    sets = load_sets(torch, config, n_sets, dev, batch)
    w0 = sets[0][0]
    code = sv.SV_BF16 if w0.dtype == "bf16" else sv.SV_F32
    ver = sv.Verifier(w0.V, code, w0.B, max(w.draft_rows for w, _ in sets), 16)
    ver.set_path(PLANS(sv)[plan])
    steps = Steps(sv, torch, ver, sets, dev)
    acc = []
    for k in range(len(sets)):
        steps(k)
        torch.cuda.synchronize()
        assert ver.status() == sv.SV_OK, ver.last_error()
        acc.append(steps.outs[k].accepted_count.cpu().numpy())
    one = ver.last_path() == sv.SV_PATH_ONE_LAUNCH  # stops reading rows at the first rejection
    key = plan_key(sv, ver)
    plan_txt = plan_name(sv, ver)
    dt, kt = timed_steps(sv, torch, ver, steps, n_steps, warmup, stride)
    ver.close()
    method = float(np.mean([method_bytes(w, n) for (w, _), n in zip(sets, acc)]))
    needed = float(np.mean([needed_bytes(w, n, one) for (w, _), n in zip(sets, acc)]))
    k_us = sum(t for _, t in kt) * 1e3
    pos = float(np.mean([w.draft_rows for w, _ in sets]))
    cfgd = synth.CONFIGS[config]
    res = {
        "workload": (f"{config}: B={w0.B} gamma={cfgd['gamma'] if w0.uniform_gamma else 'ragged 1..8'} "
                     f"V={w0.V} {w0.dtype} logits" + (", fp32 q" if w0.T > 0 else ", greedy") + f", T={w0.T:g}"),
        "plan": plan_txt, "input_sets": n_sets, "rotated_MB": n_sets * input_bytes(w0) / 1e6,
        "steps": n_steps, "us_per_step": dt * 1e6, "kernel_us": {nm: t * 1e3 for nm, t in kt},
        "kernel_us_total": k_us, "positions_per_s": pos / dt,
        "method_MB": method / 1e6, "read_MB": needed / 1e6,
        "frac_method": method / (k_us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
        "frac_read": needed / (k_us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
    }
    # counter bytes of every kernel of the step, where profiles of these sources exist
    trs = [0.0 if nm == "k_order_by_gamma" else counter_traffic(nm, traffic_tag(config, key)) for nm, _ in kt]
    tr = sum(trs) if all(t is not None for t in trs) else None
    res["traffic_MB"] = tr / 1e6 if tr else None
    res["frac_traffic"] = tr / (k_us * 1e-6) / 1e9 / HBM_PEAK_GBPS if tr else None
    log(f"[bench] {config}: {dt * 1e6:.2f} us/step ({plan_txt}; kernels "
        + ", ".join(f"{nm} {t * 1e3:.2f}" for nm, t in kt) + f" us), {pos / dt / 1e6:.2f} M positions/s, "
        f"reads {needed / 1e6:.1f} MB: {res['frac_read']:.1%} of peak over the kernels' time; "
        f"{n_sets} sets ({res['rotated_MB']:.0f} MB) rotated")
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="C3", help="workload (C3 is the measured one; others for development)")
    ap.add_argument("--sets", type=int, default=0, help="input sets rotated across steps (0: enough that 1 GiB is read between two uses of a set)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the other workloads and the follow-on measurements")
    ap.add_argument("--no-every-row", action="store_true",
                    help="skip the second timing with p(x) requested (every draft row read)")
    ap.add_argument("--plan", choices=("auto", "two", "one", "pooled"), default="auto",
                    help="launch plan (auto: the library's choice by batch size; pooled: the small-batch "
                         "one-launch plan, rows read in chunks and draws shared)")
    ap.add_argument("--batch", type=int, default=None, help="sequences per step (default: the workload's)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run plain device copies of MIB MiB (calibrates the HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the verification step shards by sequence with no "
              "exchange, so there is no multi-GPU path to time here. Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import speculative_sampling_verification_03_amd as sv
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / 5
        log(f"[bench] copy of {args.copy_calibration} MiB: {dt * 1e6:.1f} us, "
            f"{2 * n / dt / 1e9:.0f} GB/s (read + write); each copy reads {n} B and writes {n} B")
        return
    sv.load_library()

    n_sets = args.sets or auto_sets(args.config)
    log(f"[bench] generating {n_sets} input set(s) of {args.config}")
    sets = load_sets(torch, args.config, n_sets, dev, args.batch)
    w0 = sets[0][0]
    ragged = w0.uniform_gamma is None
    code = sv.SV_BF16 if w0.dtype == "bf16" else sv.SV_F32
    ver = sv.Verifier(w0.V, code, w0.B, max(w.draft_rows for w, _ in sets), 16)
    ver.set_path(PLANS(sv)[args.plan])
    step = Steps(sv, torch, ver, sets, dev)

    # untimed: outputs of each set fix the algorithmic bytes of its steps
    nb = []
    for k in range(len(sets)):
        step(k)
        torch.cuda.synchronize()
        assert ver.status() == sv.SV_OK, ver.last_error()
        nb.append(step.outs[k].accepted_count.cpu().numpy())
    stop = ver.last_path() == sv.SV_PATH_ONE_LAUNCH  # stops reading rows at the first rejection
    one_launch = ver.last_path() in (sv.SV_PATH_ONE_LAUNCH, sv.SV_PATH_POOLED)
    key = plan_key(sv, ver)
    plan_txt = plan_name(sv, ver)
    method_per_set = [method_bytes(w, n) for (w, _), n in zip(sets, nb)]
    needed_per_set = [needed_bytes(w, n, stop) for (w, _), n in zip(sets, nb)]

    # timed loop: exactly args.steps steps between two device synchronizations; per-kernel
    # HIP events (start and stop of the dispatch itself, on the launch stream) on one step
    # in every TIMING_STRIDE, which keeps their cost out of the wall clock
    sec, ktimes = timed_steps(sv, torch, ver, step, args.steps, args.warmup, TIMING_STRIDE)
    ms = sec * 1e3
    pos_per_step = np.mean([w.draft_rows for w, _ in sets])
    value = pos_per_step / (ms * 1e-3)
    path_bytes = float(np.mean([method_per_set[k % len(sets)] for k in range(args.steps)]))
    path_gbps = path_bytes / (ms * 1e-3) / 1e9
    needed = float(np.mean([needed_per_set[k % len(sets)] for k in range(args.steps)]))

    # the roofline is taken on the kernel that moves the most bytes: the whole step when
    # it is one launch (a ragged batch with more sequences than compute units first runs
    # the small ordering kernel, which moves no row data), else the row-statistics pass
    # (every draft row once)
    kt = dict(ktimes)
    k1 = ktimes[-1][0] if one_launch else ktimes[0][0]
    sl = 2 if w0.dtype == "bf16" else 4
    if one_launch:
        k1_bytes, k1_needed = path_bytes, needed
    else:
        k1_bytes = float(np.mean([w.draft_rows * (w.V * sl + 8) for w, _ in sets]))
        k1_needed = k1_bytes
    k1_s = kt[k1] * 1e-3
    k1_gbps = k1_bytes / k1_s / 1e9
    traffic = counter_traffic(k1, traffic_tag(args.config, key))

    # the same steps with p(x) requested for every draft: the one-launch plan then reads
    # every draft row, as the two-launch plan always does
    all_rows = None
    if stop and not w0.T == 0.0 and not args.no_every_row:
        step_p = Steps(sv, torch, ver, sets, dev, want_p=True)
        sec_all, kt_all = timed_steps(sv, torch, ver, step_p, args.steps, args.warmup, TIMING_STRIDE)
        ms_all = sec_all * 1e3
        all_rows = {"ms_per_step": ms_all, "value": pos_per_step / (ms_all * 1e-3),
                    "kernel_us": {nm: t * 1e3 for nm, t in kt_all},
                    "achieved_GBps": path_bytes / (kt_all[-1][1] * 1e-3) / 1e9,
                    "frac_of_peak": path_bytes / (kt_all[-1][1] * 1e-3) / 1e9 / HBM_PEAK_GBPS}
        log(f"[bench] every row read (p(x) requested): {ms_all * 1e3:.2f} us/step, "
            f"{all_rows['value'] / 1e6:.2f} M positions/s, kernel {kt_all[-1][1] * 1e3:.2f} us "
            f"({all_rows['frac_of_peak']:.1%} of peak over the method's bytes, all of which it reads)")

    # the other workloads, each on its own rotated inputs, then the follow-on rows
    next_rows = {}
    if not args.no_next and w0.T > 0:
        cfgs = {}
        for cname, n, stride in (("C1", 2000, 8), ("C2", 400, 4), ("C4", 100, 4), ("C5", 60, 2)):
            if cname != args.config:
                cfgs[cname] = bench_config(sv, torch, dev, cname, n, 20, stride)
                torch.cuda.empty_cache()
        next_rows["configs"] = cfgs
        next_rows["F1_sample"] = bench_sampling(sv, torch, sets, dev, code, args)
        next_rows["per_gpu_share"] = bench_shares(sv, torch, sets, dev, code)
        next_rows["F2_adaptive_gamma"] = bench_adaptive(sv, torch, dev)
        next_rows["F3_deterministic_drafts"] = bench_ngram(sv, torch, dev)
        next_rows["F4_vocab_parallel"] = bench_vshard(sv, torch, sets, dev, code)

    # acceptance metrics of the measured inputs
    acc = np.concatenate(nb)
    gam = np.concatenate([w.gammas for w, _ in sets]).astype(np.int64)
    alpha_hat = acc.sum() / (acc + (acc < gam)).sum()
    log(f"[bench] {args.config}: {ms * 1e3:.2f} us/step, {value / 1e6:.2f} M positions/s, "
        f"{path_gbps:.0f} GB/s ({path_gbps / HBM_PEAK_GBPS:.1%} of peak) over the method's "
        f"{path_bytes / 1e6:.1f} MB/step; this plan reads {needed / 1e6:.1f} MB/step")
    for name, t in ktimes:
        log(f"[bench]   {name:20s} {t * 1e3:8.2f} us")
    log(f"[bench] {k1}: frac {k1_gbps / HBM_PEAK_GBPS:.3f} (method bytes), "
        f"frac_read {k1_needed / k1_s / 1e9 / HBM_PEAK_GBPS:.3f} (bytes read), frac_traffic "
        + (f"{traffic / k1_s / 1e9 / HBM_PEAK_GBPS:.3f} (counter bytes)" if traffic else "n/a (no counters for these sources)"))
    log(f"[bench] acceptance: alpha_hat={alpha_hat:.4f} tokens/round={np.mean(acc + 1):.4f} "
        f"accepted/drafted={acc.sum() / gam.sum():.4f}")

    cfgd = synth.CONFIGS[args.config]
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "verified positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32/f64",
        "data": "synthetic",
        "config": {
            "workload": (f"{args.config}: B={w0.B} gamma={cfgd['gamma']} V={w0.V} {w0.dtype} logits"
                         + (", fp32 q" if w0.T > 0 else ", greedy") + f", T={w0.T:g}"),
            "B": w0.B, "gamma": cfgd["gamma"] if not ragged else "ragged 1..8", "V": w0.V,
            "logits": w0.dtype, "T": w0.T, "input_sets": len(sets),
            "rotated_MB": len(sets) * input_bytes(w0) / 1e6,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": k1,
            "achieved": k1_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": k1_gbps / HBM_PEAK_GBPS,
            "traffic": traffic,
            "bytes_per_launch": k1_bytes,
            "bytes_basis": ("the two-pass method's bytes per sequence (every draft row, the drawn row, "
                            "q of the rejected row, ids, uniforms, outputs) from this run's accepted counts"),
            "needed_bytes_per_launch": k1_needed,
            "needed_GBps": k1_needed / k1_s / 1e9,
            "frac_read": k1_needed / k1_s / 1e9 / HBM_PEAK_GBPS,
            "frac_traffic": traffic / k1_s / 1e9 / HBM_PEAK_GBPS if traffic else None,
            "kernel_us": kt[k1] * 1e3,
        },
        "path": {
            "plan": "one launch, stops reading rows at the first rejection" if stop else plan_txt,
            "method_bytes_per_step": path_bytes,
            "needed_bytes_per_step": needed,
            "achieved_GBps": path_gbps,
            "frac_of_peak": path_gbps / HBM_PEAK_GBPS,
            "kernel_us": {n: t * 1e3 for n, t in ktimes},
            "every_row_read": all_rows,
        },
        "next_rows": next_rows,
        "acceptance": {"alpha_hat": float(alpha_hat), "tokens_per_round": float(np.mean(acc + 1)),
                       "accepted_per_drafted": float(acc.sum() / gam.sum())},
    }
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle for ~{args.cpu_seconds:.0f} s")
        line["cpu_baseline"] = cpu_baseline(w0, args.cpu_seconds)
    ver.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
