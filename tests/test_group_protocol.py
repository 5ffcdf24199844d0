"""CPU model check of the small-batch plan's hand-offs between workgroups (no GPU).

In the small-batch one-launch plan every sequence has W workgroups (chunks of its draft
rows). Each stores its pass-1 record as 64-bit words, the value in the high half and the
call's tag in the low half, with no wait. Wave 0 of every workgroup of the sequence then
reads all W records, word by word, and starts over until every word it read carries this
call's tag; the workgroup's other waves wait at a barrier for it. Every wave whose unit
index is below U then sweeps its unit of the drawn row and stores the unit's sums as
tagged words (two here), with no wait. The wave of unit 0 then reads every unit's words,
starting over until all carry the tag, and writes the outputs.

The model: each step of a wave is one access to shared memory, taken atomically; a store
is issued into the wave's queue of pending stores and performed at memory later, at any
point the explorer chooses (stores of one wave to one address in order, to different
addresses in any order). The end of a kernel performs every pending store. The explorer
runs every interleaving of the waves of `calls` consecutive calls, with the workspace as
the previous call left it (the first call sees the zeroed workspace: tag 0, which no
call uses), and checks:
  * every record a wave accepts is this call's, in every word;
  * the finishing wave accepts this call's sums of every unit, in every word;
  * exactly one wave finishes per call;
  * from every reachable state the end of the last call is reachable (no wave can be
    trapped in a wait).
Three planted mistakes must each be caught: a poll that checks the tag of one word of
each record (or unit) only, records without tags, and sums without tags.
"""
import os
import re

import pytest


class Model:
    def __init__(self, W=2, U=2, wpg=1, calls=2, planted=None):
        assert 1 <= U <= W * wpg
        self.W, self.U, self.wpg, self.calls, self.planted = W, U, wpg, calls, planted
        self.nw = W * wpg  # waves: workgroup j has waves j*wpg .. j*wpg + wpg - 1
        self.recw = 2      # words per record
        self.sumw = 2      # words per unit's sums

    # shared memory: dict address -> value; addresses ("rec", j, w), ("sum", u, w), "fin"
    def initial(self):
        mem = {}
        for j in range(self.W):
            for w in range(self.recw):
                mem[("rec", j, w)] = (0, None)  # (tag, value)
        for u in range(self.U):
            for w in range(self.sumw):
                mem[("sum", u, w)] = (0, None)
        mem["fin"] = 0
        return mem

    def rec_word(self, call, j, w):
        tag = None if self.planted == "no_tag" else call
        return (tag, (call, j, w))

    def start_wave(self, i):
        j, k = divmod(i, self.wpg)
        if k == 0:
            return ("store_rec", 0, ())  # (pc, index, local view)
        return ("barrier", 0, ())

    def sum_word(self, call, u, w):
        tag = None if self.planted == "untagged_sums" else call
        return (tag, (call, u, w))

    def tag_ok(self, word, call, w, sums=False):
        tag = word[0]
        if self.planted == ("untagged_sums" if sums else "no_tag"):
            return True
        if self.planted == "one_word" and w > 0:
            return True
        return tag == call

    def steps(self, state):
        """Successor states of `state` = (call, mem (sorted tuple), waves, pending, polled)."""
        call, memt, waves, pending, polled = state
        mem = dict(memt)
        out = []
        # perform one pending store (the oldest per address of each wave)
        for i, q in enumerate(pending):
            seen = set()
            for qi, (addr, val) in enumerate(q):
                if addr in seen:
                    continue
                seen.add(addr)
                m2 = dict(mem)
                m2[addr] = val
                p2 = list(pending)
                p2[i] = q[:qi] + q[qi + 1:]
                out.append((call, tuple(sorted(m2.items(), key=repr)), waves, tuple(p2), polled))
        for i, (pc, idx, view) in enumerate(waves):
            r = self.wave_step(call, mem, i, pc, idx, view, pending[i], polled)
            if r is None:
                continue
            m2, wv, q2, pol2 = r
            w2 = list(waves)
            w2[i] = wv
            p2 = list(pending)
            p2[i] = q2
            out.append((call, tuple(sorted(m2.items(), key=repr)), tuple(w2), tuple(p2), pol2))
        # kernel boundary: every wave done -> perform every pending store, start the next call
        if all(w[0] == "done" for w in waves):
            m2 = dict(mem)
            for q in pending:
                for addr, val in q:
                    m2[addr] = val
            assert m2["fin"] == 1, ("finishes in call", call, m2["fin"])
            if call < self.calls:
                m2["fin"] = 0
                waves2 = tuple(self.start_wave(i) for i in range(self.nw))
                out.append((call + 1, tuple(sorted(m2.items(), key=repr)), waves2, ((),) * self.nw,
                            (False,) * self.W))
            else:
                out.append(("end",))
        return out

    def wave_step(self, call, mem, i, pc, idx, view, q, polled):
        """One step of wave i; None if it cannot move (blocked or done)."""
        j, k = divmod(i, self.wpg)
        W, U = self.W, self.U
        if pc == "store_rec":  # issue record word idx, no wait
            q2 = q + ((("rec", j, idx), self.rec_word(call, j, idx)),)
            nxt = ("store_rec", idx + 1, ()) if idx + 1 < self.recw else ("poll", 0, ())
            return mem, nxt, q2, polled
        if pc == "poll":  # read word idx of the group's records
            nwords = W * self.recw
            lj, w = divmod(idx, self.recw)
            view2 = view + (mem[("rec", lj, w)],)
            if idx + 1 < nwords:
                return mem, ("poll", idx + 1, view2), q, polled
            ok = all(self.tag_ok(word, call, n % self.recw) for n, word in enumerate(view2))
            if not ok:
                return mem, ("poll", 0, ()), q, polled
            for n, word in enumerate(view2):
                lj2, w2 = divmod(n, self.recw)
                assert word[1] == (call, lj2, w2), ("stale record accepted", call, n, word)
            pol = list(polled)
            pol[j] = True
            return mem, ("unit", 0, ()), q, tuple(pol)
        if pc == "barrier":  # the other waves of the workgroup wait for wave 0's poll
            if not polled[j]:
                return None
            return mem, ("unit", 0, ()), q, polled
        u = j * self.wpg + k
        if pc == "unit":  # issue sum word idx of unit u, no wait
            if u >= U:
                return mem, ("done", 0, ()), q, polled
            q2 = q + ((("sum", u, idx), self.sum_word(call, u, idx)),)
            if idx + 1 < self.sumw:
                return mem, ("unit", idx + 1, ()), q2, polled
            return mem, ("read" if u == 0 else "done", 0, ()), q2, polled
        if pc == "read":  # unit 0's wave: read word idx of every unit's sums
            uu, w = divmod(idx, self.sumw)
            view2 = view + (mem[("sum", uu, w)],)
            if idx + 1 < U * self.sumw:
                return mem, ("read", idx + 1, view2), q, polled
            ok = all(self.tag_ok(word, call, n % self.sumw, sums=True) for n, word in enumerate(view2))
            if not ok:
                return mem, ("read", 0, ()), q, polled
            for n, word in enumerate(view2):
                uu2, w2 = divmod(n, self.sumw)
                assert word[1] == (call, uu2, w2), ("stale sums accepted by the finisher", call, n, word)
            m2 = dict(mem)
            m2["fin"] = m2["fin"] + 1
            return m2, ("done", 0, ()), q, polled
        if pc == "done":
            return None
        raise AssertionError(pc)

    def explore(self):
        mem = self.initial()
        s0 = (1, tuple(sorted(mem.items(), key=repr)), tuple(self.start_wave(i) for i in range(self.nw)),
              ((),) * self.nw, (False,) * self.W)
        seen = {s0: 0}
        order = [s0]
        succ = []
        n = 0
        while n < len(order):
            s = order[n]
            n += 1
            nx = [] if s == ("end",) else self.steps(s)
            ids = []
            for t in nx:
                if t not in seen:
                    seen[t] = len(order)
                    order.append(t)
                ids.append(seen[t])
            succ.append(ids)
        # every reachable state can still reach the end
        end = seen.get(("end",))
        assert end is not None, "the last call never ends"
        pred = [[] for _ in order]
        for a, ids in enumerate(succ):
            for b in ids:
                pred[b].append(a)
        good = {end}
        stack = [end]
        while stack:
            b = stack.pop()
            for a in pred[b]:
                if a not in good:
                    good.add(a)
                    stack.append(a)
        assert len(good) == len(order), ("states that cannot reach the end", len(order) - len(good))
        return len(order)


@pytest.mark.parametrize("W,U,wpg", [(1, 1, 1), (2, 1, 1), (2, 2, 1), (1, 2, 2), (2, 2, 2), (2, 3, 2)])
def test_group_protocol_every_interleaving(W, U, wpg):
    states = Model(W=W, U=U, wpg=wpg, calls=2).explore()
    assert states > 10


@pytest.mark.parametrize("mistake,W,U", [("one_word", 2, 1), ("one_word", 1, 2), ("no_tag", 2, 1),
                                         ("untagged_sums", 1, 2)])
def test_group_protocol_planted_mistake_is_caught(mistake, W, U):
    with pytest.raises(AssertionError):
        Model(W=W, U=U, wpg=2 if U > W else 1, calls=2, planted=mistake).explore()


def test_group_code_has_no_barrier_in_the_draw():
    """After the workgroup's one barrier (behind wave 0's wait) each wave of the small-batch
    plan sweeps its unit and only the last to count finishes the draw: the functions the
    waves run from there on contain no workgroup barrier."""
    src = open(os.path.join(os.path.dirname(__file__), "..", "speculative_sampling_verification_03_amd", "csrc",
                            "spec_verify.hip"), encoding="utf-8").read()
    names = ["group_finish", "wave_resweep", "draw_sweep", "draw_select", "drawn_row", "drawn_q", "uniform_draw"]
    found = 0
    for name in names:
        m = re.search(r"__device__[^{;]*\b" + name + r"\b[^;{]*\{", src)
        if not m:
            continue
        found += 1
        depth, i = 1, m.end()
        while depth and i < len(src):
            depth += {"{": 1, "}": -1}.get(src[i], 0)
            i += 1
        body = src[m.end():i]
        assert "__syncthreads" not in body and "team_barrier" not in body, name
    assert found == len(names), found
    # in the kernel, the one barrier comes before the unit sweep
    m = re.search(r"void k_verify_group\(Args a\) \{", src)
    assert m
    body = src[m.end():src.index("\n}\n", m.end())]
    assert body.count("__syncthreads") == 1
    assert body.index("__syncthreads") < body.index("draw_sweep")
