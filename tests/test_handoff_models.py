"""CPU model checks of two hand-offs between workgroups that the kernels rely on (no GPU).

Both are explored over every interleaving of their workgroups (thread 0 of each, which
makes every shared-memory access of the protocol), over two consecutive calls, with the
memory as the previous call left it. Stores and returnless atomics are issued into the
issuing workgroup's queue and performed later, in any order the explorer picks
(s_waitcnt vmcnt(0) blocks until the queue is empty: gfx9 counts stores and returnless
atomics in vmcnt); atomics with a return value and loads are performed at once, at
system scope (past the per-XCD L2 caches), after the workgroup's own queued accesses to
the same address (one thread's accesses to one address stay in order). A kernel's end
performs every queued access.

1. The split draw of the two-launch plan (k_draw_part): S workgroups of one sequence
   each store their sums (three words), wait for the stores to complete, and add one to
   the sequence's count; the one that brings it to S resets it to 0 and reads every
   slice's sums. Checked: the reader sees this call's sums of every slice; exactly one
   reader per call; the count is 0 when the next call starts.

2. Greedy verification with helpers (k_greedy_help): the owner of a sequence resets the
   published minimum to "none" and the participant count to (epoch, 1), waits, and opens
   the claim counter at (epoch, 2) (rows 0 and 1 are its own). A helper joins if the
   counter carries this call's epoch, has rows left and no mismatch is published: it adds
   one to the participant count (returnless), waits, and claims two rows. Each
   participant walks its rows; at each row's end it claims the next row and reads the
   published minimum; a row that mismatches (or the bonus row g) is published with an
   atomic min of (row, token); it leaves on publishing, when its next row lies past g or
   past the published minimum; before leaving it waits for its atomics, then subtracts one
   from the count, and the one that brings it to 0 reads the minimum and writes the
   outputs. Checked: every write of the outputs is the right one (the first mismatching
   row and its token, or the bonus row's), so a helper that joins after the owner has
   already written (a second writer) writes the same outputs; there is at least one
   writer; every state can reach the end.

Planted mistakes that each check must catch: the split draw counting before its stores
complete; a helper that claims rows before its join is counted; a participant that
leaves before its published minimum is performed.
"""
import pytest

NONE = (1 << 31, 0)  # the published minimum when no row is published: (row, token)


class Explorer:
    """Every interleaving of processes with per-process queues of pending accesses."""

    def __init__(self, calls):
        self.calls = calls

    def run(self):
        s0 = self.first_state()
        seen = {s0: 0}
        order = [s0]
        succ = []
        i = 0
        while i < len(order):
            s = order[i]
            i += 1
            nx = [] if s == "end" else self.succ(s)
            ids = []
            for t in nx:
                if t not in seen:
                    seen[t] = len(order)
                    order.append(t)
                ids.append(seen[t])
            succ.append(ids)
        assert "end" in seen, "the last call never ends"
        pred = [[] for _ in order]
        for a, ids in enumerate(succ):
            for b in ids:
                pred[b].append(a)
        good = {seen["end"]}
        stack = [seen["end"]]
        while stack:
            b = stack.pop()
            for a in pred[b]:
                if a not in good:
                    good.add(a)
                    stack.append(a)
        assert len(good) == len(order), ("states that cannot reach the end", len(order) - len(good))
        return len(order)

    def succ(self, st):
        call, mem, procs, queues = st
        out = []
        for i, q in enumerate(queues):
            seen = set()
            for qi, op in enumerate(q):
                if op[1] in seen:
                    continue
                seen.add(op[1])
                m2 = self.perform(dict(mem), op)
                q2 = list(queues)
                q2[i] = q[:qi] + q[qi + 1:]
                out.append((call, tuple(sorted(m2.items(), key=repr)), procs, tuple(q2)))
        for i, p in enumerate(procs):
            r = self.step(call, dict(mem), i, p, queues[i])
            if r is None:
                continue
            m2, p2, q2 = r
            pl = list(procs)
            pl[i] = p2
            ql = list(queues)
            ql[i] = q2
            out.append((call, tuple(sorted(m2.items(), key=repr)), tuple(pl), tuple(ql)))
        if all(p[0] == "done" for p in procs):
            m2 = dict(mem)
            for q in queues:
                for op in q:
                    m2 = self.perform(m2, op)
            self.end_of_call(call, m2)
            if call < self.calls:
                out.append(self.next_call(call + 1, m2))
            else:
                out.append("end")
        return out

    @staticmethod
    def blocked(q, *addrs):
        """An access to addrs must wait for this workgroup's queued accesses to them."""
        return any(op[1] in addrs for op in q)

    @staticmethod
    def perform(m, op):
        kind, addr, val = op
        if kind == "store":
            m[addr] = val
        elif kind == "add":
            e, c = m[addr]
            m[addr] = (e, c + val)
        elif kind == "min":
            m[addr] = min(m[addr], val)
        return m


class SplitDraw(Explorer):
    def __init__(self, S=2, calls=2, planted=None):
        super().__init__(calls)
        self.S, self.planted = S, planted

    def first_state(self):
        mem = {"cnt": 0, "fin": 0}
        for s in range(self.S):
            for w in range(3):
                mem[("sum", s, w)] = None
        return (1, tuple(sorted(mem.items(), key=repr)), (("st", 0, ()),) * self.S, ((),) * self.S)

    def step(self, call, mem, i, p, q):
        pc, k, view = p
        if pc == "st":  # issue word k of this slice's sums
            q2 = q + (("store", ("sum", i, k), (call, i, k)),)
            return mem, (("st", k + 1, ()) if k + 1 < 3 else ("wait" if self.planted != "no_wait" else "cnt", 0, ())), q2
        if pc == "wait":
            return None if q else (mem, ("cnt", 0, ()), q)
        if pc == "cnt":
            if self.blocked(q, "cnt"):
                return None
            old = mem["cnt"]
            mem["cnt"] = old + 1
            if old == self.S - 1:
                return mem, ("read", 0, ()), q + (("store", "cnt", 0),)
            return mem, ("done", 0, ()), q
        if pc == "read":  # every slice's three words
            s, w = divmod(k, 3)
            if self.blocked(q, ("sum", s, w)):
                return None
            v = mem[("sum", s, w)]
            assert v == (call, s, w), ("the last slice read a stale sum", call, s, w, v)
            if k + 1 < 3 * self.S:
                return mem, ("read", k + 1, ()), q
            mem["fin"] += 1
            return mem, ("done", 0, ()), q
        return None

    def end_of_call(self, call, m):
        assert m["fin"] == 1, ("readers in call", call, m["fin"])
        assert m["cnt"] == 0, ("count left at", m["cnt"])

    def next_call(self, call, m):
        m = dict(m)
        m["fin"] = 0
        return (call, tuple(sorted(m.items(), key=repr)), (("st", 0, ()),) * self.S, ((),) * self.S)


class Greedy(Explorer):
    """One sequence with rows 0 .. g (row g is the bonus row); `mismatch` lists the draft
    rows whose argmax differs from the draft; the token of row i is 100 + i."""

    def __init__(self, g=2, mismatch=(1,), helpers=1, calls=2, planted=None):
        super().__init__(calls)
        self.g, self.mismatch, self.H, self.planted = g, set(mismatch), helpers, planted
        first = min(self.mismatch | {g})
        self.want = (first, 100 + first)

    def procs0(self):
        return (("o_init", ()),) + (("h_load", ()),) * self.H

    def first_state(self):
        mem = {"claim": (0, 0), "part": (0, 0), "best": (0, 0), "out": ()}
        return (1, tuple(sorted(mem.items(), key=repr)), self.procs0(), ((),) * (1 + self.H))

    def step(self, call, mem, i, p, q):
        pc, loc = p
        g = self.g
        E = call
        if pc == "done":
            return None
        if pc == "o_init":
            q2 = q + (("store", "best", NONE), ("store", "part", (E, 1)))
            return mem, ("o_wait", ()), q2
        if pc == "o_wait":
            if q:
                return None
            return mem, ("o_open", ()), q
        if pc == "o_open":
            return mem, ("row_end", (0, 1)), q + (("store", "claim", (E, 2)),)
        if pc in ("h_load", "h_claim", "row_end") and self.blocked(q, "claim", "best"):
            return None
        if pc in ("leave", "write") and self.blocked(q, "part", "best") and self.planted != "leave_early":
            return None
        if pc == "h_load":
            c = mem["claim"]
            b = mem["best"]
            join = c[0] == E and c[1] <= g and b == NONE
            if not join:
                return mem, ("done", ()), q
            q2 = q + (("add", "part", 1),)
            return mem, ("h_wait" if self.planted != "claim_first" else "h_claim", ()), q2
        if pc == "h_wait":
            if q:
                return None
            return mem, ("h_claim", ()), q
        if pc == "h_claim":
            e, r0 = mem["claim"]
            mem["claim"] = (e, r0 + 2)
            if r0 > g:
                return mem, ("leave", ()), q
            return mem, ("row_end", (r0, r0 + 1)), q
        if pc == "row_end":  # the participant has walked row rc; claim the next, read the minimum
            rc, rn = loc
            e, nc = mem["claim"]
            mem["claim"] = (e, nc + 1)
            known = mem["best"][0]
            stop = rc == g or rc in self.mismatch
            q2 = q
            if stop:
                q2 = q + (("min", "best", (rc, 100 + rc)),)
            if stop or rn > g or known < rn:
                return mem, ("leave", ()), q2
            return mem, ("row_end", (rn, nc)), q2
        if pc == "leave":
            if q and self.planted != "leave_early":
                return None
            e, c = mem["part"]
            mem["part"] = (e, c - 1)
            if c == 1:
                return mem, ("write", ()), q
            return mem, ("done", ()), q
        if pc == "write":
            row, tok = mem["best"]
            n = min(row, g)
            got = (n, tok if row <= g else None)
            assert got == self.want, ("outputs written", call, got, self.want)
            mem["out"] = mem["out"] + (got,)
            return mem, ("done", ()), q
        raise AssertionError(pc)

    def end_of_call(self, call, m):
        assert len(m["out"]) >= 1, ("no writer in call", call)

    def next_call(self, call, m):
        m = dict(m)
        m["out"] = ()
        return (call, tuple(sorted(m.items(), key=repr)), self.procs0(), ((),) * (1 + self.H))


@pytest.mark.parametrize("S", [1, 2, 3])
def test_split_draw_every_interleaving(S):
    assert SplitDraw(S=S, calls=2).run() > 5


def test_split_draw_planted_mistake_is_caught():
    with pytest.raises(AssertionError):
        SplitDraw(S=2, calls=2, planted="no_wait").run()


@pytest.mark.parametrize("g,mismatch,helpers", [(2, (), 1), (2, (0,), 1), (2, (1,), 1), (3, (2,), 1),
                                                (3, (1, 2), 1), (2, (1,), 2), (3, (), 2)])
def test_greedy_helpers_every_interleaving(g, mismatch, helpers):
    assert Greedy(g=g, mismatch=mismatch, helpers=helpers, calls=2).run() > 5


@pytest.mark.parametrize("mistake,g,mismatch", [("claim_first", 3, (2,)), ("leave_early", 3, (1,))])
def test_greedy_helpers_planted_mistake_is_caught(mistake, g, mismatch):
    with pytest.raises(AssertionError):
        Greedy(g=g, mismatch=mismatch, helpers=1, calls=2, planted=mistake).run()
