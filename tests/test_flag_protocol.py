"""CPU model of the LDS flag protocols of the split-plan state-chain kernels
(pair_inter_kernel and pair_roles_kernel in csrc/kda_pair.hip), explored over
every interleaving of the waves' LDS operations for small sizes.

Each wave is a small state machine whose steps are the kernel's LDS
operations in program order: flag loads and stores, entry writes by loaders,
entry reads (the pair's operands, V, U) and output writes by the chains and
output waves.  One LDS instruction is atomic with respect to the others and a
wave's own LDS operations complete in order, which is all the kernels rely
on.  The search checks, in every reachable state:

* no deadlock: while some wave is unfinished, some wave can take a step (so
  the bounded polls of the kernels never run out);
* no stale read: every read of a ring entry that the protocol treats as valid
  (after a flag that published it) sees the pair it expects -- which also
  rules out an early overwrite by a loader;
* (pair_inter_kernel) every pair's outputs leave the ring exactly once, after
  every chain wrote them.

It does not model the data the kernels compute, only who holds which entry.
"""
from __future__ import annotations

from collections import deque

import pytest


class Violation(AssertionError):
    pass


def _explore(init, waves, finished):
    """Breadth-first search over interleavings.  `waves` are step functions
    (state, i) -> new state | None (blocked or done); returns the number of
    states seen."""
    seen = {init}
    todo = deque([init])
    while todo:
        st = todo.popleft()
        moved = False
        for i, step in enumerate(waves):
            nxt = step(st, i)
            if nxt is None:
                continue
            moved = True
            if nxt not in seen:
                seen.add(nxt)
                todo.append(nxt)
        if not moved and not finished(st):
            raise Violation(f"deadlock in state {st}")
    return len(seen)


def _set(t, i, v):
    return t[:i] + (v,) + t[i + 1:]


# --------------------------------------------------------------- roles kernel
#
# State: (pcs, ready, done, uready, content, ucontent)
#   pcs[w]        per-wave local state tuple
#   ready[e]      last pair published in entry e (-1 none)
#   done[e][r]    last pair reader r released from entry e
#   uready[c]     last pair whose U chain c left in its entry
#   content[e]    pair whose block and V entry e holds ('w', p) while being written
#   ucontent[e][c]  pair whose U chain c left in its area of entry e

def roles_model(NP, NPAIR, NL, NCW):
    NREAD = 2 * NCW
    E = lambda p: p % NPAIR

    def loader(st, i):
        pcs, ready, done, uready, content, ucontent = st
        L = i - NREAD
        pc = pcs[i]
        if pc == "end":
            return None
        kind, p = pc
        e = E(p)
        if kind == "wait":
            if p >= NPAIR and any(done[e][r] < p - NPAIR for r in range(NREAD)):
                return None
            return (_set(pcs, i, ("dma", p)), ready, done, uready, content, ucontent)
        if kind == "dma":     # block and V land in the entry
            return (_set(pcs, i, ("vstore", p)), ready, done, uready,
                    _set(content, e, ("w", p)), ucontent)
        if kind == "vstore":  # V stores complete
            return (_set(pcs, i, ("publish", p)), ready, done, uready,
                    _set(content, e, p), ucontent)
        if kind == "publish":
            nxt = p + NL
            return (_set(pcs, i, ("wait", nxt) if nxt < NP else "end"), _set(ready, e, p),
                    done, uready, content, ucontent)
        raise AssertionError(pc)

    def chain(st, i):
        pcs, ready, done, uready, content, ucontent = st
        w = i
        pc = pcs[i]
        if pc == "end":
            return None
        kind, s, fl = pc
        e = E(s)

        def go(new_pc, **kw):
            d = dict(ready=ready, done=done, uready=uready, content=content, ucontent=ucontent)
            d.update(kw)
            return (_set(pcs, i, new_pc), d["ready"], d["done"], d["uready"], d["content"],
                    d["ucontent"])

        if kind == "start":           # spin on ready[0] >= 0, then read entry 0's first operands
            if ready[0] < 0:
                return None
            return go(("kread0", 0, 0))
        if kind == "kread0":
            if content[0] != 0:
                raise Violation(f"chain {w} read entry 0 holding {content[0]}")
            return go(("top", 0, 0))
        if kind == "top":
            if s == NP:
                return go("end")
            return go(("spin", s, fl) if fl < s else ("read", s, fl))
        if kind == "spin":            # the rare re-read of a pair read ahead of publication
            if ready[e] < s:
                return None
            return go(("reread", s, s))
        if kind == "reread":
            if content[e] != s:
                raise Violation(f"chain {w} re-read entry {e} for pair {s}: holds {content[e]}")
            return go(("read", s, fl))
        if kind == "read":            # V and the chain operands of pair s
            if content[e] != s:
                raise Violation(f"chain {w} read entry {e} for pair {s}: holds {content[e]}")
            return go(("uput", s, fl))
        if kind == "uput":
            return go(("uready", s, fl), ucontent=_set(ucontent, e, _set(ucontent[e], w, s)))
        if kind == "uready":
            return go(("release", s, fl), uready=_set(uready, w, s))
        if kind == "release":
            return go(("flag", s, fl), done=_set(done, e, _set(done[e], w, s)))
        if kind == "flag":            # fl = ready[(s + 1) % NPAIR]
            return go(("spec", s, ready[E(s + 1)]))
        if kind == "spec":            # first operands of pair s + 1, read ahead
            if s + 1 < NP and fl >= s + 1 and content[E(s + 1)] != s + 1:
                raise Violation(f"chain {w} read ahead entry {E(s + 1)} for pair {s + 1} "
                                f"after its flag showed it: holds {content[E(s + 1)]}")
            return go(("top", s + 1, fl))
        raise AssertionError(pc)

    def output(st, i):
        pcs, ready, done, uready, content, ucontent = st
        wc = i - NCW
        pc = pcs[i]
        if pc == "end":
            return None
        kind, s = pc
        e = E(s)
        if kind == "wait":
            if uready[wc] < s:
                return None
            return (_set(pcs, i, ("read", s)), ready, done, uready, content, ucontent)
        if kind == "read":            # U, the output and the update operands of pair s
            if ucontent[e][wc] != s:
                raise Violation(f"output wave {wc} read U of entry {e} for pair {s}: "
                                f"{ucontent[e][wc]}")
            if content[e] != s:
                raise Violation(f"output wave {wc} read entry {e} for pair {s}: holds {content[e]}")
            return (_set(pcs, i, ("release", s)), ready, done, uready, content, ucontent)
        if kind == "release":
            nd = _set(done, e, _set(done[e], NCW + wc, s))
            return (_set(pcs, i, ("wait", s + 1) if s + 1 < NP else "end"), ready, nd, uready,
                    content, ucontent)
        raise AssertionError(pc)

    pcs = tuple([("start", 0, 0)] * NCW + [("wait", 0)] * NCW
                + [("wait", L) if L < NP else "end" for L in range(NL)])
    init = (pcs, (-1,) * NPAIR, ((-1,) * NREAD,) * NPAIR, (-1,) * NCW, (None,) * NPAIR,
            ((None,) * NCW,) * NPAIR)
    waves = [chain] * NCW + [output] * NCW + [loader] * NL
    finished = lambda st: all(pc == "end" for pc in st[0])
    return init, waves, finished


# --------------------------------------------------------------- inter kernel
#
# State: (pcs, ready, done, content, outs, flushed)
#   outs[e][c]   pair whose outputs chain c left in entry e
#   flushed      tuple of pairs whose outputs left the ring, in order

def inter_model(NP, NPAIR, NL, NCW):
    E = lambda p: p % NPAIR
    tail = list(range(max(0, NP - NPAIR), NP))

    def loader(st, i):
        pcs, ready, done, content, outs, flushed = st
        L = i - NCW
        pc = pcs[i]
        if pc == "end":
            return None
        kind, p, k = pc            # k: index into the tail list in the tail phase

        def nxt_after_main(p):
            n = p + NL
            if n < NP:
                return ("wait", n, 0)
            return next_tail(0)

        def next_tail(j):
            while j < len(tail) and (tail[j] + NPAIR) % NL != L:
                j += 1
            return ("twait", tail[j], j) if j < len(tail) else "end"

        def flush(q):
            e = E(q)
            if content[e] != q or any(outs[e][c] != q for c in range(NCW)):
                raise Violation(f"loader {L} flushed entry {e} for pair {q}: holds "
                                f"{content[e]}, outputs {outs[e]}")
            return flushed + (q,)

        if kind == "wait":
            e = E(p)
            if p >= NPAIR:
                if any(done[e][c] < p - NPAIR for c in range(NCW)):
                    return None
                return (_set(pcs, i, ("write", p, 0)), ready, done, content, outs,
                        flush(p - NPAIR))
            return (_set(pcs, i, ("write", p, 0)), ready, done, content, outs, flushed)
        if kind == "write":
            e = E(p)
            return (_set(pcs, i, ("publish", p, 0)), ready, done, _set(content, e, p),
                    _set(outs, e, (None,) * NCW), flushed)
        if kind == "publish":
            return (_set(pcs, i, nxt_after_main(p)), _set(ready, E(p), p), done, content, outs,
                    flushed)
        if kind == "twait":
            e = E(p)
            if any(done[e][c] < p for c in range(NCW)):
                return None
            return (_set(pcs, i, next_tail(k + 1)), ready, done, content, outs, flush(p))
        raise AssertionError(pc)

    def chain(st, i):
        pcs, ready, done, content, outs, flushed = st
        w = i
        pc = pcs[i]
        if pc == "end":
            return None
        kind, s, fl = pc
        e = E(s)

        def go(new_pc, ready=ready, done=done, outs=outs):
            return (_set(pcs, i, new_pc), ready, done, content, outs, flushed)

        if kind == "start":
            if ready[0] < 0:
                return None
            return go(("kread0", 0, 0))
        if kind == "kread0":
            if content[0] != 0:
                raise Violation(f"chain {w} read entry 0 holding {content[0]}")
            return go(("top", 0, 0))
        if kind == "top":
            if s == NP:
                return go("end")
            return go(("spin", s, fl) if fl < s else ("read", s, fl))
        if kind == "spin":
            if ready[e] < s:
                return None
            return go(("reread", s, s))
        if kind == "reread":
            if content[e] != s:
                raise Violation(f"chain {w} re-read entry {e} for pair {s}: holds {content[e]}")
            return go(("read", s, fl))
        if kind == "read":
            if content[e] != s:
                raise Violation(f"chain {w} read entry {e} for pair {s}: holds {content[e]}")
            return go(("oput", s, fl))
        if kind == "oput":           # outputs over the chain's own V words
            return go(("release", s, fl), outs=_set(outs, e, _set(outs[e], w, s)))
        if kind == "release":
            return go(("flag", s, fl), done=_set(done, e, _set(done[e], w, s)))
        if kind == "flag":
            return go(("spec", s, ready[E(s + 1)]))
        if kind == "spec":
            if s + 1 < NP and fl >= s + 1 and content[E(s + 1)] != s + 1:
                raise Violation(f"chain {w} read ahead entry {E(s + 1)} for pair {s + 1} "
                                f"after its flag showed it: holds {content[E(s + 1)]}")
            return go(("top", s + 1, fl))
        raise AssertionError(pc)

    pcs = tuple([("start", 0, 0)] * NCW
                + [("wait", L, 0) if L < NP else "end" for L in range(NL)])
    # loaders with no main-phase pair go straight to their tail work
    pcs = list(pcs)
    for L in range(NL):
        if L >= NP:
            j = 0
            while j < len(tail) and (tail[j] + NPAIR) % NL != L:
                j += 1
            pcs[NCW + L] = ("twait", tail[j], j) if j < len(tail) else "end"
    pcs = tuple(pcs)
    init = (pcs, (-1,) * NPAIR, ((-1,) * NCW,) * NPAIR, (None,) * NPAIR,
            ((None,) * NCW,) * NPAIR, ())
    waves = [chain] * NCW + [loader] * NL

    def finished(st):
        if not all(pc == "end" for pc in st[0]):
            return False
        fl = st[5]
        if sorted(fl) != list(range(NP)):
            raise Violation(f"outputs left the ring as {fl}, expected each of 0..{NP - 1} once")
        return True

    return init, waves, finished


ROLE_CASES = [(NP, NPAIR, NL, 1) for NP in (1, 2, 3, 5, 7) for NPAIR in (2, 3, 5)
              for NL in (1, 2, 6)] + [(4, 2, 1, 2), (5, 3, 2, 2)]
INTER_CASES = [(NP, NPAIR, NL, NCW) for NP in (1, 2, 4, 6) for NPAIR in (2, 3, 4)
               for NL in (1, 2, 3) for NCW in (1, 2)]


@pytest.mark.parametrize("NP,NPAIR,NL,NCW", ROLE_CASES)
def test_roles_protocol(NP, NPAIR, NL, NCW):
    n = _explore(*roles_model(NP, NPAIR, NL, NCW))
    assert n > 0


@pytest.mark.parametrize("NP,NPAIR,NL,NCW", INTER_CASES)
def test_inter_protocol(NP, NPAIR, NL, NCW):
    n = _explore(*inter_model(NP, NPAIR, NL, NCW))
    assert n > 0


def test_model_finds_a_planted_early_overwrite():
    """The model is not vacuous: a loader that skips its wait for the readers
    to release an entry is caught as a stale read."""
    init, waves, finished = roles_model(4, 2, 2, 1)
    loader = waves[-1]

    def hasty_loader(st, i):
        pcs, ready, done, uready, content, ucontent = st
        pc = pcs[i]
        if pc != "end" and pc[0] == "wait":
            return (_set(pcs, i, ("dma", pc[1])), ready, done, uready, content, ucontent)
        return loader(st, i)

    with pytest.raises(Violation):
        _explore(init, waves[:-2] + [hasty_loader, hasty_loader], finished)


def test_model_finds_a_planted_deadlock():
    """...and a chain that waits for a pair no loader ever publishes is caught
    as a deadlock."""
    init, waves, finished = inter_model(3, 2, 1, 1)
    pcs = list(init[0])
    pcs[0] = ("spin", 0, -1)
    init = (tuple(pcs),) + init[1:]
    ready = list(init[1])
    ready[0] = -5
    init = (init[0], tuple(ready)) + init[2:]
    loader = waves[1]

    def lazy_loader(st, i):   # never publishes
        pc = st[0][i]
        if pc != "end" and pc[0] == "publish":
            return None
        return loader(st, i)

    with pytest.raises(Violation):
        _explore(init, [waves[0], lazy_loader], finished)
