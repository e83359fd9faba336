"""CPU model of the cross-workgroup protocol of the ring plan
(pair_ring_kernel in csrc/kda_ring.hip), explored over every interleaving of
its flag operations and its ring and entry accesses for small sizes.

One unit (one sequence and head) is split over NCT workgroups, one per
16-column tile of the state; each holds NPW producer waves, a gate wave, the
chain wave and the output wave.  Tile p mod NCT makes pair p, writes it to
ring slot p mod R in L2 once every tile has taken pair p - R, and then sets
the unit's flag ready[p mod R] = p.  The gate of each tile is the only wave
that polls L2: a round publishes done[tile] (the last pair both of its
consumers took), reads the R ready flags and the NCT done flags, sets its LDS
flag lfree to the slowest tile's done and forwards the run of published pairs
to its LDS flag lready.  The chain and the output wave of a tile read each
pair from its slot (the chain issues the loads of the next pair a whole step
ahead, once lready shows it; the output wave once uready shows U of the
current pair, which the chain stores only after that wait) and hand U and the
chain's state over NU LDS entries (flags uready and udone); each releases a
pair (ldone) once the operands it still needs have arrived (the output wave
before it reads the entry).

Steps are the kernel's flag loads and stores and its slot and entry accesses
in program order.  A slot or entry write is two steps (begun, finished): a
read between them sees a torn block.  A load of a slot is issued at one step
and may read L2 at any later time before its data is used: the model checks
that the slot holds the pair when the load is issued and that no write to
the slot begins before the use, which covers every such time.  The gate reads its
R + NCT flags one at a time (for the larger sizes, in one step).  The
search checks, over every reachable state:

* no stale read: each load of a slot and each read of an entry sees the pair
  it is meant for, so neither a producer nor the chain overwrites what a
  reader still needs;
* progress: from every reachable state some interleaving finishes (a gate
  that spins cannot hide a deadlock).

It leaves out the data, the memory ordering that makes a flag visible only
after the data it publishes (the kernel waits for its slot stores to reach
L2 before the flag's atomic; the model takes each step as atomic and in
program order) and the give-up path of the bounded waits.
"""
from __future__ import annotations

import pytest


class Violation(AssertionError):
    pass


def _set(t, i, v):
    return t[:i] + (v,) + t[i + 1:]


def _explore(init, successors, finished, limit=3_000_000):
    """Every state reachable from `init` (successors(state) lists the next
    states); raises Violation if one of them cannot reach a finished state.
    Returns the number of states."""
    index = {init: 0}
    states = [init]
    preds = [[]]
    i = 0
    while i < len(states):
        for nxt in successors(states[i]):
            j = index.get(nxt)
            if j is None:
                j = len(states)
                if j >= limit:
                    raise RuntimeError("state space beyond the limit")
                index[nxt] = j
                states.append(nxt)
                preds.append([])
            preds[j].append(i)
        i += 1
    good = bytearray(len(states))
    todo = [k for k, st in enumerate(states) if finished(st)]
    for k in todo:
        good[k] = 1
    while todo:
        k = todo.pop()
        for q in preds[k]:
            if not good[q]:
                good[q] = 1
                todo.append(q)
    for k, ok in enumerate(good):
        if not ok:
            raise Violation(f"no interleaving finishes from state {states[k]}")
    return len(states)


# tile-local LDS flags
LREADY, LFREE, LDONE0, LDONE1, UREADY, UDONE, ENTRIES = range(7)

PLANTS = ("no_free_wait", "done_from_chain_only", "any_ready", "no_udone_wait", "own_tile_free",
          "out_loads_first")


def ring_model(NP, NCT, NPW, R, NU, plant=None, each_read=True):
    """State: (pcs, ready, done, slot, tiles)
      pcs[w]       per-wave local state
      ready[r]     last pair published in slot r (-1 none), one per unit
      done[t]      last pair tile t published as taken by both consumers
      slot[r]      pair slot r holds (('w', p) while being written)
      tiles[t]     (lready, lfree, ldone0, ldone1, uready, udone, entries)
                   with entries[e] the pair whose U and state entry e holds
    A `plant` name switches one step of the protocol to a plausible mistake.
    each_read False takes the gate's R + NCT flag reads as one step: each of
    its decisions needs only that every flag it read held at least that value
    when it acts (the flags only grow), which reads in one step or in several
    both give; the single step keeps larger rings and more tiles small enough
    to search."""
    assert plant in (None,) + PLANTS
    NW = NPW + 3                         # waves per tile
    GATE, CHAIN, OUT = NPW, NPW + 1, NPW + 2
    stride = NCT * NPW

    def nxt_pair(s):
        return s + 1 if s + 1 < NP else s   # the last step reloads its own pair

    def producer(st, t, w):
        pcs, ready, done, slot, tiles = st
        i = t * NW + w
        pc = pcs[i]
        if pc == "end":
            return
        kind, p = pc
        if kind == "wait":            # slot p mod R is free once every tile took p - R
            if plant != "no_free_wait" and tiles[t][LFREE] < p - R:
                return
            yield (_set(pcs, i, ("write", p)), ready, done, slot, tiles)
        elif kind == "write":         # the block's stores begin
            for c in pcs:
                if isinstance(c, tuple) and len(c) == 3:
                    for q in c[2]:
                        if q % R == p % R:
                            raise Violation(f"tile {t} producer began pair {p} in slot {p % R} "
                                            f"while a load of pair {q} held it")
            yield (_set(pcs, i, ("reach", p)), ready, done, _set(slot, p % R, ("w", p)), tiles)
        elif kind == "reach":         # ... and have all reached L2
            yield (_set(pcs, i, ("flag", p)), ready, done, _set(slot, p % R, p), tiles)
        elif kind == "flag":
            n = p + stride
            yield (_set(pcs, i, ("wait", n) if n < NP else "end"), _set(ready, p % R, p), done,
                   slot, tiles)
        else:
            raise AssertionError(pc)

    def gate(st, t):
        pcs, ready, done, slot, tiles = st
        i = t * NW + GATE
        pc = pcs[i]
        if pc == "end":
            return
        lt = tiles[t]
        p = lt[LREADY] + 1            # the gate alone writes lready
        if pc == "top":
            if p >= NP:
                yield (_set(pcs, i, "end"), ready, done, slot, tiles)
                return
            d = lt[LDONE0] if plant == "done_from_chain_only" else min(lt[LDONE0], lt[LDONE1])
            if d > done[t]:
                done = _set(done, t, d)
            yield (_set(pcs, i, ("rd", ())), ready, done, slot, tiles)
            return
        kind, vals = pc
        if kind == "rd":              # one flag per step: R ready flags, then NCT done flags
            if each_read:
                k = len(vals)
                vals = vals + ((ready + done)[k],)
            else:
                vals = ready + done
            yield (_set(pcs, i, ("rd", vals) if len(vals) < R + NCT else ("free", vals)), ready,
                   done, slot, tiles)
        elif kind == "free":          # the slowest tile's done
            mn = vals[R + t] if plant == "own_tile_free" else min(vals[R:])
            if mn > lt[LFREE]:
                tiles = _set(tiles, t, _set(lt, LFREE, mn))
            yield (_set(pcs, i, ("fwd", vals)), ready, done, slot, tiles)
        elif kind == "fwd":           # the run of published pairs from p on
            m = 0
            for lane in range(R):
                want = p + (lane - p % R + R) % R     # the pair lane's slot holds next
                if vals[lane] >= want or (plant == "any_ready" and vals[lane] >= 0):
                    m |= 1 << lane
            sh = p % R
            run = ((m >> sh) | (m << (R - sh))) & ((1 << R) - 1)
            n = 0
            while n < R and run >> n & 1:
                n += 1
            n = min(n, NP - p)
            if n > 0:
                tiles = _set(tiles, t, _set(lt, LREADY, p + n - 1))
            yield (_set(pcs, i, "top"), ready, done, slot, tiles)
        else:
            raise AssertionError(pc)

    def issue(slot, q, who):
        """A load of pair q's slot is issued; it reads L2 at some time before
        its data is used.  It sees pair q whatever that time is exactly when
        the slot holds q now and no write to the slot begins before the use
        (a producer's write checks the loads still open)."""
        if slot[q % R] != q:
            raise Violation(f"{who} loaded slot {q % R} for pair {q}: it held {slot[q % R]}")
        return q

    def consumer(st, t, which):
        """The chain (which 0) or the output wave (which 1) of tile t.  Its
        pc is (kind, s, open) with `open` the pairs whose slot loads are
        still in flight."""
        pcs, ready, done, slot, tiles = st
        i = t * NW + (CHAIN if which == 0 else OUT)
        pc = pcs[i]
        if pc == "end":
            return
        lt = tiles[t]
        who = f"tile {t} " + ("chain" if which == 0 else "output wave")

        def go(npc, tiles=tiles):
            return (_set(pcs, i, npc), ready, done, slot, tiles)

        def with_entry(e, v):
            return _set(tiles, t, _set(lt, ENTRIES, _set(lt[ENTRIES], e, v)))

        if pc == "pro":               # pair 0 published: its loads
            if lt[LREADY] >= 0:
                yield go(("top", 0, (issue(slot, 0, who),)))
            return
        kind, s, op = pc
        if kind == "top" and which == 0:   # chain: the next pair published, entry s mod NU read
            sn = nxt_pair(s)
            if lt[LREADY] < sn:
                return
            if plant != "no_udone_wait" and lt[UDONE] < s - NU:
                return
            yield go(("use", s, op + (issue(slot, sn, who),)))
        elif kind == "top":           # output wave: U of pair s ready, which the chain stores
            # only after its own wait for pair s + 1; then the next pair's loads
            if lt[UREADY] < s and plant != "out_loads_first":
                return
            yield go(("use", s, op + (issue(slot, nxt_pair(s), who),)))
        elif kind == "use":           # pair s's operands arrived: its loads close
            j = op.index(s)
            op = op[:j] + op[j + 1:]
            if which == 0:            # the chain's writes of entry s mod NU begin
                yield go(("wdone", s, op), with_entry(s % NU, ("w", s)))
            else:                     # the output wave releases the slot at once
                yield go(("orel", s, op))
        elif kind == "orel":
            yield go(("rd", s, op), _set(tiles, t, _set(lt, LDONE1, s)))
        elif kind == "wdone":         # chain: the entry written, then uready
            yield go(("ur", s, op), with_entry(s % NU, s))
        elif kind == "ur":
            yield go(("rel", s, op), _set(tiles, t, _set(lt, UREADY, s)))
        elif kind == "rd":
            if lt[UREADY] < s:        # (only a planted early load gets here first)
                return
            got = lt[ENTRIES][s % NU]
            if got != s:
                raise Violation(f"{who} read entry {s % NU} for pair {s}: it held {got}")
            yield go(("ud", s, op))
        elif kind == "ud":            # output wave: the entry released, the products follow
            nt = _set(tiles, t, _set(lt, UDONE, s))
            yield go(("top", s + 1, op) if s + 1 < NP else ("drain", s, op), nt)
        elif kind == "rel":           # chain: pair s released (before its state update)
            nt = _set(tiles, t, _set(lt, LDONE0, s))
            yield go(("top", s + 1, op) if s + 1 < NP else ("drain", s, op), nt)
        elif kind == "drain":         # the last step's reload of its own pair lands
            yield go("end")
        else:
            raise AssertionError(pc)

    def successors(st):
        for t in range(NCT):
            for w in range(NPW):
                yield from producer(st, t, w)
            yield from gate(st, t)
            yield from consumer(st, t, 0)
            yield from consumer(st, t, 1)

    pcs = []
    for t in range(NCT):
        for w in range(NPW):
            p = t + NCT * w
            pcs.append(("wait", p) if p < NP else "end")
        pcs += ["top", "pro", "pro"]
    tile0 = (-1, -1, -1, -1, -1, -1, (None,) * NU)
    init = (tuple(pcs), (-1,) * R, (-1,) * NCT, (None,) * R, (tile0,) * NCT)
    finished = lambda st: all(pc == "end" for pc in st[0])
    return init, successors, finished


# (NP, NCT, NPW, R, NU, each_read): two tiles with the gate's reads one at a
# time; larger rings with the reads in one step; one tile with up to three
# producer waves.  Three tiles take more states than a test can search.
CASES = ([(NP, 2, 1, 2, NU, True) for NP in (1, 2, 3, 4, 5) for NU in (1, 2)]
         + [(4, 2, 1, 3, 1, False), (3, 2, 1, 3, 2, False), (5, 2, 2, 2, 1, False)]
         + [(6, 1, 1, 3, 1, True), (6, 1, 1, 2, 2, True), (4, 1, 2, 2, 2, True),
            (7, 1, 2, 3, 2, True), (6, 1, 3, 3, 2, True), (8, 1, 1, 2, 1, True)])


@pytest.mark.parametrize("NP,NCT,NPW,R,NU,each_read", CASES)
def test_ring_protocol(NP, NCT, NPW, R, NU, each_read):
    n = _explore(*ring_model(NP, NCT, NPW, R, NU, each_read=each_read))
    assert n > 0


@pytest.mark.parametrize("plant", PLANTS)
def test_model_finds_a_planted_mistake(plant):
    """The model is not vacuous: a producer that does not wait for its slot,
    a gate that publishes its tile's done from the chain alone, takes any
    published flag for the pair it waits for, or frees slots by its own
    tile's progress, a chain that does not wait for the output wave to read
    an entry, and an output wave that issues the next pair's loads before U
    of the current pair is ready are each caught as a stale read."""
    NU = 1 if plant == "no_udone_wait" else 2
    with pytest.raises(Violation, match="held"):
        _explore(*ring_model(4, 2, 1, 2, NU, plant))


def test_one_slot_deadlocks():
    """A ring needs two slots: each consumer waits for the next pair to be
    published before it releases the current one, and with one slot the next
    pair's producer waits for that release."""
    with pytest.raises(Violation, match="no interleaving finishes"):
        _explore(*ring_model(3, 2, 1, 1, 1))
