"""Host model of the K-loop synchronisation protocols, checked over every
interleaving of a few abstract wavefronts.  CPU only.

Each wavefront runs a list of events on a ring of LDS stages:

* ("w", s, t): synchronous store of its piece of K tile t into stage s
  (the register path: global load, then LDS store);
* ("wall", s, t): synchronous store over the whole stage s (every piece:
  data laid out without regard to the stages' pieces);
* ("wx", s, label): synchronous store of this wave's partial sums into its
  piece of region s, laid out over the stage's bytes without regard to its
  pieces: the other pieces' tile data is clobbered (other waves' partial
  sums in the region are kept);
* ("issue", s, t): an asynchronous direct copy of its piece of tile t into
  stage s; the write lands at any later moment the model chooses;
* ("wait", t): block until none of this wave's copies of tiles <= t is still
  in flight (s_waitcnt on the copies; t = None waits for all);
* ("r", s, t): read the whole stage s (every wave's piece), expecting tile t;
  ("r", s, t, waves): read only the pieces of those waves (a stage that one
  group of waves fills, or one wave's partial sums);
* ("b",): workgroup barrier.

A schedule is correct when every read, in every interleaving and for every
landing time of every copy, sees tile t in all pieces of stage s, and no
interleaving deadlocks.  The protocols are those of the kernels (two stages
and one barrier per tile through registers or direct copies, the pipelined
multiply whose last step runs after the barrier, the S-stage copy ring of
the 16-bit-input kernels, the K split over groups of waves with its final
exchange of partial sums through LDS); the mutants (a barrier dropped, the
stage parity flipped, the last step read after the barrier, the wait
dropped or too weak, the partial sums written before the loop's last
barrier or read without a barrier) must each be caught.  The pages argue the one-barrier protocol in
prose ("My Triton From Scratch, Part 18", section "What ping-pong changes
about synchronization"); this is a machine check of that argument and of
its pipelined extension.
"""

from __future__ import annotations

import sys

import pytest


def check(programs, stages: int):
    """Explore every interleaving; return None, or a description of the
    first violation or deadlock found."""
    waves = len(programs)
    sys.setrecursionlimit(100000)
    seen = set()
    # content[s][v]: tile in wave v's piece of stage s (-1: never written)
    start = (tuple([0] * waves), tuple(tuple([-1] * waves) for _ in range(stages)),
             tuple(frozenset() for _ in range(waves)))
    stack = [start]
    while stack:
        state = stack.pop()
        if state in seen:
            continue
        seen.add(state)
        pcs, content, pending = state
        if all(pcs[v] == len(programs[v]) for v in range(waves)):
            continue
        moves = []
        # a copy in flight may land now
        for v in range(waves):
            for (s, t) in pending[v]:
                c = [list(row) for row in content]
                c[s][v] = t
                p = list(pending)
                p[v] = pending[v] - {(s, t)}
                moves.append((pcs, tuple(tuple(row) for row in c), tuple(p)))
        # barrier: all waves at a barrier together
        if all(pcs[v] < len(programs[v]) and programs[v][pcs[v]][0] == "b" for v in range(waves)):
            moves.append((tuple(pc + 1 for pc in pcs), content, pending))
        for v in range(waves):
            if pcs[v] == len(programs[v]):
                continue
            ev = programs[v][pcs[v]]
            nxt = list(pcs)
            nxt[v] += 1
            nxt = tuple(nxt)
            kind = ev[0]
            if kind == "b":
                continue
            if kind in ("w", "wall", "wx"):
                c = [list(row) for row in content]
                if kind == "w":
                    c[ev[1]][v] = ev[2]
                elif kind == "wx":
                    c[ev[1]] = [x if isinstance(x, str) else "clobbered" for x in c[ev[1]]]
                    c[ev[1]][v] = ev[2]
                else:
                    c[ev[1]] = [ev[2]] * waves
                moves.append((nxt, tuple(tuple(row) for row in c), pending))
            elif kind == "issue":
                p = list(pending)
                p[v] = pending[v] | {(ev[1], ev[2])}
                moves.append((nxt, content, tuple(p)))
            elif kind == "wait":
                if all(ev[1] is not None and t > ev[1] for (_, t) in pending[v]):
                    moves.append((nxt, content, pending))
            elif kind == "r":
                got = content[ev[1]] if len(ev) == 3 else tuple(content[ev[1]][u] for u in ev[3])
                if any(x != ev[2] for x in got):
                    return f"wave {v} read stage {ev[1]} expecting tile {ev[2]}, pieces hold {got}"
                moves.append((nxt, content, pending))
        if not moves:
            return f"deadlock at {pcs}"
        stack.extend(moves)
    return None


# ---- the kernels' protocols (T K tiles) -------------------------------------------


def one_stage_two_barriers(T):
    ev = []
    for t in range(T):
        ev += [("w", 0, t), ("b",), ("r", 0, t), ("b",)]
    return ev


def two_stage_registers(T, parity_flip=False, drop_barrier=False):
    ev = [("w", 0, 0), ("b",)]
    for t in range(T):
        ev.append(("r", t % 2, t))
        if t + 1 < T:
            ev.append(("w", (t if parity_flip else t + 1) % 2, t + 1))
        if not drop_barrier:
            ev.append(("b",))
    return ev


def two_stage_direct(T, drop_wait=False):
    ev = [("issue", 0, 0), ("wait", None), ("b",)]
    for t in range(T):
        if t + 1 < T:
            ev.append(("issue", (t + 1) % 2, t + 1))
        ev.append(("r", t % 2, t))
        if not drop_wait:
            ev.append(("wait", None))
        ev.append(("b",))
    return ev


def pipelined(T, steps=3, last_after_barrier=False):
    """The MFMA kernel's PIPE loop: step 0 of tile t was read before the
    loop or after the previous barrier; steps 1.. are read before the
    barrier (the last one's registers are multiplied after it)."""
    ev = [("issue", 0, 0), ("wait", None), ("b",), ("r", 0, 0)]
    for t in range(T):
        if t + 1 < T:
            ev.append(("issue", (t + 1) % 2, t + 1))
        body = [("r", t % 2, t)] * (steps - 1)
        if last_after_barrier:
            ev += body[:-1] + [("wait", None), ("b",), body[-1]]
        else:
            ev += body + [("wait", None), ("b",)]
        if t + 1 < T:
            ev.append(("r", (t + 1) % 2, t + 1))
    return ev


def ring(T, S, weak_wait=False):
    """The 16-bit-input kernels' S-stage copy ring, pipelined across tiles:
    the copies of tile t+S-1 go into the stage of tile t-1; before the
    barrier each wave waits until its copies of tile t+1 have landed."""
    ev = []
    for p in range(min(S - 1, T)):
        ev.append(("issue", p % S, p))
    ev += [("wait", None), ("b",), ("r", 0, 0)]
    for t in range(T):
        nt = t + S - 1
        if nt < T:
            ev.append(("issue", nt % S, nt))
        ev.append(("r", t % S, t))
        ev.append(("wait", t if weak_wait else t + 1))
        ev.append(("b",))
        if t + 1 < T:
            ev.append(("r", (t + 1) % S, t + 1))
    return ev


def ksplit_stages(groups):
    """Model stages of the K-split kernel: 2 per group, and the exchange
    regions (p, q) at index p * groups + q, over the working stages where
    they overlap them in LDS."""
    return max(2 * groups, groups * groups)


def ksplit(TF, tail, groups, per_group, wave, drop_final_barrier=False, early_partials=False, copy_late=False):
    """The K-split kernel, as wave `wave` runs it: group q (per_group waves)
    takes K tiles q, q + groups, ... through its own stages 2q and 2q + 1;
    the TF whole tiles by direct copies, a ragged last tile (tail) through
    registers, stored after the multiply of the group's previous tile.
    Every group runs ceil(T / groups) iterations and every barrier.  Then
    each group writes its partial sums of every other group p's slice to
    region (p, q) (over the stages: index p * groups + q), a barrier, and
    each group reads the regions of its own slice (wave w reads wave w of
    each other group).  The next tile's copies are issued between the MFMA
    steps of the current one: modelled at both ends, before the stage read
    or (copy_late) after it."""
    T = TF + (1 if tail else 0)
    q, w = divmod(wave, per_group)
    members = [q * per_group + i for i in range(per_group)]
    ev = []
    if q < TF:
        ev.append(("issue", 2 * q, q))
    elif q < T:
        ev.append(("w", 2 * q, q))
    ev += [("wait", None), ("b",)]
    iters = (T + groups - 1) // groups
    for it in range(iters):
        s, ns = 2 * q + it % 2, 2 * q + 1 - it % 2
        t, tn = it * groups + q, it * groups + q + groups
        if tn < TF and not copy_late:
            ev.append(("issue", ns, tn))
        if t < T:
            ev.append(("r", s, t, members))
        if tn < TF and copy_late:
            ev.append(("issue", ns, tn))
        if TF <= tn < T:
            ev.append(("w", ns, tn))
        ev.append(("wait", None))
        if not (early_partials and it == iters - 1):
            ev.append(("b",))
    for p in range(groups):
        if p != q:
            ev.append(("wx", p * groups + q, f"P{p}{q}"))
    if early_partials:
        ev.append(("b",))
    if not drop_final_barrier:
        ev.append(("b",))
    for g in range(groups):
        if g != q:
            ev.append(("r", q * groups + g, f"P{q}{g}", [g * per_group + w]))
    return ev


def ksplit_programs(TF, tail, groups, per_group, **kw):
    return [ksplit(TF, tail, groups, per_group, v, **kw) for v in range(groups * per_group)]


@pytest.mark.parametrize("TF,tail", [(0, True), (1, False), (2, True), (3, False), (3, True), (4, True),
                                     (5, False)])
@pytest.mark.parametrize("groups,per_group", [(2, 1), (2, 2), (3, 1)])
@pytest.mark.parametrize("copy_late", [False, True])
def test_k_split_protocol_is_race_free(TF, tail, groups, per_group, copy_late):
    programs = ksplit_programs(TF, tail, groups, per_group, copy_late=copy_late)
    assert check(programs, ksplit_stages(groups)) is None


@pytest.mark.parametrize("mutant", ["drop_final_barrier", "early_partials"])
def test_k_split_mutant_is_caught(mutant):
    # two whole tiles and a tail with 2 groups: group 0 reads the tail from its
    # stage 1 in the last iteration, where group 1's partial sums of group 0's
    # slice go
    assert check(ksplit_programs(2, True, 2, 1, **{mutant: True}), ksplit_stages(2)) is not None


CORRECT = [
    ("one stage, two barriers", lambda T: one_stage_two_barriers(T), 1),
    ("two stages through registers", lambda T: two_stage_registers(T), 2),
    ("two stages, direct copies", lambda T: two_stage_direct(T), 2),
    ("pipelined multiply", lambda T: pipelined(T), 2),
    ("three-stage copy ring", lambda T: ring(T, 3), 3),
    ("four-stage copy ring", lambda T: ring(T, 4), 4),
]

MUTANTS = [
    ("two stages without the barrier", lambda T: two_stage_registers(T, drop_barrier=True), 2),
    ("stage parity flipped", lambda T: two_stage_registers(T, parity_flip=True), 2),
    ("one stage with one barrier", lambda T: [e for i, e in enumerate(one_stage_two_barriers(T)) if i % 4 != 3], 1),
    ("direct copies without the wait", lambda T: two_stage_direct(T, drop_wait=True), 2),
    ("pipelined, last step read after the barrier", lambda T: pipelined(T, last_after_barrier=True), 2),
    ("three-stage ring waiting one tile short", lambda T: ring(T, 3, weak_wait=True), 3),
]


@pytest.mark.parametrize("waves", [2, 3])
@pytest.mark.parametrize("name,make,stages", CORRECT, ids=[c[0] for c in CORRECT])
def test_protocol_is_race_free(name, make, stages, waves):
    T = 4
    assert check([make(T)] * waves, stages) is None


@pytest.mark.parametrize("name,make,stages", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, make, stages):
    T = 4
    assert check([make(T)] * 2, stages) is not None


def test_divergent_barrier_deadlocks():
    prog = two_stage_registers(3)
    short = prog[:-1]  # one wave skips the last barrier
    assert "deadlock" in (check([prog, short], 2) or "")
