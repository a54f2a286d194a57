"""CPU check of the staged decode form's copy pipeline (the explicit wait counts and the slot
reuse in fp8q_gemm.hip), by replaying one wave's sequence of vector memory instructions.

Per wave: the prologue copies pieces 0 .. kDepth (two copy instructions each); then every
piece t of the walk (items in rounds of four, the first item on its own) issues the copies of
piece t + kDepth (before its wait with one piece ahead, after its barrier otherwise; the
first item's first piece issues none), waits with vmcnt(n), passes the barrier, and in a
round's first piece issues the reduce's two stores.  Vector memory instructions complete in
order, so vmcnt(n) leaves only the newest n outstanding: each piece's copies must be older
than that.  A slot may be copied into only after the barrier that follows every read of the
piece it held, and a read must find its own piece there.  The wait rule and depth are read
from the kernel source, so a change there is checked here."""
import os
import re

import pytest

SRC = os.path.join(os.path.dirname(__file__), "..", "fp8_e4m3_quantization_amd", "csrc",
                   "fp8q_gemm.hip")


def _rule():
    s = open(SRC).read()
    depth = int(re.search(r"#define FP8Q_STAGE_DEPTH (\d+)", s).group(1))
    assert "constexpr int kAhead = kDepth == 1 ? 2 : 2 * (kDepth - 1);" in s
    assert "if constexpr (t >= 1 && t <= kDepth)\n      wait_copies_then_barrier<kAhead + 2>();" in s
    assert "if constexpr (!(decltype(first_item)::value && t == 0))" in s
    return depth


def _wait(depth, t):
    ahead = 2 if depth == 1 else 2 * (depth - 1)
    return ahead + 2 if 1 <= t <= depth else ahead


def _replay(gpw, depth, nit):
    ops = []            # ("copy", piece) or ("store",)
    slot_of = {}        # slot -> (piece, index of the barrier after which it was copied)
    barrier = 0         # barriers passed
    last_read = {}      # slot -> barrier index of the piece iteration that read it
    problems = []

    def copy(q):
        s = q % 4
        if s in last_read and last_read[s] >= barrier:
            problems.append(f"piece {q} copied into slot {s} before the barrier after its read")
        ops.extend([("copy", q), ("copy", q)])
        slot_of[s] = q

    for q in range(depth + 1):  # prologue
        copy(q)
    order = [(0, 0, True)] + [(i, j, False) for i in range(0, nit, 4) for j in range(4)
                              if i + j < nit and (j > 0 or i > 0)]
    for i, j, first in order:
        for p in range(gpw):
            t = j * gpw + p
            q = (i + j) * gpw + p
            skip = first and t == 0
            if depth == 1 and not skip:
                copy(q + depth)
            n = _wait(depth, t)
            last = max(k for k, op in enumerate(ops) if op == ("copy", q))
            newer = len(ops) - 1 - last
            if newer < n:
                problems.append(f"piece {q}: vmcnt({n}) leaves its copy outstanding ({newer} newer)")
            barrier += 1
            if depth > 1 and not skip:
                copy(q + depth)
            if t == 0:
                ops.extend([("store",), ("store",)])
            if slot_of.get(q % 4) != q:
                problems.append(f"piece {q} read from slot {q % 4} holding {slot_of.get(q % 4)}")
            last_read[q % 4] = barrier
    return problems


@pytest.mark.parametrize("gpw", range(1, 9))
@pytest.mark.parametrize("nit", [1, 2, 3, 4, 5, 8, 9, 13])
def test_committed_depth_waits_and_slots(gpw, nit):
    assert _replay(gpw, _rule(), nit) == []


@pytest.mark.parametrize("depth", [1, 2, 3])
@pytest.mark.parametrize("gpw", range(1, 9))
def test_every_depth_waits_and_slots(depth, gpw):
    assert _replay(gpw, depth, 9) == []


def test_a_planted_under_wait_is_caught():
    """The replay is not vacuous: one fewer newer op than the rule assumes is reported."""
    global _wait
    saved = _wait
    try:
        _wait = lambda depth, t: (saved(depth, t) + 2) if t == 5 else saved(depth, t)
        assert any("outstanding" in p for p in _replay(5, 3, 4))
    finally:
        _wait = saved
