"""The first product's LDS ring schedules, checked on the CPU.

The fused kernel's loader and multiplier waves share an NS-deep LDS ring and
meet only at workgroup barriers.  This test replays both roles' schedules,
barrier interval by barrier interval, as the kernel issues them
(``gemm1_loads`` with direct loads, ``gemm1_loads_reg`` with register-staged
loads, ``gemm1_mma`` on the multiplier side), and checks the protocol:

* every stage a multiplier reads has been written by the loaders in an
  earlier interval (direct loads: issued in an earlier interval and waited for
  before the barrier that ends the interval in which they must land);
* no buffer is written in an interval in which a multiplier reads it;
* a register set of the register-staged loader is written to LDS only after
  the loads of the stage it holds, and reloaded only after that write.

Intervals are numbered by the barrier that opens them: interval -1 follows
barrier -1 (the first one of the pass), interval kt follows barrier kt.
"""
import pytest


def multiplier_reads(nk2):
    """(interval, stage) pairs: the multipliers read stage 0 after barrier -1
    and stage kt + 1 after barrier kt (one stage ahead of the one they
    multiply); the read of stage nk2 is a stale read that is never used."""
    return [(-1, 0)] + [(kt, kt + 1) for kt in range(nk2)]


def direct_writes(ns, nk2):
    """(first interval, last interval, stage) over which the direct loads of a
    stage are in flight in gemm1_loads: stages 0 .. ns-2 are issued before
    barrier -1 (interval -2), stage s >= ns - 1 right after barrier s - ns + 1
    into buffer s mod ns; the wait before barrier s - 1 (at most ns - 3
    younger stages in flight, or none near the end) has stage s landed by the
    end of interval s - 2."""
    out = []
    for i in range(min(ns - 1, nk2)):
        out.append((-2, i - 2, i))
    for kt in range(nk2):
        s = kt + ns - 1
        if s < nk2:
            out.append((kt, s - 2, s))
    return out


def reg_writes(nk2):
    """gemm1_loads_reg: (interval of the LDS write, stage), and the register
    events (load into a set / write out of it, stage, interval) in program
    order.  Two sets, even and odd stages; stage s is written between
    barriers s - 2 and s - 1 (published by barrier s - 1), and its set is
    reloaded with stage s + 2 after the next barrier, so the loads are issued
    while the multipliers work."""
    writes, events = [], []
    events += [("load", "A", 0, -2), ("load", "B", 1, -2)]
    writes.append((-2, 0))
    events.append(("store", "A", 0, -2))
    events.append(("load", "A", 2, -2))
    for kt in range(0, nk2, 2):
        writes.append((kt - 1, kt + 1))
        events.append(("store", "B", kt + 1, kt - 1))
        events.append(("load", "B", kt + 3, kt))
        writes.append((kt, kt + 2))
        events.append(("store", "A", kt + 2, kt))
        events.append(("load", "A", kt + 4, kt + 1))
    return writes, events


def check_no_overlap(ns, nk2, writes):
    """writes: (first interval the buffer may be touched, last interval, stage)."""
    reads = multiplier_reads(nk2)
    read_at = {}
    for iv, st in reads:
        read_at.setdefault(iv, set()).add(st % ns)
    for first, last, st in writes:
        for iv in range(first, last + 1):
            # a write in flight during interval iv must not hit a buffer read then
            assert st % ns not in read_at.get(iv, set()), (ns, nk2, st, iv)
    # every real stage read was written (landed) before the interval that reads it
    landed = {st: last for _, last, st in writes}
    for iv, st in reads:
        if st < nk2:
            assert st in landed and landed[st] < iv, (ns, nk2, st, iv)


@pytest.mark.parametrize("ns", [3, 4, 5, 6])
@pytest.mark.parametrize("nk2", [2, 4, 6, 8, 14, 128, 256])
def test_direct_load_ring(ns, nk2):
    writes = direct_writes(ns, nk2)
    # every stage read is loaded exactly once (stages past the end are never issued)
    assert sorted(st for _, _, st in writes) == list(range(nk2))
    check_no_overlap(ns, nk2, writes)


@pytest.mark.parametrize("nk2", [2, 4, 6, 8, 14, 128, 256])
@pytest.mark.parametrize("ns", [3, 4])
def test_register_staged_ring(ns, nk2):
    writes, events = reg_writes(nk2)
    # every stage 0 .. nk2 is written once, in the interval before the barrier
    # that publishes it (stage nk2: the never-used stale read)
    assert sorted(st for _, st in writes) == list(range(nk2 + 1))
    check_no_overlap(ns, nk2, [(iv, iv, st) for iv, st in writes])
    # registers: a set holds one stage from its load to its store, and is
    # reloaded only after that store
    held = {}
    for kind, reg, st, _ in events:
        if kind == "load":
            assert reg not in held, (nk2, reg, st)
            held[reg] = st
        else:
            assert held.get(reg) == st, (nk2, reg, st)
            del held[reg]
    # the loads of a stage are issued right after a barrier and written out in
    # the next interval (stage s >= 3: loaded in interval s - 3, written in
    # interval s - 2), so they have about one interval to land
    load_iv = {st: iv for kind, _, st, iv in events if kind == "load"}
    for iv, st in writes:
        if st >= 3:
            assert iv - load_iv[st] == 1, (st, iv, load_iv[st])
