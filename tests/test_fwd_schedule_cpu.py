"""CPU check of the attention forward's LDS tile schedule (attn_fwd_bf16.hip).

The kernel's waves form two groups (waves 0-3 and 4-7, one of each on every
SIMD) that alternate a softmax phase and a matrix phase per key tile, half a
tile apart, with a workgroup barrier between phases. This model restates, in
program order for each group, what the kernel issues:

  prologue  load K(0) -> K slot 0, K(1) -> K slot 1, V(0) -> V slot 0;
            wait; barrier; read K slot 0 (scores of tile 0)
  group 1   one extra barrier
  tile t    softmax(t): load K(t+2) -> K slot (t+2) % 3
            barrier
            matrix(t):  load V(t+1) -> V slot (t+1) % 3;
                        read K slot (t+1) % 3 (scores of tile t+1),
                        read V slot t % 3 (P V of tile t); wait for own loads
            barrier
  group 0   one extra barrier

and checks that both groups pass the same number of barriers, that every read
finds the intended tile, loaded by both groups and waited for before a barrier
that precedes the read, and that no slot is written while a read of an older
tile in it is still due. A planted mistake (two slots instead of three) must be
caught."""
import pytest

N_SLOTS = 3


def program(group: int, nt: int, slots: int = N_SLOTS):
    ev = []
    if nt > 0:
        ev.append(("load", "k", 0 % slots, 0))
        if nt > 1:
            ev.append(("load", "k", 1 % slots, 1))
        ev.append(("load", "v", 0, 0))
    ev.append(("wait",))
    ev.append(("bar",))
    if nt > 0:
        ev.append(("read", "k", 0, 0))
    if group == 1:
        ev.append(("bar",))
    for t in range(nt):
        if t + 2 < nt:
            ev.append(("load", "k", (t + 2) % slots, t + 2))
        ev.append(("bar",))
        if t + 1 < nt:
            ev.append(("load", "v", (t + 1) % slots, t + 1))
            ev.append(("read", "k", (t + 1) % slots, t + 1))
        ev.append(("read", "v", t % slots, t))
        ev.append(("wait",))
        ev.append(("bar",))
    if group == 0:
        ev.append(("bar",))
    return ev


def check(nt: int, slots: int = N_SLOTS):
    progs = {g: program(g, nt, slots) for g in (0, 1)}
    bars = [sum(1 for e in progs[g] if e[0] == "bar") for g in (0, 1)]
    assert bars[0] == bars[1], f"barrier counts differ: {bars}"
    # period of an event = barriers passed before it
    timed = {}
    for g, ev in progs.items():
        p, out = 0, []
        for e in ev:
            if e[0] == "bar":
                p += 1
            else:
                out.append((p, e))
        timed[g] = out
    # each load: (array, slot, tile, group, period issued, period waited)
    loads = []
    for g, ev in timed.items():
        pending = []
        for p, e in ev:
            if e[0] == "load":
                pending.append((e[1], e[2], e[3], p))
            elif e[0] == "wait":
                loads += [(a, s, t, g, pi, p) for a, s, t, pi in pending]
                pending = []
        assert not pending, "a load is never waited for"
    for g, ev in timed.items():
        for p, e in ev:
            if e[0] != "read":
                continue
            _, arr, slot, tile = e
            into = [ld for ld in loads if ld[0] == arr and ld[1] == slot]
            for gg in (0, 1):
                done = [ld for ld in into if ld[3] == gg and ld[5] < p]
                assert done, f"group {g} reads {arr}{tile} in period {p}: no completed load by group {gg}"
                last = max(done, key=lambda ld: ld[5])
                assert last[2] == tile, f"group {g} reads {arr}{tile} in period {p}, slot holds {arr}{last[2]}"
            for ld in into:
                assert not (ld[2] > tile and ld[4] <= p), \
                    f"{arr}{ld[2]} overwrites slot {slot} before group {g} reads {arr}{tile} in period {p}"
    return bars[0]


@pytest.mark.parametrize("nt", range(0, 48))
def test_forward_tile_schedule_is_hazard_free(nt):
    check(nt)


def test_planted_two_slot_schedule_is_caught():
    with pytest.raises(AssertionError):
        for nt in range(0, 8):
            check(nt, slots=2)
