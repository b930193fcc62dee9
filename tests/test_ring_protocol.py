"""CPU model of the LDS ring protocol of the attention kernel (csrc/attention.hip)
and the token selector's key-block ring (csrc/token_select.hip), checked over
random interleavings.

The kernel streams the union of its query blocks' kept KV units through a ring
of NS slots (unit u lives in slot u mod NS). L loader wavefronts own the units
u = l, l + L, l + 2L, ...; a loader keeps up to I units in flight, and before
issuing its k-th unit it waits (s_waitcnt vmcnt) until the copies of its unit
k - I have landed (vector-memory loads complete in issue order), publishes that
unit (ready[slot] = unit), then waits until its slot is free: every compute
wave's progress word is past the slot's previous unit u - NS, and that unit was
published. Each compute wave walks only the units its query block needs: it
stores its progress (the unit it is about to read), waits for ready[slot] ==
unit, reads the slot, and moves on. The model executes these steps with every
actor (each loader, each compute wave, each loader's oldest copy landing)
taking turns in random order, copies and reads taking random time, and checks:

* a slot is never written (a copy in flight, from issue to landing) while a
  compute wave reads another unit from it, nor by two units' copies at once;
* a compute wave reads a unit only after all of its copies landed;
* every schedule finishes (no deadlock), each wave having read exactly its units.

Planted mistakes are shown to fail: the publish rule of the slot check
removed (a slot reused once the waves are past it, published or not: the hole
a unit no wave needs opens), a unit published one vmcnt step early, and a
wave announcing progress before its read has finished.

Hardware facts the model takes as given (not modelled): a wavefront's LDS
operations are performed in issue order, so the reads of a unit are done
before that wave's next progress store; and s_waitcnt vmcnt returns only
once a direct-to-LDS copy's data is in LDS, so the publish store that follows
it is seen after the data.
"""
import numpy as np
import pytest

DONE = 1 << 30


class Violation(AssertionError):
    pass


def run_schedule(n_units, needs, n_loaders, inflight, n_slots, rng, publish_rule=True, early_publish=False,
                 early_progress=False, lag=False, lag_flush=True, needers_only=False, max_steps=200000):
    """One random execution. needs[w]: ascending units compute wave w reads.
    publish_rule, early_publish and early_progress plant protocol mistakes: no
    publish check before slot reuse; a vmcnt count one too high (a unit
    published before its copies land); a wave announcing its next unit before
    its read has finished. lag: each wave reads a unit in two parts, the
    second (the V tile of the lagged PV product) during its next unit's turn;
    while it waits for that next unit its progress word still names the
    pending unit, unless the two lie more than n_slots - 1 apart, when it first
    finishes the pending read (lag_flush; False plants the mistake of always
    holding it). needers_only: the slot check asks only the waves that read
    the slot's previous unit to be past it (the others never read that unit)."""
    W = len(needs)
    need_sets = [set(n) for n in needs]
    ready = [-1] * n_slots
    prog = [0] * W
    # slot state: the unit whose copies are in flight into it, readers of it
    writing = [None] * n_slots
    landed = [-1] * n_slots            # unit whose copies have all landed there last
    readers = [dict() for _ in range(n_slots)]   # wave -> unit being read
    # loader state
    L_units = [list(range(l, n_units, n_loaders)) for l in range(n_loaders)]
    L_k = [0] * n_loaders              # next iteration
    L_phase = ["start"] * n_loaders    # start -> slotwait -> (issue) ... -> drain -> done
    L_fifo = [[] for _ in range(n_loaders)]      # units with copies in flight, issue order
    # compute state
    C_i = [0] * W                      # index into needs[w]
    C_phase = ["announce"] * W
    read_log = [[] for _ in range(W)]
    pend = [None] * W                  # lag: unit whose second part is still to be read

    def publish(l, u):
        ready[u % n_slots] = u

    def loader_step(l):
        units = L_units[l]
        k = L_k[l]
        ph = L_phase[l]
        if ph == "done":
            return False
        if ph == "start":
            if k >= len(units):
                L_phase[l] = "drain"
                return True
            if k >= inflight:
                # wait until the copies of iteration k - inflight have landed
                old = units[k - inflight]
                if old in L_fifo[l] and not early_publish:
                    return False          # still in flight: the vmcnt wait blocks
                publish(l, old)
            L_phase[l] = "slotwait"
            return True
        if ph == "slotwait":
            u = units[k]
            s = u % n_slots
            if needers_only:
                mn = min([prog[w] for w in range(W) if (u - n_slots) in need_sets[w]], default=DONE)
            else:
                mn = min(prog)
            free = mn >= u - n_slots + 1
            if publish_rule:
                free = free and (u < n_slots or ready[s] == u - n_slots)
            if not free:
                return False
            # issue: the copies are in flight into slot s from now until they land
            if writing[s] is not None:
                raise Violation(f"slot {s}: unit {u} issued while unit {writing[s]}'s copies are in flight")
            for w, ru in readers[s].items():
                raise Violation(f"slot {s}: unit {u} issued while wave {w} reads unit {ru}")
            writing[s] = u
            L_fifo[l].append(u)
            L_k[l] = k + 1
            L_phase[l] = "start"
            return True
        if ph == "drain":
            if L_fifo[l]:
                return False              # wait for every copy (vmcnt(0))
            # publish the last `inflight` units (those not yet published)
            for u in units[max(0, len(units) - inflight):]:
                publish(l, u)
            L_phase[l] = "done"
            return True
        raise AssertionError(ph)

    def land_step(l):
        if not L_fifo[l]:
            return False
        u = L_fifo[l].pop(0)              # in order
        s = u % n_slots
        if writing[s] != u:
            raise Violation(f"slot {s}: copies of {u} land but {writing[s]} is recorded in flight")
        for w, ru in readers[s].items():
            raise Violation(f"slot {s}: unit {u} lands while wave {w} reads unit {ru}")
        writing[s] = None
        landed[s] = u
        return True

    def check_landed(w, u):
        s = u % n_slots
        if writing[s] is not None or landed[s] != u:
            raise Violation(f"wave {w} reads unit {u} from slot {s}: landed {landed[s]}, in flight {writing[s]}")

    def compute_step(w):
        ph = C_phase[w]
        i = C_i[w]
        if ph == "done":
            return False
        if ph == "announce":
            if i >= len(needs[w]):
                if pend[w] is not None:     # the last pending read
                    C_phase[w] = "flush_end"
                    return True
                prog[w] = DONE
                C_phase[w] = "done"
                return True
            u = needs[w][i]
            if pend[w] is not None and lag_flush and u - pend[w] > n_slots - 1:
                C_phase[w] = "flush"
                return True
            prog[w] = pend[w] if pend[w] is not None else u
            C_phase[w] = "wait"
            return True
        if ph in ("flush", "flush_end"):
            # the pending unit's second read, then release it
            pu = pend[w]
            check_landed(w, pu)
            pend[w] = None
            C_phase[w] = "announce" if ph == "flush" else "announce"
            return True
        u = needs[w][i]
        s = u % n_slots
        if ph == "wait":
            if ready[s] != u:
                return False
            check_landed(w, u)
            readers[s][w] = u
            if pend[w] is not None:
                readers[pend[w] % n_slots][w] = pend[w]
            C_phase[w] = "read"
            if early_progress:
                prog[w] = needs[w][i + 1] if i + 1 < len(needs[w]) else DONE
            return True
        if ph == "read":
            # this unit's first part and the pending unit's second part are read;
            # the pending unit's reads have finished before the progress store
            del readers[s][w]
            if pend[w] is not None:
                pu = pend[w]
                check_landed(w, pu)
                del readers[pu % n_slots][w]
            read_log[w].append(u)
            if lag:
                pend[w] = u
                prog[w] = u
            C_i[w] = i + 1
            C_phase[w] = "announce"
            return True
        raise AssertionError(ph)

    actors = [("L", l) for l in range(n_loaders)] + [("D", l) for l in range(n_loaders)] + [("C", w) for w in range(W)]
    steps = 0
    while True:
        if all(p == "done" for p in L_phase) and all(p == "done" for p in C_phase):
            break
        order = rng.permutation(len(actors))
        moved = False
        for a in order:
            kind, x = actors[a]
            # random delays: an actor may skip its turn (copies and reads take time)
            if rng.random() < 0.5:
                continue
            ok = loader_step(x) if kind == "L" else land_step(x) if kind == "D" else compute_step(x)
            if ok:
                moved = True
                break
        if not moved:
            # nobody moved this round: check that someone could (deadlock otherwise)
            any_ok = False
            for a in order:
                kind, x = actors[a]
                ok = loader_step(x) if kind == "L" else land_step(x) if kind == "D" else compute_step(x)
                if ok:
                    any_ok = True
                    break
            if not any_ok:
                raise Violation(f"deadlock: loaders {L_phase}, waves {C_phase}, prog {prog}, ready {ready}")
        steps += 1
        if steps > max_steps:
            raise Violation("no progress bound reached")
    for w in range(W):
        assert read_log[w] == list(needs[w])


def random_needs(rng, n_units, waves, density):
    needs = []
    for _ in range(waves):
        m = rng.random(n_units) < density
        needs.append(np.nonzero(m)[0].tolist())
    return needs


@pytest.mark.parametrize("loaders,inflight,slots",
                         [(4, 1, 9), (4, 1, 8), (4, 1, 6), (4, 1, 3), (4, 1, 2), (3, 2, 9), (3, 2, 8), (4, 2, 9)])
def test_ring_protocol_random_interleavings(loaders, inflight, slots):
    """The protocol of the attention kernel (4 loaders, 1 unit in flight each,
    9 or 6 slots; the earlier form: 3 loaders, 2 in flight) and of the token
    selector (the same loaders over its key-block ring of 2 to 16 buffers),
    8 compute waves, unions of 1 to 40 units, densities from sparse (units no
    wave needs occur) to full."""
    rng = np.random.default_rng(loaders * 100 + inflight * 10 + slots)
    for trial in range(150):
        n = int(rng.integers(1, 41))
        density = float(rng.choice([0.05, 0.2, 0.5, 1.0]))
        needs = random_needs(rng, n, 8, density)
        run_schedule(n, needs, loaders, inflight, slots, rng)


@pytest.mark.parametrize("loaders,inflight,slots", [(4, 1, 9), (4, 1, 6), (4, 1, 3), (4, 1, 2), (3, 2, 9)])
def test_ring_protocol_needers_only(loaders, inflight, slots):
    """A variant of the slot check that was timed and not adopted (bitwise the
    same outputs, static launches 1% slower): a slot is refilled once the
    waves that read its previous unit are past it and that unit was
    published, so a wave that never reads the unit does not hold the slot. No
    slot is written while read, no unit is read before it landed, no schedule
    deadlocks."""
    rng = np.random.default_rng(2000 + loaders * 100 + inflight * 10 + slots)
    for trial in range(150):
        n = int(rng.integers(1, 41))
        density = float(rng.choice([0.05, 0.2, 0.5, 1.0]))
        needs = random_needs(rng, n, 8, density)
        run_schedule(n, needs, loaders, inflight, slots, rng, needers_only=True)


def test_ring_protocol_needers_only_without_publish_rule_fails():
    """With that check the publish rule is still needed: a unit
    no wave reads has no needers, and its slot would be refilled while its own
    copies may still be landing. The model finds it."""
    rng = np.random.default_rng(23)
    found = False
    for trial in range(400):
        n = int(rng.integers(10, 41))
        needs = random_needs(rng, n, 8, 0.05)
        try:
            run_schedule(n, needs, 4, 1, 9, rng, publish_rule=False, needers_only=True)
        except Violation:
            found = True
            break
    assert found


@pytest.mark.parametrize("mistake", ["early_publish", "early_progress"])
def test_ring_protocol_planted_mistakes_fail(mistake):
    """Publishing a unit one vmcnt step early, or announcing progress before a
    read completes, lets a read overlap a copy: the model finds both."""
    rng = np.random.default_rng(7)
    found = False
    for trial in range(400):
        n = int(rng.integers(10, 41))
        needs = random_needs(rng, n, 8, float(rng.choice([0.2, 1.0])))
        try:
            run_schedule(n, needs, 4, 1, 9, rng, **{mistake: True})
        except Violation:
            found = True
            break
    assert found


def test_ring_protocol_without_publish_rule_fails():
    """Reusing a slot as soon as every wave is past its unit, without waiting
    for that unit to be published, lets a unit no wave needs still be landing
    when its slot is refilled (two units' copies in flight into one slot):
    the model finds it."""
    rng = np.random.default_rng(5)
    found = False
    for trial in range(400):
        n = int(rng.integers(10, 41))
        needs = random_needs(rng, n, 8, 0.05)
        try:
            run_schedule(n, needs, 4, 1, 9, rng, publish_rule=False)
        except Violation:
            found = True
            break
    assert found


@pytest.mark.parametrize("loaders,inflight,slots", [(4, 1, 9), (4, 1, 6), (4, 1, 8)])
def test_ring_protocol_lagged_pv(loaders, inflight, slots):
    """A variant of the protocol that was timed and not adopted (no gain for
    the dense kernel, slower sparse launches): the PV product of a unit lags
    one unit behind, so a wave keeps its previous unit claimed (progress word
    = that unit) while it waits for the next one, and finishes the previous
    unit first when the two are more than slots - 1 apart. No slot is
    refilled under a pending read, and no schedule deadlocks."""
    rng = np.random.default_rng(1000 + slots)
    for trial in range(150):
        n = int(rng.integers(1, 41))
        density = float(rng.choice([0.05, 0.2, 0.5, 1.0]))
        needs = random_needs(rng, n, 8, density)
        run_schedule(n, needs, loaders, inflight, slots, rng, lag=True)


def test_ring_protocol_lag_without_flush_deadlocks():
    """Holding the pending unit while waiting for a unit more than slots - 1
    further on deadlocks: that unit's slot still holds a unit between the two,
    which the loaders may not replace while the wave's progress word names the
    pending unit. The model finds it."""
    rng = np.random.default_rng(11)
    found = False
    for trial in range(400):
        n = int(rng.integers(20, 41))
        needs = random_needs(rng, n, 8, 0.1)
        try:
            run_schedule(n, needs, 4, 1, 9, rng, lag=True, lag_flush=False)
        except Violation:
            found = True
            break
    assert found
