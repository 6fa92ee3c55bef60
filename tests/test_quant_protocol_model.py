"""CPU model of the single-launch quantiser's tensor-maximum exchange.

The resident quantiser (k_quant_resident in csrc/quantize.hip) runs at most one
workgroup per CU.  Each workgroup reduces its share of the tensor, publishes
the maximum in its own 64-bit slot tagged with the call's epoch, and polls all
slots until every one carries that epoch; a workgroup whose bounded wait
expires finds the maximum another way.  How each workgroup learns the call's
epoch is what the variants below differ in.

This module simulates that exchange step by step: every workgroup is a
generator that yields after each access to the shared workspace, and a
scheduler decides which workgroup moves next, including workgroups that only
start after others have finished (a grid that is not resident all at once).
Four variants are modelled:

  "advance_by_wg0"   the earlier kernel: workgroup 0 advances the control word
                     as soon as its own poll ends, whether it saw every slot or
                     its wait expired; an expired workgroup reads the whole
                     tensor.
  "last_arrival"     the kernel before the own-slot epochs: every workgroup, after its poll, adds
                     one to an arrival counter; the workgroup that brings it to
                     the grid size resets it and advances the control word, so
                     no workgroup of a call can read an advanced word.  An
                     expired workgroup reads directly only the shares of the
                     workgroups whose slots it has not seen.

  "arrive_before_read"  an arrival at the start, before the read of the
                     control word, and the advance after the poll (a negative
                     control).

  "own_slot"         the current kernel: no control word.  A workgroup's
                     epoch is one more than the largest tag in its own slot of
                     each of the call's tensors, and it stamps every slot
                     k + i*nwg (i >= 1) of those tensors with the new epoch as
                     it publishes slot k, so after a call every slot of every
                     tensor it touched carries the same tag whatever the grid
                     size.  Only workgroup k ever writes slot k during a call,
                     so no workgroup can see its own slot changed before it
                     reads it; no shared word is advanced, so no arrival count
                     is needed.  An expired workgroup reads directly only the
                     shares of the workgroups whose slots it has not seen.

The tests show that the first variant takes a stale maximum from the previous
call under a reachable schedule, and that the others give every workgroup the
true maximum under that schedule and under many random ones, for sequences of
calls with different grid sizes on one zero-initialised workspace ("own_slot"
also when calls take one or two tensor regions of a pool in any role).
"""

import random

import pytest

MASK48 = (1 << 48) - 1
LONG = 200            # a wait that outlasts every schedule below


class Workspace:
    """Slots and control words; every word starts at zero."""

    def __init__(self):
        self.slot = {}          # workgroup index -> (epoch, max)
        self.eword = 0          # epoch of the last completed call
        self.arrive = 0         # arrival counter of the call in flight

    def read_slot(self, p):
        return self.slot.get(p, (0, 0))


NSLOTS = 8                      # slots per tensor region (the kernel has 1024)


def own_slot_program(k, shares, regions, wait_polls, out, stamp=True):
    """One workgroup of an "own_slot" call over len(regions) tensors;
    ``shares[j][p]`` is workgroup p's share maximum of tensor j.  With
    ``stamp`` false the slots above the grid are left alone (a negative
    control)."""
    nwg = len(shares[0])
    tags = []
    for r in regions:                              # its own slot of every tensor
        tags.append(r.read_slot(k)[0])
        yield
    epoch = (max(tags) + 1) & MASK48 or 1
    for j, r in enumerate(regions):                # publish, and stamp the slots above
        r.slot[k] = (epoch, shares[j][k])
        yield
        for s in range(k + nwg, NSLOTS, nwg) if stamp else ():
            r.slot[s] = (epoch, 0)
            yield
    seen = [dict() for _ in regions]
    polls = 0
    while True:
        for j, r in enumerate(regions):
            for p in range(nwg):
                if p not in seen[j]:
                    tag, v = r.read_slot(p)
                    if tag == epoch:
                        seen[j][p] = v
        yield
        if all(len(sj) == nwg for sj in seen):
            break
        polls += 1
        if polls > wait_polls:
            break
    res = []
    for j in range(len(regions)):
        direct = [shares[j][p] for p in range(nwg) if p not in seen[j]]
        res.append(max(list(seen[j].values()) + direct))
    out[k] = res


def run_own_slot_call(shares, regions, order, wait_polls, stamp=True):
    """run_call for "own_slot": every workgroup's result is the list of its
    tensor maxima."""
    nwg = len(shares[0])
    out, gens, finished = {}, {}, set()

    def step(k):
        if k in finished:
            return
        if k not in gens:
            gens[k] = own_slot_program(k, shares, regions, wait_polls[k], out, stamp)
        try:
            next(gens[k])
        except StopIteration:
            finished.add(k)

    for k in order:
        step(k)
    while len(finished) < nwg:
        for k in range(nwg):
            step(k)
    return [out[k] for k in range(nwg)]


def wg_program(variant, k, shares, ws, wait_polls, out):
    """One workgroup of one call; yields after each workspace access.

    ``shares[p]`` is the maximum of workgroup p's share of the tensor;
    ``wait_polls`` bounds the number of poll rounds before the wait expires.
    The workgroup's result (its tensor maximum A) is stored in out[k].
    """
    nwg = len(shares)
    last = False
    if variant == "arrive_before_read":            # the order the current kernel avoids
        old = ws.arrive
        ws.arrive = old + 1
        last = old == nwg - 1
        yield
    epoch = (ws.eword + 1) & MASK48 or 1           # read the control word
    yield
    ws.slot[k] = (epoch, shares[k])                # publish this share's maximum
    yield
    seen = {}
    polls = 0
    while True:
        for p in range(nwg):                       # one round: thread p loads slot p
            if p not in seen:
                tag, v = ws.read_slot(p)
                if tag == epoch:
                    seen[p] = v
        yield
        if len(seen) == nwg:
            break
        polls += 1
        if polls > wait_polls:
            break                                  # the bounded wait expired
    if variant == "advance_by_wg0":
        if k == 0:
            ws.eword = epoch
            yield
        out[k] = max(seen.values()) if len(seen) == nwg else max(shares)
    elif variant == "arrive_before_read":
        if last:                                   # advance once the poll has ended
            ws.arrive = 0
            ws.eword = epoch
            yield
        direct = [shares[p] for p in range(nwg) if p not in seen]
        out[k] = max(list(seen.values()) + direct)
    elif variant == "last_arrival":
        old = ws.arrive                            # one atomic add
        ws.arrive = old + 1
        if old == nwg - 1:                         # the last workgroup to arrive
            ws.arrive = 0
            ws.eword = epoch
        yield
        direct = [shares[p] for p in range(nwg) if p not in seen]   # read missing shares
        out[k] = max(list(seen.values()) + direct)
    else:
        raise ValueError(variant)


def run_call(variant, shares, ws, order, wait_polls):
    """Runs one call.  ``order`` is a list of workgroup indices: each entry
    moves that workgroup by one step (starting it if needed); once the list is
    used up the unfinished workgroups take steps in turn until all are done.
    Every workgroup of the call finishes before the call returns (stream
    order)."""
    out = {}
    gens = {}
    finished = set()

    def step(k):
        if k in finished:
            return
        if k not in gens:
            gens[k] = wg_program(variant, k, shares, ws, wait_polls[k], out)
        try:
            next(gens[k])
        except StopIteration:
            finished.add(k)

    for k in order:
        step(k)
    while len(finished) < len(shares):
        for k in range(len(shares)):
            step(k)
    return [out[k] for k in range(len(shares))]


def solo(k, n=64):
    return [k] * n                                 # enough steps to finish alone


# ----------------------------------------------------------------------------
# the race of the earlier protocol


def test_wg0_advance_takes_a_stale_maximum():
    # call 1: workgroup 1 is not resident until workgroup 0 has finished; 0's
    # wait expires and it advances the control word; 1 then reads the advanced
    # word and tags its slot with the next call's epoch
    ws = Workspace()
    big = [10, 0x7F00]
    a1 = run_call("advance_by_wg0", big, ws, solo(0) + solo(1), [0, 0])
    assert a1 == [max(big)] * 2                    # the call itself is right (fallback)
    # call 2 on smaller data: workgroup 0 polls before workgroup 1 republishes
    # and accepts the stale slot as current
    small = [0x3F80, 0x3F00]
    a2 = run_call("advance_by_wg0", small, ws, solo(0) + solo(1), [1000, 1000])
    assert a2[0] == 0x7F00 != max(small)


def test_last_arrival_same_schedule_is_exact():
    ws = Workspace()
    big = [10, 0x7F00]
    assert run_call("last_arrival", big, ws, solo(0) + solo(1), [0, 0]) == [max(big)] * 2
    small = [0x3F80, 0x3F00]
    assert run_call("last_arrival", small, ws, solo(0) + solo(1), [1000, 1000]) == [max(small)] * 2
    assert ws.arrive == 0 and ws.eword == 2


def test_last_arrival_expired_wait_then_normal_wait():
    # a call whose waits all expire (the testing hook's wait of 0), then a call
    # with the normal wait on different data, on the same workspace
    ws = Workspace()
    for rep in range(20):
        d1 = [100 + 7 * p + rep for p in range(5)]
        order = [p for p in (4, 2, 0, 3, 1) for _ in range(2)]
        assert run_call("last_arrival", d1, ws, order, [0] * 5) == [max(d1)] * 5
        d2 = [p + rep for p in range(5)]
        assert run_call("last_arrival", d2, ws, [0, 1, 2, 0, 1, 2], [LONG] * 5) == [max(d2)] * 5


def random_schedule(rng, nwg):
    """A random interleaving in which some workgroups start only after others
    have taken many steps (not all resident at once)."""
    late = set(rng.sample(range(nwg), rng.randint(0, nwg - 1)))
    early = [p for p in range(nwg) if p not in late]
    order = [rng.choice(early) for _ in range(rng.randint(0, 12 * nwg))]
    for p in sorted(late, key=lambda _: rng.random()):
        early.append(p)
        order += [rng.choice(early) for _ in range(rng.randint(1, 8 * nwg))]
    return order


@pytest.mark.parametrize("seed", range(4))
def test_last_arrival_random_schedules(seed):
    rng = random.Random(seed)
    for trial in range(400):
        ws = Workspace()
        for call in range(6):
            nwg = rng.randint(1, 6)
            shares = [rng.randint(0, 0x7F7F) for _ in range(nwg)]
            waits = [rng.choice([0, 1, 2, 5, LONG]) for _ in range(nwg)]
            got = run_call("last_arrival", shares, ws, random_schedule(rng, nwg), waits)
            assert got == [max(shares)] * nwg, (seed, trial, call, shares, got)
            assert ws.arrive == 0


def test_random_schedules_find_the_earlier_race():
    # the same random search breaks the earlier protocol, so the search is
    # able to reach the failure it rules out for the current one
    rng = random.Random(123)
    failures = 0
    for trial in range(400):
        ws = Workspace()
        for call in range(6):
            nwg = rng.randint(1, 6)
            shares = [rng.randint(0, 0x7F7F) for _ in range(nwg)]
            waits = [rng.choice([0, 1, 2, 5, LONG]) for _ in range(nwg)]
            got = run_call("advance_by_wg0", shares, ws, random_schedule(rng, nwg), waits)
            failures += got != [max(shares)] * nwg
    assert failures > 0


def test_random_schedules_find_an_arrival_before_the_read():
    # arriving before reading the control word lets the last arriver advance
    # it while a late workgroup of the same call has still to read it; that
    # workgroup then tags its slot with the next call's epoch.  The search
    # reaches that failure, so the read-then-arrive order is what it checks.
    rng = random.Random(321)
    failures = 0
    for trial in range(400):
        ws = Workspace()
        for call in range(6):
            nwg = rng.randint(1, 6)
            shares = [rng.randint(0, 0x7F7F) for _ in range(nwg)]
            waits = [rng.choice([0, 1, 2, 5, LONG]) for _ in range(nwg)]
            got = run_call("arrive_before_read", shares, ws, random_schedule(rng, nwg), waits)
            failures += got != [max(shares)] * nwg
    assert failures > 0


def test_prefilled_workspace_is_outside_the_contract():
    # A workspace whose slots already carry the next epoch cannot be told from
    # a current one by any tag check, so the interface requires workspaces to
    # be zero before their first use (after that the library keeps them valid).
    ws = Workspace()
    ws.eword = 41
    ws.slot = {0: (42, 0x7F7F), 1: (42, 0x7F7F)}
    got = run_call("last_arrival", [0x3F80, 0x3F00], ws, solo(0) + solo(1), [LONG, LONG])
    assert got[0] == 0x7F7F
    ws = Workspace()                                # zeroed: exact
    assert run_call("last_arrival", [0x3F80, 0x3F00], ws, solo(0) + solo(1), [LONG] * 2) == [0x3F80] * 2


# ----------------------------------------------------------------------------
# the current protocol: epochs from the workgroups' own slots


def test_own_slot_same_schedule_is_exact():
    ws = Workspace()
    big = [10, 0x7F00]
    assert run_own_slot_call([big], [ws], solo(0) + solo(1), [0, 0]) == [[max(big)]] * 2
    small = [0x3F80, 0x3F00]
    assert run_own_slot_call([small], [ws], solo(0) + solo(1), [1000, 1000]) == [[max(small)]] * 2
    assert {ws.read_slot(s)[0] for s in range(NSLOTS)} == {2}    # every slot stamped


def test_own_slot_grid_size_changes_keep_the_slots_uniform():
    ws = Workspace()
    for call, nwg in enumerate([3, 1, 8, 5, 2, 7, 1, 4]):
        shares = [[0x100 * (call + 1) + p for p in range(nwg)]]
        got = run_own_slot_call(shares, [ws], [], [LONG] * nwg)
        assert got == [[max(shares[0])]] * nwg
        assert {ws.read_slot(s)[0] for s in range(NSLOTS)} == {call + 1}


def test_own_slot_expired_wait_then_normal_wait():
    ws = Workspace()
    for rep in range(20):
        d1 = [100 + 7 * p + rep for p in range(5)]
        order = [p for p in (4, 2, 0, 3, 1) for _ in range(2)]
        assert run_own_slot_call([d1], [ws], order, [0] * 5) == [[max(d1)]] * 5
        d2 = [p + rep for p in range(5)]
        assert run_own_slot_call([d2], [ws], [0, 1, 2, 0, 1, 2], [LONG] * 5) == [[max(d2)]] * 5


@pytest.mark.parametrize("seed", range(4))
def test_own_slot_random_schedules_and_regions(seed):
    # a pool of three tensor regions; each call takes one or two of them in
    # either role (the epoch comes from all of a call's regions), with a random
    # grid size, random waits and late workgroups
    rng = random.Random(1000 + seed)
    for trial in range(300):
        pool = [Workspace() for _ in range(3)]
        for call in range(8):
            nj = rng.randint(1, 2)
            regions = rng.sample(pool, nj)
            nwg = rng.randint(1, 6)
            shares = [[rng.randint(0, 0x7F7F) for _ in range(nwg)] for _ in range(nj)]
            waits = [rng.choice([0, 1, 2, 5, LONG]) for _ in range(nwg)]
            got = run_own_slot_call(shares, regions, random_schedule(rng, nwg), waits)
            want = [max(sj) for sj in shares]
            assert got == [want] * nwg, (seed, trial, call, shares, got)
            for r in regions:
                assert len({r.read_slot(s)[0] for s in range(NSLOTS)}) == 1


def test_own_slot_stale_slots_of_earlier_calls_are_ignored():
    # slots left uniform at epoch E holding the largest magnitude (the state an
    # earlier call leaves, with other data): the next call is exact
    ws = Workspace()
    ws.slot = {s: (0x123456789A, 0x7F7F) for s in range(NSLOTS)}
    for rep in range(3):
        got = run_own_slot_call([[0x3F80, 0x3F00, 0x3E00]], [ws], [2, 2, 1, 0], [LONG] * 3)
        assert got == [[0x3F80]] * 3
    assert {ws.read_slot(s)[0] for s in range(NSLOTS)} == {0x123456789A + 3}


def test_own_slot_prefilled_next_epoch_is_outside_the_contract():
    # slots that already carry the next epoch in a non-uniform workspace are
    # indistinguishable from current ones: workspaces must start zeroed
    ws = Workspace()
    ws.slot = {0: (41, 0), 1: (42, 0x7F7F)}
    got = run_own_slot_call([[0x3F80, 0x3F00]], [ws], solo(0) + solo(1), [LONG, LONG])
    assert got[0] == [0x7F7F]


def test_own_slot_without_stamping_fails():
    # without the stamps a smaller grid leaves the slots above it behind; a
    # later larger grid then derives different epochs in different workgroups
    rng = random.Random(77)
    failures = 0
    for trial in range(300):
        pool = [Workspace() for _ in range(2)]
        for call in range(8):
            nj = rng.randint(1, 2)
            regions = rng.sample(pool, nj)
            nwg = rng.randint(1, 6)
            shares = [[rng.randint(0, 0x7F7F) for _ in range(nwg)] for _ in range(nj)]
            waits = [rng.choice([0, 1, 2, 5, LONG]) for _ in range(nwg)]
            got = run_own_slot_call(shares, regions, random_schedule(rng, nwg), waits, stamp=False)
            failures += got != [[max(sj) for sj in shares]] * nwg
    assert failures > 0
