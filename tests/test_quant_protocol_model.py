"""CPU model of the single-launch quantiser's tensor-maximum exchange.

The resident quantiser (k_quant_resident in csrc/quantize.hip) runs at most one
workgroup per CU.  Each workgroup reduces its share of the tensor, publishes
the maximum in its own 64-bit slot tagged with the call's epoch, and polls all
slots until every one carries that epoch; a workgroup whose bounded wait
expires finds the maximum another way.  The epoch is one more than a control
word that the previous call on the same workspace left behind.

This module simulates that exchange step by step: every workgroup is a
generator that yields after each access to the shared workspace, and a
scheduler decides which workgroup moves next, including workgroups that only
start after others have finished (a grid that is not resident all at once).
Three variants are modelled:

  "advance_by_wg0"   the earlier kernel: workgroup 0 advances the control word
                     as soon as its own poll ends, whether it saw every slot or
                     its wait expired; an expired workgroup reads the whole
                     tensor.
  "last_arrival"     the current kernel: every workgroup, after its poll, adds
                     one to an arrival counter; the workgroup that brings it to
                     the grid size resets it and advances the control word, so
                     no workgroup of a call can read an advanced word.  An
                     expired workgroup reads directly only the shares of the
                     workgroups whose slots it has not seen.

  "arrive_before_read"  an arrival at the start, before the read of the
                     control word, and the advance after the poll (a negative
                     control).

The tests show that the first variant takes a stale maximum from the previous
call under a reachable schedule, and that the second gives every workgroup the
true maximum under that schedule and under many random ones, for sequences of
calls with different grid sizes on one zero-initialised workspace.
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
