"""CPU model of the single launch's cross-workgroup protocol (no GPU).

The fused kernel's workgroups are modelled as coroutines stepped by a
randomised scheduler, with the hardware's limited residency: each XCD holds
at most R workgroups at once, and the others wait in dispatch order until a
resident one exits.  Each workgroup does what the kernel does:

* reads its XCD and draws a ticket there (an atomic counter); the first
  min(chains of the XCD, MAX_CONSUMERS) tickets consume chains, the rest
  produce units;
* a producer draws units from its XCD's list with an atomic counter, and
  flags a unit's block ready at the first barrier of its next unit (or after
  its last unit);
* a consumer walks its chains in order; before each block it polls the
  block's ready flag, at most SPIN_LIMIT times (then it records a time-out
  and goes on, as the kernel does).

The model checks that every block is produced exactly once and consumed
only after it was flagged, that every chain is consumed in chunk order, that
no wait times out when every XCD can hold one producer beside its consumers
(whatever the interleaving and the dispatch order), and that when it cannot,
the waits end by time-out (the kernel then reports FLAG_TIMEOUT) instead of
hanging.  Producers never wait, so no cycle of waits exists; the draw is a
plain fetch-and-add, so there is no retry loop that could livelock.

It also checks the plan kernel's closed form for the per-XCD unit lists
(row j of XCD x holds ceil((C_j - x) / 8) entries, C_j = H * #sequences with
more than j chunks) against a brute-force chunk-major enumeration.
"""

import collections
import math
import random

import pytest

XCDS = 8
MAX_CONSUMERS = 8


def plan_lists(lengths, H):
    """The plan kernel's construction: sequences sorted by chunk count
    (longest first, ties by index); chain rank rho = i * H + h on XCD
    rho % 8; per XCD, units (chunk c, head h) row by row, C_j chains per row."""
    n = [math.ceil(L / 64) for L in lengths]
    first = [0]
    for x in n:
        first.append(first[-1] + x)
    order = sorted(range(len(n)), key=lambda s: (-n[s], s))
    nsorted = [n[s] for s in order]
    jmax = nsorted[0] if nsorted else 0
    lists = [[] for _ in range(XCDS)]
    for x in range(XCDS):
        for j in range(jmax):
            S = sum(1 for v in nsorted if v > j)
            C = H * S
            cnt = (C - x + 7) // 8 if C > x else 0
            for r in range(cnt):
                rho = 8 * r + x
                s = order[rho // H]
                lists[x].append((first[s] + j, rho % H))
    return order, first, lists


def brute_lists(lengths, H):
    """Chunk-major enumeration by definition: for each XCD and local chunk j,
    every chain of that XCD (in rank order) that has more than j chunks."""
    n = [math.ceil(L / 64) for L in lengths]
    first = [0]
    for x in n:
        first.append(first[-1] + x)
    order = sorted(range(len(n)), key=lambda s: (-n[s], s))
    chains = [(order[rho // H], rho % H) for rho in range(len(n) * H)]
    lists = [[] for _ in range(XCDS)]
    for x in range(XCDS):
        mine = [chains[rho] for rho in range(x, len(chains), 8)]
        for j in range(max(n) if n else 0):
            for s, h in mine:
                if n[s] > j:
                    lists[x].append((first[s] + j, h))
    return lists


@pytest.mark.parametrize("lengths,H", [([2048] * 4, 16), ([16384], 96), ([130, 0, 64, 17, 200, 1, 0, 95], 3),
                                       ([700, 5, 3000, 64, 65, 1, 128], 5), ([0, 0], 2)])
def test_plan_unit_lists_match_brute_force(lengths, H):
    _, _, lists = plan_lists(lengths, H)
    assert lists == brute_lists(lengths, H)
    units = sorted(u for lst in lists for u in lst)
    n = [math.ceil(L / 64) for L in lengths]
    assert len(units) == len(set(units)) == H * sum(n)


def test_plan_unit_lists_random():
    rng = random.Random(7)
    for _ in range(40):
        N = rng.randint(1, 40)
        H = rng.randint(1, 20)
        lengths = [rng.choice([0, rng.randint(1, 64), rng.randint(65, 2000)]) for _ in range(N)]
        _, _, lists = plan_lists(lengths, H)
        assert lists == brute_lists(lengths, H)


class Model:
    """One call of the fused kernel, stepped one sync point at a time."""

    def __init__(self, lengths, H, wgs_per_xcd, resident_per_xcd, spin_limit, seed, produce_steps=6):
        self.rng = random.Random(seed)
        self.H = H
        self.order, self.first, self.lists = plan_lists(lengths, H)
        self.N = len(lengths)
        self.ready = collections.defaultdict(int)   # block (c, h) -> flag
        self.produced = collections.Counter()
        self.consumed = []                           # (chain, c) in the order consumed
        self.ticket = [0] * XCDS
        self.unitctr = [0] * XCDS
        self.timeouts = 0
        self.spin_limit = spin_limit
        self.produce_steps = produce_steps
        self.wgs_per_xcd = wgs_per_xcd
        self.resident_per_xcd = resident_per_xcd

    def workgroup(self, xcd):
        t = self.ticket[xcd]
        self.ticket[xcd] += 1
        yield
        chains = self.N * self.H
        chains_x = (chains - xcd + 7) // 8 if chains > xcd else 0
        consumers = min(chains_x, MAX_CONSUMERS)
        if t < consumers:
            rho = xcd + 8 * t
            while rho < chains:
                s, h = self.order[rho // self.H], rho % self.H
                for c in range(self.first[s], self.first[s + 1]):
                    spins = 0
                    while not self.ready[(c, h)]:
                        if spins >= self.spin_limit:
                            self.timeouts += 1
                            break
                        spins += 1
                        yield
                    if self.ready[(c, h)]:
                        self.consumed.append(((s, h), c))
                    yield
                rho += 8 * consumers
            return
        lst = self.lists[xcd]
        k = self.unitctr[xcd]
        self.unitctr[xcd] += 1
        yield
        prev = None
        while k < len(lst):
            # the next unit is drawn at the start of this one
            k_next = self.unitctr[xcd]
            self.unitctr[xcd] += 1
            yield
            # first barrier: the previous unit's block is flagged ready
            if prev is not None:
                self.ready[prev] = 1
            for _ in range(self.produce_steps):
                yield
            self.produced[lst[k]] += 1
            prev = lst[k]
            k = k_next
        if prev is not None:
            self.ready[prev] = 1

    def run(self, dispatch="round_robin"):
        G = XCDS * self.wgs_per_xcd
        if dispatch == "round_robin":
            queue = [b % XCDS for b in range(G)]
        else:  # a permuted dispatch order (still wgs_per_xcd per XCD)
            queue = [b % XCDS for b in range(G)]
            self.rng.shuffle(queue)
        waiting = collections.deque(queue)
        resident = []
        per_xcd = [0] * XCDS
        steps = 0
        while waiting or resident:
            # admit in dispatch order while the head's XCD has room
            while waiting and per_xcd[waiting[0]] < self.resident_per_xcd:
                x = waiting.popleft()
                resident.append((x, self.workgroup(x)))
                per_xcd[x] += 1
            i = self.rng.randrange(len(resident))
            x, co = resident[i]
            try:
                next(co)
            except StopIteration:
                resident.pop(i)
                per_xcd[x] -= 1
            steps += 1
            assert steps < 10_000_000, "no progress"
        return self


def check_complete(m, lengths, H):
    n = [math.ceil(L / 64) for L in lengths]
    all_blocks = {(m.first[s] + j, h) for s in range(len(lengths)) for h in range(H) for j in range(n[s])}
    assert set(m.produced) == all_blocks
    assert all(v == 1 for v in m.produced.values())
    got = collections.defaultdict(list)
    for chain, c in m.consumed:
        got[chain].append(c)
    for s in range(len(lengths)):
        for h in range(H):
            assert got[(s, h)] == list(range(m.first[s], m.first[s + 1]))


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("lengths,H", [([2048] * 4, 16), ([130, 0, 64, 17, 200, 1, 0, 95], 3),
                                       ([1500] + [70] * 20, 4)])
@pytest.mark.parametrize("dispatch", ["round_robin", "shuffled"])
def test_full_residency_never_times_out(seed, lengths, H, dispatch):
    # 64 workgroups per XCD, all resident (two per CU on an idle device)
    m = Model(lengths, H, wgs_per_xcd=12, resident_per_xcd=12, spin_limit=10**6,
              seed=seed).run(dispatch)
    assert m.timeouts == 0
    check_complete(m, lengths, H)


@pytest.mark.parametrize("seed", range(6))
def test_partial_residency_with_room_for_one_producer(seed):
    # each XCD holds only its consumers plus one producer at a time (the
    # rest of the device busy elsewhere): slower, but no time-out
    lengths, H = [640] * 3 + [64, 0, 300], 8
    m = Model(lengths, H, wgs_per_xcd=14, resident_per_xcd=MAX_CONSUMERS + 1,
              spin_limit=10**6, seed=seed).run("shuffled")
    assert m.timeouts == 0
    check_complete(m, lengths, H)


def test_no_room_for_a_producer_ends_by_time_out():
    # an XCD that can hold only its consumers: they cannot make progress, and
    # every wait ends at the spin limit instead of hanging
    lengths, H = [256] * 8, 8
    m = Model(lengths, H, wgs_per_xcd=10, resident_per_xcd=MAX_CONSUMERS, spin_limit=50,
              seed=1).run()
    assert m.timeouts > 0
