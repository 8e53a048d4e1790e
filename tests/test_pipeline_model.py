"""A discrete-event model of the forward's hand-synchronised K/V ring protocols.

The forward kernels copy K/V blocks global->LDS with copies the compiler does
not track, wait for them with hand-counted `s_waitcnt vmcnt(N)`, and publish
them with fenceless barriers.  The GPU race check (test_gpu_race.py) compares
the pipelined build with a build that drains every wait; this CPU test checks
the protocols themselves, as the kernels order them, under randomised
timings:

- the ping-pong body (eight waves in two halves, a four-slot ring of K|V
  blocks, copies two intervals ahead, issued from the softmax phase);
- the pipelined single-wave body (four waves, K in two slots and V in three,
  block j+1 copied when iteration j opens);
- the serial double-buffered body (variable-length batches at D = 256);
- the backward's rings: the dQ and dK/dV kernels (four slots, copies two
  blocks ahead, the dK/dV kernel's LSE and Delta copies by waves 0 and 1,
  and wave 0's write of the LSE of rows without keys before the barrier),
  and the wide-head kernels' two-slot ring.

Each wave is a sequence of actions in the kernel's order (copy issue, vmcnt
waits, barriers, LDS reads with a duration).  A copy's share lands after a
random latency; a wave's copies retire in issue order, as the vector-memory
counter counts them.  Every LDS read must find all eight (four) shares of the
block it expects in the slot, and no share of another block may land in that
slot while it reads.  Persistent workgroups run several tiles in a row; the
barrier before a tile's first copies is what keeps the last PV of one half
from reading a slot the other half's next-tile copies overwrite, and the model
finds that race when the barrier is taken out (a planted protocol mutation).
"""
import random

import pytest


class Violation(Exception):
    pass


class Model:
    def __init__(self, waves, rng, latency, slow_wave=None, slow_factor=1.0, owners=None):
        self.waves = waves
        self.owners = owners or {}  # kind -> the waves that write it (default: every wave)
        self.rng = rng
        self.latency = latency
        self.slow_wave = slow_wave
        self.slow_factor = slow_factor
        self.lands = {}  # (kind, slot) -> list of (land_time, wave, tag)
        self.reads = []  # (reader, kind, slot, tag, start, end), checked once every copy is known

    def dur(self, wave, lo, hi):
        d = self.rng.uniform(lo, hi)
        return d * (self.slow_factor if wave == self.slow_wave else 1.0)

    def run(self, programs):
        """programs[w]: list of actions of wave w."""
        n = len(programs)
        t = [0.0] * n
        pc = [0] * n
        issued = [[] for _ in range(n)]  # per wave: landing times in issue order (retired in order)
        at_barrier = {}
        while True:
            live = [w for w in range(n) if pc[w] < len(programs[w]) and w not in at_barrier]
            if not live:
                if at_barrier:
                    if len(at_barrier) != n:
                        raise AssertionError("barrier counts differ between waves")
                    release = max(at_barrier.values())
                    for w in at_barrier:
                        t[w] = release
                        pc[w] += 1
                    at_barrier = {}
                    continue
                for r in self.reads:
                    self.check_read(*r)
                return
            w = min(live, key=lambda x: t[x])
            act = programs[w][pc[w]]
            op = act[0]
            if op == "barrier":
                at_barrier[w] = t[w]
                continue
            if op == "compute":
                t[w] += self.dur(w, act[1], act[2])
            elif op == "issue":
                _, kind, slot, tag = act
                land = t[w] + self.rng.uniform(*self.latency)
                if issued[w]:
                    land = max(land, issued[w][-1])  # in-order retirement
                issued[w].append(land)
                self.lands.setdefault((kind, slot), []).append((land, w, tag))
                t[w] += 1.0
            elif op == "write":  # an LDS store of the wave itself, waited for at once
                _, kind, slot, tag = act
                self.lands.setdefault((kind, slot), []).append((t[w] + 1.0, w, tag))
                t[w] += 2.0
            elif op == "wait":  # s_waitcnt vmcnt(max_outstanding)
                keep = act[1]
                done = issued[w][: max(0, len(issued[w]) - keep)]
                if done:
                    t[w] = max(t[w], done[-1])
            elif op == "read":
                _, kind, slot, tag, lo, hi = act
                d = self.dur(w, lo, hi)
                self.reads.append((w, kind, slot, tag, t[w], t[w] + d))
                t[w] += d
            pc[w] += 1

    def check_read(self, reader, kind, slot, tag, t0, t1):
        events = self.lands.get((kind, slot), [])
        for owner in self.owners.get(kind, range(self.waves)):
            mine = [e for e in events if e[1] == owner]
            before = [e for e in mine if e[0] <= t0]
            if not before or max(before)[2] != tag:
                raise Violation("wave %d read %s slot %d expecting %s before wave %d's share landed"
                                % (reader, kind, slot, tag, owner))
            for (land, _, other) in mine:
                if t0 < land <= t1 and other != tag:
                    raise Violation("wave %d read %s slot %d (%s) while %s landed in it"
                                    % (reader, kind, slot, tag, other))


# ---- the ping-pong body (D <= 192): two halves of four waves, 4-slot ring

def pingpong_programs(tiles, tile_barrier=True, slots=4):
    """Actions of the 8 waves for a persistent workgroup running tiles of the
    given block counts.  Per wave per block: one K copy and one V copy (its
    share), so LOADS_BLOCK = 2 in the model's units."""
    progs = []
    ring = lambda b: b % slots  # noqa: E731
    for w in range(8):
        half = w // 4
        p = []
        for ti, n in enumerate(tiles):
            tag = lambda b: (ti, b)  # noqa: E731
            p.append(("wait", 0))                  # the Q rows' load (vmcnt(0) via their pin)
            if tile_barrier:
                p.append(("barrier",))
            for b in range(min(n, 2)):
                p.append(("issue", "K", ring(b), tag(b)))
                p.append(("issue", "V", ring(b), tag(b)))
            for it in range(n + 1):
                p.append(("wait", 2 if it + 1 < n else 0))
                p.append(("barrier",))

                def matrix():
                    if it < n:
                        p.append(("read", "K", ring(it), tag(it), 600, 800))
                    if it > 0:
                        p.append(("read", "V", ring(it - 1), tag(it - 1), 700, 900))

                def softmax():
                    if it + 2 < n:
                        p.append(("issue", "K", ring(it + 2), tag(it + 2)))
                    p.append(("compute", 300, 700))
                    if it + 2 < n:
                        p.append(("issue", "V", ring(it + 2), tag(it + 2)))
                    p.append(("compute", 500, 900))

                if half == 0:
                    matrix()
                    softmax()
                else:
                    softmax()
                    matrix()
            p.append(("compute", 50, 200))         # epilogue
        progs.append(p)
    return progs


# ---- the pipelined single-wave body (D = 256): four waves, K 2 slots, V 3

def pipelined_programs(tiles, tile_barrier=True, vslots=3):
    progs = []
    for w in range(4):
        p = []
        for ti, n in enumerate(tiles):
            tag = lambda b: (ti, b)  # noqa: E731

            def issue_block(j):
                if j < n:
                    p.append(("issue", "K", j & 1, tag(j)))
                    p.append(("issue", "V", j % vslots, tag(j)))

            def open_(j):
                p.append(("wait", 1 if j < n else 0))  # K_j and V_{j-1} landed
                p.append(("barrier",))
                issue_block(j + 1)

            p.append(("wait", 0))                  # Q rows
            if tile_barrier:
                p.append(("barrier",))
            if n > 0:
                issue_block(0)
                open_(0)
                p.append(("read", "K", 0, tag(0), 900, 1300))
                p.append(("compute", 300, 600))
            for j in range(1, n):
                open_(j)
                p.append(("read", "K", j & 1, tag(j), 900, 1300))
                p.append(("read", "V", (j - 1) % vslots, tag(j - 1), 1000, 1600))
            if n > 0:
                open_(n)
                p.append(("read", "V", (n - 1) % vslots, tag(n - 1), 1000, 1600))
            p.append(("compute", 50, 200))
        progs.append(p)
    return progs


# ---- the serial double-buffered body (variable-length batches at D = 256)

def serial_programs(tiles, end_barrier=True):
    """Block j+1 is copied into the other buffer when iteration j starts;
    iteration j ends with a barrier, so the buffer of block j-1 (the same as
    block j+1's) is free, and a persistent workgroup's next tile starts with
    every wave done reading."""
    progs = []
    for w in range(4):
        p = []
        for ti, n in enumerate(tiles):
            tag = lambda b: (ti, b)  # noqa: E731
            p.append(("wait", 0))                  # Q rows
            if n > 0:
                p.append(("issue", "K", 0, tag(0)))
                p.append(("issue", "V", 0, tag(0)))
            for j in range(n):
                if j + 1 < n:
                    p.append(("issue", "K", (j + 1) & 1, tag(j + 1)))
                    p.append(("issue", "V", (j + 1) & 1, tag(j + 1)))
                    p.append(("wait", 2))
                else:
                    p.append(("wait", 0))
                p.append(("barrier",))
                p.append(("read", "K", j & 1, tag(j), 900, 1300))
                p.append(("compute", 600, 1200))
                p.append(("read", "V", j & 1, tag(j), 1000, 1600))
                if end_barrier:
                    p.append(("barrier",))
            p.append(("compute", 50, 200))
        progs.append(p)
    return progs


# ---- the backward's rings

def bwd_programs(n, stats=False, lse_fix=(), fix_after_barrier=False, slots=4):
    """dQ (stats=False) or dK/dV (stats=True) kernel at D <= 128: four waves,
    a ring of `slots` slots, block j+2 copied at the top of iteration j, one
    barrier per block and none at its end.  In dK/dV, wave 0 copies the
    block's LSE and wave 1 its Delta; for the blocks in lse_fix, wave 0 then
    overwrites the LSE of rows without keys, before the barrier."""
    progs = []
    for w in range(4):
        p = []

        def issue(j):
            p.append(("issue", "Q", j % slots, j))
            p.append(("issue", "G", j % slots, j))
            if stats and w < 2:
                p.append(("issue", "L" if w == 0 else "E", j % slots, j))
        per_block = 2 + (1 if stats and w < 2 else 0)
        for j in range(min(n, 2)):
            issue(j)
        for j in range(n):
            if j + 2 < n:
                issue(j + 2)
                p.append(("wait", 2 * per_block))
            elif j + 1 < n:
                p.append(("wait", per_block))
            else:
                p.append(("wait", 0))
            fix = stats and w == 0 and j in lse_fix
            if fix and not fix_after_barrier:
                p.append(("write", "L", j % slots, (j, "fixed")))
            p.append(("barrier",))
            if fix and fix_after_barrier:
                p.append(("write", "L", j % slots, (j, "fixed")))
            if stats:
                lt = (j, "fixed") if j in lse_fix else j
                p.append(("read", "L", j % slots, lt, 20, 60))
                p.append(("read", "E", j % slots, j, 20, 60))
            p.append(("read", "Q", j % slots, j, 800, 1400))
            p.append(("compute", 300, 900))
            p.append(("read", "G", j % slots, j, 800, 1400))
        progs.append(p)
    return progs


def wide_bwd_programs(n, slots=2):
    """The wide-head backward kernels: a two-slot ring; block j+1 copied
    right after the barrier (which drains the wave's LDS reads) that opens
    block j, into the slot of block j-1."""
    progs = []
    for w in range(4):
        p = []
        if n > 0:
            p.append(("issue", "Q", 0, 0))
        for j in range(n):
            p.append(("wait", 0))
            p.append(("barrier",))
            if j + 1 < n:
                p.append(("issue", "Q", (j + 1) % slots, j + 1))
            p.append(("read", "Q", j % slots, j, 1500, 3000))
        progs.append(p)
    return progs


BWD_OWNERS = {"L": [0], "E": [1]}


@pytest.mark.parametrize("n", [1, 2, 3, 5, 9])
@pytest.mark.parametrize("stats", [False, True], ids=["dq", "dkdv"])
def test_backward_ring_protocols_have_no_race(n, stats):
    fixes = (0, 1) if stats else ()
    for seed in range(60):
        rng = random.Random(seed * 31 + n)
        lat = (rng.choice([200, 1500]), rng.choice([2500, 6000]))
        slow = rng.randrange(4) if seed % 3 == 0 else None
        Model(4, rng, lat, slow, rng.uniform(1.0, 4.0), BWD_OWNERS).run(
            bwd_programs(n, stats, lse_fix=fixes))
        Model(4, rng, lat, slow, rng.uniform(1.0, 4.0)).run(wide_bwd_programs(n))


def test_model_finds_backward_protocol_mutations():
    """Planted mutations: the keyless rows' LSE written after the barrier
    (another wave may read the block's LSE first), a three-slot ring with
    copies two blocks ahead, and a one-slot wide ring."""
    def finds(progs, owners=None, slow=2):
        for seed in range(200):
            try:
                Model(4, random.Random(seed), (10, 50), slow, 6.0, owners).run(progs)
            except Violation:
                return True
        return False
    assert finds(bwd_programs(4, True, lse_fix=(0,), fix_after_barrier=True), BWD_OWNERS, slow=0)
    assert finds(bwd_programs(6, False, slots=3))
    assert finds(wide_bwd_programs(4, slots=1))


TILE_SETS = [[1], [2], [3], [5], [9], [4, 3], [2, 7, 1], [5, 5, 6], [8, 1, 2, 3]]


@pytest.mark.parametrize("tiles", TILE_SETS, ids=lambda t: "x".join(map(str, t)))
def test_pingpong_ring_protocol_has_no_race(tiles):
    for seed in range(60):
        rng = random.Random(seed * 1009 + len(tiles))
        lat = (rng.choice([200, 1500]), rng.choice([2500, 6000]))
        slow = rng.randrange(8) if seed % 3 == 0 else None
        Model(8, rng, lat, slow, rng.uniform(1.0, 4.0)).run(pingpong_programs(tiles))


@pytest.mark.parametrize("tiles", TILE_SETS, ids=lambda t: "x".join(map(str, t)))
def test_pipelined_body_ring_protocol_has_no_race(tiles):
    for seed in range(60):
        rng = random.Random(seed * 917 + len(tiles))
        lat = (rng.choice([200, 1500]), rng.choice([2500, 6000]))
        slow = rng.randrange(4) if seed % 3 == 0 else None
        Model(4, rng, lat, slow, rng.uniform(1.0, 4.0)).run(pipelined_programs(tiles))


@pytest.mark.parametrize("tiles", TILE_SETS, ids=lambda t: "x".join(map(str, t)))
def test_serial_body_double_buffer_has_no_race(tiles):
    for seed in range(60):
        rng = random.Random(seed * 733 + len(tiles))
        lat = (rng.choice([200, 1500]), rng.choice([2500, 6000]))
        slow = rng.randrange(4) if seed % 3 == 0 else None
        Model(4, rng, lat, slow, rng.uniform(1.0, 4.0)).run(serial_programs(tiles))


def _finds_race(programs, waves, slow_wave, latency=(10, 50)):
    for seed in range(200):
        rng = random.Random(seed)
        try:
            # short copy latency, one slow wave: a copy can land while that
            # wave still reads the slot's previous block
            Model(waves, rng, latency, slow_wave, 6.0).run(programs)
        except Violation:
            return True
    return False


def test_model_finds_the_cross_tile_race_without_the_tile_barrier():
    """Planted mutation: without the barrier before a tile's first copies, a
    half-1 wave still in the previous tile's last PV can read a ring slot that
    half 0's next-tile copies overwrite (last block in slot 0 or 1)."""
    assert _finds_race(pingpong_programs([5, 3], tile_barrier=False), 8, slow_wave=5)
    assert _finds_race(pipelined_programs([4, 3], tile_barrier=False), 4, slow_wave=2)


def test_model_finds_a_ring_one_slot_short():
    """Planted mutation: with copies two intervals ahead, a three-slot ring
    (ping-pong) or a two-slot V ring (single-wave body, V read one iteration
    after K) lets a copy overwrite a block that is still being read."""
    assert _finds_race(pingpong_programs([6], slots=3), 8, slow_wave=6)
    assert _finds_race(pipelined_programs([6], vslots=2), 4, slow_wave=1)


def test_model_finds_the_serial_body_race_without_its_end_barrier():
    assert _finds_race(serial_programs([6], end_barrier=False), 4, slow_wave=3)


def test_model_finds_a_missing_interval_wait():
    """Planted mutation: an interval that waits for no copy at all reads a
    block before its shares have landed."""
    def no_wait(tiles, tile_barrier=True):
        progs = pingpong_programs(tiles, tile_barrier)
        return [[("compute", 1, 2) if a[0] == "wait" and a[1] == 2 else a for a in p]
                for p in progs]
    found = False
    for seed in range(50):
        try:
            Model(8, random.Random(seed), (3000, 9000)).run(no_wait([6]))
        except Violation:
            found = True
            break
    assert found
