"""A CPU model of the ring protocols the kernels run, explored under random
interleavings of their waves.

Each wave is a generator that follows its kernel's sequence of operations on
the LDS ring: DMA issues (which land later, in issue order per wave), waits on
its own loads (vmcnt), arrivals on and waits for the per-stage "full" and
"empty" counters, workgroup barriers, and the span during which it reads a
stage's fragments.  A random scheduler interleaves the waves and lands loads
at random moments.  The model checks, at every step:

  - RAW: a wave starts reading a position only when every part of it has
    landed in the position's stage;
  - WAR: no load lands into or is issued to a stage while a wave reads it;
  - liveness: the run ends with every wave finished (no deadlock);
  - every position is read by exactly the waves that compute it.

The configurations mirror the kernels: the all-wave kernel with full/empty
counters (flags) and with one barrier per k-step (barrier), the loader/MFMA
split (wavespec), and loader waves with two MFMA groups taking tiles in turn
(pingpong), and the barrier kernel over the split-window ring (windows).
Injected faults -- a wrong arrival count, a skipped WAR or RAW wait, an
off-by-one RAW target, counters that do not start at zero, an announcement
lag too long for the ring, a refill or an epilogue that is not fenced by the
barrier -- must each be caught.
"""
import random

import pytest


class Violation(Exception):
    pass


class Deadlock(Exception):
    pass


class Ring:
    """Shared state: the stages' contents, the counters, the readers."""

    def __init__(self, S, parts, init_full=0, init_empty=0):
        self.S = S
        self.parts = parts                     # loading waves per position
        self.full = [init_full] * S
        self.empty = [init_empty] * S
        self.landed = [dict() for _ in range(S)]   # stage -> {part: position}
        self.readers = [set() for _ in range(S)]   # stage -> waves reading it
        self.reads = {}                            # position -> waves that read it
        self.barrier_count = 0

    def issue(self, s, q):
        if self.readers[s]:
            raise Violation("WAR: load of position %r issued into stage %d while %s read it"
                            % (q, s, sorted(self.readers[s])))

    def land(self, s, part, q):
        if self.readers[s]:
            raise Violation("WAR: load of position %r landed in stage %d while %s read it"
                            % (q, s, sorted(self.readers[s])))
        self.landed[s][part] = q

    def begin_read(self, w, s, q):
        have = self.landed[s]
        if len(have) != self.parts or any(v != q for v in have.values()):
            raise Violation("RAW: wave %d reads position %r from stage %d holding %r" % (w, q, s, have))
        self.readers[s].add(w)
        self.reads.setdefault(q, set()).add(w)

    def end_read(self, w, s):
        self.readers[s].discard(w)


class Wave:
    """A wave's generator plus its queue of DMA loads in flight."""

    def __init__(self, wid, gen):
        self.wid = wid
        self.gen = gen
        self.inflight = []          # (stage, part, position), oldest first
        self.cond = None            # callable: may the wave continue?
        self.done = False


def run(ring, waves, seed, max_steps=200000, idle_polls=0):
    """idle_polls: when no wave can move, re-evaluate the waits up to this many
    times before declaring a deadlock (time passes for waits that poll with a
    budget; unbounded waits never change their answer)."""
    rng = random.Random(seed)
    for w in waves:
        w.cond = None
    steps = 0
    while True:
        steps += 1
        if steps > max_steps:
            raise Deadlock("step limit")
        live = [w for w in waves if not w.done]
        landable = [w for w in waves if w.inflight]
        if not live and not landable:
            return
        runnable = [w for w in live if w.cond is None or w.cond()]
        for _ in range(idle_polls):
            if runnable or landable:
                break
            runnable = [w for w in live if w.cond is None or w.cond()]
        choices = [("run", w) for w in runnable] + [("land", w) for w in landable]
        if not choices:
            raise Deadlock("no wave can move: %s" % [(w.wid, w.done) for w in waves])
        kind, w = rng.choice(choices)
        if kind == "land":
            s, part, q = w.inflight.pop(0)
            ring.land(s, part, q)
            continue
        try:
            w.cond = next(w.gen)
        except StopIteration:
            w.done = True
            w.cond = None


def vm_wait(wave, n):
    """Yield until at most n of the wave's loads are in flight."""
    return lambda: len(wave.inflight) <= n


def at_least(arr, i, target):
    return lambda: arr[i] >= target


# --- loader waves (wave-specialised and ping-pong kernels) ---------------------
def loader(ring, wave, part, total, S, D, releasers, skip_war_wait=False):
    for q in range(total):
        s = q % S
        if q >= S and not skip_war_wait:
            yield at_least(ring.empty, s, (q // S) * releasers)
        ring.issue(s, q)
        wave.inflight.append((s, part, q))
        yield None
        if q >= D:
            yield vm_wait(wave, D)
            ring.full[(q - D) % S] += 1
            yield None
    yield vm_wait(wave, 0)
    for q in range(max(total - D, 0), total):
        ring.full[q % S] += 1
        yield None


# --- MFMA waves of the wave-specialised and ping-pong kernels -------------------
def consumer(ring, wave, positions, S, NP, raw_off=0):
    """positions: the flat positions this wave computes, in order (its group's
    tiles).  It waits for a position's announcement, reads it, then releases."""
    for q in positions:
        s = q % S
        yield at_least(ring.full, s, (q // S + 1) * NP - raw_off)
        ring.begin_read(wave.wid, s, q)
        yield None          # reading the stage's fragments
        yield None
        ring.end_read(wave.wid, s)
        ring.empty[s] += 1
        yield None


# --- all-wave kernel, full/empty counters ----------------------------------------
def flags_wave(ring, wave, total, S, NW, empty_target_scale=1, skip_full_wait=False, announce_first=False):
    """Each of the NW waves loads its part of every position and computes every
    position.  Prologue: positions 0 .. S-2, then position 0 announced.  Per
    k-step c: the load of position c+S-1 goes out into the stage of position
    c-1 (checked free at the end of k-step c-1), the wave reads position c,
    waits for its own loads of position c+1, then releases c and announces
    c+1 in one atomic step (the kernel's single add on a word that holds both
    counters), and waits until every wave has done both."""
    w = wave.wid
    for q in range(S - 1):
        ring.issue(q % S, q)
        wave.inflight.append((q % S, w, q))
        yield None
    # position 0 readable
    yield vm_wait(wave, S - 2)
    ring.full[0] += 1
    yield at_least(ring.full, 0, NW)
    for c in range(total):
        s_cur = c % S
        q_new = c + S - 1                       # positions past the end load zeros
        s_new = q_new % S
        ring.issue(s_new, q_new)
        wave.inflight.append((s_new, w, q_new))
        ring.begin_read(w, s_cur, c)
        yield None
        s_nxt, g_nxt = (c + 1) % S, (c + 1) // S
        if announce_first:
            # fault: the announcement of c+1 goes out while c is still read
            yield vm_wait(wave, S - 2)
            ring.full[s_nxt] += 1
            yield None
            ring.end_read(w, s_cur)
            ring.empty[s_cur] += 1
        else:
            ring.end_read(w, s_cur)
            yield vm_wait(wave, S - 2)
            ring.empty[s_cur] += 1
            ring.full[s_nxt] += 1
        full_target = 0 if skip_full_wait else (g_nxt + 1) * NW
        empty_target = (c // S + 1) * NW * empty_target_scale
        yield (lambda f=s_nxt, e=s_cur, ft=full_target, et=empty_target:
               ring.full[f] >= ft and ring.empty[e] >= et)
    yield vm_wait(wave, 0)


# --- all-wave kernel, one barrier per k-step ---------------------------------------
def barrier_wave(ring, wave, total, S, NW, barrier, skip_vm=False):
    """Loads of position c+S-1 go out after the barrier that ends k-step c-1
    (every wave has finished reading that stage).  Before the barrier that
    ends k-step c the wave waits for its own loads of position c+1."""
    w = wave.wid
    for q in range(S - 1):
        ring.issue(q % S, q)
        wave.inflight.append((q % S, w, q))
        yield None
    yield vm_wait(wave, S - 2)
    yield from barrier(wave)
    for c in range(total):
        s_cur = c % S
        q_new = c + S - 1
        ring.issue(q_new % S, q_new)
        wave.inflight.append((q_new % S, w, q_new))
        ring.begin_read(w, s_cur, c)
        yield None
        ring.end_read(w, s_cur)
        if not skip_vm:
            yield vm_wait(wave, S - 2)
        yield from barrier(wave)
    yield vm_wait(wave, 0)


def make_barrier(NW):
    state = {"arrived": 0}

    def barrier(wave):
        state["arrived"] += 1
        target = -(-state["arrived"] // NW) * NW     # the generation this wave joined
        yield lambda: state["arrived"] >= target
    return barrier


# --- all-wave kernel over the split-window ring ----------------------------------
def window_wave(ring, wave, total, KT, NW, barrier, skip_epi_barrier=False, vm_slack=0,
                early_refill=False):
    """Five windows; position q keeps its A tile in window 2q mod 5 and its B
    tile in window 2q+1 mod 5.  Every wave loads two parts of each tile.  Per
    k-step c: region 0 issues the second part of B(c+1); regions 1-2 the two
    parts of A(c+2); region 3 ends the reads of position c, waits for its own
    loads up to B(c+1), passes the barrier, issues the first part of B(c+2)
    into A(c)'s window and starts reading position c+1.  After a tile's last
    k-step the wave stages its epilogue in B(c)'s window, then a barrier,
    before A(c+3) reuses that window."""
    w = wave.wid
    win_a = lambda q: (2 * q) % 5
    win_b = lambda q: (2 * q + 1) % 5

    def issue(win, tag, q, part):
        ring.issue(win, q)
        wave.inflight.append((win, (w, part), (tag, q)))

    for part in (0, 1):
        issue(win_a(0), "A", 0, part)
    for part in (0, 1):
        issue(win_b(0), "B", 0, part)
    for part in (0, 1):
        issue(win_a(1), "A", 1, part)
    issue(win_b(1), "B", 1, 0)
    yield None
    yield vm_wait(wave, 3)                      # A(1) and B(1) part 0 may be in flight
    yield from barrier(wave)
    ring.begin_read(w, win_a(0), ("A", 0))
    ring.begin_read(w, win_b(0), ("B", 0))
    for c in range(total):
        issue(win_b(c + 1), "B", c + 1, 1)      # region 0
        yield None
        issue(win_a(c + 2), "A", c + 2, 0)      # region 1
        yield None
        issue(win_a(c + 2), "A", c + 2, 1)      # region 2
        yield None
        if early_refill:
            issue(win_b(c + 2), "B", c + 2, 0)
        ring.end_read(w, win_a(c))              # region 3: reads of c done
        ring.end_read(w, win_b(c))
        yield vm_wait(wave, 2 + vm_slack)       # only A(c+2) may be in flight
        yield from barrier(wave)
        if not early_refill:
            issue(win_b(c + 2), "B", c + 2, 0)
        if c + 1 < total:
            ring.begin_read(w, win_a(c + 1), ("A", c + 1))
            ring.begin_read(w, win_b(c + 1), ("B", c + 1))
        yield None
        if c % KT == KT - 1:                    # epilogue in B(c)'s window
            # wave-private strips: other waves' strips may share the window,
            # fragment reads and loads may not (landing checks the strips)
            busy = [r for r in ring.readers[win_b(c)] if not (isinstance(r, tuple) and r[0] == "strip")]
            if busy:
                raise Violation("epilogue strip in window %d while %s read it" % (win_b(c), busy))
            ring.readers[win_b(c)].add(("strip", w))
            yield None
            ring.readers[win_b(c)].discard(("strip", w))
            if not skip_epi_barrier:
                yield from barrier(wave)
    yield vm_wait(wave, 0)


def run_windows(NW, n_tiles, KT, seed, **faults):
    ring = Ring(5, 2 * NW)
    barrier = make_barrier(NW)
    waves = []
    for w in range(NW):
        wv = Wave(w, None)
        wv.gen = window_wave(ring, wv, n_tiles * KT, KT, NW, barrier, **faults)
        waves.append(wv)
    run(ring, waves, seed)
    for q in range(n_tiles * KT):
        assert ring.reads.get(("A", q)) == set(range(NW)), q
        assert ring.reads.get(("B", q)) == set(range(NW)), q


# --- harnesses -------------------------------------------------------------------
def run_producer_consumer(S, NP, NCWG, groups, n_tiles, KT, seed, releasers=None, D=None,
                          skip_war_wait=False, raw_off=0, init=0):
    total = n_tiles * KT
    ring = Ring(S, NP, init_full=init, init_empty=init)
    D = (min(S - 2, 2) if D is None else D)
    releasers = NCWG if releasers is None else releasers
    waves = []
    for g in range(groups):
        tiles = range(g, n_tiles, groups)
        positions = [it * KT + kt for it in tiles for kt in range(KT)]
        for i in range(NCWG):
            wv = Wave(len(waves), None)
            wv.gen = consumer(ring, wv, positions, S, NP, raw_off)
            waves.append(wv)
    for part in range(NP):
        wv = Wave(len(waves), None)
        wv.gen = loader(ring, wv, part, total, S, D, releasers, skip_war_wait)
        waves.append(wv)
    run(ring, waves, seed)
    # every position read by exactly the NCWG waves of the group that owns its tile
    for q in range(total):
        g = (q // KT) % groups
        want = set(range(g * NCWG, (g + 1) * NCWG))
        assert ring.reads.get(q) == want, (q, ring.reads.get(q), want)


def run_flags(S, NW, total, seed, empty_target_scale=1, init=0, skip_full_wait=False, announce_first=False):
    ring = Ring(S, NW, init_full=init, init_empty=init)
    waves = []
    for w in range(NW):
        wv = Wave(w, None)
        wv.gen = flags_wave(ring, wv, total, S, NW, empty_target_scale, skip_full_wait, announce_first)
        waves.append(wv)
    run(ring, waves, seed)
    for q in range(total):
        assert ring.reads.get(q) == set(range(NW)), q


def run_barrier(S, NW, total, seed, skip_vm=False):
    ring = Ring(S, NW)
    barrier = make_barrier(NW)
    waves = []
    for w in range(NW):
        wv = Wave(w, None)
        wv.gen = barrier_wave(ring, wv, total, S, NW, barrier, skip_vm)
        waves.append(wv)
    run(ring, waves, seed)
    for q in range(total):
        assert ring.reads.get(q) == set(range(NW)), q


SEEDS = range(12)


@pytest.mark.parametrize("S", [2, 3, 4])
@pytest.mark.parametrize("seed", SEEDS)
def test_wavespec_protocol(S, seed):
    run_producer_consumer(S, NP=4, NCWG=4, groups=1, n_tiles=3, KT=5, seed=seed)


@pytest.mark.parametrize("S", [2, 4])
@pytest.mark.parametrize("seed", SEEDS)
def test_wavespec_two_mfma_waves_per_simd_protocol(S, seed):
    """The 2- and 4-stage rings of the wave-specialised kernel: 8 MFMA waves
    (each releases a stage once all its reads of it have landed) beside 4
    loader waves, whose refill of a stage waits for all 8 releases."""
    run_producer_consumer(S, NP=4, NCWG=8, groups=1, n_tiles=3, KT=5, seed=seed)


@pytest.mark.parametrize("seed", SEEDS)
def test_pingpong_per_group_pipeline_protocol(seed):
    """Ping-pong with one pipeline per MFMA group (2 stages): each group's ring
    is filled by 2 loader waves (two announcements per position) and read by
    its 4 MFMA waves; the two pipelines share nothing but the workgroup."""
    run_producer_consumer(2, NP=2, NCWG=4, groups=1, n_tiles=3, KT=5, seed=seed)


@pytest.mark.parametrize("S", [2, 3, 4])
@pytest.mark.parametrize("seed", SEEDS)
def test_pingpong_protocol(S, seed):
    run_producer_consumer(S, NP=4, NCWG=4, groups=2, n_tiles=5, KT=4, seed=seed)


@pytest.mark.parametrize("S", [2, 3, 4])
@pytest.mark.parametrize("seed", SEEDS)
def test_flags_protocol(S, seed):
    run_flags(S, NW=4, total=11, seed=seed)


@pytest.mark.parametrize("S", [2, 3, 4])
@pytest.mark.parametrize("seed", SEEDS)
def test_barrier_protocol(S, seed):
    run_barrier(S, NW=4, total=11, seed=seed)


@pytest.mark.parametrize("KT", [1, 2, 3, 5])
@pytest.mark.parametrize("seed", SEEDS)
def test_window_ring_protocol(KT, seed):
    run_windows(NW=4, n_tiles=3, KT=KT, seed=seed)


def test_one_tile_pingpong_second_group_idle():
    for seed in SEEDS:
        run_producer_consumer(3, NP=4, NCWG=4, groups=2, n_tiles=1, KT=6, seed=seed)


# --- injected faults: each must be caught for some interleaving -----------------
def caught(fn, seeds=range(40)):
    for seed in seeds:
        try:
            fn(seed)
        except (Violation, Deadlock, AssertionError):
            return True
    return False


def test_fault_pingpong_release_count_of_all_mfma_waves():
    """Loaders waiting for releases by all 8 MFMA waves, when one group of 4
    releases each position, never see the stage freed."""
    assert caught(lambda sd: run_producer_consumer(3, 4, 4, 2, 4, 4, sd, releasers=8))


def test_fault_two_wave_ring_release_count_of_one_wave_per_simd():
    """Loaders of the 8-MFMA-wave ring that refill a stage after 4 releases
    (the 4-MFMA-wave layout's count) overwrite data still being read."""
    for S in (2, 4):
        assert caught(lambda sd: run_producer_consumer(S, 4, 8, 1, 3, 5, sd, releasers=4))


def test_fault_loader_skips_war_wait():
    assert caught(lambda sd: run_producer_consumer(2, 4, 4, 1, 3, 5, sd, skip_war_wait=True))


def test_fault_consumer_raw_target_off_by_one():
    assert caught(lambda sd: run_producer_consumer(3, 4, 4, 1, 3, 5, sd, raw_off=1))


def test_fault_counters_not_zeroed():
    """Counters that start at a stale value let a consumer read a stage before
    its loads land (the initialisation the counters rely on)."""
    assert caught(lambda sd: run_producer_consumer(3, 4, 4, 1, 3, 5, sd, init=4))


def test_fault_announce_lag_too_long():
    """Announcing position q - D only after issuing q, with D = S - 1, makes
    the announcement of a stage wait on its own release: no progress."""
    assert caught(lambda sd: run_producer_consumer(3, 4, 4, 1, 3, 5, sd, D=3))


@pytest.mark.parametrize("S", [2, 3, 4])
def test_flags_war_wait_is_implied_by_the_raw_wait(S):
    """Every wave releases position c no later than it announces position
    c + 1, and the refill of c's stage goes out only after every wave's
    announcement.  So the announcement wait already covers WAR: the model stays
    safe with the release check removed altogether.  (The kernel keeps the
    check; it costs nothing because both counters are read at once.)"""
    for seed in SEEDS:
        run_flags(S, 4, 11, seed, empty_target_scale=0)


def test_fault_flags_announce_before_release_without_war_check():
    """Announcing position c + 1 while still reading c is safe only because the
    release check catches it; with the check removed as well, a refill lands
    in a stage that a wave still reads."""
    assert caught(lambda sd: run_flags(2, 4, 9, sd, empty_target_scale=0, announce_first=True))


@pytest.mark.parametrize("S", [2, 3, 4])
def test_flags_release_check_guards_an_early_announcement(S):
    """The same early announcement with the release check in place stays safe:
    the check is what makes the two signals independent."""
    for seed in SEEDS:
        run_flags(S, 4, 11, seed, announce_first=True)


@pytest.mark.parametrize("S", [2, 3, 4])
def test_flags_raw_wait_is_implied_by_the_release_check(S):
    """One atomic step carries a wave's release of c and its announcement of
    c + 1, made after its own loads of c + 1 landed.  So a complete release
    count implies a complete announcement, too: each check alone is safe."""
    for seed in SEEDS:
        run_flags(S, 4, 11, seed, skip_full_wait=True)


def test_fault_flags_no_wait_at_all():
    assert caught(lambda sd: run_flags(2, 4, 9, sd, skip_full_wait=True, empty_target_scale=0))


def test_fault_barrier_without_load_wait():
    assert caught(lambda sd: run_barrier(2, 4, 9, sd, skip_vm=True))


def test_fault_window_epilogue_without_barrier():
    """Without the barrier after the epilogue, one wave's A(c+3) load can land
    in the window another wave still stages its output tile in."""
    assert caught(lambda sd: run_windows(4, 3, 2, sd, skip_epi_barrier=True))


def test_fault_window_load_wait_misses_next_b():
    assert caught(lambda sd: run_windows(4, 3, 3, sd, vm_slack=1))


def test_fault_window_refill_before_barrier():
    assert caught(lambda sd: run_windows(4, 3, 3, sd, early_refill=True))


# --- bounded waits: a failure terminates and is visible -------------------------
# The kernels' waits on ring counters give up after a bounded number of polls.
# A wave that gives up sets the workgroup's poison word before its next step,
# then runs its loops to the end; before storing a tile, every wave checks the
# word (and its own failure) and writes NaN instead of values.  The model below
# gives waits a budget of scheduler evaluations; with a fault that makes a
# counter fall short for good, it checks that every wave finishes and that
# every tile whose reads saw data the failure let through -- a stage read
# before all of its loads landed, or a load landing in a stage being read -- is
# stored flagged.  Without a failure nothing is flagged.
class BoundedRing(Ring):
    def __init__(self, S, parts):
        super().__init__(S, parts)
        self.poison = False
        self.timeouts = 0
        self.tile_of = {}               # wave -> tile it is computing
        self.corrupt = set()            # (wave, tile) whose reads saw bad data
        self.stores = []                # (wave, tile, flagged)

    def _taint(self, s):
        if not self.poison:
            return False
        for r in self.readers[s]:
            self.corrupt.add((r, self.tile_of.get(r)))
        return True

    def issue(self, s, q):
        if self.readers[s] and self._taint(s):
            return
        super().issue(s, q)

    def land(self, s, part, q):
        if self.readers[s] and self._taint(s):
            self.landed[s][part] = q
            return
        super().land(s, part, q)

    def begin_read(self, w, s, q):
        have = self.landed[s]
        if self.poison and (len(have) != self.parts or any(v != q for v in have.values())):
            self.corrupt.add((w, self.tile_of.get(w)))
            self.readers[s].add(w)
            self.reads.setdefault(q, set()).add(w)
            return
        super().begin_read(w, s, q)


def bounded(ring, wave, cond, limit):
    """A wait that gives up after `limit` evaluations: the wave's failure
    flag and the workgroup's poison word are set before it continues; a wave
    that has failed does not wait any more."""
    state = {"polls": 0}

    def check():
        if wave.failed or cond():
            return True
        state["polls"] += 1
        if state["polls"] > limit:
            wave.failed = True
            ring.poison = True
            ring.timeouts += 1
            return True
        return False
    return check


def bounded_loader(ring, wave, part, total, S, D, releasers, limit, lose=None):
    """The loader of `loader` with bounded waits.  lose = position whose
    announcement this loader never makes (the injected fault)."""
    for q in range(total):
        s = q % S
        if q >= S:
            yield bounded(ring, wave, at_least(ring.empty, s, (q // S) * releasers), limit)
        ring.issue(s, q)
        wave.inflight.append((s, part, q))
        yield None
        if q >= D:
            yield vm_wait(wave, D)
            if q - D != lose:
                ring.full[(q - D) % S] += 1
            yield None
    yield vm_wait(wave, 0)
    for q in range(max(total - D, 0), total):
        if q != lose:
            ring.full[q % S] += 1
        yield None


def bounded_consumer(ring, wave, tiles, KT, S, NP, limit, use_poison=True):
    for t in tiles:
        ring.tile_of[wave.wid] = t
        for q in range(t * KT, (t + 1) * KT):
            s = q % S
            yield bounded(ring, wave, at_least(ring.full, s, (q // S + 1) * NP), limit)
            ring.begin_read(wave.wid, s, q)
            yield None
            yield None
            ring.end_read(wave.wid, s)
            ring.empty[s] += 1
            yield None
        # the store: poison_tile checks the wave's flag and the poison word
        ring.stores.append((wave.wid, t, wave.failed or (use_poison and ring.poison)))
        yield None


def run_bounded(S, NP, NCWG, groups, n_tiles, KT, seed, limit=30, lose=None, lose_part=0, use_poison=True,
                loader_limit=None):
    total = n_tiles * KT
    ring = BoundedRing(S, NP)
    D = min(S - 2, 2)
    waves = []
    for g in range(groups):
        for i in range(NCWG):
            wv = Wave(len(waves), None)
            wv.failed = False
            wv.gen = bounded_consumer(ring, wv, list(range(g, n_tiles, groups)), KT, S, NP, limit, use_poison)
            waves.append(wv)
    for part in range(NP):
        wv = Wave(len(waves), None)
        wv.failed = False
        wv.gen = bounded_loader(ring, wv, part, total, S, D, NCWG, limit if loader_limit is None else loader_limit,
                                lose if part == lose_part else None)
        waves.append(wv)
    run(ring, waves, seed, idle_polls=min(max(limit, loader_limit or 0) + 2, 10 ** 4))   # Deadlock if stuck
    for w, t in ring.corrupt:
        assert (w, t, True) in ring.stores, ("tile computed from bad data stored unflagged", w, t)
    assert len(ring.stores) == NCWG * n_tiles
    return ring


@pytest.mark.parametrize("S", [2, 3, 4])
@pytest.mark.parametrize("groups", [1, 2], ids=["wavespec", "pingpong"])
def test_bounded_waits_without_failure_flag_nothing(S, groups):
    """Generous budgets: no wait gives up, nothing is flagged, and the run
    is the unbounded protocol's."""
    for seed in SEEDS:
        ring = run_bounded(S, 4, 4, groups, 4, 5, seed, limit=10 ** 6)
        assert ring.timeouts == 0 and not ring.poison
        assert not ring.corrupt and not any(f for _, _, f in ring.stores)


@pytest.mark.parametrize("S", [2, 3, 4])
@pytest.mark.parametrize("groups", [1, 2], ids=["wavespec", "pingpong"])
def test_lost_announcement_terminates_and_is_flagged(S, groups):
    """One loader never announces position 6: the consumers' waits for it
    give up instead of hanging, every wave finishes, the failure is counted
    and poisoned, and every tile whose reads saw bad data is stored flagged."""
    for seed in SEEDS:
        ring = run_bounded(S, 4, 4, groups, 4, 5, seed, limit=30, lose=6)
        assert ring.timeouts > 0 and ring.poison
        # the tile that needed position 6 is flagged by every one of its waves
        t6 = 6 // 5
        owners = [w for w in range(4 * groups) if (w // 4) == t6 % groups]
        for w in owners:
            assert (w, t6, True) in ring.stores


def test_lost_announcement_without_bounds_hangs():
    """The same fault with unbounded waits: no wave can move (what the bound
    turns into a flagged result)."""
    assert caught(lambda sd: run_bounded(3, 4, 4, 1, 4, 5, sd, limit=10 ** 9, lose=6))


def test_tight_budget_flags_every_tile_it_corrupts():
    """Budgets so small that waits give up while data is merely late (what the
    library's spin-limit setting forces on the GPU): whatever is read too
    early or overwritten while read, the tiles it feeds are stored flagged."""
    seen = 0
    for seed in range(40):
        ring = run_bounded(3, 4, 4, 2, 4, 5, seed, limit=1)
        seen += len(ring.corrupt) > 0
    assert seen > 0


def test_fault_flagging_by_own_failure_only():
    """Without the shared poison word a wave flags only what it computed after
    its own failure; a loader's failure then corrupts MFMA waves that never
    failed themselves, and their tiles go out unflagged."""
    assert caught(lambda sd: run_bounded(3, 4, 4, 2, 4, 5, sd, limit=10 ** 3, loader_limit=1, use_poison=False),
                  seeds=range(60))


def test_loader_failure_is_flagged_through_the_poison_word():
    """The same loader-only failures with the poison word in place: every
    corrupted tile is stored flagged."""
    seen = 0
    for seed in range(60):
        ring = run_bounded(3, 4, 4, 2, 4, 5, seed, limit=10 ** 3, loader_limit=1)
        seen += len(ring.corrupt) > 0
    assert seen > 0
