"""CPU model of the pipelined chunked prefill's launch (kda_prefill.hip, prefill_pipe_kernel):
one grid holding the chunk workgroups and, at indices pipe_first .. pipe_first + NC - 1, the
carries, which wait for the records' ready words.

The model follows the launch as the kernel relies on it:
  - workgroups go to the XCDs round-robin by index (index i to XCD i % 8), and each XCD
    starts its own workgroups in index order as its compute units free up, one workgroup
    per compute unit;
  - a chunk workgroup never waits: it writes its segment's records one chunk at a time;
  - a carry walks its pair's chunks in order and may start chunk c only once record c of
    its pair is ready (polling holds its compute unit).
The properties: with fewer carries on every XCD than that XCD has compute units, every
schedule drains (each workgroup finishes), whatever pipe_first and the workgroups' speeds
are; and the host's rule, carries on at most half the compute units, always satisfies that.
With at least as many carries on an XCD as it has compute units, a carry can hold every
compute unit while its records' workgroups wait behind it: the model finds that stall,
so it can tell the two cases apart."""
import random

import pytest

XCDS = 8


def _simulate(cus, pairs, chunks, seg, first, carries, rng, max_steps=200_000):
    """Run the launch; return True if every workgroup finished, False on a stall (every
    busy compute unit holds a carry waiting for a record no running workgroup will write,
    and the next workgroups in line on those XCDs cannot start)."""
    nsegs = (chunks + seg - 1) // seg
    items = [(j, p) for j in range(nsegs) for p in range(pairs)]  # segment-major (row j, pair p)
    grid = []
    for b in range(len(items) + carries):
        if first <= b < first + carries:
            grid.append(("carry", b - first))
        else:
            grid.append(("prod", items[b if b < first else b - carries]))
    per_xcd = [[g for i, g in enumerate(grid) if i % XCDS == x] for x in range(XCDS)]
    nxt = [0] * XCDS
    cu_per_xcd = cus // XCDS
    ready = set()
    running = [[] for _ in range(XCDS)]  # per XCD: [kind, data, progress]
    done = 0
    for _ in range(max_steps):
        # start workgroups on free compute units, in index order per XCD
        for x in range(XCDS):
            while len(running[x]) < cu_per_xcd and nxt[x] < len(per_xcd[x]):
                kind, data = per_xcd[x][nxt[x]]
                nxt[x] += 1
                running[x].append([kind, data, 0])
        if done == len(grid):
            return True
        # one step of a random subset of the running workgroups (arbitrary relative speeds)
        moved = False
        for x in range(XCDS):
            for wg in list(running[x]):
                if rng.random() < 0.5:
                    continue
                kind, data, prog = wg
                if kind == "prod":
                    j, p = data
                    c = j * seg + prog
                    if c < chunks:
                        ready.add((c, p))
                    wg[2] += 1
                    moved = True
                    if wg[2] >= seg or j * seg + wg[2] >= chunks:
                        running[x].remove(wg)
                        done += 1
                else:
                    if (prog, data) in ready:
                        wg[2] += 1
                        moved = True
                        if wg[2] >= chunks:
                            running[x].remove(wg)
                            done += 1
        if not moved:
            # nothing can move unless a producer does: a stall if every running workgroup
            # is a waiting carry and no XCD can start anything
            stalled = all(kind == "carry" and (prog, data) not in ready
                          for x in range(XCDS) for kind, data, prog in running[x])
            blocked = all(len(running[x]) >= cu_per_xcd or nxt[x] >= len(per_xcd[x]) for x in range(XCDS))
            if stalled and blocked and any(running[x] for x in range(XCDS)):
                return False
    raise AssertionError("no decision within the step bound")


@pytest.mark.parametrize("seed", range(40))
def test_half_the_compute_units_always_drains(seed):
    rng = random.Random(seed)
    cus = XCDS * rng.choice([2, 3, 4, 6])
    pairs = rng.randint(1, cus // 2)  # the host's rule: 2 * B * H <= compute units
    chunks = rng.randint(1, 12)
    seg = rng.choice([1, 2, 4])
    nitems = ((chunks + seg - 1) // seg) * pairs
    first = rng.randint(0, nitems)  # any start, early or late
    assert _simulate(cus, pairs, chunks, seg, first, pairs, rng)


@pytest.mark.parametrize("seed", range(20))
def test_fewer_carries_than_compute_units_per_xcd_drains(seed):
    rng = random.Random(100 + seed)
    cu_per_xcd = rng.choice([2, 3, 4])
    cus = XCDS * cu_per_xcd
    pairs = XCDS * (cu_per_xcd - 1)  # one compute unit per XCD left for the chunk workgroups
    chunks = rng.randint(2, 8)
    assert _simulate(cus, pairs, chunks, 2, 0, pairs, rng)


def test_carries_on_every_compute_unit_can_stall():
    # as many carries as compute units, placed first: they take every compute unit and
    # wait for records that the chunk workgroups behind them never get to write
    rng = random.Random(7)
    cus = XCDS * 2
    assert not _simulate(cus, cus, 4, 2, 0, cus, rng)


def _row_major_index(nseg, s, j):
    """The position the chunk table kernel gives segment j of sequence s (nseg: segments per
    sequence): the rows before it, then the sequences before s that reach row j."""
    return sum(min(n, j) for n in nseg) + sum(1 for t in range(s) if nseg[t] > j)


@pytest.mark.parametrize("seed", range(30))
def test_row_major_segment_order(seed):
    # the kernel's formula is a bijection onto the segments in row-major order: row j of
    # every sequence (in sequence order) before row j + 1, empty sequences skipped
    rng = random.Random(seed)
    nseg = [rng.choice([0, 0, 1, 2, 3, 5, 8]) for _ in range(rng.randint(1, 12))]
    expect = [(s, j) for j in range(max(nseg)) for s in range(len(nseg)) if j < nseg[s]]
    got = sorted(((_row_major_index(nseg, s, j), (s, j)) for s in range(len(nseg)) for j in range(nseg[s])))
    assert [i for i, _ in got] == list(range(len(expect)))
    assert [sj for _, sj in got] == expect
