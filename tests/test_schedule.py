"""The scheduling oracle against the page's example and textbook bounds, and the
persistent forward kernel's static work assignment against the oracle (CPU)."""

import itertools
import json
import os

import pytest

import oracle.schedule as sch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "lpt_example.json")


def test_page_example():
    ex = json.load(open(GOLDEN))["lpt_causal_2batches_3workers"]
    costs = sch.causal_costs(ex["batches"], 4)
    busy, _ = sch.list_schedule(costs, ex["workers"])
    assert busy == [float(x) for x in ex["printed"]["in_order_worker_blocks"]]
    assert sch.makespan(busy) == ex["printed"]["in_order_makespan"]
    lpt = sch.list_schedule(costs, ex["workers"], sch.lpt_order(costs))[0]
    assert sch.makespan(lpt) == ex["printed"]["lpt_makespan"]


def _optimum(costs, m):
    best = float("inf")
    for assign in itertools.product(range(m), repeat=len(costs)):
        loads = [0] * m
        for c, w in zip(costs, assign):
            loads[w] += c
        best = min(best, max(loads))
    return best


@pytest.mark.parametrize("seed", range(12))
def test_lpt_within_grahams_bound(seed):
    # LPT <= (4/3 - 1/(3m)) OPT; any greedy list <= (2 - 1/m) OPT (Graham 1966, 1969)
    import random
    rng = random.Random(seed)
    m = rng.choice([2, 3])
    costs = [rng.randint(1, 9) for _ in range(rng.randint(3, 8))]
    opt = _optimum(costs, m)
    lpt = sch.makespan(sch.list_schedule(costs, m, sch.lpt_order(costs))[0])
    naive = sch.makespan(sch.list_schedule(costs, m)[0])
    assert opt <= lpt <= (4 / 3 - 1 / (3 * m)) * opt + 1e-9
    assert opt <= naive <= (2 - 1 / m) * opt + 1e-9
    assert sum(sch.list_schedule(costs, m)[0]) == sum(costs)


def _kernel_items(n_tiles, bh_count, grid, xcd_order=False):
    """The persistent forward kernel's assignment (with xcd_order also the
    persistent backward kernels', whose dK/dV pass takes tile = rank), restated: the items, numbered
    longest first over all pairs (item i -> (pair, rank), pairs dealt over the 8
    XCDs) or, with xcd_order, pair by pair per XCD (the per-tile kernel's order),
    are dealt in rounds of one per work-group, even rounds in work-group order,
    odd rounds with each XCD's work-groups reversed (work-group g = 8 j + x takes
    item round * grid + 8 (grid/8 - 1 - j) + x); tile = n_tiles - 1 - rank."""
    out = {g: [] for g in range(grid)}
    total = n_tiles * bh_count
    r = 0
    while r * grid < total:
        for g in range(grid):
            it = r * grid + (8 * (grid // 8 - 1 - g // 8) + g % 8 if r % 2 else g)
            if it >= total:
                continue
            if xcd_order:
                if bh_count % 8 == 0:
                    j = it // 8
                    bh, rank = (j // n_tiles) * 8 + it % 8, j % n_tiles
                else:
                    L = (it % 8) * (total // 8) + it // 8 if total % 8 == 0 else it
                    bh, rank = L // n_tiles, L % n_tiles
            elif bh_count % 8 == 0:
                per = bh_count // 8
                j = it // 8
                bh, rank = (j % per) * 8 + it % 8, j // per
            else:
                bh, rank = it % bh_count, it // bh_count
            out[g].append((bh, n_tiles - 1 - rank))
        r += 1
    return out


@pytest.mark.parametrize("n_tiles,bh_count,grid", [(32, 128, 512), (32, 128, 504), (8, 48, 64), (5, 6, 16),
                                                   (256, 16, 512), (1, 3, 8)])
def test_persistent_assignment(n_tiles, bh_count, grid):
    items = _kernel_items(n_tiles, bh_count, grid)
    seen = [x for g in items for x in items[g]]
    # every (pair, tile) exactly once
    assert sorted(seen) == sorted((bh, t) for bh in range(bh_count) for t in range(n_tiles))
    # with a grid that is a multiple of 8, each work-group stays on its XCD's pairs
    if bh_count % 8 == 0 and grid % 8 == 0:
        for g, lst in items.items():
            assert all(bh % 8 == g % 8 for bh, _ in lst)
    # each work-group's items come longest first
    for lst in items.values():
        assert all(a[1] >= b[1] for a, b in zip(lst, lst[1:]))
    # busy time of the static dealing: within one longest item of greedy LPT
    costs = [t + 1 for bh in range(bh_count) for t in range(n_tiles)]
    lpt = sch.makespan(sch.list_schedule(costs, grid, sch.lpt_order(costs))[0])
    static = max(sum(t + 1 for _, t in lst) for lst in items.values())
    assert static <= lpt + n_tiles
    # the snake deal is within one cost unit of greedy LPT on these causal lists
    # (a round-robin deal is 9-12% above it on 32 x 128 and 256 x 16)
    assert static <= lpt + 1


@pytest.mark.parametrize("n_tiles,bh_count,grid", [(32, 128, 512), (32, 64, 512), (16, 128, 504), (8, 48, 64),
                                                   (5, 6, 16), (8, 256, 512)])
def test_persistent_assignment_xcd_order(n_tiles, bh_count, grid):
    """The order for grids of several rounds: every tile exactly once, each
    work-group on its XCD's pairs, and the items in flight on an XCD in any round
    spanning few pairs (the L2 sharing the order is for)."""
    items = _kernel_items(n_tiles, bh_count, grid, xcd_order=True)
    seen = [x for g in items for x in items[g]]
    assert sorted(seen) == sorted((bh, t) for bh in range(bh_count) for t in range(n_tiles))
    if bh_count % 8 == 0 and grid % 8 == 0:
        for g, lst in items.items():
            assert all(bh % 8 == g % 8 for bh, _ in lst)
        # round r's items on XCD x: grid / 8 consecutive items of that XCD's
        # sequence, i.e. at most ceil(grid / 8 / n_tiles) + 1 pairs
        rounds = max(len(lst) for lst in items.values())
        for r in range(rounds):
            for x in range(8):
                pairs = {lst[r][0] for g, lst in items.items() if g % 8 == x and r < len(lst)}
                assert len(pairs) <= -(-(grid // 8) // n_tiles) + 1
    # each pair's tiles reach a work-group longest first
    for lst in items.values():
        by_pair = {}
        for bh, t in lst:
            by_pair.setdefault(bh, []).append(t)
        assert all(ts == sorted(ts, reverse=True) for ts in by_pair.values())


SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "schedule.py")
MUTATIONS = {
    "lpt_ascending": ("key=lambda j: -costs[j]", "key=lambda j: costs[j]"),
    "ties_to_last_worker": ("key=lambda i: (free_at[i], i)", "key=lambda i: (free_at[i], -i)"),
    "free_time_not_advanced": ("free_at[w] += costs[j]", "free_at[w] += 0"),
    "causal_costs_flat": ("return [r + 1 for _ in range(batches) for r in range(blocks)]",
                          "return [blocks for _ in range(batches) for r in range(blocks)]"),
    "least_busy_not_first_free": ("w = min(range(workers), key=lambda i: (free_at[i], i))",
                                  "w = len(plan) % workers"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name):
    import types
    find, repl = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(find) == 1
    mod = types.ModuleType("schedule_mutant")
    exec(compile(src.replace(find, repl), "schedule_mutant", "exec"), mod.__dict__)
    global sch
    saved, sch = sch, mod
    caught = False
    try:
        for fn in (test_page_example, *(lambda s=s: test_lpt_within_grahams_bound(s) for s in range(12))):
            try:
                fn()
            except Exception:
                caught = True
                break
    finally:
        sch = saved
    assert caught, name
