"""Scheduling of attention tiles onto workers: greedy list scheduling and LPT.

TEST INFRASTRUCTURE (see the package docstring): only the tests use this module.

Source: "LLM Systems 22: Flash Attention", §4.1.5 Load Balancing: Causal
Attention.  Under the causal mask the query-row tiles of a sequence cost
different amounts (a tile sees only the keys up to its own rows), so handing
the tiles to workers in their natural order leaves some workers busy long after
the others; assigning the longest tile first (longest-processing-time-first,
LPT) evens the loads.  The page's example: 2 batches, 3 workers; in order the
workers finish 9, 5 and 6 blocks (9 units), LPT finishes in 7.

Readings:
* A worker takes the next job as soon as it is free (greedy list scheduling;
  ties go to the lowest-numbered worker); "in order" lists the jobs batch by
  batch, row by row; LPT lists them by decreasing cost (ties keep that order).
* Causal tile costs: query-row block r (0-based) of a causal sequence with
  equal block sizes costs r + 1 key blocks.  The page's example figure is not
  in the text; costs 1, 2, 3, 4 per batch reproduce every printed number.
"""

from __future__ import annotations

from typing import Sequence


def causal_costs(batches: int, blocks: int) -> list[int]:
    """Costs of the query-row blocks of `batches` causal sequences of `blocks` blocks,
    batch by batch, row by row: 1, 2, ..., blocks for each batch."""
    return [r + 1 for _ in range(batches) for r in range(blocks)]


def lpt_order(costs: Sequence[float]) -> list[int]:
    """Job indices by decreasing cost; equal costs keep their original order."""
    return sorted(range(len(costs)), key=lambda j: -costs[j])


def list_schedule(costs: Sequence[float], workers: int, order: Sequence[int] | None = None):
    """Greedy list scheduling.  Returns (per-worker busy time, [(job, worker, start)])."""
    if workers <= 0:
        raise ValueError("need at least one worker")
    order = list(range(len(costs))) if order is None else list(order)
    free_at = [0.0] * workers
    busy = [0.0] * workers
    plan = []
    for j in order:
        w = min(range(workers), key=lambda i: (free_at[i], i))
        plan.append((j, w, free_at[w]))
        free_at[w] += costs[j]
        busy[w] += costs[j]
    return busy, plan


def makespan(busy: Sequence[float]) -> float:
    return max(busy) if busy else 0.0
