"""Plain-Python schedules and dQ accumulation orders (the oracle's copy).

TEST INFRASTRUCTURE ONLY: imported by tests and the smoke check, never by the
product path.  The product's C++ schedule generator is checked against these
lists bit for bit.

Vocabulary.  A head's sequence is cut into n KV tiles and n Q blocks of the
same width (square tiling).  An *item* (kv, q) is one KV tile meeting one Q
block; under a causal mask the item exists only when q >= kv.  A *unit* is
the work one workgroup runs without interruption: a list of items, grouped by
KV tile, because a KV tile's dK/dV stay in that workgroup's registers for as
long as it works on it (explainer, "Technisches Resuemee" 2.1: one KV tile's
operations run continuously on one SM).  A *rank table* gives, for every Q
block q, the order in which the KV tiles' dQ partials are added into q's
accumulator: rank[q][kv] = position of kv in that order.

Schedules (explainer 2.2 A and B; authors' abstract (i) and (ii)):

* NAIVE - the baseline fixed order: one unit per KV tile, Q blocks visited in
  ascending order, dQ partials added in ascending kv order.
* DESCENDING - Descending Q-tile iteration: the same units and the same dQ
  order, but each unit visits its Q blocks from the last to the first.
* SHIFT, full mask - one unit per KV tile; unit i visits Q blocks cyclically
  i, i+1, ..., n-1, 0, ..., i-1 (the explainer's cyclic pattern, read as a
  cycle over Q blocks because a KV tile stays on one SM).  The dQ order of a
  block is the step at which each unit reaches it, so no two units ever touch
  the same block at the same step.
* SHIFT, causal mask (symmetric shift) - a unit pairs KV tiles w and n-1-w
  (folding the triangle into a rectangle of n+1 items per unit), run in two
  phases: the dense lower-left square (Q blocks n/2..n-1 against KV tiles
  0..n/2-1) with a cyclic shift, then the folded remainder (the two small
  triangles) with a cyclic shift over "super-rows".  Every step touches
  distinct Q blocks; the dQ order is again by step.
* ATOMIC - NAIVE's traversal with unordered adds (no rank table).

The two-phase construction and the reading of the cyclic pattern as a cycle
over Q blocks are this project's readings of passages that the pages give
only in outline.
"""
from __future__ import annotations

NAIVE = "naive"
DESCENDING = "descending"
SHIFT = "shift"
ATOMIC = "atomic"
SCHEDULES = (ATOMIC, NAIVE, DESCENDING, SHIFT)


def live(kv: int, q: int, causal: bool) -> bool:
    """Square tiling: Q block q holds queries [q*T, q*T+T), KV tile kv keys
    [kv*T, kv*T+T).  Causal: some key <= some query  <=>  kv <= q."""
    return (not causal) or kv <= q


def units(schedule: str, n: int, causal: bool):
    """Per-unit item lists [(kv, q), ...] in processing order, for one head."""
    if n < 1:
        raise ValueError("n must be >= 1")
    if schedule in (NAIVE, ATOMIC):
        return [[(kv, q) for q in range(n) if live(kv, q, causal)] for kv in range(n)]
    if schedule == DESCENDING:
        return [[(kv, q) for q in reversed(range(n)) if live(kv, q, causal)] for kv in range(n)]
    if schedule == SHIFT:
        return _symmetric_shift(n) if causal else _shift_full(n)
    raise ValueError(f"unknown schedule {schedule!r}")


def _shift_full(n):
    return [[(i, (i + t) % n) for t in range(n)] for i in range(n)]


def _symmetric_shift(n):
    """Causal shift.  n even: n/2 units; unit w owns KV tiles w then n-1-w.

    Phase 1 (dense square): step t in [0, n/2), unit w does Q block
    n/2 + ((w + t) mod n/2) on KV tile w.

    Phase 2 (folded triangles): n/2 + 1 super-rows k.  For k <= n/2 - 2,
    super-row k holds upper row k (Q block k, for KV tiles w <= k) and lower
    row n-2-k (Q block n-2-k, for KV tiles n-1-w with w > k); super-row
    n/2 - 1 is upper row n/2 - 1 (all w); super-row n/2 is lower row n-1
    (all w).  At phase-2 step s, unit w works on super-row (w + s) mod
    (n/2 + 1): on KV tile w if that super-row's part for w is an upper row,
    else on KV tile n-1-w.

    n odd and above 1 has no pairing that covers every tile; the schedule
    is then undefined and a ValueError is raised (the product reports the
    shape as unsupported).  n == 1 is a single unit.
    """
    if n == 1:
        return [[(0, 0)]]
    if n % 2:
        raise ValueError("symmetric shift needs an even number of tiles")
    h = n // 2
    out = []
    for w in range(h):
        items = [(w, h + ((w + t) % h)) for t in range(h)]
        for s in range(h + 1):
            k = (w + s) % (h + 1)
            if k <= h - 2:
                items.append((w, k) if w <= k else (n - 1 - w, n - 2 - k))
            elif k == h - 1:
                items.append((w, h - 1))
            else:  # k == h
                items.append((n - 1 - w, n - 1))
        out.append(items)
    return out


def rank_table(schedule: str, n: int, causal: bool):
    """rank[q][kv] (or None where the item does not exist); None for ATOMIC.

    NAIVE / DESCENDING: ascending kv among the block's contributors.
    SHIFT: by the step at which the unit reaches the block (the
    constructions above never put two units on one block at one step; a tie
    would be broken by unit index)."""
    if schedule == ATOMIC:
        return None
    rank = [[None] * n for _ in range(n)]
    if schedule in (NAIVE, DESCENDING):
        for q in range(n):
            r = 0
            for kv in range(n):
                if live(kv, q, causal):
                    rank[q][kv] = r
                    r += 1
        return rank
    us = units(schedule, n, causal)
    keyed = {}
    for u, items in enumerate(us):
        for step, (kv, q) in enumerate(items):
            keyed.setdefault(q, []).append((step, u, kv))
    for q, lst in keyed.items():
        lst.sort()
        for r, (_, _, kv) in enumerate(lst):
            rank[q][kv] = r
    return rank


def contributors(n: int, causal: bool, q: int) -> int:
    return sum(1 for kv in range(n) if live(kv, q, causal))


# ------------------------------------------------------------ masked tiles
#
# Windows and block masks (the summary's limitations list names special
# masks such as block-sparse ones as needing schedule extensions).  Readings:
# a tile pair (kv, q) is live when at least one of its (query, key) pairs is
# visible, and partial when it is live but some pair is hidden (the kernel
# then masks elements).  NAIVE / DESCENDING / ATOMIC visit each KV tile's
# live Q blocks ascending / descending, dQ order ascending kv.  SHIFT for a
# general tile graph keeps the pages' defining property - at every step the
# units touch distinct Q blocks - by giving each live pair a step (colour)
# such that no unit and no Q block has two pairs at one step, with as many
# steps as the busiest tile has pairs; a unit runs its pairs in step order
# and a block's dQ order is by step.  Such colourings are not unique, so the
# oracle checks a product table against these rules (``check_step_schedule``)
# instead of building its own.


def tile_liveness(mask, n_tiles: int, tile: int):
    """(live, partial): n_tiles x n_tiles lists of bools indexed [q][kv],
    from the element mask (``oracle.attention.Mask``) by brute force."""
    import numpy as np
    n = n_tiles * tile
    vis = mask.visible(np.arange(n), np.arange(n)).reshape(n_tiles, tile, n_tiles, tile)
    any_vis = vis.any(axis=(1, 3))
    all_vis = vis.all(axis=(1, 3))
    live_t = [[bool(any_vis[q, kv]) for kv in range(n_tiles)] for q in range(n_tiles)]
    part_t = [[bool(any_vis[q, kv] and not all_vis[q, kv]) for kv in range(n_tiles)]
              for q in range(n_tiles)]
    return live_t, part_t


def masked_units(schedule: str, live_t):
    """Per-KV-tile item lists for NAIVE, DESCENDING and ATOMIC."""
    n = len(live_t)
    if schedule in (NAIVE, ATOMIC):
        return [[(kv, q) for q in range(n) if live_t[q][kv]] for kv in range(n)]
    if schedule == DESCENDING:
        return [[(kv, q) for q in reversed(range(n)) if live_t[q][kv]] for kv in range(n)]
    raise ValueError(f"no fixed masked construction for {schedule!r}")


def masked_rank_table(live_t):
    """NAIVE / DESCENDING dQ order: ascending kv among the block's live tiles."""
    n = len(live_t)
    rank = [[None] * n for _ in range(n)]
    for q in range(n):
        r = 0
        for kv in range(n):
            if live_t[q][kv]:
                rank[q][kv] = r
                r += 1
    return rank


def check_step_schedule(live_t, unit_items, steps, rank, dynamic=False):
    """Validate a SHIFT table for a general tile graph.  unit_items: per unit
    [(kv, q), ...] in run order; steps: per unit the step of each item;
    rank[q][kv].  dynamic: the units are handed out in list order by a work
    counter, so every wait (an item waits for the item ranked just before
    it at its Q block) must point to an earlier unit.  Returns '' or the
    first rule broken."""
    n = len(live_t)
    deg_kv = [sum(1 for q in range(n) if live_t[q][kv]) for kv in range(n)]
    deg_q = [sum(1 for kv in range(n) if live_t[q][kv]) for q in range(n)]
    delta = max(deg_kv + deg_q + [0])
    seen = {}
    owner = {}
    for u, (items, st) in enumerate(zip(unit_items, steps)):
        if len(items) != len(st):
            return "steps do not match items"
        if any(b <= a for a, b in zip(st, st[1:])):
            return "steps not increasing within a unit"
        for (kv, q), s in zip(items, st):
            if not (0 <= kv < n and 0 <= q < n) or not live_t[q][kv]:
                return "dead or out-of-range pair"
            if (kv, q) in seen:
                return "pair twice"
            if not 0 <= s < delta:
                return "step out of range"
            if owner.setdefault(kv, u) != u:
                return "KV tile in two units"
            seen[(kv, q)] = s
    if len(seen) != sum(deg_q):
        return "live pair missing"
    for q in range(n):
        contrib = sorted((seen[(kv, q)], kv) for kv in range(n) if live_t[q][kv])
        if len({s for s, _ in contrib}) != len(contrib):
            return "two units on one block at one step"
        for r, (_, kv) in enumerate(contrib):
            if rank[q][kv] != r:
                return "dQ order is not by step"
        for kv in range(n):
            if not live_t[q][kv] and rank[q][kv] is not None:
                return "rank for a dead pair"
        if dynamic:
            for (_, kv0), (_, kv1) in zip(contrib, contrib[1:]):
                if owner[kv0] > owner[kv1]:
                    return "a wait points to a later unit under a work counter"
    return ""
