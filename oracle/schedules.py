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
# live Q blocks ascending / descending, dQ order ascending kv.
#
# SHIFT on such a mask is a *timed shift* (``timed_shift``): the pages'
# defining property - units running side by side touch distinct Q blocks,
# and a block's dQ order is the order in which units reach it - kept by
# simulating, step by step, a number of workgroup slots running one head's
# units, and taking the dQ orders from that simulated timing.  The pages'
# full-mask shift is the special case of a full mask with a slot per tile.
# Tables built that way may make a unit wait for one handed out later, so
# they carry a slot count; ``timed_slots`` and ``run_counter`` give and
# check the number of workgroups under which a work counter cannot
# deadlock on them.


def timed_shift(live_t, slots):
    """Timed shift of one head on `slots` workgroup slots.

    Units: one per KV tile with live pairs, started longest first (ties: the
    lower KV tile), each as soon as a slot is free (at step 0 the first
    `slots`; a unit that takes its last block at step t frees its slot for
    step t + 1).  At every step the running units, in start order, each
    take the one of their remaining Q blocks that no other unit has taken at
    this step and that comes first going up cyclically from the unit's own
    diagonal, i.e. with the smallest (q - kv) mod n; a unit with every
    remaining block taken idles for the step.

    Returns (units, steps, rank, starts): per unit in start order its items
    [(kv, q), ...] in step order and their steps, rank[q][kv] = the
    position of kv's step among the block's steps (None where dead), and
    the step at which each unit took its slot (a unit whose blocks are all
    taken when it starts idles, so its first item can come later)."""
    n = len(live_t)
    if slots < 1:
        raise ValueError("slots must be >= 1")
    blocks = {kv: [q for q in range(n) if live_t[q][kv]] for kv in range(n)}
    order = sorted((kv for kv in range(n) if blocks[kv]), key=lambda kv: (-len(blocks[kv]), kv))
    remaining = {kv: set(blocks[kv]) for kv in order}
    got = {kv: [] for kv in order}
    start = {}
    running, started, step = [], 0, 0
    while started < len(order) or running:
        while len(running) < slots and started < len(order):
            start[order[started]] = step
            running.append(order[started])
            started += 1
        taken = set()
        for kv in running:
            free = [q for q in remaining[kv] if q not in taken]
            if free:
                q = min(free, key=lambda q: (q - kv) % n)
                taken.add(q)
                remaining[kv].remove(q)
                got[kv].append((step, q))
        running = [kv for kv in running if remaining[kv]]
        step += 1
    units_out = [[(kv, q) for _, q in got[kv]] for kv in order]
    steps_out = [[st for st, _ in got[kv]] for kv in order]
    rank = [[None] * n for _ in range(n)]
    for q in range(n):
        by_step = sorted((st, kv) for kv in order for st, qq in got[kv] if qq == q)
        for r, (_, kv) in enumerate(by_step):
            rank[q][kv] = r
    return units_out, steps_out, rank, [start[kv] for kv in order]


def timed_slots(maxco, heads, n_units):
    """Slots per head of the timed shift for a launch on `maxco` co-resident
    workgroups and `heads` heads of `n_units` units: the largest s with
    (s - 1) * h + 1 workgroups available both in 8 XCD groups (maxco // 8
    workgroups, h = ceil(heads / 8)) and device-wide (min(maxco,
    heads * n_units) workgroups, h = heads), at most n_units, at least 1."""
    if maxco < 1 or heads < 1 or n_units < 1:
        return 1
    grid = min(maxco, heads * n_units)
    s = (grid - 1) // heads + 1
    g = maxco // 8
    if g >= 1:
        s = min(s, (g - 1) // -(-heads // 8) + 1)
    return max(1, min(s, n_units))


def run_counter(units, rank, heads, workgroups, durations, order="head"):
    """Executes tables under a work counter, one event at a time, with no
    model of time beyond the given durations: `workgroups` workers take
    units from a counter (head-major: head 0's units in list order, then
    head 1's ...; "unit": unit 0 of every head, then unit 1, ...; or an
    explicit list of (head, unit)), run their items in list order, and an
    item's dQ add waits until the block's previous contributor (by rank)
    of the same head has added.  durations(head, unit, item) > 0 is each
    item's compute time.  Returns the finish time, or None when every
    worker is stuck waiting (a deadlock)."""
    n = len(rank)
    if order == "head":
        seq = [(h, u) for h in range(heads) for u in range(len(units))]
    elif order == "unit":
        seq = [(h, u) for u in range(len(units)) for h in range(heads)]
    else:
        seq = list(order)
    prev = {}
    for q in range(n):
        chain = sorted((rank[q][kv], kv) for kv in range(n) if rank[q][kv] is not None)
        for (_, a), (_, b) in zip(chain, chain[1:]):
            prev[(b, q)] = a
    added = {}                       # (head, kv, q) -> time its add finished
    work = [None] * workgroups       # [head, unit, item index, clock] per worker
    nxt = 0
    clock = 0.0
    for w in range(workgroups):
        if nxt < len(seq):
            work[w] = [seq[nxt][0], seq[nxt][1], 0, 0.0]
            nxt += 1
    while any(x is not None for x in work):
        # the worker whose next add can happen earliest goes first
        best = None
        for w, x in enumerate(work):
            if x is None:
                continue
            h, u, i, t = x
            kv, q = units[u][i]
            ready = t + durations(h, u, i)
            p = prev.get((kv, q))
            if p is not None:
                if (h, p, q) not in added:
                    continue
                ready = max(ready, added[(h, p, q)])
            if best is None or (ready, w) < best[:2]:
                best = (ready, w)
        if best is None:
            return None
        t_add, w = best
        h, u, i, _ = work[w]
        kv, q = units[u][i]
        added[(h, kv, q)] = t_add
        clock = max(clock, t_add)
        if i + 1 < len(units[u]):
            work[w] = [h, u, i + 1, t_add]
        elif nxt < len(seq):
            work[w] = [seq[nxt][0], seq[nxt][1], 0, t_add]
            nxt += 1
        else:
            work[w] = None
    return clock


def check_timed_schedule(live_t, unit_items, steps, rank, starts, slots):
    """The timing certificate of a timed shift: every live pair once, a KV
    tile in one unit, steps increasing within a unit and distinct within a
    Q block, dQ orders by step, units listed in the order of their start
    steps, no item before its unit's start, and at most `slots` units
    between their start and their last step at any step.  Returns '' or
    the first rule broken."""
    n = len(live_t)
    seen, owner = {}, {}
    for u, (items, st) in enumerate(zip(unit_items, steps)):
        if not items or len(items) != len(st):
            return "empty unit or steps do not match items"
        if any(b <= a for a, b in zip(st, st[1:])):
            return "steps not increasing within a unit"
        for (kv, q), s in zip(items, st):
            if not (0 <= kv < n and 0 <= q < n) or not live_t[q][kv]:
                return "dead or out-of-range pair"
            if (kv, q) in seen:
                return "pair twice"
            if owner.setdefault(kv, u) != u:
                return "KV tile in two units"
            seen[(kv, q)] = s
    if len(seen) != sum(sum(1 for x in row if x) for row in live_t):
        return "live pair missing"
    if len(starts) != len(steps):
        return "starts do not match units"
    if any(st[0] < s0 for st, s0 in zip(steps, starts)):
        return "item before its unit's start"
    if any(b < a for a, b in zip(starts, starts[1:])):
        return "units not in start order"
    last = max((st[-1] for st in steps), default=-1)
    for t in range(last + 1):
        if sum(1 for st, s0 in zip(steps, starts) if s0 <= t <= st[-1]) > slots:
            return "more units running than slots"
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
    return ""


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
