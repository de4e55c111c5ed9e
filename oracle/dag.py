"""Plain-Python DAG model of the deterministic backward (the oracle's copy).

TEST INFRASTRUCTURE ONLY: imported by tests, never by the product path.  The
product's C++ critical-path calculator is checked against this module.

The model is the one the explainer sets up ("Technisches Resuemee" 2.1) and
the authors' abstract names: the backward pass of deterministic attention
is a directed acyclic graph whose nodes are compute phases (one KV tile
meeting one Q block) and reduction phases (adding that item's dQ partial into
the Q block's accumulator); edges are data dependencies plus the mandatory
accumulation order; the quantity to minimise is the length of the critical
path; and the work of one KV tile runs as one uninterrupted chain on one
processor.  Concretely, for a launch with P processor slots:

* item (kv, q) of a unit gives two nodes, C (weight c_diag on a causal
  diagonal item, else c_full) and R (weight r), with edge C -> R;
* consecutive items of a unit are chained R -> C, and consecutive units on
  one slot are chained last R -> first C;
* for a deterministic schedule, R of the contributor ranked k-1 for Q block
  q precedes R of the contributor ranked k, with latency h (the hand-off);
* start(x) = max over in-edges (finish(pred) + latency), finish = start +
  weight; the makespan is the largest finish (the critical-path length).

Slots take units in one of two ways (this project's reading of how a
persistent grid runs the explainer's "one KV tile per SM" chains):
* "dynamic": units in head-major order go to whichever slot frees first
  (ties to the lowest slot), an add waiting for its block's previous
  contributor even when that one's unit was handed out later - used for
  NAIVE, DESCENDING, ATOMIC and the timed shift of window and block masks;
* "static": head-aligned rounds, slot = u mod P' with P' the largest
  multiple of the units per head not above P - used for the pages' SHIFT
  on the full and causal masks, whose order edges point to later units of
  the same head.

Lemma 1 of the explainer (2.2 B): adding a zero-weight edge u -> v keeps the
critical path when depth(u) <= depth(v).  Read with depth(u) = earliest
finish of u and depth(v) = earliest start of v, this is checked by
``lemma1_preserves``.
"""
from __future__ import annotations

from . import schedules as S


def item_cost(kv, q, causal, cost):
    c_full, c_diag = cost[0], cost[1]
    return c_diag if (causal and kv == q) else c_full


def longest_path(weights, edges):
    """weights: list of node weights; edges: list of (u, v, latency).

    Returns (start, finish) lists, or raises ValueError on a cycle.
    Plain Kahn topological order, then one relaxation pass.
    """
    n = len(weights)
    succ = [[] for _ in range(n)]
    indeg = [0] * n
    for u, v, lat in edges:
        succ[u].append((v, lat))
        indeg[v] += 1
    order = [i for i in range(n) if indeg[i] == 0]
    head = 0
    while head < len(order):
        u = order[head]
        head += 1
        for v, _ in succ[u]:
            indeg[v] -= 1
            if indeg[v] == 0:
                order.append(v)
    if len(order) != n:
        raise ValueError("cycle in dependency graph")
    start = [0.0] * n
    finish = [0.0] * n
    for u in order:
        finish[u] = start[u] + weights[u]
        for v, lat in succ[u]:
            if finish[u] + lat > start[v]:
                start[v] = finish[u] + lat
    return start, finish


def _policy(schedule):
    return "static" if schedule == S.SHIFT else "dynamic"


def _item_costs(causal, cost, partial):
    """Compute weight of an item: c_diag on a partial item (explicit set of
    (kv, q) pairs for masked tables; the causal diagonal otherwise)."""
    if partial is None:
        return lambda kv, q: item_cost(kv, q, causal, cost)
    return lambda kv, q: cost[1] if (kv, q) in partial else cost[0]


def realize(schedule, n, causal, heads, slots, cost, tables=None, unit_major=False):
    """Assign units to slots and build the graph.

    ``unit_major`` (dynamic policy only): slots take units in the order
    unit 0 of every head, unit 1 of every head, ... instead of head after
    head (a head's own units keep their order either way).

    ``tables`` (optional) gives one head's tables explicitly, for masks the
    oracle does not construct itself: {"units": [[(kv, q), ...], ...],
    "rank": rank[q][kv] (None or negative where absent; None for ATOMIC),
    "partial": set of (kv, q) pairs costed c_diag, optional "static": whether
    the units run in head-aligned rounds (default: SHIFT only)}.

    Returns dict with 'weights', 'edges', 'assign' (unit -> slot),
    'units' (global unit list of item lists, each item (head, kv, q)) and
    for the dynamic policy the times of the event simulation used to decide
    the assignment ('sim_finish').
    """
    if tables is None:
        per_head = S.units(schedule, n, causal)
        ranks = S.rank_table(schedule, n, causal)
        icost = _item_costs(causal, cost, None)
    else:
        per_head = tables["units"]
        ranks = tables["rank"]
        if ranks is not None:
            ranks = [[None if (r is None or r < 0) else int(r) for r in row] for row in ranks]
        icost = _item_costs(causal, cost, tables["partial"])
    U = len(per_head)
    glob = []
    dynamic = (_policy(schedule) == "dynamic" if tables is None or "static" not in tables
               else not tables["static"])
    if unit_major and dynamic:
        # all heads' first units, then all heads' second units, ...
        for items in per_head:
            for hd in range(heads):
                glob.append([(hd, kv, q) for kv, q in items])
    else:
        for hd in range(heads):
            for items in per_head:
                glob.append([(hd, kv, q) for kv, q in items])
    # node ids: for unit u item k -> C = 2*idx, R = 2*idx + 1
    idx_of = {}
    weights = []
    for u, items in enumerate(glob):
        for k, (hd, kv, q) in enumerate(items):
            idx_of[(u, k)] = len(weights) // 2
            weights.append(icost(kv, q))
            weights.append(cost[2])
    r_node = {}
    for u, items in enumerate(glob):
        for k, (hd, kv, q) in enumerate(items):
            r_node[(hd, kv, q)] = 2 * idx_of[(u, k)] + 1
    order_edges = []
    if ranks is not None:
        for hd in range(heads):
            for q in range(n):
                chain = sorted((ranks[q][kv], kv) for kv in range(n) if ranks[q][kv] is not None)
                for (r0, kv0), (r1, kv1) in zip(chain, chain[1:]):
                    order_edges.append((r_node[(hd, kv0, q)], r_node[(hd, kv1, q)], cost[3]))

    policy = _policy(schedule)
    if tables is not None and "static" in tables:
        policy = "static" if tables["static"] else "dynamic"
    assign = [None] * len(glob)
    sim_finish = None
    if policy == "static":
        if U > slots:
            raise ValueError("static policy needs a whole head of units resident")
        p_eff = (slots // U) * U if U else 1
        for u in range(len(glob)):
            assign[u] = u % p_eff
    else:
        # Event simulation of the work counter: a slot that becomes free
        # takes the next unit in `glob` order; an item runs when its slot
        # reaches it, and its add waits for the block's previous
        # contributor, also when that contributor's unit was handed out
        # later (timed shift).  Events are handled in time order: an item at
        # the time its compute starts (once its predecessor's add is known),
        # a free slot at the time it frees; ties go to items, then to the
        # lower slot.
        state = [None] * slots        # [unit, item index, time] per busy slot
        free_at = [0.0] * slots       # time a free slot frees (None when busy)
        r_fin = {}
        nxt = 0
        while True:
            best = None
            for s_ in range(slots):
                if state[s_] is None:
                    if free_at[s_] is not None and nxt < len(glob):
                        key = (free_at[s_], 1, s_)
                        if best is None or key < best:
                            best = key
                    continue
                u, k, t = state[s_]
                hd, kv, q = glob[u][k]
                if ranks is not None and ranks[q][kv] > 0:
                    prev = [kv2 for kv2 in range(n) if ranks[q][kv2] == ranks[q][kv] - 1][0]
                    if (hd, prev, q) not in r_fin:
                        continue
                key = (t, 0, s_)
                if best is None or key < best:
                    best = key
            if best is None:
                break
            t, kind, s_ = best
            if kind == 1:
                assign[nxt] = s_
                state[s_] = [nxt, 0, t]
                free_at[s_] = None
                nxt += 1
                if not glob[nxt - 1]:
                    state[s_] = None
                    free_at[s_] = t
                continue
            u, k, t = state[s_]
            hd, kv, q = glob[u][k]
            t_r = t + icost(kv, q)
            if ranks is not None and ranks[q][kv] > 0:
                prev = [kv2 for kv2 in range(n) if ranks[q][kv2] == ranks[q][kv] - 1][0]
                t_r = max(t_r, r_fin[(hd, prev, q)] + cost[3])
            t = t_r + cost[2]
            r_fin[(hd, kv, q)] = t
            if k + 1 < len(glob[u]):
                state[s_] = [u, k + 1, t]
            else:
                state[s_] = None
                free_at[s_] = t
        if nxt < len(glob) or any(x is not None for x in state):
            raise ValueError("the work counter deadlocks on these tables")
        sim_finish = max(r_fin.values()) if r_fin else 0.0

    edges = list(order_edges)
    last_on_slot = {}
    for u, items in enumerate(glob):
        for k in range(len(items)):
            c_id = 2 * idx_of[(u, k)]
            edges.append((c_id, c_id + 1, 0.0))
            if k > 0:
                edges.append((2 * idx_of[(u, k - 1)] + 1, c_id, 0.0))
        s = assign[u]
        if s in last_on_slot and items:
            edges.append((last_on_slot[s], 2 * idx_of[(u, 0)], 0.0))
        if items:
            last_on_slot[s] = 2 * idx_of[(u, len(items) - 1)] + 1
    return {"weights": weights, "edges": edges, "assign": assign, "units": glob,
            "sim_finish": sim_finish, "policy": policy, "n_order": len(order_edges),
            "icost": icost}


def predict(schedule, n, causal, heads, slots, cost, tables=None, unit_major=False):
    """Returns (makespan, total_wait, max_slot_idle, lower_bound).

    total_wait: summed time R nodes spend held by their order edge beyond
    what their own chain allows; max_slot_idle: largest (makespan - busy)
    over slots; lower_bound: max(total work / slots, longest single unit)."""
    g = realize(schedule, n, causal, heads, slots, cost, tables, unit_major)
    icost = g["icost"]
    start, finish = longest_path(g["weights"], g["edges"])
    makespan = max(finish) if finish else 0.0
    # time each R node could start from its own chain alone (order edges
    # excluded); the excess of its actual start is time spent waiting
    chain_ready = [0.0] * len(g["weights"])
    for i, (u, v, lat) in enumerate(g["edges"]):
        if i >= g["n_order"]:
            chain_ready[v] = max(chain_ready[v], finish[u] + lat)
    total_wait = 0.0
    for i in range(1, len(g["weights"]), 2):
        total_wait += start[i] - chain_ready[i]
    busy = [0.0] * slots
    for u, items in enumerate(g["units"]):
        for hd, kv, q in items:
            busy[g["assign"][u]] += icost(kv, q) + cost[2]
    max_idle = max(makespan - b for b in busy) if slots else 0.0
    longest_unit = max((sum(icost(kv, q) + cost[2] for _, kv, q in items)
                        for items in g["units"]), default=0.0)
    lower = max(sum(busy) / slots, longest_unit)
    return makespan, total_wait, max_idle, lower


def lemma1_preserves(weights, edges, u, v):
    """Adds a zero-weight, zero-latency edge u -> v and reports
    (condition, preserved): condition is finish(u) <= start(v) in the
    original graph; preserved is whether the makespan is unchanged."""
    start, finish = longest_path(weights, edges)
    before = max(finish)
    start2, finish2 = longest_path(weights, edges + [(u, v, 0.0)])
    after = max(finish2)
    return finish[u] <= start[v], after == before
