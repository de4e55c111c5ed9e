"""Pins for the oracle's masked tables and its DAG model on explicit tables
and in unit-major order (CPU only).

Each pin compares the oracle with something other than itself:
* ``masked_units`` / ``masked_rank_table`` on the plain full and causal
  liveness equal ``units`` / ``rank_table``, which the schedule tests pin
  by the pages' stated properties and the golden files;
* tile liveness, the naive / descending unit lists and the dQ orders of
  three sliding windows equal lists worked by hand
  (tests/golden/window_tables_n4.txt: DASH summary, "Limitations and future
  work", under readings R20 and R21);
* ``predict`` with explicit ``tables=`` reproduces makespans derived by hand
  for a causal window (naive: a chain through every Q block; descending:
  two items per unit), and the closed forms of the plain causal schedules
  when the plain tables are passed explicitly;
* ``realize(unit_major=True)`` reproduces a makespan derived by hand
  (H heads of n equal units on H slots) that differs from head-major order;
* the event simulation equals the longest path with ``tables=`` and in
  unit-major order.
Planted mistakes (a transposed liveness index, unit-major order ignored,
partial pairs costed as full) are applied to copies of the oracle functions
here and must fail these pins.
"""
import os

import pytest

from oracle import attention as A
from oracle import dag as G
from oracle import schedules as S

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------- plain liveness reduces

def _plain_live(n, causal):
    return [[S.live(kv, q, causal) for kv in range(n)] for q in range(n)]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 7, 8, 16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("schedule", [S.NAIVE, S.DESCENDING, S.ATOMIC])
def test_masked_units_on_plain_liveness_equal_units(schedule, n, causal):
    live_t = _plain_live(n, causal)
    assert S.masked_units(schedule, live_t) == S.units(schedule, n, causal)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 7, 8, 16])
@pytest.mark.parametrize("causal", [False, True])
def test_masked_rank_on_plain_liveness_equals_rank_table(n, causal):
    live_t = _plain_live(n, causal)
    want = S.rank_table(S.NAIVE, n, causal)
    assert S.masked_rank_table(live_t) == want
    assert S.rank_table(S.DESCENDING, n, causal) == want


@pytest.mark.parametrize("causal", [False, True])
def test_plain_tile_liveness_from_the_element_mask(causal):
    n, tile = 5, 3
    live_t, part_t = S.tile_liveness(A.Mask(causal=causal), n, tile)
    assert live_t == _plain_live(n, causal)
    # causal: exactly the diagonal pairs hide elements; full: none
    assert part_t == [[causal and kv == q for kv in range(n)] for q in range(n)]


# ------------------------------------------------ hand-worked windows

def _golden_cases():
    cases = {}
    cur = None
    with open(os.path.join(GOLD, "window_tables_n4.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tok = line.split()
            if tok[0] == "case":
                kv = dict(t.split("=") for t in tok[2:])
                cur = {"causal": kv["causal"] == "1", "window": int(kv["window"]),
                       "tile": int(kv["tile"]), "n": int(kv["n"]),
                       "live": {}, "naive": {}, "descending": {}, "order": {}}
                cases[tok[1]] = cur
            elif tok[0] == "live":
                cur["live"][int(tok[1])] = [(int(t[:-1]), t[-1]) for t in tok[2:]]
            else:
                cur[tok[0]][int(tok[1])] = [int(t) for t in tok[2:]]
    return cases


CASES = _golden_cases()


def _check_window_case(case, tile_liveness, masked_units, masked_rank_table):
    """'' if the functions reproduce the hand-worked case, else what differs."""
    n = case["n"]
    m = A.Mask(causal=case["causal"], window=case["window"])
    live_t, part_t = tile_liveness(m, n, case["tile"])
    for q in range(n):
        got = [(kv, "p" if part_t[q][kv] else "f") for kv in range(n) if live_t[q][kv]]
        if got != case["live"].get(q, []):
            return f"liveness of Q block {q}"
    for sched in (S.NAIVE, S.DESCENDING):
        us = masked_units(sched, live_t)
        for kv in range(n):
            got = [q for k, q in us[kv]]
            if any(k != kv for k, _ in us[kv]) or got != case[sched].get(kv, []):
                return f"{sched} unit of KV tile {kv}"
    rank = masked_rank_table(live_t)
    for q in range(n):
        order = sorted((rank[q][kv], kv) for kv in range(n) if rank[q][kv] is not None)
        if [kv for _, kv in order] != case["order"].get(q, []):
            return f"dQ order of Q block {q}"
    return ""


@pytest.mark.parametrize("name", sorted(CASES))
def test_window_tables_match_hand_worked_lists(name):
    assert CASES, "golden file parsed"
    assert _check_window_case(CASES[name], S.tile_liveness, S.masked_units,
                              S.masked_rank_table) == ""


def _masked_units_transposed(schedule, live_t):
    # planted mistake: reads live_t[kv][q] instead of live_t[q][kv]
    n = len(live_t)
    order = range(n) if schedule != S.DESCENDING else reversed(range(n))
    return [[(kv, q) for q in order if live_t[kv][q]] for kv in range(n)]


def _rank_transposed(live_t):
    n = len(live_t)
    return S.masked_rank_table([[live_t[kv][q] for kv in range(n)] for q in range(n)])


def _liveness_wrong_partial(mask, n_tiles, tile):
    # planted mistake: the diagonal always counted as partial, nothing else
    live_t, _ = S.tile_liveness(mask, n_tiles, tile)
    return live_t, [[live_t[q][kv] and q == kv for kv in range(n_tiles)] for q in range(n_tiles)]


def test_planted_table_mistakes_fail_the_window_pins():
    for name, case in CASES.items():
        if case["causal"]:
            assert _check_window_case(case, S.tile_liveness, _masked_units_transposed,
                                      S.masked_rank_table) != "", name
            assert _check_window_case(case, S.tile_liveness, S.masked_units,
                                      _rank_transposed) != "", name
    assert any(_check_window_case(c, _liveness_wrong_partial, S.masked_units,
                                  S.masked_rank_table) != "" for c in CASES.values())


# ------------------------------------------- DAG model on explicit tables

def _tables_from_golden(case, sched):
    n = case["n"]
    units = [[(kv, q) for q in case[sched].get(kv, [])] for kv in range(n)]
    rank = [[None] * n for _ in range(n)]
    for q, kvs in case["order"].items():
        for r, kv in enumerate(kvs):
            rank[q][kv] = r
    partial = {(kv, q) for q, lst in case["live"].items() for kv, f in lst if f == "p"}
    return {"units": units, "rank": rank, "partial": partial, "static": False}


# costs (c_full, c_diag, r, h); c_diag applies to partial pairs
WCOST = (5.0, 2.0, 1.0, 0.5)


def _window_makespans(predict):
    case = CASES["causal_w5"]
    out = {}
    for sched in (S.NAIVE, S.DESCENDING):
        out[sched] = predict(sched, case["n"], True, 1, case["n"], WCOST,
                             tables=_tables_from_golden(case, sched))[0]
    return out


def test_window_makespans_derived_by_hand():
    """Causal window W = T + 1, n tiles, one slot per KV tile, every live pair
    partial (cost d), add r, hand-off h (h <= d):
    naive: unit kv adds its diagonal partial only after unit kv-1 added its
    last one, so the adds form one chain through all Q blocks:
    makespan = n*d + (2n - 1)*r + (n - 1)*h.
    descending: unit kv first adds (kv, kv+1) (rank 0), then (kv, kv), whose
    predecessor (kv-1, kv) finished at d + r: makespan = 2d + 2r."""
    c, d, r, h = WCOST
    n = CASES["causal_w5"]["n"]
    got = _window_makespans(G.predict)
    assert got[S.NAIVE] == n * d + (2 * n - 1) * r + (n - 1) * h
    assert got[S.DESCENDING] == 2 * d + 2 * r


def test_planted_partial_costing_fails_the_window_makespans():
    def predict_ignoring_partial(sched, n, causal, heads, slots, cost, tables=None, unit_major=False):
        t = dict(tables)
        t["partial"] = {(kv, kv) for kv in range(n)}  # planted: diagonal only
        return G.predict(sched, n, causal, heads, slots, cost, tables=t, unit_major=unit_major)
    c, d, r, h = WCOST
    n = CASES["causal_w5"]["n"]
    got = _window_makespans(predict_ignoring_partial)
    assert got[S.DESCENDING] != 2 * d + 2 * r


@pytest.mark.parametrize("n", [2, 4, 8])
def test_plain_tables_passed_explicitly_keep_the_closed_forms(n):
    """The causal closed forms of the schedule tests (naive unit i ends at
    n(c+r) + i*r, descending at n(c+r) - i*c) through the tables= path."""
    c, r = 3.0, 1.0
    cost = (c, c, r, 0.0)
    live_t = _plain_live(n, True)
    for sched, end in ((S.NAIVE, lambda u: n * (c + r) + u * r),
                       (S.DESCENDING, lambda u: n * (c + r) - u * c)):
        tables = {"units": S.masked_units(sched, live_t), "rank": S.masked_rank_table(live_t),
                  "partial": {(kv, kv) for kv in range(n)}, "static": False}
        g = G.realize(sched, n, True, 1, n, cost, tables=tables)
        _, fin = G.longest_path(g["weights"], g["edges"])
        pos = 0
        for u, items in enumerate(g["units"]):
            pos += len(items)
            assert fin[2 * pos - 1] == end(u), (sched, u)


# ------------------------------------------------------ unit-major order

def _unit_major_makespans(realize, n, heads, c, r, h):
    out = {}
    for um in (False, True):
        g = realize(S.NAIVE, n, False, heads, heads, (c, c, r, h), unit_major=um)
        _, fin = G.longest_path(g["weights"], g["edges"])
        out[um] = max(fin)
    return out


def test_unit_major_makespan_derived_by_hand():
    """Full mask, naive order, H heads of n units, H slots, h < n(c+r) - r.
    Unit-major: round k runs unit k of every head; unit k-1 of the head has
    finished every add a whole unit earlier, so nothing waits:
    makespan = n * n(c+r).  Head-major with H = n: the first head's n units
    start together and unit kv lags unit kv-1 by r + h; every later head
    inherits that stagger without further waits:
    makespan = H * n(c+r) + (n - 1)(r + h)."""
    n, c, r, h = 4, 3.0, 1.0, 0.5
    got = _unit_major_makespans(G.realize, n, n, c, r, h)
    assert got[True] == n * n * (c + r)
    assert got[False] == n * n * (c + r) + (n - 1) * (r + h)


def test_planted_unit_order_mistake_fails_the_unit_major_pin():
    def realize_ignoring_order(*args, unit_major=False, **kw):
        return G.realize(*args, unit_major=False, **kw)   # planted: order ignored

    n, c, r, h = 4, 3.0, 1.0, 0.5
    got = _unit_major_makespans(realize_ignoring_order, n, n, c, r, h)
    assert got[True] != n * n * (c + r)


# ------------------------------- event simulation = longest path (extended)

@pytest.mark.parametrize("schedule", [S.NAIVE, S.DESCENDING, S.ATOMIC])
@pytest.mark.parametrize("causal", [False, True])
def test_unit_major_simulation_equals_longest_path(schedule, causal):
    for heads, slots, n in ((3, 5, 4), (4, 7, 8), (5, 3, 6)):
        cost = (2.5, 1.5, 0.75, 0.25)
        g = G.realize(schedule, n, causal, heads, slots, cost, unit_major=True)
        _, fin = G.longest_path(g["weights"], g["edges"])
        assert abs(max(fin) - g["sim_finish"]) < 1e-9


def _masked_tables(sched, mask, n, tile):
    live_t, part_t = S.tile_liveness(mask, n, tile)
    return {"units": S.masked_units(sched, live_t),
            "rank": None if sched == S.ATOMIC else S.masked_rank_table(live_t),
            "partial": {(kv, q) for q in range(n) for kv in range(n) if part_t[q][kv]},
            "static": False}


@pytest.mark.parametrize("schedule", [S.NAIVE, S.DESCENDING, S.ATOMIC])
@pytest.mark.parametrize("unit_major", [False, True])
def test_masked_tables_simulation_equals_longest_path(schedule, unit_major):
    import numpy as np
    rng = np.random.default_rng(3)
    masks = [A.Mask(causal=True, window=7), A.Mask(causal=False, window=9),
             A.Mask(causal=True, block=rng.random((4, 4)) < 0.6, block_size=8),
             A.Mask(causal=False, block=rng.random((4, 4)) < 0.4, block_size=8)]
    for m in masks:
        t = _masked_tables(schedule, m, 8, 4)
        for heads, slots in ((2, 3), (3, 8), (4, 5)):
            g = G.realize(schedule, 8, m.causal, heads, slots, (2.5, 1.5, 0.75, 0.25),
                          tables=t, unit_major=unit_major)
            _, fin = G.longest_path(g["weights"], g["edges"])
            assert abs(max(fin) - g["sim_finish"]) < 1e-9
