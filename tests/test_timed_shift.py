"""Pins of the timed shift (SHIFT on window and block masks) and of the
work-counter condition under which its tables cannot deadlock (CPU only).

The oracle's construction (oracle/schedules.py timed_shift) is pinned to
a hand-worked case (tests/golden/timed_shift_n5.txt), to the pages' cyclic
shift (a full mask with a slot per tile), to a closed form on the causal
triangle, and to its timing certificate on random masks.  The deadlock
condition W >= (s - 1) h + 1 is checked by executing tables with random
item durations under a work counter (oracle run_counter) in head-major,
unit-major and random head interleavings, and shown to matter by a case
that deadlocks with fewer workgroups.  The library's tables equal the
oracle's for random masks, slot counts and head counts, and the oracle's
DAG model refuses tables run on too few slots.
"""
import os
import random

import numpy as np
import pytest

import deterministic_attention_backward_attn_amd as D
from oracle import dag as OD
from oracle import schedules as OS

GOLD = os.path.join(os.path.dirname(__file__), "golden", "timed_shift_n5.txt")


def _golden():
    g = {"live": {}, "units": [], "order": {}}
    for line in open(GOLD):
        w = line.split()
        if not w or w[0].startswith("#"):
            continue
        if w[0] == "n":
            g["n"] = int(w[1])
        elif w[0] == "live":
            g["live"][int(w[1])] = [int(x) for x in w[2:]]
        elif w[0] == "slots":
            g["slots"] = int(w[1])
        elif w[0] == "unit":
            kv = int(w[1])
            start = int(w[3])
            items = [tuple(int(y) for y in x.split("@")) for x in w[5:]]
            g["units"].append((kv, start, items))
        elif w[0] == "order":
            g["order"][int(w[1])] = [int(x) for x in w[2:]]
        elif w[0] == "deadlock_workgroups":
            g["deadlock"] = int(w[1])
    n = g["n"]
    live = [[q in g["live"].get(kv, []) for kv in range(n)] for q in range(n)]
    return g, live


def test_golden_worked_example():
    g, live = _golden()
    units, steps, rank, starts = OS.timed_shift(live, g["slots"])
    assert [u[0][0] for u in units] == [kv for kv, _, _ in g["units"]]
    assert starts == [s for _, s, _ in g["units"]]
    for (kv, _, items), u, st in zip(g["units"], units, steps):
        assert [(q, s) for (_, q), s in zip(u, st)] == items
    for q, kvs in g["order"].items():
        assert [kv for kv in sorted(range(g["n"]), key=lambda k: (rank[q][k] is None, rank[q][k]))
                if rank[q][kv] is not None] == kvs
    assert OS.check_timed_schedule(live, units, steps, rank, starts, g["slots"]) == ""
    one = lambda h, u, i: 1.0  # noqa: E731
    assert OS.run_counter(units, rank, 1, g["deadlock"], one) is None
    assert OS.run_counter(units, rank, 1, g["deadlock"] + 1, one) is not None


def test_golden_through_the_library():
    """The same mask as a block mask (block = tile): with 16 co-resident
    workgroups and one head the library times it on 2 slots per head
    (min of 16 device-wide and 16 / 8 in XCD groups) and builds the
    hand-worked tables."""
    g, live = _golden()
    n = g["n"]
    block = np.array([[1 if live[q][kv] else 0 for kv in range(n)] for q in range(n)], np.uint8)
    t = D.mask_schedule_tables(1, 1, 64 * n, 64, "f32", False, "shift", block_mask=block,
                               block_size=64, slots=16)
    assert t["slots_per_head"] == g["slots"] and not t["static"]
    for (kv, _, items), u, st in zip(g["units"], t["units"], t["steps"]):
        assert [(q, s) for (_, q), s in zip(u, st)] == items and all(k == kv for k, _ in u)


@pytest.mark.parametrize("n", [1, 2, 5, 8, 13])
def test_full_mask_with_a_slot_per_tile_is_the_cyclic_shift(n):
    live = [[True] * n for _ in range(n)]
    units, steps, rank, starts = OS.timed_shift(live, n)
    assert units == OS.units(OS.SHIFT, n, False)
    assert rank == OS.rank_table(OS.SHIFT, n, False)
    assert starts == [0] * n and all(st == list(range(n)) for st in steps)


@pytest.mark.parametrize("n", [2, 6, 9])
def test_full_block_mask_through_the_library_is_the_pages_shift(n):
    """An all-ones block mask (the full mask spelled as a block mask) with a
    slot per tile gives the pages' cyclic shift, item for item."""
    block = np.ones((n, n), np.uint8)
    t = D.mask_schedule_tables(1, 1, 64 * n, 64, "f32", False, "shift", block_mask=block,
                               block_size=64, slots=8 * n)
    units, rank = D.schedule_tables(n, False, "shift")
    assert t["units"] == units and np.array_equal(t["rank"], rank)


@pytest.mark.parametrize("n", [1, 4, 7])
def test_causal_triangle_closed_form(n):
    """Causal triangle, a slot per tile: unit kv walks kv, kv+1, ..., n-1
    from step 0, and block q's contributors come nearest first (rank q-kv)."""
    live = [[kv <= q for kv in range(n)] for q in range(n)]
    units, steps, rank, starts = OS.timed_shift(live, n)
    assert units == [[(kv, q) for q in range(kv, n)] for kv in range(n)]
    assert starts == [0] * n
    for q in range(n):
        for kv in range(n):
            assert rank[q][kv] == (q - kv if kv <= q else None)


def _random_live(rng, n, p, causal):
    return [[(rng.random() < p) and (kv <= q or not causal) for kv in range(n)]
            for q in range(n)]


def test_certificate_on_random_masks():
    rng = random.Random(11)
    for _ in range(60):
        n = rng.randint(1, 12)
        live = _random_live(rng, n, rng.choice([0.2, 0.5, 0.9]), rng.random() < 0.5)
        s = rng.randint(1, n + 1)
        units, steps, rank, starts = OS.timed_shift(live, s)
        assert OS.check_timed_schedule(live, units, steps, rank, starts, s) == ""


def test_counter_never_deadlocks_with_enough_workgroups():
    """Tables timed on s slots per head, h heads, W = (s - 1) h + 1
    workgroups: every head interleaving and random durations finish."""
    rng = random.Random(5)
    for trial in range(80):
        n = rng.randint(2, 9)
        live = _random_live(rng, n, rng.choice([0.3, 0.6, 1.0]), rng.random() < 0.5)
        if not any(any(r) for r in live):
            continue
        s = rng.randint(1, 5)
        h = rng.randint(1, 3)
        units, steps, rank, starts = OS.timed_shift(live, s)
        W = (s - 1) * h + 1
        seqs = ["head", "unit"]
        mixed = [(hd, u) for hd in range(h) for u in range(len(units))]
        # a random interleaving that keeps each head's own unit order
        heads_left = {hd: list(range(len(units))) for hd in range(h)}
        order = []
        while any(heads_left.values()):
            hd = rng.choice([x for x in heads_left if heads_left[x]])
            order.append((hd, heads_left[hd].pop(0)))
        seqs.append(order)
        assert len(order) == len(mixed)
        for seq in seqs:
            dur = {}
            f = lambda hd, u, i: dur.setdefault((hd, u, i), rng.uniform(0.2, 3.0))  # noqa: E731
            assert OS.run_counter(units, rank, h, W, f, seq) is not None, (trial, seq)


def test_fewer_workgroups_can_deadlock():
    """The condition matters: among random masks some deadlock with one
    workgroup fewer than (s - 1) h + 1 (so the check above is not vacuous)."""
    rng = random.Random(8)
    found = 0
    for _ in range(200):
        n = rng.randint(3, 8)
        live = _random_live(rng, n, 0.5, False)
        s, h = rng.randint(2, 4), rng.randint(1, 2)
        units, steps, rank, starts = OS.timed_shift(live, s)
        if not units:
            continue
        W = (s - 1) * h
        if OS.run_counter(units, rank, h, W, lambda hd, u, i: 1.0) is None:
            found += 1
    assert found > 0


def test_timed_slots_is_the_largest_safe_count():
    rng = random.Random(3)
    for _ in range(300):
        maxco = rng.randint(1, 600)
        heads = rng.randint(1, 300)
        units = rng.randint(1, 200)
        s = OS.timed_slots(maxco, heads, units)
        assert 1 <= s <= units
        grid = min(maxco, heads * units)
        ok = lambda x: ((x - 1) * heads + 1 <= grid and  # noqa: E731
                        (maxco // 8 < 1 or (x - 1) * -(-heads // 8) + 1 <= maxco // 8))
        if s > 1 or ok(1):
            assert ok(s)
        if s < units:
            assert not ok(s + 1)


@pytest.mark.parametrize("seed", range(6))
def test_library_tables_equal_the_oracle(seed):
    """Random block masks, workgroup and head counts: the library's timed
    shift (through the C ABI) equals the oracle's for the slot count the
    oracle's timed_slots gives."""
    rng = np.random.default_rng(100 + seed)
    nb = int(rng.integers(2, 12))
    causal = bool(seed % 2)
    block = (rng.random((nb, nb)) < rng.choice([0.3, 0.6])).astype(np.uint8)
    block[0, 0] = 1
    maxco = int(rng.choice([8, 16, 40, 256]))
    B, H = 1, int(rng.integers(1, 20))
    t = D.mask_schedule_tables(B, H, 64 * nb, 64, "f32", causal, "shift", block_mask=block,
                               block_size=64, slots=maxco)
    live = [[bool(block[q, kv]) and (kv <= q or not causal) for kv in range(nb)]
            for q in range(nb)]
    n_units = sum(1 for kv in range(nb) if any(live[q][kv] for q in range(nb)))
    s = OS.timed_slots(maxco, B * H, n_units)
    assert t["slots_per_head"] == s
    units, steps, rank, starts = OS.timed_shift(live, s)
    assert t["units"] == units and t["steps"] == steps
    assert np.array_equal(t["rank"], np.array([[-1 if x is None else x for x in r] for r in rank]))


def test_dag_model_reports_a_deadlock():
    """The golden tables on one slot: the oracle's DAG realization refuses
    (the work counter would deadlock); on two it runs."""
    g, live = _golden()
    units, steps, rank, starts = OS.timed_shift(live, g["slots"])
    tables = {"units": units, "rank": rank, "partial": set(), "static": False}
    with pytest.raises(ValueError):
        OD.predict(OS.SHIFT, g["n"], False, 1, 1, (1.0, 0.5, 0.1, 0.1), tables)
    assert OD.predict(OS.SHIFT, g["n"], False, 1, 2, (1.0, 0.5, 0.1, 0.1), tables)[0] > 0


@pytest.mark.parametrize("schedule", ["naive", "descending", "shift", "atomic"])
def test_mask_with_no_live_pair(schedule):
    """A block mask that hides everything: no unit, nothing timed."""
    t = D.mask_schedule_tables(1, 2, 256, 64, "f32", True, schedule,
                               block_mask=np.zeros((4, 4), np.uint8), block_size=64)
    assert t["units"] == [] and t["slots_per_head"] == 0 and not t["static"]
    assert OS.timed_shift([[False] * 4 for _ in range(4)], 3)[0] == []


@pytest.mark.parametrize("schedule", ["naive", "descending", "shift"])
def test_launch_prediction_of_a_mask_with_no_live_pair(schedule):
    """AUTO predicts every candidate under the launch's placement; with no
    live pair the prediction is an empty launch, not an error."""
    r, info = D.bwd_predict(1, 2, 256, 64, "f32", True, schedule, slots=256,
                            cost=(1.0, 0.5, 0.05, 0.05),
                            block_mask=np.zeros((4, 4), np.uint8), block_size=64)
    assert r == (0.0, 0.0, 0.0, 0.0)
