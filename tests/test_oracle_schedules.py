"""Pins for the oracle's schedules and its DAG model (CPU only).

Schedules are pinned by the properties the pages state (coverage of every
live tile pair, one KV tile's work kept together, the cyclic order of shift
scheduling, the reversed Q order of descending iteration, the pairing of
symmetric shift, conflict-free steps) and by the golden fixtures under
tests/golden/.  The DAG model is pinned by closed forms derived by hand from
the model (uniform costs, one head, one slot per unit), by its own event
simulation, and by Lemma 1 on random graphs.
"""
import os
import random

import pytest

from oracle import dag as G
from oracle import schedules as S

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _check_common(schedule, n, causal):
    us = S.units(schedule, n, causal)
    seen = [(kv, q) for items in us for kv, q in items]
    want = [(kv, q) for kv in range(n) for q in range(n) if S.live(kv, q, causal)]
    assert sorted(seen) == sorted(want), "every live pair exactly once"
    assert len(seen) == len(set(seen))
    for items in us:
        kvs = [kv for kv, _ in items]
        # a KV tile's items are contiguous within the unit
        changes = sum(1 for a, b in zip(kvs, kvs[1:]) if a != b)
        assert changes == len(set(kvs)) - 1
    ranks = S.rank_table(schedule, n, causal)
    if ranks is not None:
        for q in range(n):
            rs = sorted(ranks[q][kv] for kv in range(n) if ranks[q][kv] is not None)
            assert rs == list(range(S.contributors(n, causal, q)))
    return us, ranks


@pytest.mark.parametrize("n", [1, 2, 3, 4, 7, 8, 16, 32])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("schedule", [S.NAIVE, S.DESCENDING, S.ATOMIC])
def test_one_tile_schedules(schedule, n, causal):
    us, ranks = _check_common(schedule, n, causal)
    assert len(us) == n
    for kv, items in enumerate(us):
        qs = [q for _, q in items]
        assert all(k == kv for k, _ in items)
        if schedule == S.DESCENDING:
            assert qs == sorted(qs, reverse=True)
        else:
            assert qs == sorted(qs)
    if ranks is not None:
        for q in range(n):
            order = sorted((ranks[q][kv], kv) for kv in range(n) if ranks[q][kv] is not None)
            assert [kv for _, kv in order] == sorted(kv for _, kv in order)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 8, 32, 128])
def test_shift_full(n):
    us, ranks = _check_common(S.SHIFT, n, False)
    for i, items in enumerate(us):
        assert [q for _, q in items] == [(i + t) % n for t in range(n)]
    for t in range(n):
        qs = [items[t][1] for items in us]
        assert len(set(qs)) == n, "no two units on one Q block at one step"
    for i, items in enumerate(us):
        for t, (kv, q) in enumerate(items):
            assert ranks[q][kv] == (q - kv) % n


def test_shift_full_golden():
    gold = [[int(x) for x in row] for row in _read_golden("shift_full_n4.txt")]
    us = S.units(S.SHIFT, 4, False)
    assert [[q for _, q in items] for items in us] == gold


@pytest.mark.parametrize("n", [2, 4, 6, 8, 16, 32, 64, 128])
def test_symmetric_shift(n):
    us, ranks = _check_common(S.SHIFT, n, True)
    assert len(us) == n // 2
    for w, items in enumerate(us):
        assert len(items) == n + 1, "triangle folded into a balanced rectangle"
        kvs = [kv for kv, _ in items]
        assert set(kvs) == {w, n - 1 - w}
        first = kvs.index(n - 1 - w)
        assert all(k == w for k in kvs[:first]) and all(k == n - 1 - w for k in kvs[first:])
        # phase 1: the dense lower-left square
        h = n // 2
        assert sorted(q for _, q in items[:h]) == list(range(h, n))
    for t in range(n + 1):
        qs = [items[t][1] for items in us]
        assert len(set(qs)) == len(qs), "conflict-free steps"


def test_symmetric_shift_golden():
    rows = _read_golden("symmetric_shift_n4.txt")
    gold = [[tuple(int(v) for v in it.split(":")) for it in row] for row in rows]
    assert S.units(S.SHIFT, 4, True) == gold
    ranks = S.rank_table(S.SHIFT, 4, True)
    order = {q: [kv for _, kv in sorted((ranks[q][kv], kv) for kv in range(4)
                                         if ranks[q][kv] is not None)] for q in range(4)}
    assert order == {0: [0], 1: [1, 0], 2: [0, 1, 2], 3: [1, 0, 2, 3]}


def test_symmetric_shift_odd_unsupported():
    with pytest.raises(ValueError):
        S.units(S.SHIFT, 5, True)


# ---------------------------------------------------------------- DAG model

COST = (3.0, 2.0, 1.0, 0.0)  # c_full, c_diag, r, h


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16])
def test_closed_form_naive_full(n):
    c, r = 3.0, 1.0
    mk, wait, idle, lb = G.predict(S.NAIVE, n, False, 1, n, (c, c, r, 0.0))
    assert mk == n * (c + r) + (n - 1) * r
    assert lb == n * (c + r)


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16])
def test_closed_form_shift_full(n):
    c, r = 3.0, 1.0
    mk, wait, idle, lb = G.predict(S.SHIFT, n, False, 1, n, (c, c, r, 0.0))
    assert mk == n * (c + r) == lb
    assert wait == 0.0


@pytest.mark.parametrize("n", [2, 4, 8, 16])
def test_closed_form_causal_naive_and_descending(n):
    c, r = 3.0, 1.0
    cost = (c, c, r, 0.0)
    g = G.realize(S.NAIVE, n, True, 1, n, cost)
    _, fin = G.longest_path(g["weights"], g["edges"])
    # unit i (KV tile i) ends at n(c+r) + i*r under the ascending baseline
    for u, items in enumerate(g["units"]):
        last_r = max(i for i in range(len(fin)) if i % 2 == 1 and _unit_of(g, i) == u)
        assert fin[last_r] == n * (c + r) + u * r
    g = G.realize(S.DESCENDING, n, True, 1, n, cost)
    _, fin = G.longest_path(g["weights"], g["edges"])
    # descending: unit i ends at n(c+r) - i*c, so late KV tiles free early
    for u, items in enumerate(g["units"]):
        last_r = max(i for i in range(len(fin)) if i % 2 == 1 and _unit_of(g, i) == u)
        assert fin[last_r] == n * (c + r) - u * c


def _unit_of(g, node):
    item = node // 2
    acc = 0
    for u, items in enumerate(g["units"]):
        if item < acc + len(items):
            return u
        acc += len(items)
    raise IndexError


@pytest.mark.parametrize("n", [2, 4, 8, 16])
def test_closed_form_symmetric_shift(n):
    c, r = 3.0, 1.0
    mk, wait, idle, lb = G.predict(S.SHIFT, n, True, 1, n // 2, (c, c, r, 0.0))
    assert mk == (n + 1) * (c + r) == lb
    assert wait == 0.0


def test_atomic_has_no_order_edges():
    mk, wait, idle, lb = G.predict(S.ATOMIC, 8, False, 1, 8, (3.0, 3.0, 1.0, 5.0))
    assert mk == 8 * 4.0 and wait == 0.0


@pytest.mark.parametrize("schedule", [S.NAIVE, S.DESCENDING, S.ATOMIC])
@pytest.mark.parametrize("causal", [False, True])
def test_dynamic_simulation_equals_longest_path(schedule, causal):
    for heads, slots, n in ((3, 5, 4), (4, 7, 8), (2, 16, 8)):
        cost = (2.5, 1.5, 0.75, 0.25)
        g = G.realize(schedule, n, causal, heads, slots, cost)
        _, fin = G.longest_path(g["weights"], g["edges"])
        assert abs(max(fin) - g["sim_finish"]) < 1e-9


def test_static_policy_needs_whole_head():
    with pytest.raises(ValueError):
        G.realize(S.SHIFT, 8, False, 2, 7, COST)


def test_cycle_rejected():
    with pytest.raises(ValueError):
        G.longest_path([1.0, 1.0, 1.0], [(0, 1, 0.0), (1, 2, 0.0), (2, 0, 0.0)])


def _latest_start(weights, edges, makespan, finish):
    succ = [[] for _ in weights]
    for u, v, lat in edges:
        succ[u].append((v, lat))
    # reverse topological order via decreasing earliest finish is not safe in
    # general; iterate to a fixed point instead (small graphs only)
    ls = [makespan - w for w in weights]
    changed = True
    while changed:
        changed = False
        for u in range(len(weights)):
            for v, lat in succ[u]:
                cand = ls[v] - lat - weights[u]
                if cand < ls[u]:
                    ls[u] = cand
                    changed = True
    return ls


def test_lemma1_on_random_dags():
    """Adding a zero-weight edge u -> v keeps the critical path exactly when
    finish(u) <= latest start(v); finish(u) <= earliest start(v) is the
    sufficient form used by the schedules (rank by step)."""
    rnd = random.Random(5)
    checked_pos = checked_neg = 0
    for _ in range(300):
        n = rnd.randint(3, 12)
        weights = [float(rnd.randint(1, 5)) for _ in range(n)]
        edges = [(u, v, 0.0) for u in range(n) for v in range(u + 1, n) if rnd.random() < 0.3]
        start, finish = G.longest_path(weights, edges)
        mk = max(finish)
        ls = _latest_start(weights, edges, mk, finish)
        u, v = sorted(rnd.sample(range(n), 2))
        cond, preserved = G.lemma1_preserves(weights, edges, u, v)
        assert preserved == (finish[u] <= ls[v])
        if cond:
            assert preserved
            checked_pos += 1
        else:
            checked_neg += 1
    assert checked_pos > 20 and checked_neg > 20
