"""Masked schedule tables and DAG prediction (CPU only, host calls).

The library's tables for sliding windows and block masks are checked
against the oracle: tile liveness and partial flags from the element mask
by brute force; NAIVE / DESCENDING / ATOMIC item lists and dQ orders
exactly; SHIFT (the timed shift) exactly against the oracle's own timed
shift and against the timing certificate; the DAG prediction on the
library's own tables against the oracle's DAG.
"""
import itertools

import numpy as np
import pytest

import deterministic_attention_backward_attn_amd as D
from oracle import attention as A
from oracle import dag as OD
from oracle import schedules as OS

T = 64  # fp32 tile
rng = np.random.default_rng(23)
BLOCKS = {
    "rand8": rng.random((8, 8)) < 0.55,
    "rand4": rng.random((4, 4)) < 0.7,
}
DEAD = np.ones((8, 8), dtype=bool)
DEAD[3, :] = False   # a query block that sees nothing
DEAD[:, 5] = False   # a key block no query sees
BLOCKS["dead"] = DEAD

# (N, causal, window, block name, block_size)
CASES = [
    (512, True, 100, None, 0),
    (512, True, 64, None, 0),
    (512, True, 1, None, 0),
    (512, False, 130, None, 0),
    (512, False, 0, "rand8", 64),
    (512, True, 0, "rand8", 64),
    (512, False, 0, "rand4", 128),
    (512, True, 200, "rand4", 128),
    (512, False, 0, "dead", 64),
    (512, True, 0, "dead", 64),
    (1024, True, 300, None, 0),
]


def _ids(c):
    return f"N{c[0]}_{'c' if c[1] else 'f'}_w{c[2]}_{c[3]}"


def _oracle_mask(N, causal, window, block, bs):
    return A.Mask(causal=causal, window=window,
                  block=None if block is None else BLOCKS[block], block_size=bs)


def _kw(window, block, bs):
    return dict(window=window, block_mask=None if block is None else BLOCKS[block].astype(np.uint8),
                block_size=bs)


@pytest.mark.parametrize("case", CASES, ids=_ids)
@pytest.mark.parametrize("schedule", ["naive", "descending", "atomic", "shift"])
def test_masked_tables_against_oracle(case, schedule):
    N, causal, window, block, bs = case
    n = N // T
    live, part = OS.tile_liveness(_oracle_mask(N, causal, window, block, bs), n, T)
    t = D.mask_schedule_tables(1, 1, N, 64, "f32", causal, schedule, **_kw(window, block, bs))
    assert t["n"] == n
    # partial flags
    for items, flags in zip(t["units"], t["partial"]):
        for (kv, q), f in zip(items, flags):
            assert f == part[q][kv], (kv, q)
    plain = window == 0 and block is None
    if schedule == "shift":
        n_units = sum(1 for kv in range(n) if any(live[q][kv] for q in range(n)))
        ws = OS.timed_slots(256, 1, n_units)
        assert t["slots_per_head"] == ws and not t["static"]
        units, steps, rank, starts = OS.timed_shift(live, ws)
        assert t["units"] == units and t["steps"] == steps
        assert np.array_equal(t["rank"], np.array([[-1 if x is None else x for x in row]
                                                   for row in rank]))
        assert OS.check_timed_schedule(live, units, steps, rank, starts, ws) == ""
        return
    want_units = [u for u in OS.masked_units(schedule, live) if u]
    assert t["units"] == want_units
    if schedule == "atomic":
        assert np.all(t["rank"] == -1)
    else:
        want = OS.masked_rank_table(live)
        assert np.array_equal(t["rank"], np.array([[-1 if x is None else x for x in row]
                                                   for row in want]))
    assert not plain


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("schedule", ["naive", "descending", "shift"])
def test_covering_window_gives_the_plain_tables(causal, schedule):
    N = 512
    units, rank = D.schedule_tables(N // T, causal, schedule)
    for w in (0, N, 4 * N):
        t = D.mask_schedule_tables(1, 1, N, 64, "f32", causal, schedule, window=w)
        assert t["units"] == units and np.array_equal(t["rank"], rank)
        if schedule == "shift":
            assert all(s == list(range(len(s))) for s in t["steps"])


def test_causal_band_shift_runs_each_tile_from_its_diagonal():
    """A causal window of whole tiles: with a slot per unit every KV tile
    starts on its diagonal block and walks up one block per step, so at
    block q the contributors come nearest first (rank q - kv) and every
    hand-off is one step."""
    n, w = 16, 3 * T
    t = D.mask_schedule_tables(1, 1, n * T, 64, "f32", True, "shift", window=w, slots=8 * n)
    assert t["slots_per_head"] == n
    for items, steps in zip(t["units"], t["steps"]):
        kv = items[0][0]
        assert [q for _, q in items] == list(range(kv, min(n, kv + 4)))
        assert steps == list(range(len(items)))
    for q in range(n):
        for kv in range(n):
            want = q - kv if 0 <= q - kv <= 3 else -1
            assert t["rank"][q, kv] == want


def test_timed_checker_catches_broken_tables():
    """The oracle's certificate checker rejects tables with planted
    mistakes (steps clashing on a block, units out of start order, a dQ
    order not by step, a missing unit, more units running than slots)."""
    n = 8
    live, _ = OS.tile_liveness(A.Mask(causal=True, window=3 * T), n, T)
    units, steps, rank, starts = OS.timed_shift(live, 3)
    ok = lambda u, st, r, s0, k: OS.check_timed_schedule(live, u, st, r, s0, k)  # noqa: E731
    assert ok(units, steps, rank, starts, 3) == ""
    assert ok(units, steps, rank, starts, 2) != ""
    # two units on one block at one step
    bad = [list(x) for x in steps]
    i = next(i for i in range(1, len(units)) if units[i][0][1] == units[0][1][1])
    bad[i] = [steps[0][1] + k for k in range(len(bad[i]))]
    assert ok(units, bad, rank, starts, 3) != ""
    assert ok(units[::-1], steps[::-1], rank, starts[::-1], 3) != ""
    late = list(starts)
    late[1] = steps[1][0] + 1
    assert ok(units, steps, rank, late, 3) != ""
    bad_rank = [list(r) for r in rank]
    q = units[2][0][1]
    kvs = [kv for kv in range(n) if bad_rank[q][kv] is not None]
    bad_rank[q][kvs[0]], bad_rank[q][kvs[-1]] = bad_rank[q][kvs[-1]], bad_rank[q][kvs[0]]
    assert ok(units, steps, bad_rank, starts, 3) != ""
    assert ok(units[:-1], steps[:-1], rank, starts[:-1], 3) != ""


def test_oracle_tile_liveness_closed_forms():
    n = 6
    live, part = OS.tile_liveness(A.Mask(causal=True), n, T)
    for q in range(n):
        for kv in range(n):
            assert live[q][kv] == OS.live(kv, q, True)
            assert part[q][kv] == (kv == q)
    live, part = OS.tile_liveness(A.Mask(), n, T)
    assert all(all(r) for r in live) and not any(any(r) for r in part)
    # a causal window of exactly one tile: the diagonal and the tile below
    # it are live, both partial
    live, part = OS.tile_liveness(A.Mask(causal=True, window=T), n, T)
    for q in range(n):
        for kv in range(n):
            assert live[q][kv] == (q - kv in (0, 1))
            assert part[q][kv] == live[q][kv]


@pytest.mark.parametrize("case", CASES[:8], ids=_ids)
@pytest.mark.parametrize("schedule", ["naive", "descending", "shift", "atomic"])
def test_masked_predict_matches_oracle_dag(case, schedule):
    N, causal, window, block, bs = case
    n = N // T
    kw = _kw(window, block, bs)
    heads, slots = 3, 5
    # the tables a launch on `slots` workgroups runs for `heads` heads (the
    # timed shift's slots per head depend on both)
    t = D.mask_schedule_tables(1, heads, N, 64, "f32", causal, schedule, slots=slots, **kw)
    tables = {"units": t["units"],
              "rank": None if schedule == "atomic" else t["rank"].tolist(),
              "partial": {it for items, fl in zip(t["units"], t["partial"])
                          for it, f in zip(items, fl) if f},
              "static": t["static"]}
    cost = (1.0, 0.6, 0.2, 0.1)
    assert not t["static"]
    for um in (False, True):
        got = D.mask_schedule_predict(1, heads, N, 64, "f32", causal, schedule, slots=slots,
                                      cost=cost, unit_major=um, **kw)
        want = OD.predict(schedule, n, causal, heads, slots, cost, tables, unit_major=um)
        for g, w in zip(got, want):
            assert abs(g - w) <= 1e-9 * max(1.0, abs(w)), (um, got, want)


def test_mask_argument_errors():
    with pytest.raises(D.DashError) as e:   # block size not a multiple of the tile
        D.mask_schedule_tables(1, 1, 512, 64, "f32", False, "naive",
                               block_mask=np.ones((16, 16)), block_size=32)
    assert e.value.code == 2
    with pytest.raises(D.DashError) as e:   # block size does not divide N
        D.mask_schedule_tables(1, 1, 512, 64, "f32", False, "naive",
                               block_mask=np.ones((2, 2)), block_size=192)
    assert e.value.code == 2
    with pytest.raises(D.DashError) as e:   # negative window
        D.mask_schedule_tables(1, 1, 512, 64, "f32", False, "naive", window=-1)
    assert e.value.code == 1
    with pytest.raises(D.DashError) as e:   # too many tiles with a special mask
        D.mask_schedule_tables(1, 1, 64 * 4096, 64, "f32", True, "naive", window=100)
    assert e.value.code == 2


def test_workload_visible_pairs_match_the_oracle_mask():
    """The bench's FLOP count for masked workloads (exact visible pairs,
    counted per tile pair) equals a brute-force count of the oracle's mask."""
    from dataclasses import replace
    from synth import WORKLOADS
    base = WORKLOADS["b1h32_n16k_d128_swa4k"]
    for extra, causal in [({"window": 300}, True), ({"window": 200}, False),
                          ({"block": {"size": 128, "band": 1, "globals": 1, "density": 0.2}}, True),
                          ({"block": {"size": 256, "band": 0, "globals": 1, "density": 0.3}}, False),
                          ({"window": 150, "block": {"size": 128, "band": 2, "globals": 0,
                                                     "density": 0.1}}, True)]:
        w = replace(base, N=1024, extra=extra)
        mk = w.mask_args()
        m = A.Mask(causal=causal, window=mk["window"], block=mk["block_mask"],
                   block_size=mk["block_size"])
        assert w.visible_pairs(causal) == int(m.visible(np.arange(1024), np.arange(1024)).sum())


def test_unit_major_order_on_a_block_sparse_mask():
    """Long units (global key blocks seen by every query) next to short
    ones: taking unit k of every head before unit k+1 lets every head's long
    units start at once; the model predicts a much shorter makespan, and
    never a longer one for the plain causal triangle under DESCENDING."""
    from synth import WORKLOADS
    w = WORKLOADS["b1h32_n16k_d128_blocksparse"]
    mk = w.mask_args()
    cost = (1.0, 0.5, 0.05, 0.05)
    hm = D.mask_schedule_predict(1, 4, w.N, w.d, "bf16", True, "descending", slots=32, cost=cost,
                                 **mk)[0]
    um = D.mask_schedule_predict(1, 4, w.N, w.d, "bf16", True, "descending", slots=32, cost=cost,
                                 unit_major=True, **mk)[0]
    assert um < 0.7 * hm
    hm = D.mask_schedule_predict(1, 4, 4096, 128, "bf16", True, "descending", slots=32,
                                 cost=cost)[0]
    um = D.mask_schedule_predict(1, 4, 4096, 128, "bf16", True, "descending", slots=32, cost=cost,
                                 unit_major=True)[0]
    assert um <= hm * 1.0001


def test_table_export_protocol():
    """Two-call export: sizes first; arrays of other sizes are refused; a
    negative workgroup count is refused."""
    import ctypes
    lib = D.load()
    desc = D._desc(1, 1, 512, 64, "f32", True, None, 100)
    sizes = (ctypes.c_int32 * 5)()
    assert lib.dash_attn_schedule_tables(ctypes.byref(desc), 2, 256, sizes, None, None, None,
                                         None, None, None) == 0
    n, nu, ni = sizes[0], sizes[1], sizes[2]
    assert n == 8 and nu == 8 and ni > 0 and sizes[3] == 0 and sizes[4] == 0
    arr = lambda m: (ctypes.c_int32 * max(m, 1))()
    bad = (ctypes.c_int32 * 5)(n, nu, ni + 1, 0, 0)
    assert lib.dash_attn_schedule_tables(ctypes.byref(desc), 2, 256, bad, arr(nu + 1), arr(ni),
                                         arr(ni), arr(ni), (ctypes.c_uint8 * ni)(),
                                         arr(n * n)) == 1
    assert lib.dash_attn_schedule_tables(ctypes.byref(desc), 9, 256, sizes, None, None, None,
                                         None, None, None) == 1
    assert lib.dash_attn_schedule_tables(ctypes.byref(desc), 2, -1, sizes, None, None, None,
                                         None, None, None) == 1
    assert lib.dash_attn_schedule_tables(None, 2, 256, sizes, None, None, None, None, None,
                                         None) == 1
    # SHIFT on the window: a timed shift for min(256 / 8, 8) slots per head
    assert lib.dash_attn_schedule_tables(ctypes.byref(desc), 3, 256, sizes, None, None, None,
                                         None, None, None) == 0
    assert sizes[3] == 0 and sizes[4] == 8


def test_bench_dag_prediction_on_the_plain_workloads():
    """The bench's DAG view of each ordered schedule, as the launch places
    it: on the full and causal masks shift meets its lower bound with no
    waits (the pages' conflict-free construction), descending needs no
    longer than naive, the dynamic schedules run in 8 XCD groups of 32
    workgroups, and shift runs grouped exactly when its units per head fit
    a group (32 at 4K full, 64 at 16K causal: device-wide)."""
    import bench
    from synth import WORKLOADS
    # the default costs of the one-stage kernel and of the two-stage pipeline
    for name, cost in itertools.product(
            ("b1h32_n16k_d128_causal", "b4h32_n4k_d128_full", "b2h16_n2k_d128_causal"),
            ((1.0, 0.5, 0.05, 0.05), (1.0, 0.5, 0.3, 0.3))):
        w = WORKLOADS[name]
        causal = w.masks[0] == "causal"
        pred = {s: bench.dag_prediction(D, w, causal, s, w.mask_args(), 256, cost)
                for s in ("naive", "descending", "shift")}
        for p in pred.values():
            assert p is not None
            assert p["slots"] * p["groups"] == 256
            assert p["heads_modelled"] <= -(-w.B * w.H // p["groups"])
            assert p["makespan_items"] >= p["lower_bound_items"] - 1e-6
            assert 0.0 <= p["wait_frac"] < 1.0
        assert pred["shift"]["makespan_items"] == pytest.approx(pred["shift"]["lower_bound_items"])
        assert pred["shift"]["wait_frac"] == 0.0
        assert pred["descending"]["makespan_items"] <= pred["naive"]["makespan_items"] + 1e-6
        assert pred["naive"]["groups"] == pred["descending"]["groups"] == 8
        n = w.N // 128
        shift_units = n // 2 if causal else n
        assert pred["shift"]["groups"] == (8 if shift_units <= 32 else 1)
