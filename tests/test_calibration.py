"""Fitting the DAG model's costs to measured kernel times (CPU, host calls).

The fit (dash_schedule_fit_costs) is checked on times the model itself
produced for known costs: it must find costs that reproduce those times
up to one common scale (zero residual), with that scale as the time per
cost unit.  Also: masked problems (the timed shift), argument errors.
"""
import math

import numpy as np
import pytest

import deterministic_attention_backward_attn_amd as D

SCHED = ("naive", "descending", "shift")


def _pred(B, H, N, d, causal, cost, slots, **kw):
    return [D.bwd_predict(B, H, N, d, "f32", causal, s, slots=slots, cost=cost, **kw)[0][0]
            for s in SCHED]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("true_cost", [(1.0, 0.5, 0.05, 0.05), (1.0, 0.75, 0.1, 0.2),
                                       (1.0, 1.0, 0.3, 0.0)])
def test_fit_reproduces_model_times(causal, true_cost):
    B, H, N, d, slots = 1, 8, 64 * 16, 64, 16
    unit = 0.0371
    ms = [unit * m for m in _pred(B, H, N, d, causal, true_cost, slots)]
    cost, res, got_unit = D.fit_costs(B, H, N, d, "f32", causal, slots=slots, ms=ms)
    assert res < 1e-9
    again = _pred(B, H, N, d, causal, cost, slots)
    for m, g in zip(ms, again):
        assert abs(got_unit * g - m) <= 1e-9 * m
    assert cost[0] == 1.0


def test_fit_on_a_block_mask():
    rng = np.random.default_rng(4)
    block = (rng.random((12, 12)) < 0.4).astype(np.uint8)
    block[:, 0] = 1
    kw = dict(block_mask=block, block_size=64)
    B, H, N, d, slots = 1, 6, 64 * 12, 64, 24
    true_cost = (1.0, 0.75, 0.05, 0.1)
    ms = [2.0 * m for m in _pred(B, H, N, d, True, true_cost, slots, **kw)]
    cost, res, unit = D.fit_costs(B, H, N, d, "f32", True, slots=slots, ms=ms, **kw)
    assert res < 1e-9
    for m, g in zip(ms, _pred(B, H, N, d, True, cost, slots, **kw)):
        assert abs(unit * g - m) <= 1e-9 * m


def test_fit_needs_two_times_and_no_negative_one():
    args = (1, 4, 64 * 8, 64, "f32", True)
    with pytest.raises(D.DashError) as e:
        D.fit_costs(*args, slots=8, ms=(1.0, None, None))
    assert e.value.code == 1
    with pytest.raises(D.DashError) as e:
        D.fit_costs(*args, slots=8, ms=(1.0, -2.0, 1.0))
    assert e.value.code == 1
    cost, res, unit = D.fit_costs(*args, slots=8, ms=(1.0, None, 1.1))
    assert math.isfinite(res) and unit > 0


def test_bench_reports_the_fit():
    """The bench's dag_fit on kernel times the model produced: zero error,
    and the fitted ratios are the times' ratios."""
    import bench
    from synth import WORKLOADS
    w = WORKLOADS["b2h16_n2k_d128_causal"]
    cost = (1.0, 1.0, 0.1, 0.05)
    results = {s: {"kernel_ms": 0.01 * D.bwd_predict(w.B, w.H, w.N, w.d, w.dtype, True, s,
                                                      slots=256, cost=cost)[0][0]}
               for s in SCHED}
    fit = bench.dag_fit(D, w, True, w.mask_args(), results, 256)
    assert fit["rel_rms_error"] < 1e-6
    for s in ("naive", "descending"):
        assert fit["fitted_vs_shift"][s] == pytest.approx(
            results[s]["kernel_ms"] / results["shift"]["kernel_ms"], rel=2e-3)
