"""Calibration on the GPU (collected after the other GPU files: it changes
the costs "auto" uses for fp32 d = 64 for the rest of the process).

dash_attn_bwd_calibrate times the ordered schedules, fits the DAG model's
costs and records them; "auto" then predicts with them, and a pick that
dash_attn_bwd_tune measured keeps precedence."""
import math

import pytest
import torch

import deterministic_attention_backward_attn_amd as D
from tests.gpu_common import device_inputs, log, require_gpu

pytestmark = pytest.mark.gpu

SCHED = ("naive", "descending", "shift")


def test_calibrate_records_the_costs_auto_uses():
    require_gpu()
    B, H, N, d, dt = 1, 8, 1024, 64, "f32"
    dev, _ = device_inputs(B, H, N, d, dt, 9100)
    o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    delta = D.attn_bwd_preprocess(o, dev["do"])
    before = D.bwd_costs(B, H, N, d, dt, True)
    assert before == (1.0, 0.5, 0.05, 0.05)
    costs, res, times = D.attn_bwd_calibrate(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta,
                                             causal=True, reps=3)
    log(f"calibrated costs {costs} residual {res:.3f} times {times}")
    assert all(math.isfinite(t) and t > 0 for t in times.values())
    assert math.isfinite(res) and costs[0] == 1.0
    assert D.bwd_costs(B, H, N, d, dt, True) == costs
    # the fit on the host from the same times gives the same costs for the
    # launch's co-resident count (one or two workgroups per compute unit)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ms = [times[s] for s in SCHED]
    fits = {D.fit_costs(B, H, N, d, dt, True, slots=k * cus, ms=ms)[0] for k in (1, 2)}
    assert costs in fits
    # "auto" = the model's pick under the recorded costs
    picked = D.resolve_schedule(B, H, N, d, dt, True, "auto")
    picks = set()
    for k in (1, 2):
        pred = {s: D.bwd_predict(B, H, N, d, dt, True, s, slots=k * cus, cost=costs)[0][0]
                for s in SCHED}
        best = min(pred.values())
        # ties go to shift, then descending
        picks.add([s for s in reversed(SCHED) if pred[s] == best][0])
    assert picked in picks
    # other dtypes and head dims keep their costs (bf16 with d = 128 or 64
    # runs the two-stage pipeline, whose default model weighs the ordered add
    # more; fp32 with d = 128 the one-stage kernel)
    assert D.bwd_costs(B, H, N, 128, "bf16", True) == (1.0, 0.5, 0.3, 0.3)
    assert D.bwd_costs(B, H, N, 64, "bf16", True) == (1.0, 0.5, 0.3, 0.3)
    assert D.bwd_costs(B, H, N, 128, "f32", True) == (1.0, 0.5, 0.05, 0.05)
    # a measured pick keeps precedence
    tuned, _ = D.attn_bwd_tune(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, causal=True,
                               reps=2)
    assert D.resolve_schedule(B, H, N, d, dt, True, "auto") == tuned
