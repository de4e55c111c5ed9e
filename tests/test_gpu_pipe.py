"""GPU tests of the two-stage pipeline layout of the backward (bf16, d = 128 and 64).

The layout computes every product, exponential and add with the same
operands in the same order as the one-stage kernel, so its results are
compared bit for bit with the one-stage kernel's (which runs every other
dtype and head dim and which the parity tests tie to the oracle there); and
directly with the oracle at one small shape.  It is what an automatic launch
runs for bf16 with d = 128, so every other bf16 d = 128 GPU test runs it too.

* Bit-identical to the one-stage kernel for every ordered schedule on causal,
  full, sliding-window and block-sparse masks, on repeated runs; the
  automatic layout is the pipeline.
* The atomic schedule (unordered fp32 adds) within the bf16 tolerance.
* Placement (device-wide or XCD groups, L2- or device-coherent accumulator)
  and unit order change no bit.
* Order replay: dQ equals the fp32 sum of the per-KV-tile partials in the
  schedule's rank order.
* Timing perturbation before every ordered add changes no bit.
* A forced time-out ends the kernel normally and is reported.
* d = 64 (Q sub-tiles of 64 rows): the oracle, bit identity with the
  one-stage kernel and the order replay as above.
* Other dtypes are refused; the phase timer changes no bit.
"""
import numpy as np
import pytest
import torch

import deterministic_attention_backward_attn_amd as D
from oracle import attention as A
from oracle import schedules as OS
from tests.gpu_common import TOL, device_inputs, log, rel_err, require_gpu

pytestmark = pytest.mark.gpu

ORDERED = ["naive", "descending", "shift"]
PIPE = {"layout": 2}
ONE = {"layout": 3}  # the one-stage kernel


def _same(x, y):
    return torch.equal(x.view(torch.int16), y.view(torch.int16))


def _run(dev, lse, delta, sched, causal, ws, debug=None, **mkw):
    out = D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, schedule=sched,
                     causal=causal, workspace=ws, debug=debug, **mkw)
    D.attn_bwd_status(ws)  # each launch clears the word: check every compared run
    return [t.clone() for t in out]


@pytest.mark.parametrize("d", [128, 64])
def test_pipe_matches_the_oracle(d):
    require_gpu()
    B, H, N = 1, 2, 512
    for causal in (True, False):
        log(f"pipe vs oracle B={B} H={H} N={N} d={d} causal={causal}")
        dev, ex = device_inputs(B, H, N, d, "bf16", 9100)
        o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal)
        delta = D.attn_bwd_preprocess(o, dev["do"])
        refs = A.backward(ex["q"], ex["k"], ex["v"], ex["do"], causal, 1.0 / np.sqrt(d))
        for sched in ORDERED + ["atomic"]:
            ws = D.alloc_workspace(dev["q"], causal, sched)
            got = _run(dev, lse, delta, sched, causal, ws, PIPE)
            for name, g, r in zip(("dQ", "dK", "dV"), got, refs):
                err = rel_err(g, r)
                assert err <= TOL["bf16"], (sched, name, err)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("mask", ["causal", "full", "window", "block"])
def test_pipe_layout_is_bit_identical(mask, d):
    require_gpu()
    B, H, N = 2, 16, 2048
    causal = mask in ("causal", "window", "block")
    mkw = {}
    if mask == "window":
        mkw = {"window": 300}
    elif mask == "block":
        n = N // 128
        live = np.zeros((n, n), dtype=np.uint8)
        for i in range(n):
            for j in range(i + 1):
                if j == 0 or i - j <= 1 or (i + j) % 5 == 0:
                    live[i, j] = 1
        mkw = {"block_mask": live, "block_size": 128}
    log(f"pipe bit identity B={B} H={H} N={N} d={d} mask={mask}")
    dev, _ = device_inputs(B, H, N, d, "bf16", 9200)
    o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, **mkw)
    delta = D.attn_bwd_preprocess(o, dev["do"])
    for sched in ORDERED + ["atomic"]:
        ws = D.alloc_workspace(dev["q"], causal, sched, **mkw)
        ref = _run(dev, lse, delta, sched, causal, ws, ONE, **mkw)
        for rep in range(3):
            # the automatic layout (no debug options) runs the pipeline
            out = _run(dev, lse, delta, sched, causal, ws, PIPE if (rep or d != 128) else None, **mkw)
            for x, y in zip(ref, out):
                if sched == "atomic":
                    err = (x.float() - y.float()).abs().max() / x.float().abs().max()
                    assert float(err) <= TOL["bf16"], (sched, float(err))
                else:
                    assert _same(x, y), (sched, rep)
        log(f"  {sched}: pipeline matches")


@pytest.mark.parametrize("causal", [True, False])
def test_pipe_placement_and_unit_order_change_no_bit(causal):
    require_gpu()
    log(f"pipe placement/unit order causal={causal}")
    dev, _ = device_inputs(2, 16, 2048, 128, "bf16", 9300)
    o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal)
    delta = D.attn_bwd_preprocess(o, dev["do"])
    for sched in ORDERED:
        ws = D.alloc_workspace(dev["q"], causal, sched)
        ref = _run(dev, lse, delta, sched, causal, ws, dict(PIPE, placement=1))
        for place in (0, 2, 3):
            out = _run(dev, lse, delta, sched, causal, ws, dict(PIPE, placement=place))
            assert all(_same(x, y) for x, y in zip(ref, out)), (sched, place)
        if sched != "shift":
            for order in (1, 2):
                out = _run(dev, lse, delta, sched, causal, ws, dict(PIPE, unit_order=order))
                assert all(_same(x, y) for x, y in zip(ref, out)), (sched, order)


def _bf16_rne(x32):
    u = x32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("sched", ORDERED)
@pytest.mark.parametrize("causal", [False, True])
def test_pipe_order_replay(causal, sched, d):
    require_gpu()
    B, H, N = 1, 2, 512
    log(f"pipe order replay causal={causal} {sched} d={d}")
    dev, _ = device_inputs(B, H, N, d, "bf16", 9400)
    o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal)
    delta = D.attn_bwd_preprocess(o, dev["do"])
    tile = D.tile(B, H, N, d, "bf16")
    n = N // tile
    partials = torch.zeros((B * H, n, N, d), dtype=torch.float32, device="cuda")
    ws = D.alloc_workspace(dev["q"], causal, sched)
    dq, _, _ = _run(dev, lse, delta, sched, causal, ws, dict(PIPE, partials=partials))
    part = partials.cpu().numpy()
    _, rank = D.schedule_tables(n, causal, sched)
    ref_rank = OS.rank_table(sched, n, causal)
    assert all(rank[q, kv] == (-1 if ref_rank[q][kv] is None else ref_rank[q][kv])
               for q in range(n) for kv in range(n))
    scale = np.float32(1.0 / np.sqrt(d))
    acc = np.zeros((B * H, N, d), dtype=np.float32)
    for qb in range(n):
        order = sorted((rank[qb, kv], kv) for kv in range(n) if rank[qb, kv] >= 0)
        rows = slice(qb * tile, (qb + 1) * tile)
        for _, kv in order:
            acc[:, rows] = acc[:, rows] + part[:, kv, rows]
    want = (acc * scale).astype(np.float32)
    got = dq.reshape(B * H, N, d)
    assert np.array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16), _bf16_rne(want))


@pytest.mark.parametrize("causal", [True, False])
def test_pipe_timing_perturbation_changes_no_bit(causal):
    require_gpu()
    log(f"pipe jitter causal={causal}")
    dev, _ = device_inputs(1, 8, 1024, 128, "bf16", 9500)
    o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal)
    delta = D.attn_bwd_preprocess(o, dev["do"])
    for sched in ORDERED:
        ws = D.alloc_workspace(dev["q"], causal, sched)
        ref = _run(dev, lse, delta, sched, causal, ws, ONE)
        for seed in (3, 11):
            out = _run(dev, lse, delta, sched, causal, ws, dict(PIPE, jitter_seed=seed))
            assert all(_same(x, y) for x, y in zip(ref, out)), (sched, seed)


def test_pipe_fifty_runs_bit_identical():
    require_gpu()
    B, H, N, d = 2, 16, 2048, 128
    log(f"pipe determinism B={B} H={H} N={N} d={d} causal")
    dev, _ = device_inputs(B, H, N, d, "bf16", 9600)
    o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    delta = D.attn_bwd_preprocess(o, dev["do"])
    for sched in ORDERED:
        ws = D.alloc_workspace(dev["q"], True, sched)
        ref = _run(dev, lse, delta, sched, True, ws, PIPE)
        for run in range(49):
            out = D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, schedule=sched,
                             causal=True, workspace=ws, debug=PIPE)
            assert all(_same(x, y) for x, y in zip(ref, out)), (sched, run)
        D.attn_bwd_status(ws)


def test_pipe_forced_timeout_is_reported_and_terminates():
    require_gpu()
    log("pipe forced time-out")
    dev, _ = device_inputs(1, 2, 512, 128, "bf16", 9700)
    o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    delta = D.attn_bwd_preprocess(o, dev["do"])
    ws = D.alloc_workspace(dev["q"], True, "naive")
    D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, schedule="naive", causal=True,
               workspace=ws, debug=dict(PIPE, poison_q=2, spin_limit=2000))
    with pytest.raises(D.DashError) as e:
        D.attn_bwd_status(ws)
    assert e.value.code == 6
    _run(dev, lse, delta, "naive", True, ws, PIPE)


def test_pipe_rejects_other_shapes():
    require_gpu()
    dev, _ = device_inputs(1, 2, 512, 128, "f32", 9800)
    o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    delta = D.attn_bwd_preprocess(o, dev["do"])
    with pytest.raises(D.DashError) as e:
        D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, schedule="shift",
                   causal=True, debug=PIPE)
    assert e.value.code == 2  # DASH_ERR_UNSUPPORTED


def test_pipe_phase_timer_changes_no_bit():
    """The phase timer of the pipeline layout (a test hook) changes no result
    bit, and both stages' phases fit inside each wave's run."""
    require_gpu()
    B, H, N, d = 2, 16, 2048, 128
    dev, _ = device_inputs(B, H, N, d, "bf16", 9900)
    o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    delta = D.attn_bwd_preprocess(o, dev["do"])
    for sched in ORDERED + ["atomic"]:
        ws = D.alloc_workspace(dev["q"], True, sched)
        st = torch.zeros(16 * 4096 * 8, dtype=torch.int64, device="cuda")
        timed = _run(dev, lse, delta, sched, True, ws, dict(PIPE, phase_stats=st))
        plain = _run(dev, lse, delta, sched, True, ws, PIPE)
        if sched != "atomic":
            assert all(_same(x, y) for x, y in zip(timed, plain)), sched
        a = st.view(-1, 16).cpu().numpy()
        a = a[a[:, 15] > 0]
        assert set(a[:, 14].tolist()) == {1, 2}
        assert (a[:, :8].sum(axis=1) <= a[:, 15]).all()
        log(f"  {sched}: {len(a)} waves timed")
