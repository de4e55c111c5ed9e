"""GPU tests of the fixed accumulation order.

* Every ordered schedule gives bit-identical dQ, dK, dV over 50 runs.
* Where two schedules share the dQ order (naive, descending) dQ is
  bit-identical; where they share the traversal (naive, atomic) dK and dV are.
* Order replay: the per-KV-tile dQ partials, summed on the host in fp32 in
  the rank order of the schedule tables, reproduce dQ bit for bit.
* Timing perturbation (random sleeps before each ordered add) changes no bit.
* Ordering litmus across all XCDs: order-sensitive fp32 sums come out
  exactly as the host's sequential sum in turn order.
* A forced time-out (a wait that can never succeed, with a tiny spin limit)
  ends the kernel normally and is reported as DASH_ERR_ORDER_TIMEOUT.
* Causal: KV tiles never read earlier Q blocks, so perturbing those leaves
  their dK, dV bit-identical.
* Placement (device-wide or XCD groups, L2- or device-coherent accumulator)
  changes no bit.
* The phase timer (a test hook) changes no bit and its phases fit inside
  each wave's run.
* The wave-pair layout gives the same bits as the default kernel.
"""
import numpy as np
import pytest
import torch

import deterministic_attention_backward_attn_amd as D
from oracle import schedules as OS
from tests.gpu_common import device_inputs, log, require_gpu

pytestmark = pytest.mark.gpu

ORDERED = ["naive", "descending", "shift"]


def _prep(B, H, N, d, dtype, causal, seed):
    dev, _ = device_inputs(B, H, N, d, dtype, seed)
    o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal)
    delta = D.attn_bwd_preprocess(o, dev["do"])
    return dev, lse, delta


def _bwd(dev, lse, delta, sched, causal, ws=None, debug=None, check=True):
    """One backward; with `check`, its status word is read right after it
    (each launch clears the word, so every compared run is checked)."""
    if ws is None:
        ws = D.alloc_workspace(dev["q"], causal, sched)
    out = D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, schedule=sched,
                     causal=causal, workspace=ws, debug=debug)
    if check:
        D.attn_bwd_status(ws)
    return out


# every kernel instantiation the ordered schedules run: bf16 d = 128,
# bf16 d = 64, fp32 d = 64 (the fp32 workload)
FIFTY = [("bf16", (2, 16, 2048, 128)), ("f32", (1, 2, 256, 64)), ("bf16", (1, 8, 1024, 64))]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dtype,shape", FIFTY)
def test_fifty_runs_bit_identical(dtype, shape, causal):
    require_gpu()
    B, H, N, d = shape
    log(f"determinism {dtype} B={B} H={H} N={N} d={d} causal={causal}")
    dev, lse, delta = _prep(B, H, N, d, dtype, causal, 2000)
    iv = (lambda t: t.view(torch.int32)) if dtype == "f32" else (lambda t: t.view(torch.int16))
    for sched in ORDERED:
        ws = D.alloc_workspace(dev["q"], causal, sched)
        ref = [t.clone() for t in _bwd(dev, lse, delta, sched, causal, ws)]
        D.attn_bwd_status(ws)
        for run in range(49):
            out = _bwd(dev, lse, delta, sched, causal, ws)
            for a, b in zip(ref, out):
                assert torch.equal(iv(a), iv(b)), (sched, run)
        D.attn_bwd_status(ws)
        log(f"  {sched}: 50 runs identical")
    if dtype != "bf16" or d != 128:
        return
    # the unordered reference: report how many distinct dQ results occur
    ws = D.alloc_workspace(dev["q"], causal, "atomic")
    seen = set()
    for _ in range(10):
        dq, _, _ = _bwd(dev, lse, delta, "atomic", causal, ws)
        seen.add(hash(dq.view(torch.int16).cpu().numpy().tobytes()))
    log(f"  atomic: {len(seen)} distinct dQ bit patterns in 10 runs")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dtype,shape", [("bf16", (2, 4, 1024, 128)), ("f32", (1, 2, 256, 64)),
                                         ("bf16", (1, 4, 1024, 64))])
def test_cross_schedule_bit_relations(dtype, shape, causal):
    require_gpu()
    log(f"cross-schedule {dtype} {shape} causal={causal}")
    dev, lse, delta = _prep(*shape, dtype, causal, 3100)
    naive = _bwd(dev, lse, delta, "naive", causal)
    desc = _bwd(dev, lse, delta, "descending", causal)
    atom = _bwd(dev, lse, delta, "atomic", causal)
    iv = (lambda t: t.view(torch.int32)) if dtype == "f32" else (lambda t: t.view(torch.int16))
    assert torch.equal(iv(naive[0]), iv(desc[0])), "same dQ order -> same dQ bits"
    assert torch.equal(iv(naive[1]), iv(atom[1])) and torch.equal(iv(naive[2]), iv(atom[2])), \
        "same traversal -> same dK/dV bits"


def _bf16_rne(x32):
    u = x32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("sched", ORDERED)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,shape", [("f32", (1, 2, 256, 64)), ("bf16", (1, 2, 512, 128)),
                                         ("bf16", (1, 2, 512, 64))])
def test_order_replay(dtype, shape, causal, sched):
    require_gpu()
    B, H, N, d = shape
    log(f"order replay {dtype} {shape} causal={causal} {sched}")
    dev, lse, delta = _prep(B, H, N, d, dtype, causal, 4100)
    tile = D.tile(B, H, N, d, dtype)
    n = N // tile
    partials = torch.zeros((B * H, n, N, d), dtype=torch.float32, device="cuda")
    ws = D.alloc_workspace(dev["q"], causal, sched)
    dq, _, _ = _bwd(dev, lse, delta, sched, causal, ws, debug={"partials": partials})
    D.attn_bwd_status(ws)
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
            acc[:, rows] = acc[:, rows] + part[:, kv, rows]   # one fp32 add per partial
    want = (acc * scale).astype(np.float32)
    got = dq.reshape(B * H, N, d)
    if dtype == "f32":
        assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))
    else:
        assert np.array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16), _bf16_rne(want))


@pytest.mark.parametrize("causal", [True, False])
def test_timing_perturbation_changes_no_bit(causal):
    require_gpu()
    log(f"jitter causal={causal}")
    dev, lse, delta = _prep(1, 8, 1024, 128, "bf16", causal, 5100)
    for sched in ORDERED:
        ref = _bwd(dev, lse, delta, sched, causal)
        for seed in (1, 7, 1234):
            out = _bwd(dev, lse, delta, sched, causal, debug={"jitter_seed": seed})
            for a, b in zip(ref, out):
                assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (sched, seed)


def test_litmus_across_xcds():
    require_gpu()
    W, L = 1024, 256
    log(f"litmus W={W} L={L}")
    rng = np.random.default_rng(77)
    turn = rng.permutation(W).astype(np.int32)
    # wide dynamic range so that any other order changes the bits
    vals = (rng.standard_normal((W, L)) * np.exp2(rng.integers(-20, 20, size=(W, L)))).astype(np.float32)
    by_turn = np.argsort(turn)
    want = np.zeros(L, dtype=np.float32)
    for w in by_turn:
        want = want + vals[w]
    shuffled = np.zeros(L, dtype=np.float32)
    for w in range(W):
        shuffled = shuffled + vals[w]
    assert not np.array_equal(want, shuffled), "values must be order-sensitive"
    acc = torch.zeros(L, dtype=torch.float32, device="cuda")
    counters = torch.zeros(2, dtype=torch.int32, device="cuda")
    D.litmus_ordered_add(torch.from_numpy(turn).cuda(), torch.from_numpy(vals).cuda(), acc, counters)
    assert np.array_equal(acc.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_forced_timeout_is_reported_and_terminates():
    require_gpu()
    log("forced time-out")
    dev, lse, delta = _prep(1, 2, 256, 64, "f32", True, 6100)
    ws = D.alloc_workspace(dev["q"], True, "naive")
    _bwd(dev, lse, delta, "naive", True, ws, debug={"poison_q": 2, "spin_limit": 2000},
         check=False)
    with pytest.raises(D.DashError) as e:
        D.attn_bwd_status(ws)
    assert e.value.code == 6
    # the next normal call on the same workspace is clean again
    _bwd(dev, lse, delta, "naive", True, ws)
    D.attn_bwd_status(ws)


def test_causal_tiles_ignore_earlier_q_blocks():
    require_gpu()
    B, H, N, d = 1, 4, 1024, 128
    log("causal invariance")
    dev, lse, delta = _prep(B, H, N, d, "bf16", True, 7100)
    ref = _bwd(dev, lse, delta, "descending", True)
    tile = D.tile(B, H, N, d, "bf16")
    J = 3
    dev2 = {k: v.clone() for k, v in dev.items()}
    g = torch.Generator(device="cpu").manual_seed(5)
    noise = torch.randn((B, H, J * tile, d), generator=g).to(torch.bfloat16).cuda()
    dev2["q"][:, :, : J * tile] += noise
    dev2["do"][:, :, : J * tile] -= noise
    o2, lse2 = D.attn_fwd(dev2["q"], dev2["k"], dev2["v"], causal=True)
    delta2 = D.attn_bwd_preprocess(o2, dev2["do"])
    out = _bwd(dev2, lse2, delta2, "descending", True)
    for a, b in zip(ref[1:], out[1:]):
        assert torch.equal(a[:, :, J * tile:].view(torch.int16), b[:, :, J * tile:].view(torch.int16))
        assert not torch.equal(a[:, :, :J * tile], b[:, :, :J * tile])


@pytest.mark.parametrize("causal", [True, False])
def test_placement_changes_no_bit(causal):
    """Units of a head on one XCD (automatic) or spread over the device:
    same dQ order, so bit-identical results."""
    require_gpu()
    log(f"placement causal={causal}")
    dev, lse, delta = _prep(2, 16, 2048, 128, "bf16", causal, 8100)
    for sched in ORDERED:
        ref = [t.clone() for t in _bwd(dev, lse, delta, sched, causal, debug={"placement": 1})]
        for place in (0, 2, 3):
            out = _bwd(dev, lse, delta, sched, causal, debug={"placement": place})
            for x, y in zip(ref, out):
                assert torch.equal(x.view(torch.int16), y.view(torch.int16)), (sched, place)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(2, 16, 2048, 128), (1, 4, 1152, 128), (1, 64, 1024, 64)])
def test_auto_runs_its_resolved_schedule(shape, causal):
    """"auto" is bit-identical to the ordered schedule it resolves to, and
    that schedule is the DAG model's pick for the launch's co-resident
    workgroups."""
    require_gpu()
    B, H, N, d = shape
    picked = D.resolve_schedule(B, H, N, d, "bf16", causal, "auto")
    log(f"auto {shape} causal={causal} -> {picked}")
    assert picked in ORDERED
    for s in ORDERED + ["atomic"]:
        assert D.resolve_schedule(B, H, N, d, "bf16", causal, s) == s
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    # the DAG model's pick under the costs the library uses for this dtype
    # and head dim, on one or two workgroups per compute unit (the kernel's
    # occupancy); ties go to shift, then descending
    cost = D.bwd_costs(B, H, N, d, "bf16", causal)
    picks = set()
    for k in (1, 2):
        pred = {}
        for s in ORDERED:
            try:
                pred[s] = D.bwd_predict(B, H, N, d, "bf16", causal, s, slots=k * cus,
                                        cost=cost)[0][0]
            except D.DashError as e:  # a schedule that cannot run (causal shift, odd n)
                assert e.code == 2 and s == "shift", (s, e.code)
        best = min(pred.values())
        picks.add([s for s in reversed(ORDERED) if pred.get(s) == best][0])
    assert picked in picks
    dev, lse, delta = _prep(B, H, N, d, "bf16", causal, 8200)
    ref = _bwd(dev, lse, delta, picked, causal)
    for _ in range(3):
        out = _bwd(dev, lse, delta, "auto", causal)
        for x, y in zip(ref, out):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("causal", [True, False])
def test_unit_order_changes_no_bit(causal):
    """Units taken head by head or unit-major: a head's units keep their
    order, so results are bit-identical."""
    require_gpu()
    log(f"unit order causal={causal}")
    dev, lse, delta = _prep(2, 16, 2048, 128, "bf16", causal, 8300)
    for sched in ("naive", "descending"):
        ref = [t.clone() for t in _bwd(dev, lse, delta, sched, causal, debug={"unit_order": 1})]
        for order in (0, 2):
            out = _bwd(dev, lse, delta, sched, causal, debug={"unit_order": order})
            for x, y in zip(ref, out):
                assert torch.equal(x.view(torch.int16), y.view(torch.int16)), (sched, order)


@pytest.mark.parametrize("causal", [True, False])
def test_tune_records_the_fastest_for_auto(causal):
    """Profiling-driven choice: the timed pick is the fastest candidate, and
    later "auto" launches of the shape run it (bit-identical)."""
    require_gpu()
    B, H, N, d = 1, 16, 2048, 128
    log(f"tune causal={causal}")
    dev, lse, delta = _prep(B, H, N, d, "bf16", causal, 8400)
    picked, times = D.attn_bwd_tune(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta,
                                    causal=causal, reps=3)
    log(f"  times {times} -> {picked}")
    finite = {k: v for k, v in times.items() if v == v}
    assert picked == min(finite, key=finite.get)
    assert D.resolve_schedule(B, H, N, d, "bf16", causal, "auto") == picked
    ref = _bwd(dev, lse, delta, picked, causal)
    out = _bwd(dev, lse, delta, "auto", causal)
    for x, y in zip(ref, out):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("causal", [True, False])
def test_phase_timer_changes_no_bit(causal):
    """The phase timer (a test hook) changes no result bit, and its phase
    cycles of every wave add up to no more than that wave's whole run."""
    require_gpu()
    B, H, N, d = 2, 16, 2048, 128
    log(f"phase timer B={B} H={H} N={N} d={d} causal={causal}")
    dev, lse, delta = _prep(B, H, N, d, "bf16", causal, 2400)
    for sched in ORDERED + ["atomic"]:
        ws = D.alloc_workspace(dev["q"], causal, sched)
        st = torch.zeros(16 * 4096 * 4, dtype=torch.int64, device="cuda")
        # the one-stage kernel's phases (the pipeline's have their own test)
        timed = _bwd(dev, lse, delta, sched, causal, ws, debug={"layout": 3, "phase_stats": st})
        D.attn_bwd_status(ws)
        a = st.view(-1, 16).cpu().numpy()
        a = a[a[:, 15] > 0]
        assert len(a) > 0 and (a >= 0).all()
        assert (a[:, :11].sum(axis=1) <= a[:, 15]).all()
        # every wave that ran a sub-tile spent cycles in its products
        ran = a[:, :11].sum(axis=1) > 0
        assert ran.any() and (a[ran, 1] > 0).all() and (a[ran, 4] > 0).all()
        if sched != "atomic":
            plain = _bwd(dev, lse, delta, sched, causal, ws, debug={"layout": 3})
            for x, y in zip(timed, plain):
                assert torch.equal(x.view(torch.int16), y.view(torch.int16)), sched
        log(f"  {sched}: {len(a)} waves, ordered-add share "
            f"{a[:, 6].sum() / a[:, 15].sum():.3f}")


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 300)])
def test_wave_pair_layout_is_bit_identical(causal, window):
    """The wave-pair layout of the backward (two waves per KV slice) computes
    every product, exponential and add in the same order as the default
    kernel: bit-identical dQ, dK, dV for every ordered schedule, the same
    bits again on a second run; the atomic schedule runs and matches within
    the bf16 tolerance."""
    require_gpu()
    B, H, N, d = 2, 16, 2048, 128
    log(f"wave pairs B={B} H={H} N={N} d={d} causal={causal} window={window}")
    dev, _ = device_inputs(B, H, N, d, "bf16", 2500)
    o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, window=window)
    delta = D.attn_bwd_preprocess(o, dev["do"])

    def run(sched, layout, ws):
        return D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, schedule=sched,
                          causal=causal, workspace=ws, window=window,
                          debug={"layout": layout} if layout else None)

    for sched in ORDERED + ["atomic"]:
        ws = D.alloc_workspace(dev["q"], causal, sched)
        ref = [t.clone() for t in run(sched, 0, ws)]
        D.attn_bwd_status(ws)  # each launch clears the word: check every compared run
        for rep in range(2):
            out = run(sched, 1, ws)
            D.attn_bwd_status(ws)
            for x, y in zip(ref, out):
                if sched == "atomic":
                    err = (x.float() - y.float()).abs().max() / x.float().abs().max()
                    assert float(err) <= 2e-2, (sched, float(err))
                else:
                    assert torch.equal(x.view(torch.int16), y.view(torch.int16)), (sched, rep)
        log(f"  {sched}: wave pairs match")


def test_wave_pair_layout_rejects_other_shapes():
    require_gpu()
    dev, _ = device_inputs(1, 2, 512, 64, "bf16", 2600)
    o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    delta = D.attn_bwd_preprocess(o, dev["do"])
    with pytest.raises(D.DashError) as e:
        D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, schedule="shift",
                   causal=True, debug={"layout": 1})
    assert e.value.code == 2  # DASH_ERR_UNSUPPORTED


def test_wave_pair_phase_timer_changes_no_bit():
    """The phase timer of the wave-pair layout changes no result bit and
    records both roles' phases inside each wave's run."""
    require_gpu()
    B, H, N, d = 2, 16, 2048, 128
    dev, lse, delta = _prep(B, H, N, d, "bf16", True, 2700)
    for sched in ORDERED:
        ws = D.alloc_workspace(dev["q"], True, sched)
        st = torch.zeros(16 * 4096 * 4, dtype=torch.int64, device="cuda")
        timed = _bwd(dev, lse, delta, sched, True, ws, debug={"layout": 1, "phase_stats": st})
        D.attn_bwd_status(ws)  # each launch clears the word: check every compared run
        plain = _bwd(dev, lse, delta, sched, True, ws, debug={"layout": 1})
        D.attn_bwd_status(ws)
        for x, y in zip(timed, plain):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16)), sched
        a = st.view(-1, 16).cpu().numpy()
        a = a[a[:, 15] > 0]
        assert set(a[:, 14].tolist()) == {1, 2}
        assert (a[:, :9].sum(axis=1) <= a[:, 15]).all()
        log(f"  {sched}: {len(a)} waves timed")
