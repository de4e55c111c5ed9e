"""GPU parity and ordering with sliding windows and block masks.

The HIP forward and backward against the fp64 oracle's masked definition
(same metric and bounds as the plain masks: 1e-4 fp32, 2e-2 bf16), for
every schedule including auto; rows that see no key (LSE = -inf, zero
gradients); bitwise run-to-run determinism of the ordered schedules; the
cross-schedule bit relations that hold for any mask (naive and descending
share the dQ order; naive and atomic share the traversal)."""
import numpy as np
import pytest
import torch

import deterministic_attention_backward_attn_amd as D
from oracle import attention as A
from tests.gpu_common import TOL, device_inputs, log, rel_err, require_gpu

pytestmark = pytest.mark.gpu

SCHEDS = ["atomic", "naive", "descending", "shift", "auto"]
rng = np.random.default_rng(77)
BLOCK8 = rng.random((8, 8)) < 0.5
DEAD8 = np.ones((8, 8), dtype=bool)
DEAD8[2, :] = False
DEAD8[:, 6] = False


def _lse_err(lse, ref):
    g = lse.detach().float().cpu().numpy().astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    dead = np.isneginf(ref)
    assert np.array_equal(np.isneginf(g), dead), "rows without keys must have LSE = -inf"
    if dead.all():
        return 0.0
    return float(np.max(np.abs(g[~dead] - ref[~dead])) / np.max(np.abs(ref[~dead])))


def _run(B, H, N, d, dtype, causal, window, block, seed, schedules=SCHEDS):
    require_gpu()
    bs = 0 if block is None else N // block.shape[0]
    log(f"mask case B={B} H={H} N={N} d={d} {dtype} causal={causal} window={window} "
        f"block={None if block is None else block.shape} seed={seed}")
    kw = dict(window=window, block_mask=block, block_size=bs)
    dev, ex = device_inputs(B, H, N, d, dtype, seed)
    s = 1.0 / np.sqrt(d)
    m = A.Mask(causal=causal, window=window, block=block, block_size=bs)
    o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, **kw)
    o_ref, lse_ref = A.forward(ex["q"], ex["k"], ex["v"], m, s)
    dq_ref, dk_ref, dv_ref = A.backward(ex["q"], ex["k"], ex["v"], ex["do"], m, s,
                                        o=o_ref, lse=lse_ref)
    tol = TOL[dtype]
    e_o, e_l = rel_err(o, o_ref), _lse_err(lse, lse_ref)
    log(f"  fwd  O {e_o:.2e}  LSE {e_l:.2e}")
    assert e_o <= tol and e_l <= tol
    delta = D.attn_bwd_preprocess(o, dev["do"])
    # With one visible key per row (a window of 1) dS vanishes analytically
    # and dQ, dK are rounding noise around 0: their error is then measured
    # against the dV scale instead of their own (zero) maximum.
    floor = float(np.max(np.abs(dv_ref))) if window == 1 else 0.0
    vis = m.visible(np.arange(N), np.arange(N))
    dead_q, dead_k = ~vis.any(axis=1), ~vis.any(axis=0)
    outs = {}
    for sched in schedules:
        ws = D.alloc_workspace(dev["q"], causal, sched)
        # stale values in the outputs must not survive (cleared dead tiles)
        dq, dk, dv = (torch.full_like(dev["q"], 7.0) for _ in range(3))
        D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, schedule=sched,
                   causal=causal, workspace=ws, out=(dq, dk, dv), **kw)
        D.attn_bwd_status(ws)
        errs = (rel_err(dq, dq_ref, floor), rel_err(dk, dk_ref, floor), rel_err(dv, dv_ref))
        ran = D.resolve_schedule(B, H, N, d, dtype, causal, sched, **kw)
        log(f"  {sched:10s} ({ran}) dQ {errs[0]:.2e} dK {errs[1]:.2e} dV {errs[2]:.2e}")
        assert max(errs) <= tol, (sched, errs)
        for g, cut in ((dq, dead_q), (dk, dead_k), (dv, dead_k)):
            gz = (g.float() == 0).all(dim=-1).cpu().numpy()   # [B, H, N]
            assert np.all(gz[:, :, cut]), "rows the mask cuts off must be exactly zero"
        outs[sched] = (dq, dk, dv)
    return dev, lse, delta, kw, outs


@pytest.mark.parametrize("window", [300, 128, 1])
def test_causal_window_bf16(window):
    _run(1, 3, 1024, 128, "bf16", True, window, None, 5000 + window)


def test_causal_window_d64_bf16():
    _run(2, 2, 1152, 64, "bf16", True, 257, None, 5100)


def test_bidirectional_window_bf16():
    _run(1, 2, 1024, 128, "bf16", False, 200, None, 5200)


@pytest.mark.parametrize("causal", [False, True])
def test_block_mask_bf16(causal):
    _run(1, 2, 1024, 128, "bf16", causal, 0, BLOCK8, 5300 + causal)


@pytest.mark.parametrize("causal", [False, True])
def test_block_mask_with_dead_tiles_bf16(causal):
    _run(1, 2, 1024, 64, "bf16", causal, 0, DEAD8, 5400 + causal)


def test_window_and_block_f32():
    blk = np.ones((4, 4), dtype=bool)
    blk[3, 1] = False
    _run(1, 2, 512, 64, "f32", True, 150, blk, 5500)


def test_window_f32_d128():
    _run(1, 2, 384, 128, "f32", False, 70, None, 5600)


def test_coarse_block_mask_with_window_leaves_rows_empty_bf16():
    """A block mask that hides the diagonal blocks plus a narrow causal
    window: some query rows see no key at all inside live tiles."""
    blk = np.tril(np.ones((8, 8), dtype=bool), -1)
    blk[0, 0] = True
    _run(1, 2, 1024, 128, "bf16", True, 100, blk, 5700)


@pytest.mark.parametrize("causal,window,block", [(True, 300, None), (False, 0, BLOCK8)])
def test_masked_determinism_and_bit_relations(causal, window, block):
    dev, lse, delta, kw, outs = _run(2, 4, 1024, 128, "bf16", causal, window, block, 5800,
                                     schedules=["atomic", "naive", "descending", "shift"])
    iv = lambda t: t.view(torch.int16)
    assert torch.equal(iv(outs["naive"][0]), iv(outs["descending"][0]))
    assert torch.equal(iv(outs["naive"][1]), iv(outs["atomic"][1]))
    assert torch.equal(iv(outs["naive"][2]), iv(outs["atomic"][2]))
    for sched in ("naive", "descending", "shift"):
        ws = D.alloc_workspace(dev["q"], causal, sched)
        for run in range(10):
            out = D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, schedule=sched,
                             causal=causal, workspace=ws, **kw)
            for a, b in zip(outs[sched], out):
                assert torch.equal(iv(a), iv(b)), (sched, run)
        D.attn_bwd_status(ws)
        log(f"  {sched}: 10 further runs identical")


def test_block_mask_unit_order_changes_no_bit():
    """The block-sparse case the unit-major order is for: same bits either way."""
    dev, lse, delta, kw, outs = _run(1, 8, 1024, 128, "bf16", True, 0, BLOCK8, 5900,
                                     schedules=["descending"])
    for sched in ("naive", "descending"):
        ref = None
        for order in (1, 2, 0):
            out = D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, schedule=sched,
                             causal=True, debug={"unit_order": order}, **kw)
            if ref is None:
                ref = [t.clone() for t in out]
                continue
            for x, y in zip(ref, out):
                assert torch.equal(x.view(torch.int16), y.view(torch.int16)), (sched, order)


@pytest.mark.parametrize("sched", ["atomic", "naive", "descending", "shift", "auto"])
def test_mask_that_hides_everything(sched):
    """No visible pair at all: O = 0, LSE = -inf, and every gradient is
    exactly zero (no unit runs; the cleared tiles are all of them)."""
    require_gpu()
    B, H, N, d = 1, 2, 512, 128
    blk = np.zeros((4, 4), dtype=bool)
    dev, _ = device_inputs(B, H, N, d, "bf16", 6100)
    o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True, block_mask=blk)
    assert torch.all(o.float() == 0) and torch.all(torch.isneginf(lse))
    delta = D.attn_bwd_preprocess(o, dev["do"])
    outs = tuple(torch.full_like(dev["q"], 3.0) for _ in range(3))
    D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, schedule=sched, causal=True,
               block_mask=blk, out=outs)
    torch.cuda.synchronize()
    for t in outs:
        assert torch.all(t.float() == 0)


def _bf16_rne(x32):
    u = x32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("block,causal", [(BLOCK8, True), (DEAD8, False)])
def test_timed_shift_order_replay(block, causal):
    """SHIFT on a block mask (the timed shift): dQ equals a host fp32 sum of
    the kernel's own partials in the rank order of the tables the launch
    ran (fetched for this device's co-resident count), bit for bit; head
    by head, unit-major and jittered timing give the same bits."""
    require_gpu()
    B, H, N, d = 1, 16, 1024, 128
    log(f"timed shift replay causal={causal} block={block.shape}")
    bs = N // block.shape[0]
    kw = dict(block_mask=block, block_size=bs)
    dev, _ = device_inputs(B, H, N, d, "bf16", 6300)
    o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, **kw)
    delta = D.attn_bwd_preprocess(o, dev["do"])
    t = D.mask_schedule_tables(B, H, N, d, "bf16", causal, "shift", slots=0, **kw)
    assert t["slots_per_head"] >= 1 and not t["static"]
    n = t["n"]
    tile = N // n
    partials = torch.zeros((B * H, n, N, d), dtype=torch.float32, device="cuda")
    ws = D.alloc_workspace(dev["q"], causal, "shift", **kw)
    dq, _, _ = D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, schedule="shift",
                          causal=causal, workspace=ws, debug={"partials": partials}, **kw)
    D.attn_bwd_status(ws)
    part = partials.cpu().numpy()
    rank = t["rank"]
    acc = np.zeros((B * H, N, d), dtype=np.float32)
    for qb in range(n):
        rows = slice(qb * tile, (qb + 1) * tile)
        for _, kv in sorted((rank[qb, kv], kv) for kv in range(n) if rank[qb, kv] >= 0):
            acc[:, rows] = acc[:, rows] + part[:, kv, rows]
    want = _bf16_rne((acc * np.float32(1.0 / np.sqrt(d))).astype(np.float32))
    seen = (rank >= 0).any(axis=1)
    for qb in range(n):
        if not seen[qb]:
            want[:, qb * tile:(qb + 1) * tile] = 0
    got = dq.reshape(B * H, N, d).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)
    ref = D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, schedule="shift",
                     causal=causal, workspace=ws, **kw)
    for dbg in ({"unit_order": 1}, {"unit_order": 2}, {"jitter_seed": 9},
                {"placement": 1}):
        out = D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, schedule="shift",
                         causal=causal, workspace=ws, debug=dbg, **kw)
        D.attn_bwd_status(ws)
        for a, b in zip(ref, out):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), dbg
