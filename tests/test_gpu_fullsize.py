"""GPU parity at the workloads' full sizes, in the launch configuration the
bench times, on sampled rows the oracle computes one by one.

For each full-size workload and mask (the sliding-window and block-sparse
workloads included), every schedule (auto too) runs the whole backward on
the GPU; for eight heads the oracle computes the forward statistics and
then O, LSE, dQ, dK and dV at rows on tile edges, at the middle and at the
ends of the sequence.  The ordered schedules deal heads round-robin to the
8 XCD groups (head b*H + h to group (b*H + h) mod 8), so the eight heads are
one per group, from the first head to the last.  Error metric:
max|gpu - oracle| / max|oracle| over the sampled rows of each tensor,
bound 2e-2 (bf16 inputs and outputs, fp32 accumulation).
"""
import numpy as np
import pytest
import torch

import deterministic_attention_backward_attn_amd as D
from oracle import attention as A
from synth import WORKLOADS, exact_of, make_storage
from tests.gpu_common import TOL, log, require_gpu, to_device

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

CASES = [("b4h32_n4k_d128_full", "full"), ("b1h32_n16k_d128_causal", "causal"),
         ("b8h64_n8k_d64", "causal"), ("b8h64_n8k_d64", "full"),
         ("b1h32_n16k_d128_swa4k", "causal"), ("b1h32_n16k_d128_blocksparse", "causal")]


def _rows(n):
    r = [0, 1, 127, 128, n // 2 - 1, n // 2, n - 129, n - 128, n - 2, n - 1]
    return sorted(set(r))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wl,mask", CASES)
def test_full_size_sampled_rows(wl, mask):
    require_gpu()
    w = WORKLOADS[wl]
    causal = mask == "causal"
    log(f"full size {wl} {mask}: generating inputs")
    host = make_storage(w.B, w.H, w.N, w.d, w.dtype, w.seed_base)
    dev = {k: to_device(v, w.dtype) for k, v in host.items()}
    mkw = w.mask_args()
    mask = (A.Mask(causal=causal, window=mkw["window"], block=mkw["block_mask"],
                   block_size=mkw["block_size"]) if (w.window or w.block_spec) else causal)
    o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, **mkw)
    delta = D.attn_bwd_preprocess(o, dev["do"])
    rows = _rows(w.N)
    scale = 1.0 / np.sqrt(w.d)
    bh = w.B * w.H
    # one head per XCD group: flat index i (mod 8) from 0 up to bh - 1
    flat = [i + 8 * ((bh // 8 - 1) * i // 7) for i in range(8)]
    assert flat[0] == 0 and flat[-1] == bh - 1 and len({f % 8 for f in flat}) == 8
    heads = [divmod(f, w.H) for f in flat]
    refs = {}
    for (b, h) in heads:
        ex = {k: exact_of(host[k][b, h], w.dtype) for k in host}
        rq, rk, rv, ro, rl = A.sampled_backward(ex["q"], ex["k"], ex["v"], ex["do"], mask, scale,
                                                rows, rows, with_forward=True)
        refs[(b, h)] = (rq, rk, rv)
        # the forward at the same rows
        for name, gpu, ref in (("O", o[b, h, rows], ro), ("LSE", lse[b, h, rows], rl)):
            g = gpu.float().cpu().numpy().astype(np.float64)
            err = float(np.max(np.abs(g - ref)) / max(np.max(np.abs(ref)), 1e-30))
            assert err <= TOL[w.dtype], (name, (b, h), err)
        log(f"  oracle head ({b},{h}) done; forward rows match")
    ws = D.alloc_workspace(dev["q"], causal, "naive")
    for sched in ("atomic", "naive", "descending", "shift", "auto"):
        dq, dk, dv = D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta,
                                schedule=sched, causal=causal, workspace=ws, **mkw)
        D.attn_bwd_status(ws)
        worst = 0.0
        for (b, h), (rq, rk, rv) in refs.items():
            for name, gpu, ref in (("dQ", dq[b, h, rows], rq), ("dK", dk[b, h, rows], rk),
                                   ("dV", dv[b, h, rows], rv)):
                g = gpu.float().cpu().numpy().astype(np.float64)
                err = float(np.max(np.abs(g - ref)) / max(np.max(np.abs(ref)), 1e-30))
                assert err <= TOL[w.dtype], (sched, (b, h), name, err)
                worst = max(worst, err)
        log(f"  {sched}: sampled rows, worst relative error {worst:.2e}")
