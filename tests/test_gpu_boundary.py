"""GPU checks of the C-ABI boundary's conventions: the library allocates no
device memory (not even for a shape, mask or schedule it has not seen
before), the schedule tables it runs live in the caller's workspace, and
the status word is read with dash_status_query after the stream was
synchronized."""
import numpy as np
import pytest
import torch

import deterministic_attention_backward_attn_amd as D
from tests.gpu_common import device_inputs, log, require_gpu

pytestmark = pytest.mark.gpu


def _free_bytes():
    torch.cuda.synchronize()
    return torch.cuda.mem_get_info()[0]


def test_first_seen_shapes_allocate_no_device_memory():
    require_gpu()
    # load every kernel the cases run once (code-object loading and the
    # scratch a kernel's first launch sets up are the runtime's, not ours):
    # d = 128 runs the two-stage pipeline, d = 64 the one-stage kernel, each
    # with and without masked pairs, ordered and atomic
    for d in (64, 128):
        dev, _ = device_inputs(1, 2, 512, d, "bf16", 3100)
        for causal in (True, False):
            o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal)
            for sched in ("shift", "atomic"):
                D.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, schedule=sched,
                           causal=causal)
    torch.cuda.synchronize()
    block = np.random.default_rng(5).random((6, 6)) < 0.5
    cases = [dict(causal=True), dict(causal=False), dict(causal=True, window=300),
             dict(causal=False, block_mask=block)]
    for i, mk in enumerate(cases):
        B, H, N, d = 1, 3, 768, 64 + 64 * (i % 2)
        log(f"boundary case {mk} B={B} H={H} N={N} d={d}")
        dev, _ = device_inputs(B, H, N, d, "bf16", 3200 + i)
        causal = mk.pop("causal")
        o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, **mk)
        delta = D.attn_bwd_preprocess(o, dev["do"])
        for sched in ("naive", "descending", "shift", "atomic", "auto"):
            ws = D.alloc_workspace(dev["q"], causal, sched, **mk)
            out = tuple(torch.empty_like(dev["q"]) for _ in range(3))
            before = _free_bytes()
            D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, schedule=sched,
                       causal=causal, workspace=ws, out=out, **mk)
            after = _free_bytes()
            D.status_query(ws)
            assert after == before, (mk, sched, before - after)


def test_status_query_reports_a_forced_time_out():
    require_gpu()
    dev, _ = device_inputs(1, 2, 512, 128, "bf16", 3300)
    o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    delta = D.attn_bwd_preprocess(o, dev["do"])
    ws = D.alloc_workspace(dev["q"], True, "naive")
    # the first contributor of Q sub-tile 2 of head 0 waits for a counter
    # value that never comes; the bounded spin gives up and sets the word
    D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, schedule="naive",
               causal=True, workspace=ws, debug=dict(poison_q=3, spin_limit=2000))
    torch.cuda.synchronize()
    with pytest.raises(D.DashError) as e:
        D.status_query(ws)
    assert e.value.code == 6
    # the next launch clears the word
    D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, schedule="naive",
               causal=True, workspace=ws)
    torch.cuda.synchronize()
    D.status_query(ws)
