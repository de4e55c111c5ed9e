"""The allocation-free backward (dash_attn_bwd_noalloc) against dash_attn_bwd
on the same inputs, through the C ABI: bit-identical dQ, dK, dV for every
ordered schedule and the oracle's tolerance for the atomic reference, on
two calls in a row, the second with a smaller input (the built-in array
keeps the first call's contents).  No device memory is allocated by the
call, and its status word reads clean."""
import pytest
import torch

import deterministic_attention_backward_attn_amd as D
from tests.gpu_common import TOL, device_inputs, log, rel_err, require_gpu

pytestmark = pytest.mark.gpu

CASES = [(2, 16, 2048, 128, True, 7100), (1, 2, 512, 64, False, 7200)]


def _prep(B, H, N, d, causal, seed):
    dev, _ = device_inputs(B, H, N, d, "bf16", seed)
    o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal)
    delta = D.attn_bwd_preprocess(o, dev["do"])
    return dev, lse, delta


def _load_scratch():
    """The first call on a GPU loads the code object that holds the built-in
    array (the runtime's one-time allocation of it); later calls allocate
    nothing."""
    dev, lse, delta = _prep(1, 1, 128, 64, True, 7000)
    D.attn_bwd_noalloc(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, causal=True)
    torch.cuda.synchronize()


@pytest.mark.parametrize("schedule", ["naive", "descending", "shift", "auto", "atomic"])
def test_noalloc_matches_the_workspace_entry_point(schedule):
    require_gpu()
    _load_scratch()
    for B, H, N, d, causal, seed in CASES:
        log(f"noalloc {schedule} B={B} H={H} N={N} d={d} causal={causal} seed={seed}")
        dev, lse, delta = _prep(B, H, N, d, causal, seed)
        ref = D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta,
                         schedule=schedule, causal=causal)
        out = tuple(torch.full_like(dev["q"], 7.0) for _ in range(3))
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        got = D.attn_bwd_noalloc(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta,
                                 schedule=schedule, causal=causal, out=out)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0
        D.status_query("noalloc")
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            if schedule == "atomic":
                err = rel_err(g, r.float().cpu().numpy())
                assert err <= TOL["bf16"], (name, err)
            else:
                assert torch.equal(g.view(torch.int16), r.view(torch.int16)), name


def test_noalloc_refuses_what_it_cannot_hold():
    require_gpu()
    dev, lse, delta = _prep(1, 2, 512, 64, True, 7300)
    with pytest.raises(D.DashError) as e:
        D.attn_bwd_noalloc(*(torch.empty(1, 32, 4096, 128, dtype=torch.bfloat16, device="cuda")
                             for _ in range(4)),
                           torch.empty(1, 32, 4096, dtype=torch.float32, device="cuda"),
                           torch.empty(1, 32, 4096, dtype=torch.float32, device="cuda"),
                           schedule="naive", causal=True)
    assert e.value.code == 3  # 64 MiB accumulator alone: beyond the array
