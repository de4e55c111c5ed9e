"""Pins for the oracle's masks (CPU only): sliding windows and block masks.

Each check ties the masked oracle to something other than its own mask
code: per-element definitions written as plain loops, reductions to the
plain causal and full cases, closed forms (a window of one key), the
composition of independent problems (a block-diagonal mask is one full
problem per block; a query block that sees nothing drops out), torch's
float64 autograd with masks built from torch's own triangle routines, and
finite differences of <dO, O>.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from synth import gaussian

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _inputs(n, d, seed, h=1):
    return tuple(gaussian((1, h, n, d), seed + i) for i in range(4))


def _visible_loop(m, n):
    out = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for j in range(n):
            ok = True
            if m.causal and j > i:
                ok = False
            if m.window:
                dist = i - j if m.causal else abs(i - j)
                if dist >= m.window:
                    ok = False
            if m.block is not None and not m.block[i // m.block_size][j // m.block_size]:
                ok = False
            out[i, j] = ok
    return out


def _masks(n=24):
    rng = np.random.default_rng(5)
    blk = rng.random((n // 4, n // 4)) < 0.6
    return [
        A.Mask(causal=True, window=5),
        A.Mask(causal=False, window=4),
        A.Mask(causal=False, block=blk, block_size=4),
        A.Mask(causal=True, block=blk, block_size=4),
        A.Mask(causal=True, window=7, block=blk, block_size=4),
    ]


def test_visible_matches_elementwise_definition():
    n = 24
    for m in _masks(n):
        assert np.array_equal(m.visible(np.arange(n), np.arange(n)), _visible_loop(m, n))


@pytest.mark.parametrize("causal", [False, True])
def test_window_covering_everything_is_the_plain_mask(causal):
    q, k, v, do = _inputs(40, 8, 101)
    ref = A.backward(q, k, v, do, causal, 0.3)
    fo, fl = A.forward(q, k, v, causal, 0.3)
    for w in (40, 41, 1000):
        m = A.Mask(causal=causal, window=w)
        got = A.backward(q, k, v, do, m, 0.3)
        o, lse = A.forward(q, k, v, m, 0.3)
        assert np.array_equal(o, fo) and np.array_equal(lse, fl)
        for a, b in zip(ref, got):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_window_of_one_key_closed_form(causal):
    """Each query sees only its own key: P = I, O = V, LSE_i = s<q_i, k_i>,
    dV = dO, and dS = P (dP - D) = 0 so dQ = dK = 0."""
    q, k, v, do = _inputs(20, 8, 111)
    m = A.Mask(causal=causal, window=1)
    o, lse = A.forward(q, k, v, m, 0.4)
    assert np.allclose(o, v, rtol=0, atol=1e-15)
    assert np.allclose(lse[0, 0], 0.4 * np.sum(q[0, 0] * k[0, 0], axis=1), rtol=0, atol=1e-14)
    dq, dk, dv = A.backward(q, k, v, do, m, 0.4)
    assert np.allclose(dv, do, rtol=0, atol=1e-15)
    assert np.max(np.abs(dq)) < 1e-14 and np.max(np.abs(dk)) < 1e-14


def test_block_diagonal_mask_is_independent_full_problems():
    n, bs = 24, 6
    q, k, v, do = _inputs(n, 8, 121)
    m = A.Mask(block=np.eye(n // bs, dtype=bool), block_size=bs)
    dq, dk, dv = A.backward(q, k, v, do, m, 0.35)
    o, lse = A.forward(q, k, v, m, 0.35)
    for b in range(n // bs):
        sl = slice(b * bs, (b + 1) * bs)
        part = [x[:, :, sl] for x in (q, k, v, do)]
        ro, rl = A.forward(*part[:3], False, 0.35)
        rq, rk, rv = A.backward(*part, False, 0.35)
        assert np.allclose(o[:, :, sl], ro, rtol=0, atol=1e-13)
        assert np.allclose(lse[:, :, sl], rl, rtol=0, atol=1e-13)
        for a, r in ((dq, rq), (dk, rk), (dv, rv)):
            assert np.allclose(a[:, :, sl], r, rtol=0, atol=1e-13)


def test_lower_triangular_blocks_with_causal_is_causal():
    n, bs = 32, 8
    q, k, v, do = _inputs(n, 8, 131)
    m = A.Mask(causal=True, block=np.tril(np.ones((4, 4), dtype=bool)), block_size=bs)
    for a, b in zip(A.backward(q, k, v, do, m, 0.3), A.backward(q, k, v, do, True, 0.3)):
        assert np.array_equal(a, b)


def test_query_block_that_sees_nothing_drops_out():
    """A dead query block: O = 0, LSE = -inf, dQ = 0 there, and dK, dV equal
    those of the problem without those queries."""
    n, bs = 24, 6
    q, k, v, do = _inputs(n, 8, 141)
    blk = np.ones((4, 4), dtype=bool)
    blk[2, :] = False
    m = A.Mask(block=blk, block_size=bs)
    o, lse = A.forward(q, k, v, m, 0.3)
    dq, dk, dv = A.backward(q, k, v, do, m, 0.3)
    dead = slice(12, 18)
    assert np.all(o[:, :, dead] == 0) and np.all(np.isneginf(lse[:, :, dead]))
    assert np.all(dq[:, :, dead] == 0)
    keep = np.r_[0:12, 18:24]
    # the reduced problem: 18 queries against all 24 keys (rectangular), by
    # explicit softmax in torch float64
    tq = torch.tensor(q[0, 0, keep], requires_grad=True)
    tk = torch.tensor(k[0, 0], requires_grad=True)
    tv = torch.tensor(v[0, 0], requires_grad=True)
    (torch.softmax(0.3 * (tq @ tk.T.contiguous()), dim=-1) @ tv).backward(
        torch.tensor(do[0, 0, keep]))
    assert np.allclose(dk[0, 0], tk.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(dv[0, 0], tv.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(dq[0, 0, keep], tq.grad.numpy(), rtol=0, atol=1e-12)


def _torch_mask(n, causal, window, block, bs):
    full = torch.ones(n, n, dtype=torch.bool)
    m = full.clone()
    if causal:
        m &= full.tril()
        if window:
            m &= full.triu(-(window - 1))
    elif window:
        m &= full.tril(window - 1) & full.triu(-(window - 1))
    if block is not None:
        m &= torch.kron(torch.tensor(block, dtype=torch.int64),
                        torch.ones(bs, bs, dtype=torch.int64)).bool()
    return m


@pytest.mark.parametrize("case", range(5))
def test_masked_backward_against_torch_autograd(case):
    n, d, bs = 24, 8, 4
    m = _masks(n)[case]
    q, k, v, do = _inputs(n, d, 151 + case, h=2)
    tm = _torch_mask(n, m.causal, m.window, m.block, bs)
    live_rows = tm.any(dim=1).numpy()
    dq, dk, dv = A.backward(q, k, v, do, m, 0.31)
    o, lse = A.forward(q, k, v, m, 0.31)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = (0.31 * torch.matmul(tq, tk.transpose(-1, -2).contiguous())).masked_fill(~tm, float("-inf"))
    p = torch.softmax(s, dim=-1).nan_to_num(0.0)   # fully masked rows: P = 0
    to = p @ tv
    to.backward(torch.tensor(do))
    assert np.allclose(o, to.detach().numpy(), rtol=0, atol=1e-13)
    ref_lse = torch.logsumexp(s, dim=-1).detach().numpy()
    assert np.allclose(lse[..., live_rows], ref_lse[..., live_rows], rtol=0, atol=1e-13)
    assert np.all(np.isneginf(lse[..., ~live_rows]))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        ref = ref.numpy()
        assert np.max(np.abs(mine - ref)) <= 1e-12 * np.max(np.abs(ref))


def _loss(q, k, v, do, m, scale):
    o, _ = A.forward(q, k, v, m, scale)
    return float(np.sum(do * o))


@pytest.mark.parametrize("case", [0, 1, 4])
def test_masked_finite_differences(case):
    n, d = 16, 4
    rng = np.random.default_rng(9)
    ms = [A.Mask(causal=True, window=5), A.Mask(window=3),
          None, None, A.Mask(causal=True, window=6, block=rng.random((4, 4)) < 0.7, block_size=4)]
    m = ms[case]
    q, k, v, do = _inputs(n, d, 161 + case)
    dq, dk, dv = A.backward(q, k, v, do, m, 0.5)
    inputs = {"q": q, "k": k, "v": v}
    for name, g in (("q", dq), ("k", dk), ("v", dv)):
        fd = np.zeros_like(g)
        for idx in np.ndindex(g.shape):
            args = dict(inputs)
            x = args[name].copy()
            x[idx] += 1e-5
            args[name] = x
            lp = _loss(args["q"], args["k"], args["v"], do, m, 0.5)
            x[idx] -= 2e-5
            lm = _loss(args["q"], args["k"], args["v"], do, m, 0.5)
            fd[idx] = (lp - lm) / 2e-5
        assert np.max(np.abs(fd - g)) <= 1e-6 * np.max(np.abs(g)), name


@pytest.mark.parametrize("case", range(5))
def test_masked_sampled_rows_match_whole_backward(case):
    n = 24
    m = _masks(n)[case]
    q, k, v, do = (x[0, 0] for x in _inputs(n, 8, 171 + case))
    dq, dk, dv = A.backward(q[None, None], k[None, None], v[None, None], do[None, None], m, 0.3)
    rows = [0, 3, 4, 11, 12, 23]
    sq, sk, sv, so, sl = A.sampled_backward(q, k, v, do, m, 0.3, rows, rows[::-1],
                                            with_forward=True)
    fo, fl = A.forward(q[None, None], k[None, None], v[None, None], m, 0.3)
    assert np.array_equal(so, fo[0, 0, rows]) and np.array_equal(sl, fl[0, 0, rows])
    assert np.allclose(sq, dq[0, 0, rows], rtol=0, atol=1e-13)
    assert np.allclose(sk, dk[0, 0, rows[::-1]], rtol=0, atol=1e-13)
    assert np.allclose(sv, dv[0, 0, rows[::-1]], rtol=0, atol=1e-13)
