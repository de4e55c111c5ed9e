"""Pins for the fp64 attention oracle (CPU only).

Each check ties the oracle to something other than itself: central finite
differences of the scalar loss <dO, O>, the softmax-backward identity
sum_j dS_ij = 0, causal zero patterns, closed forms, and torch's float64
autograd of explicit softmax attention.  A dropped term, a wrong sign, a
wrong index or a transposed operand in the oracle fails at least one of them
(see test_planted_mistakes_are_caught).
"""
import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention as A
from synth import gaussian

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _loss(q, k, v, do, causal, scale):
    o, _ = A.forward(q, k, v, causal, scale)
    return float(np.sum(do * o))


def _small(n=16, d=8, seed=7, h=1):
    q = gaussian((1, h, n, d), seed)
    k = gaussian((1, h, n, d), seed + 1)
    v = gaussian((1, h, n, d), seed + 2)
    do = gaussian((1, h, n, d), seed + 3)
    return q, k, v, do


def _fd_grad(x_name, idx, inputs, causal, scale, eps=1e-5):
    args = {k: v.copy() for k, v in inputs.items()}
    args[x_name][idx] += eps
    lp = _loss(args["q"], args["k"], args["v"], args["do"], causal, scale)
    args[x_name][idx] -= 2 * eps
    lm = _loss(args["q"], args["k"], args["v"], args["do"], causal, scale)
    return (lp - lm) / (2 * eps)


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences_all_elements(causal):
    q, k, v, do = _small()
    scale = 0.37
    dq, dk, dv = A.backward(q, k, v, do, causal, scale)
    inputs = {"q": q, "k": k, "v": v, "do": do}
    for name, g in (("q", dq), ("k", dk), ("v", dv)):
        fd = np.zeros_like(g)
        for idx in np.ndindex(g.shape):
            fd[idx] = _fd_grad(name, idx, inputs, causal, scale)
        err = np.max(np.abs(fd - g)) / np.max(np.abs(g))
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences_sampled_tiny_workload(causal):
    """200 sampled elements per gradient at the 1x2x256x64 shape."""
    rng = np.random.default_rng(11)
    q, k, v, do = (gaussian((1, 2, 256, 64), 1000 + i) for i in range(4))
    scale = 1.0 / 8.0
    dq, dk, dv = A.backward(q, k, v, do, causal, scale)
    inputs = {"q": q, "k": k, "v": v, "do": do}
    for name, g in (("q", dq), ("k", dk), ("v", dv)):
        gmax = np.max(np.abs(g))
        for _ in range(200):
            idx = tuple(int(rng.integers(0, s)) for s in g.shape)
            fd = _fd_grad(name, idx, inputs, causal, scale)
            assert abs(fd - g[idx]) / gmax < 1e-6, (name, idx)


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_backward_row_identity(causal):
    q, k, v, do = (x[0, 0] for x in _small(n=64, d=16, seed=3))
    it = A.backward_intermediates(q, k, v, do, causal, 0.25)
    row_sum = np.sum(it["dS"], axis=1)
    # rounding scale of the two terms that cancel: sum_j P_ij dP_ij and D_i
    bound = 1e-12 * (np.sum(it["P"] * np.abs(it["dP"]), axis=1) + np.abs(it["D"]))
    assert np.all(np.abs(row_sum) <= bound)
    # consequence: sum_j dK_j = s * sum_i (sum_j dS_ij) Q_i = 0
    assert np.max(np.abs(np.sum(it["dK"], axis=0))) < 1e-12 * np.max(np.abs(it["dK"])) * 64
    # probabilities normalise
    assert np.allclose(np.sum(it["P"], axis=1), 1.0, rtol=0, atol=1e-14)


def test_dk_column_sum_zero_batched():
    q, k, v, do = _small(n=48, d=8, seed=21, h=3)
    for causal in (False, True):
        _, dk, _ = A.backward(q, k, v, do, causal, 0.5)
        s = np.sum(dk, axis=2)
        assert np.max(np.abs(s)) < 1e-12 * np.max(np.abs(dk)) * 48


def test_causal_zero_patterns():
    q, k, v, do = (x[0, 0] for x in _small(n=32, d=8, seed=5))
    it = A.backward_intermediates(q, k, v, do, True, 0.3)
    upper = np.triu(np.ones((32, 32), dtype=bool), 1)
    assert np.all(it["P"][upper] == 0.0)
    assert np.all(it["dS"][upper] == 0.0)
    # the first query sees one key: P = 1 and dS = dP - D = 0, so dQ_0 = 0
    # (up to the rounding of dO_0.V_0 against dO_0.O_0)
    assert it["P"][0, 0] == 1.0
    assert np.max(np.abs(it["dQ"][0])) < 1e-13 * np.max(np.abs(it["dQ"]))


def test_causal_dk_dv_ignore_earlier_queries():
    """dK_j and dV_j depend only on queries i >= j under a causal mask."""
    q, k, v, do = _small(n=24, d=8, seed=9)
    _, dk, dv = A.backward(q, k, v, do, True, 0.4)
    j = 10
    q2, do2 = q.copy(), do.copy()
    q2[0, 0, :j] += gaussian((j, 8), 99)
    do2[0, 0, :j] += gaussian((j, 8), 98)
    _, dk2, dv2 = A.backward(q2, k, v, do2, True, 0.4)
    assert np.array_equal(dk[0, 0, j:], dk2[0, 0, j:])
    assert np.array_equal(dv[0, 0, j:], dv2[0, 0, j:])
    assert not np.array_equal(dk[0, 0, :j], dk2[0, 0, :j])


@pytest.mark.parametrize("causal", [False, True])
def test_closed_form_zero_queries(causal):
    n, d = 40, 8
    _, k, v, do = _small(n=n, d=d, seed=13)
    q = np.zeros_like(k)
    o, lse = A.forward(q, k, v, causal, 0.7)
    dq, dk, dv = A.backward(q, k, v, do, causal, 0.7)
    cnt = np.arange(1, n + 1) if causal else np.full(n, n)
    assert np.allclose(lse[0, 0], np.log(cnt), rtol=0, atol=1e-13)
    vv, dd = v[0, 0], do[0, 0]
    if causal:
        mean_v = np.cumsum(vv, axis=0) / cnt[:, None]
        # dV_j = sum_{i >= j} dO_i / (i + 1)
        w = dd / cnt[:, None]
        dv_ref = np.cumsum(w[::-1], axis=0)[::-1]
    else:
        mean_v = np.broadcast_to(vv.mean(axis=0), vv.shape)
        dv_ref = np.broadcast_to(dd.sum(axis=0) / n, vv.shape)
    assert np.allclose(o[0, 0], mean_v, rtol=0, atol=1e-13)
    assert np.all(dk == 0.0)
    assert np.allclose(dv[0, 0], dv_ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_closed_form_constant_values(causal):
    """All V rows equal: O = V_0, dS = 0, so dQ = dK = 0 up to rounding."""
    q, k, v, do = _small(n=32, d=8, seed=17)
    v = np.broadcast_to(v[:, :, :1, :], v.shape).copy()
    o, _ = A.forward(q, k, v, causal, 0.5)
    assert np.allclose(o, v, rtol=0, atol=1e-14)
    dq, dk, dv = A.backward(q, k, v, do, causal, 0.5)
    assert np.max(np.abs(dq)) < 1e-13
    assert np.max(np.abs(dk)) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_forward_against_scipy(causal):
    q, k, v, _ = (x[0, 0] for x in _small(n=50, d=16, seed=23))
    o, lse = A.forward(q[None, None], k[None, None], v[None, None], causal, 0.25)
    s = 0.25 * q @ k.T
    if causal:
        s = np.where(np.tril(np.ones_like(s, dtype=bool)), s, -np.inf)
    assert np.allclose(lse[0, 0], scipy.special.logsumexp(s, axis=1), rtol=0, atol=1e-13)
    assert np.allclose(o[0, 0], scipy.special.softmax(s, axis=1) @ v, rtol=0, atol=1e-13)
    assert np.all(lse[0, 0] >= np.max(s, axis=1))


@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_autograd_float64(causal):
    q, k, v, do = _small(n=33, d=12, seed=31, h=2)
    scale = 0.29
    dq, dk, dv = A.backward(q, k, v, do, causal, scale)
    o, lse = A.forward(q, k, v, causal, scale)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = scale * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
    if causal:
        mask = torch.ones(33, 33, dtype=torch.bool).tril()
        s = s.masked_fill(~mask, float("-inf"))
    to = torch.softmax(s, dim=-1) @ tv
    to.backward(torch.tensor(do, dtype=torch.float64))
    assert np.allclose(o, to.detach().numpy(), rtol=0, atol=1e-13)
    assert np.allclose(lse, torch.logsumexp(s, dim=-1).detach().numpy(), rtol=0, atol=1e-13)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        ref = ref.numpy()
        assert np.max(np.abs(mine - ref)) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_rows_against_torch_autograd(causal):
    """The row-by-row backward used for full-length checks equals torch's
    float64 autograd at the requested rows (first, last, tile edges)."""
    n, d, scale = 150, 16, 0.21
    q, k, v, do = (x[0, 0] for x in _small(n=n, d=d, seed=57))
    rows = [0, 1, 63, 64, 127, 128, 149]
    dq, dk, dv = A.sampled_backward(q, k, v, do, causal, scale, rows, rows[::-1])
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    sc = scale * (tq @ tk.T.contiguous())
    if causal:
        sc = sc.masked_fill(~torch.ones(n, n, dtype=torch.bool).tril(), float("-inf"))
    (torch.softmax(sc, dim=-1) @ tv).backward(torch.tensor(do, dtype=torch.float64))
    for mine, ref in ((dq, tq.grad.numpy()[rows]), (dk, tk.grad.numpy()[rows[::-1]]),
                      (dv, tv.grad.numpy()[rows[::-1]])):
        assert np.max(np.abs(mine - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_row_chunking_matches_whole(monkeypatch):
    """Chunked rows equal whole-matrix rows (the chunk is a plain slice)."""
    q, k, v, do = _small(n=100, d=8, seed=41)
    ref = A.backward(q, k, v, do, True, 0.3)
    monkeypatch.setattr(A, "_ROW_CHUNK", 7)
    got = A.backward(q, k, v, do, True, 0.3)
    for a, b in zip(ref, got):
        assert np.allclose(a, b, rtol=0, atol=1e-13)


def _plant(monkeypatch, which):
    """Plant one plausible mistake in the oracle (CPU only)."""
    orig_head = A._head_backward

    def wrong_head(q, k, v, o, do, lse, causal, scale):
        dq, dk, dv = orig_head(q, k, v, o, do, lse, causal, scale)
        if which == "drop_D":
            d_row = np.sum(do * o, axis=1)
            p = A._probs(A._scores(q, k, scale, 0, causal), lse)
            dq = dq + scale * ((p * d_row[:, None]) @ k)
        elif which == "transpose_dv":
            dv = dv.T[: dv.shape[0], : dv.shape[1]] if dv.shape[0] == dv.shape[1] else dv[::-1]
        elif which == "sign_dk":
            dk = -dk
        elif which == "no_scale_dq":
            dq = dq / scale
        elif which == "shift_index":
            dk = np.roll(dk, 1, axis=0)
        return dq, dk, dv

    monkeypatch.setattr(A, "_head_backward", wrong_head)


@pytest.mark.parametrize("which", ["drop_D", "transpose_dv", "sign_dk", "no_scale_dq", "shift_index"])
def test_planted_mistakes_are_caught(monkeypatch, which):
    q, k, v, do = _small(n=8, d=8, seed=3)
    scale = 0.37
    _plant(monkeypatch, which)
    dq, dk, dv = A.backward(q, k, v, do, False, scale)
    inputs = {"q": q, "k": k, "v": v, "do": do}
    worst = 0.0
    for name, g in (("q", dq), ("k", dk), ("v", dv)):
        for idx in np.ndindex(g.shape):
            fd = _fd_grad(name, idx, inputs, False, scale)
            worst = max(worst, abs(fd - g[idx]) / max(np.max(np.abs(g)), 1e-30))
    assert worst > 1e-3, which
