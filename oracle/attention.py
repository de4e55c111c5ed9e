"""fp64 CPU oracle for softmax attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this module; the product path never does.

What it computes is the plain definition of the attention gradients.  The
DASH pages ("DASH: Deterministic Attention Scheduling for High-throughput
Reproducible LLM Training") change only the order and placement of the
backward's operations: the summary page (euno.news, "Results") states that
the schedules only reshuffle existing operations, and the explainer
(gist.science, "Technisches Resuemee" section 1 and section 3) places the
whole cost in how gradient reductions are scheduled, not in what they sum.
So the exact result (up to rounding order) is the textbook backward of
O = softmax(s * Q K^T) V, written out here step by step in float64:

  1. S_ij = s * <Q_i, K_j>           (masked to -inf where j > i if causal)
  2. LSE_i = m_i + ln sum_j exp(S_ij - m_i),  m_i = max_j S_ij
  3. P_ij = exp(S_ij - LSE_i)         (exactly 0 where masked)
  4. O_i = sum_j P_ij V_j
  5. D_i = <dO_i, O_i>
  6. dV_j = sum_i P_ij dO_i
  7. dP_ij = <dO_i, V_j>
  8. dS_ij = P_ij (dP_ij - D_i)
  9. dQ_i = s * sum_j dS_ij K_j ;  dK_j = s * sum_i dS_ij Q_i

The backward's inputs (Q, K, V, O, dO, LSE -> dQ, dK, dV) are the ones the
explainer's problem statement and the summary's method section name (the
backward's matrix products, score computation and gradient reduction).
Step 5 (the row-wise D) is not named on the pages; it is the identity
D_i = sum_j P_ij dP_ij, used because it needs only O and dO.

Rows are processed in chunks so that P is never formed whole for long
sequences; a chunk is a plain slice of the definition, not a reordering of
any sum (each row's sums run over the full key range in one matmul).

Masks.  ``causal`` may be a bool or a ``Mask``.  A Mask states which keys
each query sees: causal (key j only if j <= i), a sliding window of W keys
(causal: i - j < W; otherwise |i - j| < W) and a block mask (query block
i // bs and key block j // bs visible only where the block entry is
nonzero); all given constraints hold together.  The summary page
("Limitations and future work") names block-sparse and other special
masks as the coverage gap of full and causal; these definitions are this
project's reading of that item.  A row that sees no key has LSE = -inf,
P = 0 and O = 0, so its gradients are zero.

Pins (tests/test_oracle_attention.py): central finite differences of
L = <dO, O>; sum_j dS_ij = 0; sum_j dK_j = 0; causal zero patterns; the
closed forms for Q = 0 and for constant V rows; torch float64 autograd;
the sampled rows of ``sampled_backward`` against the whole backward.
"""
from __future__ import annotations

import numpy as np

__all__ = ["Mask", "forward", "backward", "backward_intermediates", "default_scale",
           "sampled_backward"]

_ROW_CHUNK = 1024


def default_scale(d: int) -> float:
    return 1.0 / np.sqrt(d)


class Mask:
    """Which keys each query sees (see the module notes)."""

    def __init__(self, causal: bool = False, window: int = 0, block=None,
                 block_size: int = 0):
        self.causal = bool(causal)
        self.window = int(window)
        self.block = None if block is None else np.asarray(block, dtype=bool)
        self.block_size = int(block_size)
        if self.window < 0:
            raise ValueError("window must be >= 0")
        if self.block is not None and self.block_size < 1:
            raise ValueError("a block mask needs block_size >= 1")

    def visible(self, rows, cols):
        """Boolean [len(rows), len(cols)]: query rows[a] sees key cols[b]."""
        i = np.asarray(rows, dtype=np.int64)[:, None]
        j = np.asarray(cols, dtype=np.int64)[None, :]
        vis = np.ones((i.shape[0], j.shape[1]), dtype=bool)
        if self.causal:
            vis &= j <= i
        if self.window:
            vis &= (i - j < self.window) if self.causal else (np.abs(i - j) < self.window)
        if self.block is not None:
            vis &= self.block[i // self.block_size, j // self.block_size]
        return vis

    def is_plain(self):
        return self.window == 0 and self.block is None


def _mask_of(causal) -> Mask:
    return causal if isinstance(causal, Mask) else Mask(causal=bool(causal))


def _scores(q_rows, k, scale, row0, causal):
    """Step 1 for a block of query rows starting at global row ``row0``."""
    s = scale * (q_rows @ k.T)
    mask = _mask_of(causal)
    if mask.causal or not mask.is_plain():
        vis = mask.visible(np.arange(row0, row0 + s.shape[0]), np.arange(s.shape[1]))
        s = np.where(vis, s, -np.inf)
    return s


def _lse(s):
    """Step 2, with the guard for fully masked rows (LSE = -inf)."""
    m = np.max(s, axis=1)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    with np.errstate(under="ignore"):
        z = np.sum(np.exp(s - m_safe[:, None]), axis=1)
    lse = np.where(finite, m_safe + np.log(np.where(finite, z, 1.0)), -np.inf)
    return lse


def _probs(s, lse):
    """Step 3: exactly zero where masked or where the row is fully masked."""
    finite = np.isfinite(lse)
    lse_safe = np.where(finite, lse, 0.0)
    with np.errstate(under="ignore"):
        p = np.exp(s - lse_safe[:, None])
    p[~finite, :] = 0.0
    return p


def _head_forward(q, k, v, causal, scale):
    n = q.shape[0]
    o = np.empty((n, v.shape[1]), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    for r0 in range(0, n, _ROW_CHUNK):
        r1 = min(n, r0 + _ROW_CHUNK)
        s = _scores(q[r0:r1], k, scale, r0, causal)
        l = _lse(s)
        p = _probs(s, l)
        o[r0:r1] = p @ v          # step 4
        lse[r0:r1] = l
    return o, lse


def _head_backward(q, k, v, o, do, lse, causal, scale):
    n = q.shape[0]
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    d_row = np.sum(do * o, axis=1)                       # step 5
    for r0 in range(0, n, _ROW_CHUNK):
        r1 = min(n, r0 + _ROW_CHUNK)
        s = _scores(q[r0:r1], k, scale, r0, causal)
        p = _probs(s, lse[r0:r1])                        # step 3 with the given LSE
        dv += p.T @ do[r0:r1]                            # step 6
        dp = do[r0:r1] @ v.T                             # step 7
        ds = p * (dp - d_row[r0:r1, None])               # step 8
        dq[r0:r1] = scale * (ds @ k)                     # step 9
        dk += scale * (ds.T @ q[r0:r1])
    return dq, dk, dv


def _as64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def forward(q, k, v, causal, scale: float | None = None):
    """O [B,H,N,d] and LSE [B,H,N] (natural log of the scaled scores), fp64."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, d = q.shape
    if scale is None:
        scale = default_scale(d)
    o = np.empty((B, H, N, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = _head_forward(q[b, h], k[b, h], v[b, h], causal, scale)
    return o, lse


def backward(q, k, v, do, causal, scale: float | None = None, o=None, lse=None):
    """dQ, dK, dV [B,H,N,d] in fp64.

    ``o`` and ``lse`` default to this module's own forward; callers that
    compare against the GPU pass nothing here, so no GPU value enters.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, H, N, d = q.shape
    if scale is None:
        scale = default_scale(d)
    if o is None or lse is None:
        o, lse = forward(q, k, v, causal, scale)
    o, lse = _as64(o), _as64(lse)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = _head_backward(
                q[b, h], k[b, h], v[b, h], o[b, h], do[b, h], lse[b, h], causal, scale)
    return dq, dk, dv


def head_forward_backward(q, k, v, do, causal, scale: float):
    """One (b, h) head end to end: returns (o, lse, dq, dk, dv).  Used by the
    CPU-baseline timing, which runs heads in a process pool."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    o, lse = _head_forward(q, k, v, causal, scale)
    dq, dk, dv = _head_backward(q, k, v, o, do, lse, causal, scale)
    return o, lse, dq, dk, dv


def backward_intermediates(q, k, v, do, causal, scale: float | None = None):
    """Single head [N,d] inputs: returns dict with S, P, LSE, O, D, dP, dS, dQ,
    dK, dV formed whole (small N only; used by the pins)."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    n, d = q.shape
    if scale is None:
        scale = default_scale(d)
    s = _scores(q, k, scale, 0, causal)
    lse = _lse(s)
    p = _probs(s, lse)
    o = p @ v
    d_row = np.sum(do * o, axis=1)
    dp = do @ v.T
    ds = p * (dp - d_row[:, None])
    return {
        "S": s, "LSE": lse, "P": p, "O": o, "D": d_row, "dP": dp, "dS": ds,
        "dV": p.T @ do, "dQ": scale * (ds @ k), "dK": scale * (ds.T @ q),
    }


def sampled_backward(q, k, v, do, causal, scale: float, rows_q, rows_kv, with_forward=False):
    """One head ([N, d] inputs): the forward statistics for every row, then
    only the requested rows of the gradients, each from the same steps 1-9
    applied to one row of P (dQ_i) or one column of P (dK_j, dV_j).  Cost is
    one forward plus O(N d) per requested row, so full-length sequences can
    be checked row by row.  Returns (dq[rows_q], dk[rows_kv], dv[rows_kv]),
    followed by (o[rows_q], lse[rows_q]) if with_forward."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    o, lse = _head_forward(q, k, v, causal, scale)        # steps 1-4
    d_row = np.sum(do * o, axis=1)                        # step 5
    n = q.shape[0]
    rows_q = np.asarray(rows_q, dtype=np.int64)
    rows_kv = np.asarray(rows_kv, dtype=np.int64)
    dq = np.empty((len(rows_q), k.shape[1]))
    for t, i in enumerate(rows_q):
        s_i = _scores(q[i:i + 1], k, scale, int(i), causal)   # row i of S
        p_i = _probs(s_i, lse[i:i + 1])[0]
        dp_i = v @ do[i]                                     # row i of dP
        ds_i = p_i * (dp_i - d_row[i])
        dq[t] = scale * (ds_i @ k)
    dk = np.empty((len(rows_kv), q.shape[1]))
    dv = np.empty((len(rows_kv), v.shape[1]))
    for t, j in enumerate(rows_kv):
        s_j = scale * (q @ k[j])                             # column j of S
        s_j = np.where(_mask_of(causal).visible(np.arange(n), [int(j)])[:, 0], s_j, -np.inf)
        finite = np.isfinite(lse)
        with np.errstate(under="ignore"):
            p_j = np.where(finite, np.exp(s_j - np.where(finite, lse, 0.0)), 0.0)
        dv[t] = p_j @ do                                     # step 6
        dp_j = do @ v[j]                                     # column j of dP
        ds_j = p_j * (dp_j - d_row)
        dk[t] = scale * (ds_j @ q)                           # step 9
    if with_forward:
        return dq, dk, dv, o[rows_q], lse[rows_q]
    return dq, dk, dv
