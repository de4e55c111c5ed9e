"""Deterministic attention backward for MI355X (gfx950): Python binding.

Thin marshalling over the C ABI in include/dash_attn.h (libdash_attn.so).
Tensors are torch tensors on the GPU, used only as device memory; every
step of the computation runs in the library's HIP kernels on the caller's
current stream.  The host-only calls (schedule tables, DAG prediction,
longest path) take and return plain Python / numpy values.

Public calls (same names as the C entry points, without the prefix):
  attn_fwd, attn_bwd_preprocess, attn_bwd_workspace_size, attn_bwd,
  status_query, attn_bwd_status, backward (preprocess + bwd),
  schedule_tables, schedule_predict, dag_longest_path, litmus_ordered_add.
"""
from __future__ import annotations

import ctypes

import numpy as np

from ._lib import (DTYPES, NOALLOC_SCRATCH_BYTES, NOALLOC_WORKSPACE, SCHEDULES, DashError, Debug,
                   Desc, check, header_symbols, load)

__all__ = [
    "DashError", "SCHEDULES", "attn_fwd", "attn_bwd_preprocess", "attn_bwd_workspace_size",
    "attn_bwd", "attn_bwd_status", "status_query", "attn_bwd_noalloc", "attn_bwd_tune", "backward", "schedule_tables", "schedule_predict", "schedule_choose",
    "resolve_schedule", "mask_schedule_tables", "mask_schedule_predict", "bwd_predict",
    "dag_longest_path", "litmus_ordered_add", "tile", "subtile", "header_symbols", "load",
]


# ----------------------------------------------------------------- helpers

def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return DTYPES["f32"]
    if t.dtype == torch.bfloat16:
        return DTYPES["bf16"]
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _set_mask(desc: Desc, window=0, block_mask=None, block_size=0) -> Desc:
    """Window and block mask fields (see the C header); the descriptor keeps
    the block mask's host buffer alive."""
    desc.window = int(window)
    if block_mask is not None:
        bm = np.ascontiguousarray(np.asarray(block_mask) != 0, dtype=np.uint8)
        if bm.ndim != 2 or bm.shape[0] != bm.shape[1]:
            raise ValueError("block_mask must be a square 2-D array")
        desc.block_size = int(block_size) if block_size else desc.N // bm.shape[0]
        desc.block_mask = bm.ctypes.data
        desc._keep = bm
    return desc


def _desc_from(q, causal: bool, scale, window=0, block_mask=None, block_size=0) -> Desc:
    if q.dim() != 4:
        raise ValueError("expected a [B, H, N, d] tensor")
    B, H, N, d = (int(x) for x in q.shape)
    return _set_mask(Desc(B, H, N, d, _dtype_code(q), 1 if causal else 0,
                          float(scale) if scale is not None else 0.0),
                     window, block_mask, block_size)


def _desc(B, H, N, d, dtype: str, causal: bool, scale=None, window=0, block_mask=None,
          block_size=0) -> Desc:
    return _set_mask(Desc(B, H, N, d, DTYPES[dtype], 1 if causal else 0,
                          float(scale) if scale is not None else 0.0),
                     window, block_mask, block_size)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _sched(schedule) -> int:
    if isinstance(schedule, int):
        return schedule
    try:
        return SCHEDULES[schedule]
    except KeyError:
        raise ValueError(f"unknown schedule {schedule!r}; one of {sorted(SCHEDULES)}") from None


def _same_shape(ref, *ts):
    for t in ts:
        if tuple(t.shape) != tuple(ref.shape) or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError("tensors must share shape, dtype and device")


# ------------------------------------------------------------------ device

def tile(B, H, N, d, dtype="bf16") -> int:
    lib = load()
    return int(lib.dash_attn_tile(ctypes.byref(_desc(B, H, N, d, dtype, False))))


def subtile(B, H, N, d, dtype="bf16") -> int:
    lib = load()
    return int(lib.dash_attn_bwd_subtile(ctypes.byref(_desc(B, H, N, d, dtype, False))))


def attn_fwd(q, k, v, causal: bool = False, scale=None, stream=None, *, window=0,
             block_mask=None, block_size=0, out=None):
    """Returns (o, lse): o like q, lse float32 [B, H, N] (written to `out`
    = (o, lse) if given).  Mask: causal, window (sliding window of keys,
    0 = none) and block_mask (square host array over blocks of block_size
    rows; default N / its side), as in the C header."""
    torch = _torch()
    lib = load()
    _same_shape(q, k, v)
    desc = _desc_from(q, causal, scale, window, block_mask, block_size)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _same_shape(q, o)
        if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(q.shape[:3]):
            raise ValueError("lse must be float32 [B, H, N]")
    nws = int(lib.dash_attn_fwd_workspace_size(ctypes.byref(desc)))
    ws = torch.empty(nws, dtype=torch.uint8, device=q.device) if nws else None
    check(lib.dash_attn_fwd_ws(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                               _ptr(ws), ctypes.c_size_t(nws), _stream(stream)),
          "dash_attn_fwd_ws")
    return o, lse


def attn_bwd_preprocess(o, do, out=None, stream=None):
    """delta = rowsum(dO * O) in float32 [B, H, N] (written to `out` if given)."""
    torch = _torch()
    lib = load()
    _same_shape(o, do)
    desc = _desc_from(o, False, None)
    if out is None:
        delta = torch.empty(o.shape[:3], dtype=torch.float32, device=o.device)
    else:
        delta = out
        if delta.dtype != torch.float32 or tuple(delta.shape) != tuple(o.shape[:3]):
            raise ValueError("out must be float32 [B, H, N]")
    check(lib.dash_attn_bwd_preprocess(ctypes.byref(desc), _ptr(o), _ptr(do), _ptr(delta),
                                       _stream(stream)), "dash_attn_bwd_preprocess")
    return delta


def attn_bwd_workspace_size(B, H, N, d, dtype="bf16", causal=False, schedule="naive", *,
                            window=0, block_mask=None, block_size=0) -> int:
    """Workspace bytes of the backward (the same for every schedule)."""
    lib = load()
    desc = _desc(B, H, N, d, dtype, causal, None, window, block_mask, block_size)
    n = int(lib.dash_attn_bwd_workspace_size(ctypes.byref(desc), _sched(schedule)))
    if n == 0:
        raise DashError(2, "dash_attn_bwd_workspace_size")
    return n


def resolve_schedule(B, H, N, d, dtype="bf16", causal=False, schedule="auto", *, window=0,
                     block_mask=None, block_size=0) -> str:
    """The schedule attn_bwd runs for `schedule` on the current device
    ("auto" -> the predicted best ordered schedule; others unchanged)."""
    lib = load()
    out = ctypes.c_int(-1)
    desc = _desc(B, H, N, d, dtype, causal, None, window, block_mask, block_size)
    check(lib.dash_attn_bwd_resolve_schedule(ctypes.byref(desc),
                                             _sched(schedule), ctypes.byref(out)),
          "dash_attn_bwd_resolve_schedule")
    return {v: k for k, v in SCHEDULES.items()}[out.value]


def alloc_workspace(q, causal=False, schedule="naive", *, window=0, block_mask=None,
                    block_size=0):
    torch = _torch()
    B, H, N, d = (int(x) for x in q.shape)
    dt = "f32" if q.dtype == torch.float32 else "bf16"
    n = attn_bwd_workspace_size(B, H, N, d, dt, causal, schedule, window=window,
                                block_mask=block_mask, block_size=block_size)
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def attn_bwd(q, k, v, do, lse, delta, *, schedule="naive", causal=False, scale=None,
             workspace=None, out=None, debug=None, stream=None, window=0, block_mask=None,
             block_size=0):
    """Returns (dq, dk, dv).  `workspace`: uint8 GPU tensor of at least
    attn_bwd_workspace_size bytes (allocated if None).  `out`: optional
    preallocated (dq, dk, dv).  `debug`: optional dict with keys spin_limit,
    jitter_seed, poison_q (1-based, 0 = off), partials (float32 tensor),
    kernel_events (two raw hipEvent_t handles), wait_stats (int64 tensor of
    at least 4*4096*4 entries), phase_stats (int64 tensor of at least
    16*4096*4 entries: cycles per phase of each wave's sub-tiles, see the
    header), layout (0 automatic: the two-stage pipeline for bf16 d=128 or 64, else
    the one-stage kernel; 1 wave pairs: bf16 d=128 only, 2 pipeline: bf16 d=128 or 64; 3
    one-stage kernel; bit-identical results), placement (0 automatic, 1 device-wide, 2 XCD
    groups with L2-coherent accumulator, 3 XCD groups device-coherent),
    unit_order (0 automatic, 1 head by head, 2 unit-major).
    Mask arguments as for attn_fwd."""
    torch = _torch()
    lib = load()
    _same_shape(q, k, v, do)
    desc = _desc_from(q, causal, scale, window, block_mask, block_size)
    if workspace is None:
        workspace = alloc_workspace(q, causal, schedule, window=window, block_mask=block_mask,
                                    block_size=block_size)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        _same_shape(q, dq, dk, dv)
    for t, shp in ((lse, q.shape[:3]), (delta, q.shape[:3])):
        if t.dtype != torch.float32 or tuple(t.shape) != tuple(shp):
            raise ValueError("lse and delta must be float32 [B, H, N]")
    args = [ctypes.byref(desc), _sched(schedule), _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse),
            _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
            ctypes.c_size_t(workspace.numel() * workspace.element_size())]
    if debug is None:
        check(lib.dash_attn_bwd(*args, _stream(stream)), "dash_attn_bwd")
    else:
        dbg = Debug(int(debug.get("spin_limit", 0)), int(debug.get("jitter_seed", 0)),
                    int(debug.get("poison_q", 0)),
                    _ptr(debug["partials"]) if debug.get("partials") is not None else None)
        dbg.placement = int(debug.get("placement", 0))
        dbg.unit_order = int(debug.get("unit_order", 0))
        if debug.get("wait_stats") is not None:
            dbg.wait_stats = _ptr(debug["wait_stats"])
        if debug.get("phase_stats") is not None:
            dbg.phase_stats = _ptr(debug["phase_stats"])
        dbg.layout = int(debug.get("layout", 0))
        ev = debug.get("kernel_events")
        if ev is not None:
            dbg.kernel_events[0] = ctypes.c_void_p(int(ev[0]))
            dbg.kernel_events[1] = ctypes.c_void_p(int(ev[1]))
        check(lib.dash_attn_bwd_debug(*args, ctypes.byref(dbg), _stream(stream)),
              "dash_attn_bwd_debug")
    return dq, dk, dv


def attn_bwd_tune(q, k, v, do, lse, delta, *, causal=False, scale=None, reps=3, workspace=None,
                  out=None, stream=None, window=0, block_mask=None, block_size=0):
    """Time naive, descending and shift on these inputs and record the
    fastest for "auto" launches of this shape (see dash_attn_bwd_tune).
    Returns (name, {name: ms per launch}); overwrites `out` (or scratch
    outputs) and the workspace."""
    torch = _torch()
    lib = load()
    _same_shape(q, k, v, do)
    desc = _desc_from(q, causal, scale, window, block_mask, block_size)
    if workspace is None:
        workspace = alloc_workspace(q, causal, "auto", window=window, block_mask=block_mask,
                                    block_size=block_size)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = out
    _same_shape(q, dq, dk, dv)
    choice = ctypes.c_int(-1)
    t = (ctypes.c_float * 3)()
    check(lib.dash_attn_bwd_tune(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(do),
                                 _ptr(lse), _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv),
                                 _ptr(workspace),
                                 ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                                 int(reps), ctypes.byref(choice), t, _stream(stream)),
          "dash_attn_bwd_tune")
    names = {v: k for k, v in SCHEDULES.items()}
    return names[choice.value], {"naive": t[0], "descending": t[1], "shift": t[2]}


def attn_bwd_calibrate(q, k, v, do, lse, delta, *, causal=False, scale=None, reps=3,
                       workspace=None, out=None, stream=None, window=0, block_mask=None,
                       block_size=0):
    """Time naive, descending and shift on these inputs, fit the DAG model's
    costs to the times and record them for "auto" launches of this dtype
    and head dim on this device (see dash_attn_bwd_calibrate).  Returns
    (costs (c_full, c_diag, r, h), relative RMS residual, {name: ms})."""
    torch = _torch()
    lib = load()
    _same_shape(q, k, v, do)
    desc = _desc_from(q, causal, scale, window, block_mask, block_size)
    if workspace is None:
        workspace = alloc_workspace(q, causal, "auto", window=window, block_mask=block_mask,
                                    block_size=block_size)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = out
    _same_shape(q, dq, dk, dv)
    c = (ctypes.c_double * 4)()
    res = ctypes.c_double(0.0)
    t = (ctypes.c_float * 3)()
    check(lib.dash_attn_bwd_calibrate(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(do),
                                      _ptr(lse), _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv),
                                      _ptr(workspace),
                                      ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                                      int(reps), c, ctypes.byref(res), t, _stream(stream)),
          "dash_attn_bwd_calibrate")
    return tuple(c), res.value, {"naive": t[0], "descending": t[1], "shift": t[2]}


def bwd_costs(B, H, N, d, dtype="bf16", causal=False):
    """The costs "auto" uses on the current device for this dtype and d."""
    lib = load()
    desc = _desc(B, H, N, d, dtype, causal)
    c = (ctypes.c_double * 4)()
    check(lib.dash_attn_bwd_costs(ctypes.byref(desc), c), "dash_attn_bwd_costs")
    return tuple(c)


def fit_costs(B, H, N, d, dtype="bf16", causal=False, *, slots, ms, window=0, block_mask=None,
              block_size=0):
    """Host-only fit of the DAG model's costs to measured times ms =
    (naive, descending, shift) (None or <= 0: not measured).  Returns
    (costs, relative RMS residual, time of one cost unit)."""
    lib = load()
    desc = _desc(B, H, N, d, dtype, causal, None, window, block_mask, block_size)
    m = (ctypes.c_double * 3)(*[float("nan") if x is None else float(x) for x in ms])
    c = (ctypes.c_double * 4)()
    res = ctypes.c_double(0.0)
    unit = ctypes.c_double(0.0)
    check(lib.dash_schedule_fit_costs(ctypes.byref(desc), int(slots), m, c, ctypes.byref(res),
                                      ctypes.byref(unit)), "dash_schedule_fit_costs")
    return tuple(c), res.value, unit.value


def attn_bwd_status(workspace, stream=None):
    """Synchronizes the stream and raises DashError if an ordered add timed out."""
    lib = load()
    check(lib.dash_attn_bwd_status(_ptr(workspace), _stream(stream)), "dash_attn_bwd_status")


def status_query(workspace):
    """Status word of the last backward on `workspace` (call after the
    stream was synchronized); raises DashError on a time-out.  "noalloc"
    reads the word of attn_bwd_noalloc's built-in array on this GPU."""
    lib = load()
    ptr = ctypes.c_void_p(NOALLOC_WORKSPACE) if isinstance(workspace, str) else _ptr(workspace)
    if isinstance(workspace, str) and workspace != "noalloc":
        raise ValueError("workspace must be a tensor or 'noalloc'")
    check(lib.dash_status_query(ptr), "dash_status_query")


def attn_bwd_noalloc(q, k, v, do, lse, delta, *, schedule="naive", causal=False, scale=None,
                     out=None, stream=None):
    """attn_bwd without a workspace: the library's built-in device array
    (NOALLOC_SCRATCH_BYTES per GPU) serves as one; full and causal masks
    only.  Calls on one GPU share that array and must not overlap.  The
    library allocates nothing; `out` = (dq, dk, dv) avoids the output
    allocations here too."""
    torch = _torch()
    lib = load()
    _same_shape(q, k, v, do)
    desc = _desc_from(q, causal, scale)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        _same_shape(q, dq, dk, dv)
    for t in (lse, delta):
        if t.dtype != torch.float32 or tuple(t.shape) != tuple(q.shape[:3]):
            raise ValueError("lse and delta must be float32 [B, H, N]")
    check(lib.dash_attn_bwd_noalloc(ctypes.byref(desc), _sched(schedule), _ptr(q), _ptr(k),
                                    _ptr(v), _ptr(do), _ptr(lse), _ptr(delta), _ptr(dq),
                                    _ptr(dk), _ptr(dv), _stream(stream)),
          "dash_attn_bwd_noalloc")
    return dq, dk, dv


def backward(q, k, v, o, do, lse, *, schedule="naive", causal=False, scale=None,
             workspace=None, stream=None, window=0, block_mask=None, block_size=0):
    """preprocess + bwd: returns (dq, dk, dv)."""
    delta = attn_bwd_preprocess(o, do, stream=stream)
    return attn_bwd(q, k, v, do, lse, delta, schedule=schedule, causal=causal, scale=scale,
                    workspace=workspace, stream=stream, window=window, block_mask=block_mask,
                    block_size=block_size)


def litmus_ordered_add(turn, values, acc, counters, spin_limit=0, stream=None):
    """Device litmus of the ordered hand-off (see the C header)."""
    lib = load()
    W, L = (int(x) for x in values.shape)
    check(lib.dash_litmus_ordered_add(W, L, _ptr(turn), _ptr(values), _ptr(acc), _ptr(counters),
                                      int(spin_limit), _stream(stream)),
          "dash_litmus_ordered_add")


# --------------------------------------------------------------- host only

def schedule_tables(n: int, causal: bool, schedule):
    """Returns (units, rank): units = list of [(kv, q), ...] per unit,
    rank = int32 array [n, n] (rank[q, kv], -1 where absent)."""
    lib = load()
    cap = max(1, n * n)
    n_units = ctypes.c_int32(0)
    off = (ctypes.c_int32 * (n + 1))()
    kv = (ctypes.c_int32 * cap)()
    qq = (ctypes.c_int32 * cap)()
    rank = (ctypes.c_int32 * cap)()
    check(lib.dash_schedule_tables(n, 1 if causal else 0, _sched(schedule), ctypes.byref(n_units),
                                   off, kv, qq, rank), "dash_schedule_tables")
    units = []
    for u in range(n_units.value):
        units.append([(kv[i], qq[i]) for i in range(off[u], off[u + 1])])
    return units, np.frombuffer(rank, dtype=np.int32).reshape(n, n).copy()


def mask_schedule_tables(B, H, N, d, dtype="bf16", causal=False, schedule="naive", *, window=0,
                         block_mask=None, block_size=0, slots=256):
    """The backward's tables for a masked problem, as a launch on `slots`
    co-resident workgroups runs them (0: this device's count; 256 is
    MI355X's for the backward).  Returns a dict: n (tiles per side), units
    (per unit [(kv, q), ...]), steps (per unit, the lockstep or timed step
    of each item; SHIFT only, else None), partial (per unit, per item
    bool), rank (int32 [n, n], rank[q, kv], -1 where absent), static (units
    run in head-aligned rounds), slots_per_head (timed shift: the slots per
    head it was timed on; 0 otherwise)."""
    lib = load()
    desc = _desc(B, H, N, d, dtype, causal, None, window, block_mask, block_size)
    sizes = (ctypes.c_int32 * 5)()
    check(lib.dash_attn_schedule_tables(ctypes.byref(desc), _sched(schedule), int(slots), sizes,
                                        None, None, None, None, None, None),
          "dash_attn_schedule_tables")
    n, nu, ni = sizes[0], sizes[1], sizes[2]
    off = np.zeros(nu + 1, dtype=np.int32)
    kv = np.zeros(max(ni, 1), dtype=np.int32)
    qq = np.zeros(max(ni, 1), dtype=np.int32)
    st = np.zeros(max(ni, 1), dtype=np.int32)
    pa = np.zeros(max(ni, 1), dtype=np.uint8)
    rank = np.zeros(n * n, dtype=np.int32)
    ip = ctypes.POINTER(ctypes.c_int32)
    check(lib.dash_attn_schedule_tables(ctypes.byref(desc), _sched(schedule), int(slots), sizes,
                                        off.ctypes.data_as(ip), kv.ctypes.data_as(ip),
                                        qq.ctypes.data_as(ip), st.ctypes.data_as(ip),
                                        pa.ctypes.data, rank.ctypes.data_as(ip)),
          "dash_attn_schedule_tables")
    units, steps, partial = [], [], []
    for u in range(nu):
        sl = range(off[u], off[u + 1])
        units.append([(int(kv[i]), int(qq[i])) for i in sl])
        steps.append([int(st[i]) for i in sl])
        partial.append([bool(pa[i]) for i in sl])
    shift = _sched(schedule) == SCHEDULES["shift"]
    return {"n": n, "units": units, "steps": steps if shift else None, "partial": partial,
            "rank": rank.reshape(n, n), "static": bool(sizes[3]), "slots_per_head": int(sizes[4])}


def mask_schedule_predict(B, H, N, d, dtype="bf16", causal=False, schedule="naive", *, slots,
                          cost, window=0, block_mask=None, block_size=0, unit_major=False):
    """DAG prediction for a masked problem with B*H heads: (makespan,
    total_wait, max_slot_idle, lower_bound); unit_major: dynamic schedules
    take unit 0 of every head, then unit 1, ..."""
    lib = load()
    desc = _desc(B, H, N, d, dtype, causal, None, window, block_mask, block_size)
    c = (ctypes.c_double * 4)(*[float(x) for x in cost])
    out = (ctypes.c_double * 4)()
    check(lib.dash_attn_schedule_predict(ctypes.byref(desc), _sched(schedule), int(slots),
                                         1 if unit_major else 0, c, out),
          "dash_attn_schedule_predict")
    return tuple(out)


def schedule_predict(n: int, causal: bool, schedule, heads: int, slots: int, cost):
    """DAG prediction for `heads` heads of n tiles under the full or causal
    mask (a descriptor with B = 1, H = heads, fp32 64-row tiles, N = 64 n).
    Returns (makespan, total_wait, max_slot_idle, lower_bound)."""
    lib = load()
    desc = _desc(1, int(heads), 64 * int(n), 64, "f32", causal)
    c = (ctypes.c_double * 4)(*[float(x) for x in cost])
    out = (ctypes.c_double * 4)()
    check(lib.dash_schedule_predict(ctypes.byref(desc), _sched(schedule), int(slots), c, out),
          "dash_schedule_predict")
    return tuple(out)


def bwd_predict(B, H, N, d, dtype="bf16", causal=False, schedule="naive", *, slots, cost,
                window=0, block_mask=None, block_size=0):
    """DAG prediction of a launch on `slots` co-resident workgroups, with the
    library's placement (XCD groups when the schedule's units fit one) and
    unit order.  Returns (makespan, total_wait, max_slot_idle, lower_bound)
    of one group's share and a dict groups, unit_major, heads, slots."""
    lib = load()
    desc = _desc(B, H, N, d, dtype, causal, None, window, block_mask, block_size)
    c = (ctypes.c_double * 4)(*[float(x) for x in cost])
    out = (ctypes.c_double * 4)()
    info = (ctypes.c_int32 * 4)()
    check(lib.dash_attn_bwd_predict(ctypes.byref(desc), _sched(schedule), int(slots), c, out,
                                    info), "dash_attn_bwd_predict")
    return tuple(out), {"groups": info[0], "unit_major": bool(info[1]), "heads": info[2],
                        "slots": info[3]}


def schedule_choose(n: int, causal: bool, heads: int, slots: int, cost=None):
    """The ordered schedule DASH_SCHED_AUTO resolves to: returns (name,
    {name: predicted makespan}) over naive, descending and shift (NaN where
    a schedule cannot run).  cost None = the library's default model."""
    lib = load()
    c = None if cost is None else (ctypes.c_double * 4)(*[float(x) for x in cost])
    choice = ctypes.c_int(0)
    pred = (ctypes.c_double * 3)()
    check(lib.dash_schedule_choose(n, 1 if causal else 0, heads, slots, c, ctypes.byref(choice),
                                   pred), "dash_schedule_choose")
    names = {v: k for k, v in SCHEDULES.items()}
    return names[choice.value], {"naive": pred[0], "descending": pred[1], "shift": pred[2]}


def dag_longest_path(weights, edges):
    """weights: node weights; edges: (src, dst, latency) triples.
    Returns (start, finish) numpy arrays."""
    lib = load()
    w = np.ascontiguousarray(weights, dtype=np.float64)
    e = list(edges)
    src = np.ascontiguousarray([x[0] for x in e], dtype=np.int32)
    dst = np.ascontiguousarray([x[1] for x in e], dtype=np.int32)
    lat = np.ascontiguousarray([x[2] for x in e], dtype=np.float64)
    start = np.zeros_like(w)
    finish = np.zeros_like(w)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    check(lib.dash_dag_longest_path(len(w), w.ctypes.data_as(dp), len(e), src.ctypes.data_as(ip),
                                    dst.ctypes.data_as(ip), lat.ctypes.data_as(dp),
                                    start.ctypes.data_as(dp), finish.ctypes.data_as(dp)),
          "dash_dag_longest_path")
    return start, finish
