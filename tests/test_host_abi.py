"""C-ABI tests that need no GPU: the library loads and exports every symbol
the header declares; host-only calls (schedule tables, DAG prediction,
longest path) match the oracle exactly; argument errors come back as status
codes before any launch."""
import ctypes
import os
import random

import numpy as np
import pytest

import deterministic_attention_backward_attn_amd as D
from deterministic_attention_backward_attn_amd import _lib
from oracle import dag as OD
from oracle import schedules as OS


def test_library_exports_every_header_symbol():
    lib = D.load()
    syms = D.header_symbols()
    assert len(syms) >= 12
    for s in syms:
        assert hasattr(lib, s), s
    assert lib.dash_status_string(6) == b"ordered dQ add timed out"
    assert lib.dash_status_string(99) == b"unknown status"


@pytest.mark.parametrize("schedule", OS.SCHEDULES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 6, 8, 16, 32, 64, 128])
def test_schedule_tables_match_oracle(schedule, causal, n):
    if schedule == OS.SHIFT and causal and n % 2 and n > 1:
        with pytest.raises(D.DashError) as e:
            D.schedule_tables(n, causal, schedule)
        assert e.value.code == 2
        return
    units, rank = D.schedule_tables(n, causal, schedule)
    assert units == OS.units(schedule, n, causal)
    ref = OS.rank_table(schedule, n, causal)
    if ref is None:
        assert np.all(rank == -1)
    else:
        want = np.array([[-1 if x is None else x for x in row] for row in ref], dtype=np.int32)
        assert np.array_equal(rank, want)


@pytest.mark.parametrize("schedule", OS.SCHEDULES)
@pytest.mark.parametrize("causal", [False, True])
def test_predict_matches_oracle(schedule, causal):
    rnd = random.Random(3)
    for n, heads, slots in ((4, 3, 4), (8, 2, 8), (8, 5, 13), (16, 3, 40)):
        if schedule == OS.SHIFT:
            slots = max(slots, len(OS.units(schedule, n, causal)))
        cost = (rnd.uniform(1, 3), rnd.uniform(0.5, 2), rnd.uniform(0.1, 1), rnd.uniform(0, 0.5))
        got = D.schedule_predict(n, causal, schedule, heads, slots, cost)
        want = OD.predict(schedule, n, causal, heads, slots, cost)
        for g, w in zip(got, want):
            assert abs(g - w) <= 1e-9 * max(1.0, abs(w)), (got, want)


def test_predict_closed_forms():
    c, r = 3.0, 1.0
    for n in (2, 8, 32):
        mk = D.schedule_predict(n, False, "naive", 1, n, (c, c, r, 0.0))[0]
        assert mk == n * (c + r) + (n - 1) * r
        mk = D.schedule_predict(n, False, "shift", 1, n, (c, c, r, 0.0))[0]
        assert mk == n * (c + r)
        mk = D.schedule_predict(n, True, "shift", 1, n // 2, (c, c, r, 0.0))[0]
        assert mk == (n + 1) * (c + r)


def test_predict_rejects_shift_without_resident_head():
    with pytest.raises(D.DashError) as e:
        D.schedule_predict(8, False, "shift", 2, 7, (1, 1, 1, 0))
    assert e.value.code == 2


_CANDIDATES = (OS.NAIVE, OS.DESCENDING, OS.SHIFT)


def _oracle_choice(n, causal, heads, slots, cost):
    """Argmin of the oracle's predicted makespan over the ordered schedules
    that can run; ties go to the later candidate."""
    best, best_s, preds = None, None, {}
    for s in _CANDIDATES:
        if s == OS.SHIFT and ((causal and n % 2 and n > 1)
                              or len(OS.units(s, n, causal)) > slots):
            continue
        mk = OD.predict(s, n, causal, heads, slots, cost)[0]
        preds[s] = mk
        if best is None or mk <= best:
            best, best_s = mk, s
    return best_s, preds


def test_choose_is_argmin_of_oracle_prediction():
    rnd = random.Random(17)
    cases = [(n, c, h, sl) for n in (1, 2, 3, 5, 8, 16) for c in (False, True)
             for h, sl in ((1, 4), (3, 8), (4, 16), (2, 3))]
    for n, causal, heads, slots in cases:
        cost = (rnd.uniform(1, 3), rnd.uniform(0.3, 2), rnd.uniform(0.01, 1.5),
                rnd.uniform(0, 0.8))
        want, preds = _oracle_choice(n, causal, heads, slots, cost)
        got, pred = D.schedule_choose(n, causal, heads, slots, cost)
        assert got == want, (n, causal, heads, slots, cost, pred, preds)
        for s in _CANDIDATES:
            if s in preds:
                assert abs(pred[s] - preds[s]) <= 1e-9 * max(1.0, preds[s])
            else:
                assert np.isnan(pred[s])


def test_choose_follows_the_pages_ordering():
    # with every head's units resident and a costly dQ hand-off the DAG
    # model ranks shift first for full masks and for causal masks with an
    # even tile count, descending before naive for causal masks, and ties
    # naive and descending for full masks
    cost = (1.0, 0.5, 0.3, 0.3)
    for n in (8, 16, 32):
        got, pred = D.schedule_choose(n, False, 4, 4 * n, cost)
        assert got == OS.SHIFT and pred[OS.SHIFT] < pred[OS.NAIVE] == pred[OS.DESCENDING]
        got, pred = D.schedule_choose(n, True, 4, 2 * n, cost)
        assert got == OS.SHIFT and pred[OS.SHIFT] < pred[OS.DESCENDING] < pred[OS.NAIVE]
    # shift cannot run: odd causal tile count, or a head's units do not fit
    got, pred = D.schedule_choose(9, True, 4, 64, cost)
    assert got == OS.DESCENDING and np.isnan(pred[OS.SHIFT])
    got, pred = D.schedule_choose(16, False, 4, 15, cost)
    assert got == OS.DESCENDING and np.isnan(pred[OS.SHIFT])
    # default cost model: the same shape of answer
    assert D.schedule_choose(128, True, 32, 256)[0] == OS.SHIFT
    assert D.schedule_choose(129, True, 32, 256)[0] == OS.DESCENDING


def test_longest_path_and_cycle():
    rnd = random.Random(9)
    for _ in range(50):
        n = rnd.randint(1, 20)
        w = [float(rnd.randint(0, 7)) for _ in range(n)]
        edges = [(u, v, float(rnd.randint(0, 3))) for u in range(n) for v in range(u + 1, n)
                 if rnd.random() < 0.25]
        s, f = D.dag_longest_path(w, edges)
        s2, f2 = OD.longest_path(w, edges)
        assert np.array_equal(s, np.array(s2)) and np.array_equal(f, np.array(f2))
    with pytest.raises(D.DashError) as e:
        D.dag_longest_path([1.0, 1.0], [(0, 1, 0.0), (1, 0, 0.0)])
    assert e.value.code == 5


def _desc(B=1, H=2, N=256, d=64, dtype=0, causal=0):
    return _lib.Desc(B, H, N, d, dtype, causal, 0.0)


FAKE = ctypes.c_void_p(0x100000)


def test_argument_errors_without_launch():
    lib = D.load()
    ws_size = lib.dash_attn_bwd_workspace_size
    n0 = ws_size(ctypes.byref(_desc()), 1)
    assert n0 > 4 * 2 * 256 * 64
    # the longest plain sequence whose units fit the kernel's work list
    # (1024 tiles); beyond that the size query reports 0 (unsupported)
    largest = _desc(B=1, H=1, N=1024 * 128, d=128, dtype=1)
    assert ws_size(ctypes.byref(largest), 1) > 4 * 1024 * 128 * 128
    assert ws_size(ctypes.byref(_desc(B=1, H=1, N=1025 * 128, d=128, dtype=1)), 1) == 0
    # same size for every schedule (schedules only reorder work)
    for s in range(5):
        assert ws_size(ctypes.byref(_desc()), s) == n0
    bad = [
        (_desc(d=96), 2), (_desc(N=200), 2), (_desc(dtype=1, N=192), 2), (_desc(B=0), 1),
        (_desc(dtype=7), 1), (_desc(causal=2), 1),
        # one head's fp32 accumulator must stay below 2^31 bytes
        (_desc(B=1, H=1, N=1 << 22, d=128, dtype=1), 2),
    ]
    for desc, code in bad:
        assert ws_size(ctypes.byref(desc), 1) == 0
        assert lib.dash_attn_fwd(ctypes.byref(desc), FAKE, FAKE, FAKE, FAKE, FAKE, None) == code
        assert lib.dash_attn_fwd_workspace_size(ctypes.byref(desc)) == 0
    assert ws_size(ctypes.byref(_desc()), 9) == 0
    assert ws_size(None, 1) == 0
    size = ctypes.c_size_t(n0)
    desc = _desc()
    args = [FAKE] * 10
    ws_ok = ctypes.c_size_t(size.value)
    # null pointer
    assert lib.dash_attn_bwd(ctypes.byref(desc), 1, None, *args[1:], ws_ok, None) == 1
    # workspace too small, or misaligned
    assert lib.dash_attn_bwd(ctypes.byref(desc), 1, *args, ctypes.c_size_t(size.value - 4), None) == 3
    mis = args[:9] + [ctypes.c_void_p(0x100010)]
    assert lib.dash_attn_bwd(ctypes.byref(desc), 1, *mis, ws_ok, None) == 3
    # bad schedule enum
    assert lib.dash_attn_bwd(ctypes.byref(desc), 5, *args, ws_ok, None) == 1
    assert lib.dash_attn_bwd(ctypes.byref(desc), -1, *args, ws_ok, None) == 1
    # debug struct required for the debug entry point; poison out of range
    assert lib.dash_attn_bwd_debug(ctypes.byref(desc), 1, *args, ws_ok, None, None) == 1
    dbg = _lib.Debug(0, 0, 10_000, None)
    assert lib.dash_attn_bwd_debug(ctypes.byref(desc), 1, *args, ws_ok, ctypes.byref(dbg), None) == 1
    for bad in (-1, 4):  # placement out of range
        dbg = _lib.Debug()
        dbg.placement = bad
        assert lib.dash_attn_bwd_debug(ctypes.byref(desc), 1, *args, ws_ok, ctypes.byref(dbg),
                                       None) == 1
    for bad in (-1, 3):  # unit order out of range
        dbg = _lib.Debug()
        dbg.unit_order = bad
        assert lib.dash_attn_bwd_debug(ctypes.byref(desc), 1, *args, ws_ok, ctypes.byref(dbg),
                                       None) == 1
    # host-only argument checks
    cost = (ctypes.c_double * 4)(1, 1, 1, 0)
    out = (ctypes.c_double * 4)()
    assert lib.dash_schedule_predict(None, 1, 1, cost, out) == 1
    assert lib.dash_schedule_predict(ctypes.byref(desc), 1, 0, cost, out) == 1
    assert lib.dash_schedule_predict(ctypes.byref(desc), 1, 1, None, out) == 1
    assert lib.dash_schedule_predict(ctypes.byref(_desc(d=96)), 1, 1, cost, out) == 2
    choice = ctypes.c_int(-1)
    assert lib.dash_schedule_choose(0, 0, 1, 1, None, ctypes.byref(choice), None) == 1
    assert lib.dash_schedule_choose(8, 2, 1, 1, None, ctypes.byref(choice), None) == 1
    assert lib.dash_schedule_choose(8, 0, 1, 0, None, ctypes.byref(choice), None) == 1
    assert lib.dash_schedule_choose(8, 0, 1, 8, None, None, None) == 1
    tune_args = [FAKE] * 10 + [ws_ok]
    assert lib.dash_attn_bwd_tune(None, *tune_args, 3, ctypes.byref(choice), None, None) == 1
    assert lib.dash_attn_bwd_tune(ctypes.byref(desc), *tune_args, 0, ctypes.byref(choice), None,
                                  None) == 1
    assert lib.dash_attn_bwd_tune(ctypes.byref(desc), *tune_args, 3, None, None, None) == 1
    assert lib.dash_attn_bwd_resolve_schedule(None, 4, ctypes.byref(choice)) == 1
    assert lib.dash_attn_bwd_resolve_schedule(ctypes.byref(desc), 5, ctypes.byref(choice)) == 1
    assert lib.dash_attn_bwd_resolve_schedule(ctypes.byref(desc), 4, None) == 1
    assert lib.dash_attn_bwd_resolve_schedule(ctypes.byref(_desc(d=96)), 4,
                                              ctypes.byref(choice)) == 2
    assert lib.dash_litmus_ordered_add(0, 1, FAKE, FAKE, FAKE, FAKE, 0, None) == 1
    assert lib.dash_attn_bwd_status(None, None) == 1
    assert lib.dash_status_query(None) == 1
    assert lib.dash_attn_tile(None) == 0 and lib.dash_attn_bwd_subtile(None) == 0
    assert lib.dash_attn_tile(ctypes.byref(_desc(dtype=1, N=256))) == 128
    assert lib.dash_attn_bwd_subtile(ctypes.byref(_desc(d=128))) == 32


def _header_struct_fields(name):
    """Field names of a typedef'd struct in include/dash_attn.h, in order."""
    import re
    text = open(_lib.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    m = re.search(r"typedef struct \{([^{}]*)\}\s*" + name + r";", text)
    assert m, name
    fields = []
    for decl in m.group(1).split(";"):
        decl = decl.strip()
        if not decl:
            continue
        # "type a, b" declares several fields; arrays keep their name
        for part in decl.split(","):
            fields.append(re.match(r".*?(\w+)\s*(\[\d+\])?$", part.strip()).group(1))
    return fields


def test_ctypes_structs_mirror_the_header():
    """The binding's ctypes structures list the header's fields in the same
    order (the binding passes them by pointer to the library)."""
    assert [f[0] for f in _lib.Desc._fields_] == _header_struct_fields("dash_attn_desc")
    assert [f[0] for f in _lib.Debug._fields_] == _header_struct_fields("dash_bwd_debug")


@pytest.mark.parametrize("causal", [False, True])
def test_device_closed_form_tables_equal_the_host_tables(causal):
    """The backward writes the full and causal masks' tables on the device
    from closed forms; the library compares them item for item with its
    general builder (whose tables the oracle pins) before they are used,
    here through the table export, which fails on any difference."""
    for n in list(range(1, 41)) + [64, 127, 128]:
        for sched in ("atomic", "naive", "descending", "shift"):
            B, H, N, d = 1, 1, 64 * n, 64
            if sched == "shift" and causal and n > 1 and n % 2:
                with pytest.raises(D.DashError) as e:
                    D.mask_schedule_tables(B, H, N, d, "f32", causal, sched)
                assert e.value.code == 2
                continue
            t = D.mask_schedule_tables(B, H, N, d, "f32", causal, sched)
            units = OS.units(sched, n, causal)
            assert t["units"] == units, (n, sched)
            want = OS.rank_table(sched, n, causal)
            if want is not None:
                got = [[None if r < 0 else int(r) for r in row] for row in t["rank"]]
                assert got == want, (n, sched)


def test_library_imports_no_device_allocator():
    """The library allocates no device memory: its dynamic symbol table
    imports none of HIP's device allocators (pinned host memory for the
    tables of special masks is host memory)."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    names = {line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()}
    device_alloc = {n for n in names if n.startswith(("hipMalloc", "hipFree", "hipExtMalloc",
                                                      "hipMallocAsync", "hipMemPool"))
                    and n not in ("hipFreeHost",)}
    assert not device_alloc, sorted(device_alloc)
    assert "hipMemcpyAsync" in names


def test_noalloc_refusals_happen_before_any_device_call():
    """dash_attn_bwd_noalloc refuses problems whose workspace exceeds its
    built-in array and masks whose tables need host memory, before it
    touches the device."""
    lib = D.load()
    args = [FAKE] * 9
    big = _desc(B=1, H=32, N=4096, d=128, dtype=1, causal=1)
    assert lib.dash_attn_bwd_workspace_size(ctypes.byref(big), 1) > _lib.NOALLOC_SCRATCH_BYTES
    assert lib.dash_attn_bwd_noalloc(ctypes.byref(big), 1, *args, None) == 3
    win = _desc(B=1, H=1, N=1024, d=64, dtype=1, causal=1)
    win.window = 200
    assert lib.dash_attn_bwd_noalloc(ctypes.byref(win), 1, *args, None) == 2
    assert lib.dash_attn_bwd_noalloc(ctypes.byref(_desc(d=96)), 1, *args, None) == 2
    assert lib.dash_attn_bwd_noalloc(ctypes.byref(_desc()), 9, *args, None) == 1
    assert lib.dash_attn_bwd_noalloc(None, 1, *args, None) == 1


def test_profile_hash_covers_every_kernel_include():
    """The freshness hash of the committed traffic summaries covers the
    backward kernels' sources (the one-stage kernel and the two-stage
    pipeline) and every file they include from this package."""
    import re
    from deterministic_attention_backward_attn_amd import rocprof_summary as RS
    kdir = "deterministic_attention_backward_attn_amd/csrc/kernels/"
    seen, todo = set(), ["attn_bwd.hip", "attn_bwd_pipe.hip"]
    while todo:
        f = todo.pop()
        if f in seen:
            continue
        seen.add(f)
        text = open(os.path.join(RS.ROOT, kdir + f)).read()
        todo += re.findall(r'#include\s+"([^"]+)"', text)
    assert {kdir + f for f in seen} == set(RS.KERNEL_SOURCES)
