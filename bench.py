#!/usr/bin/env python3
"""Throughput of the deterministic attention backward on one MI355X.

A step is one pass of the whole backward path over one batch of synthetic
input already resident in HBM: the row term delta (preprocess), the
workspace clear, the persistent backward kernel with the chosen schedule,
and the dQ conversion.  O and LSE come from the library's forward before
timing.  Default workload: B=1, H=32, N=16384, d=128, bf16, causal mask.

Every schedule (atomic, naive, descending, shift, and auto, the library's
own pick from its DAG model) is timed the same way; `value` is the backward
TFLOP/s of auto (or of --primary), FLOPs counted as 2.5x the forward's
4*B*H*N^2*d, halved for a causal mask (with a window or block mask:
2.5x 4*B*H*d times the exact number of visible query-key pairs; the
workloads ..._swa4k and ..._blocksparse).  Also reported:
% of the dense bf16 MFMA peak, the deterministic / atomic throughput ratio
per schedule, the backward kernel's own roofline figures (HIP events around
its launch), the share of cycles the ordered schedules spend waiting for
their turn (one extra untimed, instrumented launch each), the forward alone
and a synthetic attention block (forward, then preprocess and backward with
the reported schedule; forward FLOPs 4*B*H*N^2*d, halved when causal), and
the fp64 CPU oracle timed on a bounded sample of heads.

Prints one JSON line.  --gpus above 1 is refused: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "deterministic attn-bwd TFLOP/s + % bf16 MFMA peak; det/non-det throughput ratio"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X dense MFMA (bf16), fp32 MFMA
def kernel_source_hash() -> str:
    """Hash of the backward kernel's sources and build flags, as recorded in
    the committed traffic summaries."""
    from deterministic_attention_backward_attn_amd.rocprof_summary import kernel_source_hash as h
    return h()


def read_traffic(workload: str, schedule: str):
    """Bytes per launch moved past L2 by the backward kernel, from the
    committed rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, calibrated
    against a plain copy), or None if absent or taken on other kernel
    sources."""
    path = os.path.join(ROOT, "profiles", f"attn_bwd_{workload}_{schedule}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != kernel_source_hash():
        return None
    return float(m_b.group(1))


# ------------------------------------------------------------ CPU baseline

def _oracle_head(args):
    """Worker: fp64 oracle backward of one head (forward untimed first)."""
    q, k, v, do, causal, scale = args
    from threadpoolctl import threadpool_limits
    from oracle import attention as A
    with threadpool_limits(1):
        o, lse = A._head_forward(q, k, v, causal, scale)
        t0 = time.perf_counter()
        A._head_backward(q, k, v, o, do, lse, causal, scale)
        t1 = time.perf_counter()
    return t1 - t0


def cpu_baseline(exact, w, causal, max_workers):
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    import numpy as np
    cores = max(1, min(len(os.sched_getaffinity(0)), max_workers, w.B * w.H))
    scale = 1.0 / np.sqrt(w.d)
    mask = causal
    if w.window or w.block_spec:
        from oracle import attention as A
        mk = w.mask_args()
        mask = A.Mask(causal=causal, window=mk["window"], block=mk["block_mask"],
                      block_size=mk["block_size"])
    jobs = []
    for i in range(cores):
        b, h = divmod(i, w.H)
        jobs.append((exact["q"][b, h], exact["k"][b, h], exact["v"][b, h], exact["do"][b, h],
                     mask, scale))
    with ProcessPoolExecutor(max_workers=cores, mp_context=mp.get_context("spawn")) as ex:
        times = list(ex.map(_oracle_head, jobs))
    per_head = w.flops_bwd(causal) / (w.B * w.H)
    tflops = cores * per_head / max(times) / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{cores} of {w.B * w.H} heads, one per process (1 BLAS thread each), "
                      f"fp64 backward given the oracle's own O/LSE; time = slowest head "
                      f"({max(times):.1f} s)"}


# ------------------------------------------------------- ordering waits

def order_wait(D, dev, lse, delta, sched, causal, ws, out, mkw, lay=None):
    """One extra, untimed launch of the instrumented kernel (wait statistics
    on): the share of the waves' cycles spent waiting for ordered-add turns,
    and the share of ordered adds whose turn had not come at the first poll."""
    import torch
    st = torch.zeros(4 * 4096 * 4, dtype=torch.int64, device="cuda")
    D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, schedule=sched,
               causal=causal, workspace=ws, out=out, debug=dict(lay or {}, wait_stats=st), **mkw)
    torch.cuda.synchronize()
    D.attn_bwd_status(ws)
    a = st.view(-1, 4).cpu().numpy()
    a = a[a[:, 3] > 0]
    wait, waits, spun, busy = (float(a[:, i].sum()) for i in range(4))
    return {"order_wait_frac": wait / max(busy, 1.0), "order_adds": int(waits),
            "order_polled_frac": spun / max(waits, 1.0)}


PHASES = ("item/KV change", "S,dP products", "counter check", "softmax,dS", "dV,dK products",
          "staging", "ordered add", "barrier", "dQ product", "hand-off", "prefetch,partial")
# wave-pair layout: phases of the two roles
PHASES_A = ("item/KV change", "S products", "softmax,P", "P barrier", "dV products", "staging",
            "barrier", "dQ product,partial", "prefetch")
PHASES_B = ("item/KV change", "dP products,counter check", "-", "P barrier", "dS,dK products",
            "staging", "ordered add,barrier", "hand-off", "prefetch,counter read")
# two-stage pipeline layout: stage A (S, dP, P, dS, dV of sub-tile t) and
# stage B (dK, dQ and the ordered add of sub-tile t - 1)
PIPE_A = ("item/KV change,loads", "S,dP products", "softmax,dS", "dV product", "barrier")
PIPE_B = ("item/KV change", "turn check,acc reads", "dK product", "hand-off", "dQ product",
          "ordered add", "barrier")


def phase_shares(D, dev, lse, delta, sched, causal, ws, out, mkw, lay=None, kind="single"):
    """One extra, untimed launch with the phase timer on: the share of the
    waves' cycles spent in each phase of their Q sub-tiles (the timer's own
    clock reads slow the launch down; the shares are the result)."""
    import torch
    st = torch.zeros(16 * 4096 * 4, dtype=torch.int64, device="cuda")
    D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, schedule=sched,
               causal=causal, workspace=ws, out=out, debug=dict(lay or {}, phase_stats=st),
               **mkw)
    torch.cuda.synchronize()
    D.attn_bwd_status(ws)
    a = st.view(-1, 16).cpu().numpy().astype("float64")
    a = a[a[:, 15] > 0]
    if kind == "single":
        total = a[:, 15].sum()
        return {name: round(float(a[:, k].sum() / total), 4) for k, name in enumerate(PHASES)}
    res = {}
    pipe = kind == "pipe"
    for role, tag, names in ((1, "A", PIPE_A if pipe else PHASES_A),
                             (2, "B", PIPE_B if pipe else PHASES_B)):
        r = a[a[:, 14] == role]
        total = r[:, 15].sum()
        res.update({f"{tag}: {n}": round(float(r[:, k].sum() / total), 4)
                    for k, n in enumerate(names) if n != "-"})
    return res


def dag_prediction(D, w, causal, sched, mkw, coresident, cost=None):
    """The host DAG model's view of one ordered schedule on this workload, as
    the launch places it (dash_attn_bwd_predict: XCD groups when the
    schedule's units fit one, the library's unit order): predicted makespan
    and its lower bound in units of one full item, for one group's share,
    and the predicted share of slot time spent waiting for ordered-add
    turns, with `cost` (full item, partial item, dQ add, hand-off), by
    default the costs the library's "auto" uses for this dtype and head dim
    (dash_attn_bwd_costs, a device query).  None if the launch cannot run
    it."""
    try:
        if cost is None:
            cost = D.bwd_costs(w.B, w.H, w.N, w.d, w.dtype, causal)
        (mk, wait, _, lb), info = D.bwd_predict(w.B, w.H, w.N, w.d, w.dtype, causal, sched,
                                                slots=coresident, cost=cost, **mkw)
    except D.DashError:
        return None
    slots = info["slots"]
    return {"makespan_items": round(mk, 1), "lower_bound_items": round(lb, 1),
            "wait_frac": round(wait / (slots * mk), 4) if mk > 0 else 0.0,
            "groups": info["groups"], "unit_major": info["unit_major"],
            "heads_modelled": info["heads"], "slots": slots}


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="b1h32_n16k_d128_causal")
    ap.add_argument("--mask", choices=["causal", "full"], default=None,
                    help="mask (default: the workload's first)")
    ap.add_argument("--schedules", default="atomic,naive,descending,shift,auto")
    ap.add_argument("--primary", default="auto",
                    help="schedule reported as value (default: auto, the library's choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-workers", type=int, default=16)
    ap.add_argument("--no-wait-stats", action="store_true",
                    help="skip the untimed instrumented launch per ordered schedule")
    ap.add_argument("--tune", action="store_true",
                    help="time naive/descending/shift first (dash_attn_bwd_tune) so that auto "
                         "runs the measured fastest instead of the DAG model's pick")
    ap.add_argument("--no-fwd", action="store_true",
                    help="skip the forward and forward+backward timings")
    ap.add_argument("--layout", choices=["auto", "single", "pairs", "pipe"], default="auto",
                    help="backward kernel layout: default, wave pairs or the two-stage "
                         "pipeline (bf16 d=128 or 64; bit-identical results)")
    ap.add_argument("--phases", action="store_true",
                    help="one extra launch per schedule with the phase timer: share of wave "
                         "cycles per phase of a Q sub-tile")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="run one plain device copy of BYTES before timing (a reference "
                         "dispatch of known traffic for hardware-counter runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this backward runs on one GPU; --gpus {args.gpus} is not supported "
              "(heads shard across GPUs with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import deterministic_attention_backward_attn_amd as D
    from synth import WORKLOADS, make_workload_inputs

    D.load()  # fails loudly if the library is missing
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    w = WORKLOADS[args.workload]
    mask = args.mask or w.masks[0]
    causal = mask == "causal"
    scheds = [s for s in args.schedules.split(",") if s]
    if args.primary and args.primary not in scheds:
        scheds.append(args.primary)
    if not any(s != "atomic" for s in scheds):
        scheds.append("auto")

    t_gen = time.perf_counter()
    raw = make_workload_inputs(w)
    if w.dtype == "bf16":
        dev = {k: torch.from_numpy(v[0].view(np.int16)).view(torch.bfloat16).cuda()
               for k, v in raw.items()}
    else:
        dev = {k: torch.from_numpy(v[0]).cuda() for k, v in raw.items()}
    exact = {k: v[1] for k, v in raw.items()} if not args.no_cpu_baseline else None
    del raw
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] {w.name} {mask}: inputs ready in {t_gen:.1f}s", file=sys.stderr, flush=True)

    if args.copy_calibration > 0:
        src = torch.ones(args.copy_calibration // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    mkw = w.mask_args()
    o, lse = D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, **mkw)
    delta = torch.empty_like(lse)
    dq, dk, dv = (torch.empty_like(dev["q"]) for _ in range(3))
    ws = D.alloc_workspace(dev["q"], causal, "naive")
    flops = w.flops_bwd(causal)

    lay = {"auto": {}, "single": {"layout": 3}, "pairs": {"layout": 1},
           "pipe": {"layout": 2}}[args.layout]
    # the kernel that runs (the library's automatic choice: the pipeline for
    # bf16 with d = 128 or 64), for the phase names and the report
    kind = args.layout if args.layout != "auto" else (
        "pipe" if w.dtype == "bf16" and w.d in (128, 64) else "single")

    def step(sched, events=None):
        D.attn_bwd_preprocess(o, dev["do"], out=delta)
        dbg = dict(lay, **({} if events is None else {"kernel_events": events}))
        D.attn_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, schedule=sched,
                   causal=causal, workspace=ws, out=(dq, dk, dv), debug=dbg or None, **mkw)

    tuned = None
    if args.tune:
        D.attn_bwd_preprocess(o, dev["do"], out=delta)
        pick, times = D.attn_bwd_tune(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta,
                                      causal=causal, reps=3, workspace=ws, out=(dq, dk, dv), **mkw)
        tuned = {"choice": pick, "ms": {k: round(v, 4) for k, v in times.items()}}
        print(f"[bench] tuned: {tuned}", file=sys.stderr, flush=True)

    results = {}
    for sched in scheds:
        for _ in range(args.warmup):
            step(sched)
        torch.cuda.synchronize()
        kev = []
        for _ in range(args.steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            b.record()
            kev.append((a, b))
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(args.steps):
            step(sched, (kev[i][0].cuda_event, kev[i][1].cuda_event))
        t1.record()
        torch.cuda.synchronize()
        D.attn_bwd_status(ws)
        ms = t0.elapsed_time(t1) / args.steps
        kms = sum(a.elapsed_time(b) for a, b in kev) / args.steps
        results[sched] = {"ms_per_step": ms, "tflops": flops / ms / 1e9,
                          "kernel_ms": kms, "kernel_tflops": flops / kms / 1e9}
        if sched not in ("atomic", "auto") and not args.no_wait_stats:
            results[sched].update(order_wait(D, dev, lse, delta, sched, causal, ws, (dq, dk, dv),
                                             mkw, lay))
        if args.phases:
            results[sched]["phases"] = phase_shares(D, dev, lse, delta, sched, causal, ws,
                                                    (dq, dk, dv), mkw, lay, kind)
            print(f"[bench] {sched:10s} phases " + "  ".join(
                f"{k} {v:.3f}" for k, v in results[sched]["phases"].items()), file=sys.stderr,
                flush=True)
        if sched not in ("atomic", "auto"):
            results[sched]["dag"] = dag_prediction(D, w, causal, sched, mkw,
                                                   torch.cuda.get_device_properties(0)
                                                   .multi_processor_count)
        print(f"[bench] {sched:10s} step {ms:8.3f} ms  {flops / ms / 1e9:7.1f} TFLOP/s   "
              f"kernel {kms:8.3f} ms  {flops / kms / 1e9:7.1f} TFLOP/s", file=sys.stderr,
              flush=True)

    peak = PEAK_TFLOPS[w.dtype]
    primary = args.primary or min((s for s in results if s != "atomic"),
                                  key=lambda s: results[s]["ms_per_step"])
    ran = D.resolve_schedule(w.B, w.H, w.N, w.d, w.dtype, causal, primary, **mkw)
    # the ordered add's share of the primary schedule's wave cycles (one
    # extra untimed launch with the phase timer, unless --phases ran it)
    add_share = None
    if ran != "atomic" and not args.no_wait_stats:
        ph = results[primary].get("phases") or phase_shares(D, dev, lse, delta, ran, causal, ws,
                                                            (dq, dk, dv), mkw, lay, kind)
        if kind == "single":
            add_share = round(sum(ph[k] for k in ("counter check", "ordered add", "hand-off")), 4)
        elif kind == "pipe":
            # the stage that adds (half of the waves)
            add_share = round(sum(ph[f"B: {k}"] for k in ("turn check,acc reads", "ordered add",
                                                          "hand-off")), 4)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps

    fwd_stats = None
    if not args.no_fwd:
        # the forward alone, and a synthetic attention block: forward, then
        # the backward pass (preprocess + kernel) with the primary schedule
        def fwd():
            D.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, out=(o, lse), **mkw)

        def block():
            fwd()
            step(primary)

        f_fwd = flops / 2.5
        ms_f = timed(fwd)
        ms_b = timed(block)
        D.attn_bwd_status(ws)
        fwd_stats = {"forward": {"ms": round(ms_f, 4), "tflops": round(f_fwd / ms_f / 1e9, 2),
                                 "pct_peak": round(100.0 * f_fwd / ms_f / 1e9 / peak, 2)},
                     "fwd_bwd_block": {"ms": round(ms_b, 4),
                                       "tflops": round((f_fwd + flops) / ms_b / 1e9, 2),
                                       "schedule": primary}}
        print(f"[bench] forward    {ms_f:8.3f} ms  {f_fwd / ms_f / 1e9:7.1f} TFLOP/s   "
              f"fwd+bwd {ms_b:8.3f} ms  {(f_fwd + flops) / ms_b / 1e9:7.1f} TFLOP/s",
              file=sys.stderr, flush=True)
    prim = results[primary]
    out = {
        "metric": METRIC,
        "value": round(prim["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(prim["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: i.i.d. N(0,1) Q/K/V/dO from PCG64 seeds, O/LSE from the library's forward",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "mask": mask + (f" window {w.window}" if w.window else "")
                   + (" block " + json.dumps(w.block_spec) if w.block_spec else ""),
                   "schedule": primary if ran == primary else f"{primary} ({ran})",
                   "parallelism": "single GPU",
                   "layout": {"single": "one-stage", "pairs": "wave pairs",
                              "pipe": "two-stage pipeline"}[kind]},
        "pct_peak": round(100.0 * prim["tflops"] / peak, 2),
        "det_nondet_ratio": ({s: round(r["tflops"] / results["atomic"]["tflops"], 4)
                              for s, r in results.items() if s != "atomic"}
                             if "atomic" in results else None),
        # what that ratio measures on this chip, and the cost of ordering itself
        "ordering_cost": {
            "det_nondet_ratio_measures": "throughput against the atomic reference, whose "
                                         "unordered fp32 atomic dQ adds are themselves bound by "
                                         "the chip's fp32 atomic throughput (not a free baseline)",
            "ordered_add_share_of_wave_cycles": add_share,
            "schedule": ran,
            "source": "phase timer of the backward kernel (one instrumented launch): counter "
                      "check + ordered add + hand-off phases"
                      + (" of the adding stage's waves" if kind == "pipe" else "")},
        "dag_vs_measured": dag_vs_measured(results),
        "dag_fit": dag_fit(D, w, causal, mkw, results,
                           torch.cuda.get_device_properties(0).multi_processor_count),
        "schedules": {s: {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
                      for s, r in results.items()},
    }
    achieved = flops / (prim["kernel_ms"] * 1e-3) / 1e12
    traffic = read_traffic(w.name, ran)
    out["roofline"] = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                       "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                       "traffic": traffic,
                       "hbm_GBps": (round(traffic / (prim["kernel_ms"] * 1e-3) / 1e9, 1)
                                    if traffic else None),
                       "kernel": f"{'bwd_pipe_kernel' if kind == 'pipe' else 'bwd_kernel'} ({ran})"}
    if fwd_stats:
        out.update(fwd_stats)
    if tuned:
        out["tuned"] = tuned
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample of heads", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(exact, w, causal, args.cpu_workers)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    # release device memory while every library (a profiler's included) is
    # still live, so that nothing is left to free during interpreter exit
    del dev, o, lse, delta, dq, dk, dv, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def dag_fit(D, w, causal, mkw, results, coresident):
    """The DAG model's costs fitted to this run's measured kernel times of
    naive, descending and shift (dash_schedule_fit_costs: what
    dash_attn_bwd_calibrate would record for "auto"), the fit's relative RMS
    error, the kernel time of one cost unit, and the fitted model's
    makespans of naive and descending relative to shift's."""
    ms = [results.get(s, {}).get("kernel_ms") for s in ("naive", "descending", "shift")]
    if sum(m is not None for m in ms) < 2:
        return None
    try:
        cost, res, unit = D.fit_costs(w.B, w.H, w.N, w.d, w.dtype, causal, slots=coresident,
                                      ms=ms, **mkw)
        pred = {s: D.bwd_predict(w.B, w.H, w.N, w.d, w.dtype, causal, s, slots=coresident,
                                 cost=cost, **mkw)[0][0]
                for s in ("naive", "descending", "shift")}
    except D.DashError:
        return None
    return {"cost": [round(c, 4) for c in cost], "rel_rms_error": round(res, 4),
            "ms_per_cost_unit": round(unit, 6),
            "fitted_vs_shift": {s: round(pred[s] / pred["shift"], 3)
                                for s in ("naive", "descending")}}


def dag_vs_measured(results):
    """For naive and descending: the DAG model's predicted makespan relative
    to shift's, next to the measured kernel-time ratio."""
    sh = results.get("shift", {})
    if not sh.get("dag") or not sh.get("kernel_ms"):
        return None
    out = {}
    for s in ("naive", "descending"):
        r = results.get(s, {})
        if r.get("dag") and r.get("kernel_ms"):
            out[s] = {"predicted_vs_shift": round(r["dag"]["makespan_items"]
                                                  / sh["dag"]["makespan_items"], 3),
                      "measured_vs_shift": round(r["kernel_ms"] / sh["kernel_ms"], 3)}
    return out or None


if __name__ == "__main__":
    main()
