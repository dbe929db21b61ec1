"""Benchmark of the MiniMind FFN / top-k MoE forward (or backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--cold | --warm]
                    [--pass fwd | bwd | train] [--no-others]

A step is one full forward (every kernel of the path) over one batch of
synthetic inputs already resident in device memory.  Default workload: the
dense bf16 SwiGLU FFN, 16384 tokens, H 2048, I 6464 (the largest
configuration).  W untimed steps, then exactly K timed steps.  By default
each timed step starts with cold caches: L2 and the 256 MB Infinity Cache are
flushed before every step, outside the step's own start / stop events, by
reading a 1 GiB buffer (a read leaves clean lines; a write would leave the
caches full of dirty lines whose write-back then competes with the step), and
``value`` / ``ms_per_step`` come from those events.  The same K steps back to
back with warm caches (bracketed by device synchronisation) and a captured
graph replayed K times are reported alongside (``warm_ms_per_step``,
``graph_ms_per_step``).  A further pass of K steps records HIP events around
every stage on the library's stream to get per-kernel durations, from which
the dominant kernel's roofline fraction is computed.  The other workloads'
cold step times follow as ``other_workloads`` (``--no-others`` skips them).
The fp64 CPU oracle is then timed on a bounded sample of the workload (rank
0, one GPU only): median of 3 passes.

With ``--pass bwd`` a step is one backward instead (routing and gate/up
activations recomputed, then every gradient); its line carries its own metric
and the same roofline / cpu_baseline objects.  With ``--pass train`` a step
is one training step: the training forward, which keeps g, u (and the
routing) for the backward, then the backward that takes them instead of
recomputing them.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FFN/MoE fwd tokens/s + TFLOP/s (% bf16 MFMA peak) / GB/s (% HBM) on 1 GPU"
METRIC_BWD = "FFN/MoE bwd tokens/s + TFLOP/s (% bf16 MFMA peak) on 1 GPU"
METRIC_TRAIN = "FFN/MoE train step (fwd + bwd) tokens/s + TFLOP/s (% bf16 MFMA peak) on 1 GPU"
DEFAULT_WORKLOAD = "dense_bf16_n16384_h2048_i6464"
# the other configurations, timed cold after the headline (forward only)
OTHER_WORKLOADS = ["moe_top1_n4096_h768_e4", "moe_top2_skew_n16384_h768_e8",
                   "moe_decode_n32_h2048_e16", "dense_fp32_n100_h768_i2432"]

# MI355X published peaks
PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


GEMM_SOURCES = ["top_moe_layer_amd/csrc/gemm_impl.h", "top_moe_layer_amd/csrc/gemm_bf16.hip",
                "top_moe_layer_amd/csrc/plan.cpp"]


def gemm_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` measured with rocprofv3 counters and
    stored in profiles/traffic.json (under "<workload>:bwd" for the backward);
    None if absent or if the GEMM sources have changed since the counters were
    taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh).get(workload, {}).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != gemm_source_hash():
        return None
    return rec.get("bytes_per_launch")


def stage_units(w):
    """Algorithmic work of each stage of one forward: (flops, bytes).  Bytes
    count each tensor the stage must read or write once; re-reads, the h round
    trip and k-slot traffic are implementation costs, not credited."""
    el = w.elem_bytes()
    N, H, I, E, k = w.N, w.H, w.I, w.E, w.k
    rows = N * k
    if w.kind == "dense":
        return {
            "gateup_gemm": (4.0 * N * H * I, N * H * el + 2 * I * H * el + N * I * el),
            "down_gemm": (2.0 * N * H * I, N * I * el + H * I * el + N * H * el),
        }
    touched = min(E, rows)  # upper bound; exact count is reported from the run
    return {
        "router": (2.0 * N * H * E, N * H * el + E * H * 4 + N * k * 8),
        "permute": (0.0, N * k * 4 * 2),
        "gateup_gemm": (4.0 * rows * H * I, N * H * el + 2 * touched * I * H * el + rows * I * el),
        "down_gemm": (2.0 * rows * H * I, rows * I * el + touched * H * I * el + N * H * el),
        "combine": (0.0, (rows * H * 4 + N * H * el) if k > 1 else 0.0),
    }


def stage_units_bwd(w, touched=None):
    """Algorithmic work of each stage of one backward: (flops, bytes).  GEMM
    stages are credited with the contraction flops they execute (including the
    recomputed gate and up projections); memory stages
    with each tensor they must read or write once."""
    el = w.elem_bytes()
    N, H, I, E, k = w.N, w.H, w.I, w.E, w.k
    rows = N * k
    ex = 1 if w.kind == "dense" else (touched if touched is not None else min(E, rows))
    Ew = 1 if w.kind == "dense" else E
    u = {
        "transpose_w": (0.0, 2 * 3 * Ew * H * I * el),
        "transpose_act": (0.0, 2 * 2 * rows * H * el),
        "gu_gemm": (4.0 * rows * H * I, N * H * el + 2 * ex * H * I * el + 3 * rows * I * el),
        "dh_gemm": (2.0 * rows * H * I, N * H * el + ex * H * I * el + 6 * rows * I * el),
        "dx_gemm": (4.0 * rows * H * I, 2 * rows * I * el + 2 * ex * H * I * el + rows * H * el),
        "dwgu_gemm": (4.0 * rows * H * I, 2 * rows * I * el + rows * H * el + 2 * Ew * H * I * el),
        "dwd_gemm": (2.0 * rows * H * I, rows * I * el + rows * H * el + Ew * H * I * el),
    }
    if w.kind == "moe":
        u.update({
            "router": (2.0 * N * H * E, N * H * el + E * H * 4 + N * k * 8 + N * E * 4),
            "permute": (0.0, N * k * 4 * 2),
            "router_bwd": (0.0, N * E * 8 + N * k * 8),
            "dx_combine": (2.0 * N * H * E, rows * H * el + N * H * el + N * E * 4),
            "dwr": (2.0 * N * H * E, N * H * el + N * E * 4 + E * H * 4),
        })
    return u


def flops_bwd(w):
    """Algorithmic FLOPs of one backward given the forward's activations:
    12 * N*k * H * I for the three projections' input and weight gradients
    (the recomputation of g and u is not credited), plus 4 * N * H * E for
    the router's."""
    f = 12.0 * w.N * w.k * w.H * w.I
    if w.kind == "moe":
        f += 4.0 * w.N * w.H * w.E
    return f


def host_info():
    """The CPU the oracle runs on: model name, CPUs in this process's affinity
    mask, and the BLAS threads numpy's matmuls actually use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = affinity
    return model, affinity, int(threads)


def timed_sample(run, N, budget_s):
    """Median rate of 3 passes of the oracle over the first n tokens, n grown
    by 4x (at most N) until one pass takes a sixth of the budget."""
    n = min(N, 64)
    dt = run(n)
    while n < N and dt < budget_s / 6:
        n = min(N, n * 4)
        dt = run(n)
    times = sorted([dt] + [run(n) for _ in range(2)])
    return n, times


def baseline_record(n, times, N, what):
    model, affinity, threads = host_info()
    med = times[1]
    return {
        "value": n / med,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{what}: first {n} of {N} tokens, median of 3 passes "
                  f"({', '.join(f'{t:.2f}' for t in times)} s)",
        "cpu_model": model,
        "affinity_cpus": affinity,
        "blas_threads": threads,
    }


def cpu_baseline_bwd(w, inputs, dy, budget_s=20.0):
    """Time the fp64 oracle's backward (as it stands) on a bounded sample:
    the first n tokens as a batch of their own."""
    from oracle.cases import widen
    from oracle import swiglu_ffn_bwd, moe_ffn_bwd
    from workloads import to_f64

    f = widen(inputs)
    g = to_f64(dy, w.dtype)

    def run(n):
        t0 = time.perf_counter()
        if w.kind == "dense":
            swiglu_ffn_bwd(f["x"][:n], f["Wg"], f["Wu"], f["Wd"], g[:n])
        else:
            moe_ffn_bwd(f["x"][:n], f["Wr"], f["Wg"], f["Wu"], f["Wd"], w.k, w.coef, g[:n], 1.0,
                        w.norm_topk_prob)
        return time.perf_counter() - t0

    n, times = timed_sample(run, w.N, budget_s)
    return baseline_record(n, times, w.N, f"fp64 numpy oracle backward on {w.name} (the first n "
                                          f"tokens as one batch)")


def cpu_baseline_train(w, inputs, dy):
    """A training step of the oracle: its forward and its backward timed as in
    the other passes, the per-token times added."""
    f = cpu_baseline(w, inputs, budget_s=12.0)
    b = cpu_baseline_bwd(w, inputs, dy, budget_s=12.0)
    return dict(f, value=1.0 / (1.0 / f["value"] + 1.0 / b["value"]),
                sample=f"forward: {f['sample']}; backward: {b['sample']}; per-token times added")


def cpu_baseline(w, inputs, budget_s=20.0):
    """Time the fp64 oracle (as it stands) on a bounded sample of the workload:
    the outputs of the first n tokens."""
    import numpy as np
    from oracle.cases import widen
    from oracle import dense_ffn, moe_ffn, moe_route

    f = widen(inputs)

    def run(n):
        rows = np.arange(n)
        t0 = time.perf_counter()
        if w.kind == "dense":
            dense_ffn(f["x"], f["Wg"], f["Wu"], f["Wd"], rows=rows)
        else:
            # routing always covers all N tokens (aux and the lists need them);
            # it is charged pro rata to the n tokens whose outputs are computed
            t1 = time.perf_counter()
            route = moe_route(f["x"], f["Wr"], w.k, w.coef)
            tr = time.perf_counter() - t1
            moe_ffn(f["x"], f["Wr"], f["Wg"], f["Wu"], f["Wd"], w.k, w.coef, rows=rows, route=route)
            return time.perf_counter() - t0 - tr + tr * n / w.N
        return time.perf_counter() - t0

    n, times = timed_sample(run, w.N, budget_s)
    return baseline_record(n, times, w.N, f"fp64 numpy oracle on {w.name}" +
                           (" (routing of all tokens charged pro rata)" if w.kind == "moe" else ""))


def forward_step(tm, w, d, dev, stream):
    """One forward of the workload on preallocated outputs and workspace:
    returns step(stage_events=None, stream=stream) and the device expert
    offsets (MoE) or None."""
    import torch

    tdt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    N, H, I, E, k = w.N, w.H, w.I, w.E, w.k
    y = torch.empty((N, H), dtype=tdt, device=dev)
    if w.kind == "dense":
        ws = torch.empty(tm.ffn_workspace_bytes(N, H, I, tdt), dtype=torch.uint8, device=dev)

        def step(ev=None, st=stream):
            tm.ffn_swiglu_fwd(d["x"], d["Wg"], d["Wu"], d["Wd"], y=y, workspace=ws,
                              stream=st, stage_events=ev)
        return step, None
    ws = torch.empty(tm.moe_workspace_bytes(N, H, I, E, k, tdt), dtype=torch.uint8, device=dev)
    idx = torch.empty((N, k), dtype=torch.int32, device=dev)
    alpha = torch.empty((N, k), dtype=torch.float32, device=dev)
    aux = torch.empty((1,), dtype=torch.float32, device=dev)
    offs = torch.empty((E + 1,), dtype=torch.int32, device=dev)

    def step(ev=None, st=stream):
        tm.moe_ffn_fwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], k, w.coef, y=y,
                       topk_idx=idx, alpha=alpha, aux_loss=aux, expert_offsets=offs,
                       norm_topk_prob=w.norm_topk_prob, return_lists=False, workspace=ws,
                       stream=st, stage_events=ev)
    return step, offs


def step_bytes(w, touched):
    """Algorithmic bytes of one forward: x read and y written once, the
    weights of the experts that receive tokens once, W_router."""
    el = w.elem_bytes()
    ex = 1 if w.kind == "dense" else touched
    b = 2 * w.N * w.H * el + 3 * ex * w.H * w.I * el
    if w.kind == "moe":
        b += w.E * w.H * 4
    return b


def time_other_workloads(tm, names, steps, warmup, dev, stream, flush):
    """Cold step times of other workloads' forwards (caches flushed before each
    step, events around the step only)."""
    import numpy as np
    import torch
    from workloads import get, make_inputs

    out = {}
    for name in names:
        w = get(name)
        inputs = make_inputs(w)
        t = lambda a: (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
                       .view(torch.bfloat16) if w.dtype == "bf16"
                       else torch.from_numpy(np.ascontiguousarray(a)).to(dev))
        d = {n: t(inputs[n]) for n in ("x", "Wg", "Wu", "Wd")}
        if w.kind == "moe":
            d["Wr"] = torch.from_numpy(np.ascontiguousarray(inputs["Wr"])).to(dev)
        step, offs = forward_step(tm, w, d, dev, stream)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        per = []
        for _ in range(steps):
            flush()
            s0.record(stream)
            step()
            s1.record(stream)
            s1.synchronize()
            per.append(s0.elapsed_time(s1))
        ms = float(np.mean(per))
        touched = int((np.diff(offs.cpu().numpy()) > 0).sum()) if offs is not None else 1
        tf = w.flops() / (ms * 1e-3) / 1e12
        gbs = step_bytes(w, touched) / (ms * 1e-3) / 1e9
        rec = {"ms_per_step": round(ms, 5), "tokens_per_s": round(w.N / (ms * 1e-3), 1),
               "tflops": round(tf, 2), "frac_of_peak_flops": round(tf / PEAK_TFLOPS[w.dtype], 4),
               "hbm_gbs": round(gbs, 1), "frac_of_hbm": round(gbs / PEAK_HBM_GBS, 4),
               "dtype": w.dtype, "cache": "cold", "steps": steps}
        out[w.name] = rec
        log(f"other workload {w.name}: {rec}")
        del d, step, offs
        torch.cuda.synchronize()
    return out


class _EventPair:
    """The forward's and the backward's stage events of one training step."""

    def __init__(self, a, b):
        self.a, self.b = a, b

    def elapsed_ms(self):
        return list(self.a.elapsed_ms()) + list(self.b.elapsed_ms())

    def close(self):
        self.a.close()
        self.b.close()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    cache = ap.add_mutually_exclusive_group()
    cache.add_argument("--cold", action="store_const", const="cold", dest="cache",
                       help="headline steps with L2 and the Infinity Cache flushed before each, "
                            "timed one by one with events (default)")
    cache.add_argument("--warm", action="store_const", const="warm", dest="cache",
                       help="headline steps back to back with warm caches (then the cold steps "
                            "are the ones reported alongside)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-alongside", action="store_true",
                    help="skip the steps in the other cache mode (field warm_ms_per_step or "
                         "cold_ms_per_step)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replay timing (extra field graph_ms_per_step)")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the cold step times of the other workloads (field other_workloads)")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd", "train"), default="fwd",
                    help="time the forward (default), the backward, or a training step (the "
                         "forward keeping g, u + the backward taking them)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run 5 plain device-to-device copies of BYTES (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import top_moe_layer_amd as tm
    from workloads import get, make_inputs, make_upstream

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_probe:
        src = torch.ones(args.copy_probe, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe, "copies": 5}), flush=True)
        return
    w = get(args.workload)
    bwd = args.which == "bwd"
    train = args.which == "train"
    log(f"workload {w.name}: N={w.N} H={w.H} I={w.I} E={w.E} k={w.k} {w.dtype} {args.which}")
    decode_like = w.kind == "moe" and w.N * w.k <= 256
    cold = (args.cache or "cold") == "cold"
    inputs = make_inputs(w)

    def dev_t(a, stored=True):
        if stored and w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    d = {n: dev_t(inputs[n]) for n in ("x", "Wg", "Wu", "Wd")}
    if w.kind == "moe":
        d["Wr"] = dev_t(inputs["Wr"], stored=False)
    tdt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    N, H, I, E, k = w.N, w.H, w.I, w.E, w.k
    stream = torch.cuda.current_stream(dev)
    dy_host = make_upstream(inputs) if (bwd or train) else None

    if train:
        dyd = dev_t(dy_host)
        y = torch.empty((N, H), dtype=tdt, device=dev)
        if w.kind == "dense":
            ws = torch.empty(tm.ffn_workspace_bytes(N, H, I, tdt), dtype=torch.uint8, device=dev)
            saved = torch.empty(tm.ffn_bwd_workspace_bytes(N, H, I, tdt), dtype=torch.uint8,
                                device=dev)
            fnames, bnames = tm.FFN_STAGE_NAMES, tm.FFN_BWD_STAGE_NAMES
            nf, nb = tm.FFN_STAGES, tm.FFN_BWD_STAGES

            def step(ev=None, st=stream):
                tm.ffn_swiglu_fwd(d["x"], d["Wg"], d["Wu"], d["Wd"], y=y, workspace=ws,
                                  saved=saved, stream=st, stage_events=ev and ev.a)
                tm.ffn_swiglu_bwd(d["x"], d["Wg"], d["Wu"], d["Wd"], dyd, workspace=saved,
                                  from_saved=True, stream=st, stage_events=ev and ev.b)
        else:
            ws = torch.empty(tm.moe_workspace_bytes(N, H, I, E, k, tdt), dtype=torch.uint8,
                             device=dev)
            saved = torch.empty(tm.moe_bwd_workspace_bytes(N, H, I, E, k, tdt),
                                dtype=torch.uint8, device=dev)
            idx = torch.empty((N, k), dtype=torch.int32, device=dev)
            alpha = torch.empty((N, k), dtype=torch.float32, device=dev)
            aux = torch.empty((1,), dtype=torch.float32, device=dev)
            offs = torch.empty((E + 1,), dtype=torch.int32, device=dev)
            fnames, bnames = tm.MOE_STAGE_NAMES, tm.MOE_BWD_STAGE_NAMES
            nf, nb = tm.MOE_STAGES, tm.MOE_BWD_STAGES

            def step(ev=None, st=stream):
                tm.moe_ffn_fwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], k, w.coef, y=y,
                               topk_idx=idx, alpha=alpha, aux_loss=aux, expert_offsets=offs,
                               norm_topk_prob=w.norm_topk_prob, return_lists=False,
                               workspace=ws, saved=saved, stream=st, stage_events=ev and ev.a)
                tm.moe_ffn_bwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], dyd, k, w.coef,
                               norm_topk_prob=w.norm_topk_prob, workspace=saved,
                               from_saved=True, stream=st, stage_events=ev and ev.b)
        names = ["fwd:" + n for n in fnames] + ["bwd:" + n for n in bnames]
        make_events = lambda: _EventPair(tm.StageEvents(nf), tm.StageEvents(nb))
    elif bwd:
        dyd = dev_t(dy_host)
        new = lambda shape, dt_=tdt: torch.empty(shape, dtype=dt_, device=dev)
        if w.kind == "dense":
            ws = torch.empty(tm.ffn_bwd_workspace_bytes(N, H, I, tdt), dtype=torch.uint8, device=dev)
            names = tm.FFN_BWD_STAGE_NAMES
            make_events = lambda: tm.StageEvents(tm.FFN_BWD_STAGES)

            def step(ev=None, st=stream):
                tm.ffn_swiglu_bwd(d["x"], d["Wg"], d["Wu"], d["Wd"], dyd, workspace=ws,
                                  stream=st, stage_events=ev)
        else:
            ws = torch.empty(tm.moe_bwd_workspace_bytes(N, H, I, E, k, tdt), dtype=torch.uint8,
                             device=dev)
            names = tm.MOE_BWD_STAGE_NAMES
            make_events = lambda: tm.StageEvents(tm.MOE_BWD_STAGES)

            def step(ev=None, st=stream):
                tm.moe_ffn_bwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], dyd, k, w.coef,
                               norm_topk_prob=w.norm_topk_prob, workspace=ws, stream=st,
                               stage_events=ev)
    else:
        step, offs = forward_step(tm, w, d, dev, stream)
        names = tm.FFN_STAGE_NAMES if w.kind == "dense" else tm.MOE_STAGE_NAMES
        nst = tm.FFN_STAGES if w.kind == "dense" else tm.MOE_STAGES
        make_events = lambda: tm.StageEvents(nst)

    flush_buf = torch.zeros(1 << 28, dtype=torch.int32, device=dev)

    def flush():  # evict L2 and the Infinity Cache with clean lines
        flush_buf.sum()

    warm_ev = make_events()
    for i in range(args.warmup):
        step(warm_ev if i == 0 else None)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    def time_cold(nsteps):
        """Per-step milliseconds, caches flushed before each step (outside
        the step's events)."""
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        out = []
        torch.cuda.synchronize()
        for _ in range(nsteps):
            flush()
            s0.record(stream)
            step()
            s1.record(stream)
            s1.synchronize()
            out.append(s0.elapsed_time(s1))
        torch.cuda.synchronize()
        return out

    def time_warm(nsteps):
        """Milliseconds per step of nsteps back-to-back steps."""
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(nsteps):
            step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / nsteps

    step_pct = None
    if cold:
        per = time_cold(args.steps)
        ms_step = sum(per) / len(per)
        step_pct = {q: round(float(np.percentile(per, p_)), 5)
                    for q, p_ in (("p10", 10), ("p50", 50), ("p90", 90))}
    else:
        ms_step = time_warm(args.steps)
    log(f"timed {args.steps} {'cold' if cold else 'warm'} steps: {ms_step:.4f} ms/step")

    # The same K steps in the other cache mode, reported alongside.
    warm_ms = cold_ms = None
    if not args.no_alongside:
        if cold:
            warm_ms = time_warm(args.steps)
            log(f"warm steps: {warm_ms:.4f} ms/step")
        else:
            per = time_cold(args.steps)
            cold_ms = sum(per) / len(per)
            log(f"cold steps: {cold_ms:.4f} ms/step")

    # The same step captured once in a HIP graph and replayed K times (warm):
    # the launch overhead that a caller capturing its loop saves.
    graph_ms = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(None, torch.cuda.current_stream(dev))
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        del g
        log(f"graph replays (warm): {graph_ms:.4f} ms/step")

    # Per-kernel durations: the same K steps again, each with its own start /
    # stop events per stage, stamped by the kernel dispatches themselves
    # (hipExtLaunchKernel) on the library's stream, so each pair brackets
    # exactly one kernel.  Attaching the events costs a few microseconds of
    # dispatch per kernel, which is why the step time above is taken without.
    ev_sets = [make_events() for _ in range(args.steps)]
    for i in range(args.steps):
        if cold:
            flush()
        step(ev_sets[i])
    torch.cuda.synchronize()
    per_step = np.array([e.elapsed_ms() for e in ev_sets])  # [steps, stages]
    # Stages that enqueue no kernel here still get their two events, recorded
    # back to back; they read a few microseconds of event overhead, not work.
    empty = set()
    if w.kind == "moe" and k == 1 and not bwd:
        empty.add(("fwd:" if train else "") + "combine")  # y written by the down GEMM
    if train:
        empty.add("bwd:gu_gemm")  # g, u kept by the forward
        if w.kind == "moe":
            empty.update(("bwd:router", "bwd:permute"))  # so is the routing
    for n in empty:
        per_step[:, names.index(n)] = 0.0
    per = per_step.mean(axis=0)
    pct = lambda v: {q: round(float(np.percentile(v, p)), 5) for q, p in (("p10", 10), ("p50", 50), ("p90", 90))}
    for e in ev_sets:
        e.close()
    stages_ms = {n: round(float(v), 5) for n, v in zip(names, per)}
    log(f"stage kernel ms: {stages_ms}")

    units = stage_units(w)
    touched = None
    if train:
        units = {**{"fwd:" + n: v for n, v in stage_units(w).items()},
                 **{"bwd:" + n: v for n, v in stage_units_bwd(w).items()}}
        el = w.elem_bytes()
        rows = N * k
        ex = 1 if w.kind == "dense" else min(E, rows)
        # the gate/up projection also writes g, u (kept) besides h
        units["fwd:gateup_gemm"] = (4.0 * rows * H * I,
                                    N * H * el + 2 * ex * I * H * el + 3 * rows * I * el)
        units["bwd:gu_gemm"] = (0.0, 0.0)  # skipped: g, u come from the forward
    elif bwd:
        units = stage_units_bwd(w)
    elif w.kind == "moe":
        cnt = np.diff(offs.cpu().numpy())
        touched = int((cnt > 0).sum())
        units = {**units}
        el = w.elem_bytes()
        rows = N * k
        units["gateup_gemm"] = (4.0 * rows * H * I, N * H * el + 2 * touched * I * H * el + rows * I * el)
        units["down_gemm"] = (2.0 * rows * H * I, rows * I * el + touched * H * I * el + N * H * el)

    total_flops = (w.flops() + flops_bwd(w)) if train else (flops_bwd(w) if bwd else w.flops())
    tflops = total_flops / (ms_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    dom = "gateup_gemm"
    if train:  # the longest GEMM stage of the step
        dom = max((n for n in names if n.endswith("_gemm")), key=lambda n: stages_ms[n])
    elif bwd:  # the longest GEMM stage
        dom = max(("gu_gemm", "dh_gemm", "dx_gemm", "dwgu_gemm", "dwd_gemm"),
                  key=lambda n: stages_ms[n])
    dom_ms = stages_ms[dom]
    dom_pct = pct(per_step[:, names.index(dom)])
    dflops, dbytes = units[dom]
    if train:  # each stage is the same kernel as in the fwd / bwd passes but the gate/up one
        tkey, tkern = ((w.name, dom[4:]) if dom.startswith("fwd:") and dom != "fwd:gateup_gemm"
                       else (w.name + ":bwd", dom[4:]) if dom.startswith("bwd:") else (None, None))
        traffic = recorded_traffic(tkey, tkern) if tkey else None
    else:
        traffic = recorded_traffic(w.name + (":bwd" if bwd else ""), dom)
    if decode_like and not bwd and not train:
        achieved = dbytes / (dom_ms * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": traffic,
                "algorithmic_bytes": dbytes, "avg_launch_ms": dom_ms, "launch_ms": dom_pct}
    else:
        achieved = dflops / (dom_ms * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": traffic,
                "algorithmic_flops": dflops, "avg_launch_ms": dom_ms, "launch_ms": dom_pct}

    result = {
        "metric": METRIC_TRAIN if train else (METRIC_BWD if bwd else METRIC),
        "value": round(N / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded, shapes and distributions of the workload)",
        "config": {"workload": w.name, "N": N, "H": H, "I": I, "E": E if w.kind == "moe" else None,
                   "k": k if w.kind == "moe" else None, "batch": w.batch, "seq": w.seq,
                   "cache": "cold (L2 + Infinity Cache flushed per step)" if cold else "warm"},
        "tflops": round(tflops, 2),
        "mfma_frac": round(tflops / peak, 4),
        "stages_ms": stages_ms,
        "kernel_ms_per_step": pct(per_step.sum(axis=1)),
        "step_ms": step_pct,
        "warm_ms_per_step": None if warm_ms is None else round(warm_ms, 5),
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 5),
        "cold_ms_per_step": None if cold_ms is None else round(cold_ms, 5),
        "experts_touched": touched,
        "pass": args.which,
        "roofline": roof,
    }
    if not bwd and not train:
        # the whole step against HBM: x, y, the touched weights and W_r once
        gbs = step_bytes(w, touched if touched is not None else 1) / (ms_step * 1e-3) / 1e9
        result["step_hbm_gbs"] = round(gbs, 1)
        result["step_hbm_frac"] = round(gbs / PEAK_HBM_GBS, 4)
    if not args.no_others and not bwd and not train:
        others = [n for n in OTHER_WORKLOADS if n != w.name]
        result["other_workloads"] = time_other_workloads(tm, others, min(args.steps, 20), 3,
                                                         dev, stream, flush)
    if not args.no_cpu_baseline:
        log("timing the fp64 CPU oracle on a bounded sample")
        if train:
            result["cpu_baseline"] = cpu_baseline_train(w, inputs, dy_host)
        else:
            result["cpu_baseline"] = (cpu_baseline_bwd(w, inputs, dy_host) if bwd
                                      else cpu_baseline(w, inputs))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
