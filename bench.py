"""Benchmark of the batched speculative-verify causal conv1d update on one MI355X.

One step = one launch of the whole hot path (conv + SiLU + per-head L2 + every
rollback window + committed state) over one batch of seeded synthetic inputs.
Default workload: dedup_bs128_t8 (n_seq 128, d_inner 10240, T 8, bf16, dedup rows,
bias on) - the GB300 workload of sglang PR 46184's benchmark table.

    python bench.py [--steps K] [--warmup W] [--workload KEY]

KEY: 0 1 2 3 4 4b 4s (the chain verify workloads), 4t 4bt (the stress problems with
conv_state stored time-major), b1 b64 t16 (the pages' table rows:
bs 1 and 64 at T 8, bs 128 at T 16), 2t (time-major rows), 2v (packed
rows), 1t (tree verify), 2r / 4r / 4rt / 4rtt (accepted-prefix restore at the headline / stress
shape, the last two into a time-major state, 4rtt from time-major rows: the step is the restore
launch after an untimed verify), p (prefill: the step is the prefill conv plus the separate
q|k L2; the roofline is the prefill conv alone).

Prints ONE JSON line.  `value` is achieved algorithmic HBM bandwidth (GB/s): the
bytes one step must move (for the verify: x, out, the conv_state window read and the
committed window write, the rollback windows, weight and bias; active rows only)
divided by the mean step time measured with HIP events on the launch stream.  The
inputs rotate over enough buffer sets that the working set is >= 8x the 256 MB
Infinity Cache (so each stream's buffers outgrow it), and data is fetched from HBM.

With the default workload the line also carries `stress`: the stress problem (512
rows x T 16, offsets, ~10% padded rows) at d 10240 and d 10200, with conv_state stored
channel-major and time-major, each timed the same way with its own roofline fraction
(--also picks other keys, --also none skips them).  `cpu_baseline` times the oracle
(unchanged) on a bounded sample: one thread, and all the host threads this process
may use over disjoint row slices, each the median of 3 runs.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import numpy as np  # noqa: E402

import workloads  # noqa: E402

METRIC = "µs/launch and achieved HBM GB/s (% of peak) for verify conv1d+L2, 1 MI355X"
PEAK_GBS = 8000.0
MALL_BYTES = 256 * 2 ** 20
KERNEL_SRCS = [os.path.join(ROOT, "causal_conv1d_verify_amd", "csrc", f)
               for f in ("cv_kernels.hip", "cv_aux_kernels.hip", "cv_device.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def _code_of(text: str) -> str:
    """The source text without its comments and blank lines (string literals in the
    device sources hold no comment markers), so that a comment edit keeps the hash."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_hash() -> str:
    """sha256[:16] over the code of the device sources (every kernel the steps launch),
    comments left out."""
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(_code_of(open(f, encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None when the
    kernel source changed since they were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE)).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_sha") != kernel_hash():
        return None
    return rec.get("bytes_per_launch")


def step_kind(wl) -> str:
    """What one timed step launches: the verify, the restore after a verify, or the
    prefill conv followed by the separate L2."""
    return "prefill" if wl.prefill else "restore" if wl.restore else "verify"


def step_bytes(wl, inp) -> int:
    kind = step_kind(wl)
    if kind == "restore":
        return workloads.restore_bytes(wl, inp)
    if kind == "prefill":
        return workloads.algorithmic_bytes(wl, inp) + workloads.l2_bytes(wl, inp)
    return workloads.algorithmic_bytes(wl, inp)


def _oracle_l2(out, wl):
    """The oracle's separate L2 over every row of a packed out (a copy)."""
    import oracle

    out = out.copy()
    oracle.l2norm(out.reshape(-1, out.shape[-1]), d_inner=wl.d_inner,
                  qk_channels=wl.qk_channels, head_dim=wl.head_dim, l2_eps=wl.l2_eps,
                  x_dtype=wl.x_dtype)
    return out


def _oracle_step(inp):
    """The oracle's result of one step (the restore includes its verify)."""
    import gpu_harness as gh

    wl = inp.wl
    kind = step_kind(wl)
    ref = gh.oracle_general(inp, restore=kind == "restore")
    if kind == "prefill":
        ref["out"] = _oracle_l2(ref["out"], wl)
    return ref


def host_threads() -> int:
    """Threads the CPU legs may use: this process's CPU affinity, capped by
    OMP_NUM_THREADS when set (the share of the host that goes with one GPU) and at 16."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, min(n, 16))


def _oracle_rows(inp, bufs, i0, i1):
    """One pass of the unchanged oracle over rows [i0, i1) of the problem, writing into
    bufs (state, out, windows).  Rows own distinct slots, so slices run concurrently."""
    import oracle

    wl = inp.wl
    kind = step_kind(wl)
    n = wl.n_seq
    sl = slice(i0, i1)
    slots = inp.slot_idx if inp.slot_idx is not None else np.arange(n, dtype=np.int32)
    cut = lambda a: None if a is None else a[sl]   # noqa: E731
    packed = inp.cu_seqlens is not None
    x = inp.x if packed else inp.x[sl]
    out = bufs["out"] if packed else bufs["out"][sl]
    cu = inp.cu_seqlens[i0:i1 + 1] if packed else None
    if kind == "prefill":
        oracle.prefill(x, inp.weight, inp.bias, bufs["conv_state"], out, cu,
                       d_inner=wl.d_inner, x_dtype=wl.x_dtype, state_dtype=wl.state_dtype,
                       slot_idx=slots[sl], has_init=cut(inp.has_init))
        rows = bufs["out"][int(cu[0]):int(cu[-1])]
        oracle.l2norm(rows.reshape(-1, rows.shape[-1]), d_inner=wl.d_inner,
                      qk_channels=wl.qk_channels, head_dim=wl.head_dim, l2_eps=wl.l2_eps,
                      x_dtype=wl.x_dtype)
        return
    oracle.verify_general(x, inp.weight, inp.bias, bufs["conv_state"], out, bufs["windows"],
                          T=wl.T, d_inner=wl.d_inner, qk_channels=wl.qk_channels,
                          head_dim=wl.head_dim, l2_eps=wl.l2_eps, x_dtype=wl.x_dtype,
                          state_dtype=wl.state_dtype, layout=wl.layout, slot_idx=slots[sl],
                          num_accept_tokens=cut(inp.num_accept_tokens), cu_seqlens=cu,
                          parent=cut(inp.parent), commit=not wl.tree)
    if kind == "restore":
        oracle.restore(bufs["conv_state"], bufs["windows"], inp.restore_k[sl], T=wl.T,
                       d_conv=wl.d_conv, state_dtype=wl.state_dtype, layout=wl.layout,
                       slot_idx=slots[sl])


def _cpu_leg(inp, alg_bytes, threads, run_s, runs=3):
    """Median over `runs` of the oracle's rate (GB/s of the step's algorithmic bytes) with
    the rows split into `threads` contiguous slices on as many threads; each run repeats
    whole passes for about run_s seconds."""
    from concurrent.futures import ThreadPoolExecutor

    wl = inp.wl
    bufs = {"conv_state": inp.conv_state.copy(),
            "out": workloads.poison(inp.x.shape, wl.x_dtype),
            "windows": None if wl.prefill else workloads.poison_like_windows(wl)}
    bounds = np.linspace(0, wl.n_seq, threads + 1).astype(int)
    parts = [(int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    rates, passes = [], []
    with ThreadPoolExecutor(max_workers=len(parts)) as pool:
        for _ in range(runs):
            k, t0 = 0, time.perf_counter()
            while True:
                list(pool.map(lambda r: _oracle_rows(inp, bufs, *r), parts))
                k += 1
                el = time.perf_counter() - t0
                if el >= run_s:
                    break
            rates.append(alg_bytes * k / el / 1e9)
            passes.append(k)
    return float(np.median(rates)), rates, passes


def cpu_baseline(inp, alg_bytes, run_s_single=3.0, run_s_all=1.5):
    """The C oracle as it stands on the host: one thread, then every thread this process
    may use (over disjoint row slices), each the median of 3 timed runs."""
    wl = inp.wl
    threads = host_threads()
    one, one_runs, one_passes = _cpu_leg(inp, alg_bytes, 1, run_s_single)
    allv, all_runs, all_passes = _cpu_leg(inp, alg_bytes, threads, run_s_all)
    what = {"verify": "", "restore": " (verify + restore; bytes of the restore)",
            "prefill": " (prefill conv + separate L2)"}[step_kind(wl)]
    return {"value": round(allv, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"whole passes over the {wl.name} problem{what}; median of 3 runs of "
                      f"~{run_s_all:g} s on {threads} threads (rows split into {threads} "
                      f"slices; {all_passes} passes) and of ~{run_s_single:g} s on one "
                      f"thread ({one_passes} passes)",
            "single_thread": round(one, 3), "single_thread_runs": [round(r, 3) for r in one_runs],
            "all_threads_runs": [round(r, 3) for r in all_runs],
            "nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}


def _launches(cv, wl, p, stream, setup=True):
    """Zero-argument launch callables of one step on problem p (timed), and of its
    dominant kernel alone (for the roofline).  setup: run the restore's verify first."""
    kw = dict(qk_channels=wl.qk_channels, head_dim=wl.head_dim, l2_eps=wl.l2_eps, stream=stream)
    kind = step_kind(wl)
    if kind == "prefill":
        pre = cv.prepare("prefill", p.x, p.weight, p.bias, p.conv_state, p.out, p.cu,
                         max_len=wl.T, slot_idx=p.slot_idx, has_initial_state=p.has_init,
                         stream=stream)
        l2 = cv.prepare("l2", p.out, **kw)
        return [pre, l2], pre
    if kind == "restore":
        if setup:
            p.verify(stream)   # the windows the restore reads
        rst = cv.prepare("restore", p.conv_state, p.windows, p.restore_k, layout=p.layout,
                         d_conv=wl.d_conv, slot_idx=p.slot_idx, stream=stream)
        return [rst], rst
    args = [p.x, p.weight, p.bias, p.conv_state, p.out, p.windows] + ([p.parent] if wl.tree else [])
    ver = cv.prepare("tree" if wl.tree else "update", *args, layout=p.layout,
                     slot_idx=p.slot_idx, num_accept_tokens=p.nat, cu_seqlens=p.cu, **kw)
    return [ver], ver


def _graph_time(torch, cv, wl, problems, steps, stream):
    """Mean step time (ms) when one step per buffer set is captured in a HIP graph and
    the graph is replayed; the launches are prepared on the capture stream."""
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for p in problems:
            for f in _launches(cv, wl, p, side, setup=False)[0]:
                f()
    reps = max(1, steps // len(problems))
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / (reps * len(problems))


def _time(torch, fns_per_set, steps, warmup, stream):
    sets = len(fns_per_set)
    for i in range(warmup):
        for f in fns_per_set[i % sets]:
            f()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        for f in fns_per_set[i % sets]:
            f()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def _say(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def measure(torch, cv, gh, key, args, stream):
    """Parity at full size (unless --no-check), then the timed launches of one workload.
    Returns what the JSON line reports about it."""
    wl = workloads.WORKLOADS[key]
    _say(f"{wl.name}: inputs")
    inp = workloads.make_inputs(wl)
    kind = step_kind(wl)
    alg = step_bytes(wl, inp)
    dom_bytes = workloads.algorithmic_bytes(wl, inp) if kind == "prefill" else alg
    sb = 4 if wl.state_dtype == "f32" else 2
    set_bytes = workloads.algorithmic_bytes(wl, inp) + wl.n_slots * wl.d_inner * wl.state_len * sb
    # Every stream must outgrow the 256 MB Infinity Cache across the rotation, not only the
    # whole set: with 2x the MALL in total, buffers of a single stream (out, say) still fit
    # in it and were measured up to 12% faster than HBM allows.  8x keeps each stream of the
    # workloads here at >= 1.5x the MALL (the 32-set cap is reached only by small sets).
    sets = args.sets or max(1, min(32, math.ceil(8 * MALL_BYTES / set_bytes)))

    check = None
    if not args.no_check:
        _say(f"{wl.name}: full-size parity against the oracle")
        p0 = gh.GeneralProblem(inp)
        step, _ = _launches(cv, wl, p0, stream)
        if kind == "prefill":
            # each stage against the oracle on the same input: the prefill conv, then
            # the L2 over the GPU's own prefill output
            step[0]()
            got = p0.results()
            check = gh.compare_general(got, gh.oracle_general(inp), inp)
            ref_l2 = _oracle_l2(got["out"], wl)
            step[1]()
            check["l2"] = gh.compare_general(p0.results(), {"out": ref_l2}, inp)
        else:
            for f in step:
                f()
            check = gh.compare_general(p0.results(), _oracle_step(inp), inp)
        del p0

    _say(f"{wl.name}: {sets} buffer sets, {args.steps} timed launches")
    problems = [gh.GeneralProblem(inp) for _ in range(sets)]
    built = [_launches(cv, wl, p, stream) for p in problems]
    ms = _time(torch, [b[0] for b in built], args.steps, args.warmup, stream)
    dom_ms = ms if kind != "prefill" else _time(torch, [[b[1]] for b in built], args.steps,
                                                args.warmup, stream)
    graph_us = None
    if args.graph:
        graph_us = _graph_time(torch, cv, wl, problems, args.steps, stream) * 1e3
    del built, problems
    torch.cuda.empty_cache()
    return {"wl": wl, "inp": inp, "kind": kind, "alg": alg, "dom_bytes": dom_bytes,
            "sets": sets, "ms": ms, "dom_ms": dom_ms, "check": check, "graph_us": graph_us}


def _summary(m) -> dict:
    """The per-workload record of an extra workload on the line."""
    wl = m["wl"]
    gbs = m["dom_bytes"] / (m["dom_ms"] * 1e-3) / 1e9
    rec = {"workload": wl.name, "n_seq": wl.n_seq, "T": wl.T, "d_inner": wl.d_inner,
           "layout": wl.layout,
           "conv_state": "time-major" if wl.state_tm else "channel-major",
           "us_per_launch": round(m["dom_ms"] * 1e3, 3), "algorithmic_bytes": m["dom_bytes"],
           "achieved": round(gbs, 1), "frac": round(gbs / PEAK_GBS, 4),
           "buffer_sets": m["sets"], "traffic": measured_traffic(wl.name)}
    if m["check"] is not None:
        rec["parity"] = m["check"]
    return rec


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="2")
    ap.add_argument("--also", default="auto",
                    help="comma-separated workload keys timed after the main one and reported "
                         "under `stress` (auto: 4,4b,4t,4bt with the default workload, none "
                         "otherwise; none: skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true", help="skip the full-size parity check")
    ap.add_argument("--sets", type=int, default=0, help="buffer sets (0: auto, >= 8x MALL)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the steps replayed from a captured HIP graph (one graph "
                         "holds one step per buffer set), reported as config.graph_us_per_step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 256 MiB -> 256 MiB elementwise copy (10 dispatches), "
                         "the reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the verify conv shards by sequence or by "
              "channel with no exchange, and the library runs on a single MI355X "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import torch

    import causal_conv1d_verify_amd as cv
    import gpu_harness as gh

    if args.calibrate_copy:
        n = 64 * 2 ** 20   # fp32 elements: 256 MiB read + 256 MiB written per dispatch
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "elementwise copy", "read_bytes": 4 * n,
                          "write_bytes": 4 * n, "dispatches": 10}), flush=True)
        return 0

    key = int(args.workload) if args.workload.isdigit() else args.workload
    if args.also == "auto":
        also = ["4", "4b", "4t", "4bt"] if args.workload == "2" else []
    elif args.also in ("", "none"):
        also = []
    else:
        also = [k.strip() for k in args.also.split(",") if k.strip()]
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    m = measure(torch, cv, gh, key, args, stream)
    wl, kind, alg, ms = m["wl"], m["kind"], m["alg"], m["ms"]
    us = ms * 1e3
    gbs = alg / (ms * 1e-3) / 1e9
    dom_gbs = m["dom_bytes"] / (m["dom_ms"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "step": kind, "n_seq": wl.n_seq, "T": wl.T,
            "d_inner": wl.d_inner, "d_conv": wl.d_conv, "qk_channels": wl.qk_channels,
            "head_dim": wl.head_dim, "layout": wl.layout, "packed_rows": wl.varlen,
            "tree": wl.tree, "storage": f"x {wl.x_dtype}, state {wl.state_dtype}",
            "conv_state": "time-major" if wl.state_tm else "channel-major",
            "bias": wl.bias, "us_per_step": round(us, 3), "algorithmic_bytes": alg,
            "buffer_sets": m["sets"], "pct_of_peak": round(100 * gbs / PEAK_GBS, 1),
        },
        "roofline": {
            "bound": "hbm", "achieved": round(dom_gbs, 1), "peak": PEAK_GBS, "unit": "GB/s",
            "frac": round(dom_gbs / PEAK_GBS, 4), "traffic": measured_traffic(wl.name),
        },
    }
    if m["check"] is not None:
        line["config"]["parity"] = m["check"]
    if m["graph_us"] is not None:
        line["config"]["graph_us_per_step"] = round(m["graph_us"], 3)
    if kind == "prefill":
        line["roofline"]["kernel"] = (f"prefill conv alone: {m['dom_bytes']} bytes in "
                                      f"{m['dom_ms'] * 1e3:.3f} us")
    if also:
        extra_args = argparse.Namespace(**{**vars(args), "graph": False})
        line["stress"] = [_summary(measure(torch, cv, gh, int(k) if k.isdigit() else k,
                                           extra_args, stream)) for k in also]
    if not args.no_cpu_baseline:
        _say(f"{wl.name}: CPU oracle legs")
        line["cpu_baseline"] = cpu_baseline(m["inp"], alg)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
