"""Benchmark of the batched speculative-verify causal conv1d update on one MI355X.

One step = one launch of the whole hot path (conv + SiLU + per-head L2 + every
rollback window + committed state) over one batch of seeded synthetic inputs.
Default workload: dedup_bs128_t8 (n_seq 128, d_inner 10240, T 8, bf16, dedup rows,
bias on) - the GB300 workload of sglang PR 46184's benchmark table.

    python bench.py [--steps K] [--warmup W] [--workload 2|0|1|3|4|4b|4s]

Prints ONE JSON line.  `value` is achieved algorithmic HBM bandwidth (GB/s): the
bytes one launch must move (x, out, the conv_state window read and the committed
window write, the rollback windows, weight and bias; active rows only) divided by the
mean launch time measured with HIP events on the launch stream.  The inputs rotate
over enough buffer sets that the working set is >= 2x the 256 MB Infinity Cache, so
data is fetched from HBM.  The CPU oracle is timed on a bounded sample beside it.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
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
KERNEL_SRC = os.path.join(ROOT, "causal_conv1d_verify_amd", "csrc", "cv_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


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


def cpu_baseline(inp, alg_bytes, budget_s=10.0, max_reps=50):
    """The C oracle, single-threaded, on the full problem repeated for ~budget_s."""
    import oracle

    wl = inp.wl
    state = inp.conv_state.copy()
    out = workloads.poison(inp.x.shape, wl.x_dtype)
    win = workloads.poison_like_windows(wl)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.conv_verify(inp.x, inp.weight, inp.bias, state, out, win, d_inner=wl.d_inner,
                           qk_channels=wl.qk_channels, head_dim=wl.head_dim,
                           l2_eps=wl.l2_eps, x_dtype=wl.x_dtype, state_dtype=wl.state_dtype,
                           layout=wl.layout, slot_idx=inp.slot_idx,
                           num_accept_tokens=inp.num_accept_tokens)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= max_reps:
            break
    return {"value": round(alg_bytes * reps / el / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"the whole {wl.name} problem, {reps} calls in {el:.1f} s "
                      f"({el / reps * 1e3:.0f} ms/call), one thread"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true", help="skip the full-size parity check")
    ap.add_argument("--sets", type=int, default=0, help="buffer sets (0: auto, >= 2x MALL)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 256 MiB -> 256 MiB elementwise copy (10 dispatches), "
                         "the reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the verify conv shards by sequence or by "
              "channel with no exchange, and this build runs on a single MI355X "
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
    wl = workloads.WORKLOADS[key]
    inp = workloads.make_inputs(wl)
    alg = workloads.algorithmic_bytes(wl, inp)
    torch.cuda.set_device(0)

    set_bytes = alg + wl.n_slots * wl.d_inner * wl.state_len * (4 if wl.state_dtype == "f32" else 2)
    sets = args.sets or max(1, min(32, math.ceil(2 * MALL_BYTES / set_bytes)))
    problems = [gh.DeviceProblem(inp) for _ in range(sets)]
    stream = torch.cuda.current_stream()

    check = None
    if not args.no_check:
        import oracle

        problems[0].run(stream)
        check = gh.compare(problems[0].results(), oracle.run_inputs(inp), wl,
                           gh.active_rows(inp))

    dedup = wl.layout == "dedup"
    launches = [cv.prepare(dedup, p.x, p.weight, p.bias, p.conv_state, p.out, p.windows,
                           qk_channels=wl.qk_channels, head_dim=wl.head_dim,
                           l2_eps=wl.l2_eps, slot_idx=p.slot_idx, num_accept_tokens=p.nat,
                           stream=stream) for p in problems]
    for i in range(args.warmup):
        launches[i % sets]()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        launches[i % sets]()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    us = ms * 1e3
    gbs = alg / (ms * 1e-3) / 1e9

    traffic = measured_traffic(wl.name)
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
            "workload": wl.name, "n_seq": wl.n_seq, "T": wl.T, "d_inner": wl.d_inner,
            "d_conv": wl.d_conv, "qk_channels": wl.qk_channels, "head_dim": wl.head_dim,
            "layout": wl.layout, "storage": f"x {wl.x_dtype}, state {wl.state_dtype}",
            "bias": wl.bias, "us_per_launch": round(us, 3), "algorithmic_bytes": alg,
            "buffer_sets": sets, "pct_of_peak": round(100 * gbs / PEAK_GBS, 1),
        },
        "roofline": {
            "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_GBS, 4), "traffic": traffic,
        },
    }
    if check is not None:
        line["config"]["parity"] = check
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, alg)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
