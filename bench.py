#!/usr/bin/env python3
"""Route + align benchmark on one MI355X.

One step = one mr_route_align launch (gate contraction, bf16 rounding, top-k,
softmax + renormalise, shared slot, moe_align_block_size) over one layer's
inputs.  Inputs rotate over R independent copies (x, gate rows, shared row)
whose total size exceeds the 256 MB last-level cache and the L2s, so every
launch streams its gate rows from HBM, as a model's layers do.  The R
launches are captured once into a HIP graph and replayed; HIP events on the
launch stream bracket exactly `steps` launches.

Prints one JSON line (see the keys below).  `--gpus N` with N > 1 exits: this
benchmark runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "route+align µs/layer at M=4 (E=512,k=10); rows/s at M=2048; % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
ROTATE_BYTES = 512 << 20        # inputs rotated per replay


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=8192)
    ap.add_argument("--warmup", type=int, default=512)
    ap.add_argument("--workload", default="m4", choices=["m4", "m2048", "c3", "c4"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time spent timing the CPU oracle (0 disables)")
    ap.add_argument("--secondary-steps", type=int, default=1024,
                    help="launches timed on the M=2048 workload reported beside the M=4 line (0 disables)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain device copy of known size (HBM counter calibration)")
    return ap.parse_args()


def workload(name):
    from moe_token_routing_amd import workloads as W

    return {"m4": W.ROUTER_E512_M4, "m2048": W.sweep_workload(2048), "c3": W.PREFILL_E128_M128,
            "c4": W.PREFILL_E128_M2048_ZIPF}[name]


def make_copies(wl, R, device):
    """Copy 0 is the seeded workload input; copies 1..R-1 draw the same
    distributions from a seeded torch generator on the device."""
    import numpy as np
    import torch

    from moe_token_routing_amd import workloads as W

    d = W.workload_inputs(wl)

    def dev(b):
        return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(device)

    copies = [(dev(d["x"]), dev(d["w"]), dev(d["ws"]) if d["ws"] is not None else None)]
    g = torch.Generator(device=device)
    g.manual_seed(1234)
    for _ in range(1, R):
        x = torch.randn(wl.M, wl.H, generator=g, device=device, dtype=torch.float32)
        w = torch.randn(wl.E, wl.H, generator=g, device=device, dtype=torch.float32) * 0.02
        if wl.dist == "zipf":
            x[:, 0] = 1.0
            w[:, 0] = copies[0][1][:, 0].float()
        ws = (torch.randn(1, wl.H, generator=g, device=device) * 0.02).to(torch.bfloat16) if wl.shared else None
        copies.append((x.to(torch.bfloat16), w.to(torch.bfloat16), ws))
    return d, copies


def algorithmic_bytes(wl, npp, A):
    """Bytes one launch must move: every input element once and every output
    element once (sorted_token_ids up to npp, expert_ids up to npp/A)."""
    Ep = wl.E + int(wl.shared)
    read = Ep * wl.H * 2 + wl.M * wl.H * 2
    write = wl.M * wl.S * 8 + npp * 4 + (npp // A) * 4 + 4
    return read + write


def cpu_baseline(d, wl, seconds):
    import oracle

    threads = os.cpu_count() or 1
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        threads = max(1, min(threads, int(os.environ["OMP_NUM_THREADS"])))
    n = 0
    t0 = time.perf_counter()
    while True:
        r = oracle.route(d["x"], d["w"], d["ws"], wl.k, wl.scale, nthreads=threads)
        oracle.align(r["ids"], wl.num_experts, oracle.select_alignment(wl.M, wl.k, wl.E))
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    per = dt / n
    if wl.M >= 512:
        value, unit = wl.M / per, "rows/s"
    else:
        value, unit = per * 1e6, "us/layer"
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{n} full oracle route+align calls on the {wl.name} input (seed 0), {dt:.1f} s"}


def calibrate_copy():
    import torch

    nbytes = 256 << 20
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    torch.cuda.synchronize()
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": nbytes, "bytes_written": nbytes, "launches": 10}))


def source_digest(kernel):
    """sha256 over the sources the kernel is compiled from."""
    import hashlib

    csrc = os.path.join(ROOT, "moe_token_routing_amd", "csrc")
    main = {"route_small_kernel": "route_small.hip", "route_mfma_kernel": "route_mfma.hip"}[kernel]
    h = hashlib.sha256()
    for f in [main, "device_common.h", "kernels.h"]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profiled_traffic(kernel, wl_name):
    """HBM bytes per launch from the committed counter summary for this
    kernel and workload (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled
    by what the counter reads for a device copy of known size), or None when
    there is none or it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{wl_name}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line:
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    if fields.get("source_sha256") != source_digest(kernel) or "hbm_bytes_per_launch" not in fields:
        return None
    return int(float(fields["hbm_bytes_per_launch"]))


def measure(wl, steps, warmup):
    """Times `steps` route+align launches on workload `wl`; returns the seeded
    input and the result fields."""
    import torch

    import moe_token_routing_amd as mr

    device = "cuda:0"
    per_copy = (wl.E + int(wl.shared)) * wl.H * 2 + wl.M * wl.H * 2
    R = max(8, math.ceil(ROTATE_BYTES / per_copy))
    d, copies = make_copies(wl, R, device)
    A = mr.mr_select_alignment(wl.M, wl.k, wl.E)
    ws = mr.new_workspace(wl.M, wl.E, wl.k, wl.shared, device=device)
    outs = []
    for (x, w, s) in copies:
        o = mr.mr_route_align(x, w, s, wl.k, wl.scale, A, workspace=ws)
        outs.append(o)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream(device=device)
    graphs = {}

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                x, w, s = copies[i % R]
                o = outs[i % R]
                mr.mr_route_align(x, w, s, wl.k, wl.scale, A, workspace=ws, topk_ids=o["topk_ids"],
                                  topk_weights=o["topk_weights"], sorted_token_ids=o["sorted_token_ids"],
                                  expert_ids=o["expert_ids"], npp=o["npp"])
        return g

    graphs[R] = capture(R)
    rem = steps % R
    if rem:
        graphs[rem] = capture(rem)

    cur = torch.cuda.current_stream(device)
    for _ in range(max(1, math.ceil(warmup / R))):
        graphs[R].replay()
    torch.cuda.synchronize()

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(cur)
    for _ in range(steps // R):
        graphs[R].replay()
    if rem:
        graphs[rem].replay()
    end.record(cur)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / steps

    npps = [int(o["npp"].item()) for o in outs]
    mean_npp = sum(npps) / len(npps)
    for n in npps:
        assert n % A == 0 and n > 0
    nbytes = algorithmic_bytes(wl, mean_npp, A)
    launch_s = ms_per_step * 1e-3
    achieved_gbs = nbytes / launch_s / 1e9
    flops = 2.0 * wl.M * (wl.E + int(wl.shared)) * wl.H

    if wl.M >= 512:
        value, unit, hib = wl.M / launch_s, "rows/s", True
    else:
        value, unit, hib = ms_per_step * 1e3, "us/layer", False
    mfma_tflops = flops / launch_s / 1e12
    if wl.M >= 512 and flops / nbytes > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": round(mfma_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(mfma_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None}
    else:
        roof = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": None}
    roof["kernel"] = "route_small_kernel" if wl.M <= 16 else "route_mfma_kernel"
    roof["traffic"] = profiled_traffic(roof["kernel"], wl.name)
    roof["bytes_per_launch"] = int(nbytes)
    roof["flops_per_launch"] = int(flops)

    result = {
        "value": round(value, 3) if unit == "us/layer" else round(value, 1),
        "unit": unit,
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": hib,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "M": wl.M, "E": wl.E, "shared": wl.shared, "H": wl.H, "k": wl.k,
                   "A": A, "rotation_copies": R, "rotation_bytes": R * per_copy,
                   "timing": "HIP graph of launches over rotated inputs; HIP events on the launch stream"},
        "roofline": roof,
    }
    return d, result


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (routing shards by token: "
              "each GPU would run this same launch on its own tokens)", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.calibrate_copy:
        calibrate_copy()
        return
    import moe_token_routing_amd as mr

    mr._binding.lib()
    torch.cuda.set_device(0)
    wl = workload(args.workload)
    d, result = measure(wl, args.steps, args.warmup)
    result = {"metric": METRIC, **result}
    if args.secondary_steps > 0 and args.workload == "m4":
        _, sec = measure(workload("m2048"), args.secondary_steps, min(args.warmup, 256))
        result["secondary"] = {kk: sec[kk] for kk in ["value", "unit", "ms_per_step", "steps", "config", "roofline"]}
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(d, wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
