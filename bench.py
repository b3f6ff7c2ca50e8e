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
FLUSH_BYTES = 512 << 20         # the fill before each call in the memset method
SWEEP_M = (1, 2, 3, 4, 5, 8, 9, 12, 16, 17, 24, 32, 40, 64, 128, 512, 2048)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=8192)
    ap.add_argument("--warmup", type=int, default=512)
    ap.add_argument("--workload", default="m4", choices=[f"m{m}" for m in SWEEP_M] + ["c3", "c4", "argmax", "align_ep", "consumer"],
                    help="m<M>: E=512+1, H=4096, k=10 at M tokens (m4 is the headline); c3: E=128, H=2048, "
                         "k=8, M=128; c4: the same at M=2048 with Zipf-skewed gate rows; argmax: row-wise fp32 "
                         "argmax of [16, 248320] (the sampling shape); align_ep: mr_align over all 513 experts vs "
                         "mr_align_local for one of 8 expert-parallel ranks, on M=2048 routing ids; consumer: the "
                         "padding study (align + grouped-expert GEMM at A = 64 and 128 over a token sweep)")
    ap.add_argument("--align", type=int, default=None, choices=[64, 128],
                    help="force the alignment A (default: the M-aware tier)")
    ap.add_argument("--method", default="rotate", choices=["rotate", "memset"],
                    help="rotate: graph replay over rotated inputs (default); memset: a 512 MB fill before "
                         "each call, per-call time = (fills + calls) - (fills alone)")
    ap.add_argument("--stream-read", action="store_true",
                    help="time only the plain streaming-read kernel at 4 MiB and 512 MiB")
    ap.add_argument("--cpu-only", action="store_true", help="time only the CPU oracle on the workload")
    ap.add_argument("--cpu-threads", type=int, default=None,
                    help="oracle threads (default: every host core, capped by OMP_NUM_THREADS)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time spent timing the CPU oracle (0 disables)")
    ap.add_argument("--secondary-steps", type=int, default=1024,
                    help="launches timed on the M=2048 workload reported beside the M=4 line (0 disables)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain device copy of known size (HBM counter calibration)")
    return ap.parse_args()


def workload(name):
    from moe_token_routing_amd import workloads as W

    if name == "m4":
        return W.ROUTER_E512_M4
    if name.startswith("m"):
        return W.sweep_workload(int(name[1:]))
    return {"c3": W.PREFILL_E128_M128, "c4": W.PREFILL_E128_M2048_ZIPF}[name]


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


def cpu_baseline(d, wl, seconds, threads=None, A=None):
    """The oracle as it stands, timed on the host: full route+align calls on
    the workload's seeded input until `seconds` have passed (at least one);
    the value is the median call."""
    import oracle

    if threads is None:
        threads = os.cpu_count() or 1
        if os.environ.get("OMP_NUM_THREADS", "").isdigit():
            threads = max(1, min(threads, int(os.environ["OMP_NUM_THREADS"])))
    if A is None:
        A = oracle.select_alignment(wl.M, wl.k, wl.E)
    times = []
    t0 = time.perf_counter()
    while True:
        t1 = time.perf_counter()
        r = oracle.route(d["x"], d["w"], d["ws"], wl.k, wl.scale, nthreads=threads)
        oracle.align(r["ids"], wl.num_experts, A)
        times.append(time.perf_counter() - t1)
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    per = sorted(times)[len(times) // 2]
    if wl.M >= 512:
        value, unit = wl.M / per, "rows/s"
    else:
        value, unit = per * 1e6, "us/layer"
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle", "us_per_call": round(per * 1e6, 1),
            "sample": f"median of {len(times)} full oracle route+align calls on the {wl.name} input (seed 0), "
                      f"{dt:.1f} s"}


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
    files = {"route_small_kernel": ["route_small.hip", "device_common.h", "kernels.h"],
             "route_mfma_kernel": ["route_mfma.hip", "device_common.h", "kernels.h"],
             "argmax_kernel": ["argmax.hip", "argmax.h", "device_common.h"]}[kernel]
    h = hashlib.sha256()
    for f in files:
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


def result_fields(wl, A, ms_per_step, mean_npp, npps, steps, warmup, timing):
    """The bench line's fields for one timed workload."""
    for n in npps:
        assert n % A == 0 and n > 0
    nbytes = algorithmic_bytes(wl, mean_npp, A)
    launch_s = ms_per_step * 1e-3
    achieved_gbs = nbytes / launch_s / 1e9
    flops = 2.0 * wl.M * (wl.E + int(wl.shared)) * wl.H
    mfma_tflops = flops / launch_s / 1e12

    if wl.M >= 512:
        value, unit, hib = wl.M / launch_s, "rows/s", True
    else:
        value, unit, hib = ms_per_step * 1e3, "us/layer", False
    hbm = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": None}
    mfma = {"bound": "mfma", "achieved": round(mfma_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(mfma_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None}
    if wl.M >= 512 and flops / nbytes > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        roof = dict(mfma, hbm_frac=hbm["frac"])
    else:
        roof = dict(hbm, mfma_frac=mfma["frac"]) if wl.M >= 512 else hbm
    roof["kernel"] = "route_small_kernel" if wl.M <= 16 else "route_mfma_kernel"
    roof["traffic"] = profiled_traffic(roof["kernel"], wl.name)
    roof["bytes_per_launch"] = int(nbytes)
    roof["flops_per_launch"] = int(flops)
    return {
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
                   "A": A, "timing": timing},
        "roofline": roof,
    }


def measure_memset(wl, calls, reps, A=None):
    """The pages' method: a 512 MB fill before every call evicts the L2s and
    the memory-side cache, so each call reads its inputs from HBM.  Per call
    = (replay of fill+call pairs - replay of the fills alone) / calls, the
    medians over `reps` replays of each."""
    import torch

    import moe_token_routing_amd as mr

    device = "cuda:0"
    d, copies = make_copies(wl, 1, device)
    x, w, s = copies[0]
    if A is None:
        A = mr.mr_select_alignment(wl.M, wl.k, wl.E)
    ws = mr.new_workspace(wl.M, wl.E, wl.k, wl.shared, device=device)
    o = mr.mr_route_align(x, w, s, wl.k, wl.scale, A, workspace=ws)
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device=device)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream(device=device)

    def capture(with_call):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(calls):
                flush.zero_()
                if with_call:
                    mr.mr_route_align(x, w, s, wl.k, wl.scale, A, workspace=ws, topk_ids=o["topk_ids"],
                                      topk_weights=o["topk_weights"], sorted_token_ids=o["sorted_token_ids"],
                                      expert_ids=o["expert_ids"], npp=o["npp"])
        return g

    graphs = {True: capture(True), False: capture(False)}
    cur = torch.cuda.current_stream(device)
    for g in graphs.values():
        g.replay()
    torch.cuda.synchronize()
    times = {True: [], False: []}
    for _ in range(reps):
        for key, g in graphs.items():
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(cur)
            g.replay()
            e1.record(cur)
            torch.cuda.synchronize()
            times[key].append(e0.elapsed_time(e1))
    med = {key: sorted(t)[len(t) // 2] for key, t in times.items()}
    ms_per_call = (med[True] - med[False]) / calls
    npp = int(o["npp"].item())
    timing = (f"pages' method: a {FLUSH_BYTES >> 20} MiB fill before each call; per call = (graph of fill+call "
              f"- graph of fills) / {calls}, medians of {reps} replays each")
    result = result_fields(wl, A, ms_per_call, npp, [npp], calls * reps, calls, timing)
    result["config"]["fill_ms_per_call"] = round(med[False] / calls, 4)
    return d, result


def stream_read(reps=20):
    """One plain streaming-read launch at 4 MiB and at 512 MiB: the 4 MiB
    launches rotate over a 512 MiB buffer (each reads from HBM), as the route
    launches do; graph replay, HIP events on the launch stream."""
    import torch

    import moe_token_routing_amd as mr

    device = "cuda:0"
    words = ROTATE_BYTES // 4
    buf = torch.arange(words, dtype=torch.int32, device=device)
    out = torch.zeros(mr.MR_STREAM_READ_OUT_WORDS, dtype=torch.int32, device=device)
    stream = torch.cuda.Stream(device=device)
    cur = torch.cuda.current_stream(device)
    rows = []
    for size in (4 << 20, 512 << 20):
        R = ROTATE_BYTES // size
        n = max(R, 8)
        views = [buf[(i % R) * (size // 4):((i % R) + 1) * (size // 4)] for i in range(n)]
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for v in views:
                mr.mr_debug_stream_read(v, out)
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        for _ in range(reps):
            g.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * n)
        gbs = size / (us * 1e-6) / 1e9
        rows.append({"bytes": size, "launches": reps * n, "us_per_launch": round(us, 3), "GB/s": round(gbs, 1),
                     "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
    return {"stream_read": rows, "timing": "HIP graph replay, HIP events on the launch stream"}


ARGMAX_R, ARGMAX_N = 16, 248320


def argmax_input(seed=0):
    """[16, 248320] fp32 logits ~ N(0, 1) with a few planted NaNs, ties and
    signed zeros (seeded)."""
    import numpy as np

    rng = np.random.default_rng(seed)
    x = rng.standard_normal((ARGMAX_R, ARGMAX_N)).astype(np.float32)
    x[1, rng.choice(ARGMAX_N, 3, replace=False)] = np.nan
    x[2, rng.choice(ARGMAX_N, 40, replace=False)] = 8.0
    x[3] = rng.choice(np.array([0.0, -0.0, -1.0], dtype=np.float32), ARGMAX_N)
    return x


def measure_argmax(steps, warmup, cpu_seconds):
    """Times mr_argmax_rows_f32 on [16, 248320] fp32: graph replay over R
    rotated copies totalling >= 512 MiB (cold: every launch reads HBM) and
    over one copy (hot: the 15.9 MB input stays in the memory-side cache);
    torch.argmax(dim=1) in the same harness for context."""
    import numpy as np
    import torch

    import moe_token_routing_amd as mr
    import oracle

    device = "cuda:0"
    nbytes = ARGMAX_R * ARGMAX_N * 4
    R = max(8, math.ceil(ROTATE_BYTES / nbytes))
    x0 = argmax_input()
    g = torch.Generator(device=device)
    g.manual_seed(99)
    copies = [torch.from_numpy(x0).to(device)] + [torch.randn(ARGMAX_R, ARGMAX_N, generator=g, device=device)
                                                  for _ in range(R - 1)]
    ws = mr.new_argmax_workspace(ARGMAX_R, ARGMAX_N, device=device)
    out = torch.empty(ARGMAX_R, dtype=torch.int64, device=device)
    got = mr.mr_argmax_rows_f32(copies[0], workspace=ws, out=out).cpu().numpy()
    assert np.array_equal(got, oracle.argmax_rows(x0)), "argmax differs from the oracle"
    stream = torch.cuda.Stream(device=device)
    cur = torch.cuda.current_stream(device)

    def timed(fn, n_rot):
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(n_rot):
                fn(copies[i % R])
        reps = max(1, steps // n_rot)
        for _ in range(max(1, warmup // n_rot)):
            graph.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        for _ in range(reps):
            graph.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * n_rot), reps * n_rot

    ours = lambda x: mr.mr_argmax_rows_f32(x, workspace=ws, out=out)  # noqa: E731
    theirs = lambda x: torch.argmax(x, dim=1)  # noqa: E731
    ms_cold, n_cold = timed(ours, R)
    ms_hot, _ = timed(lambda x: ours(copies[0]), R)
    ms_torch_cold, _ = timed(theirs, R)
    ms_torch_hot, _ = timed(lambda x: theirs(copies[0]), R)
    alg = nbytes + ARGMAX_R * 8
    gbs = alg / (ms_cold * 1e-3) / 1e9
    result = {
        "metric": "row-wise fp32 argmax (PyTorch semantics) us/call at [16, 248320]",
        "value": round(ms_cold * 1e3, 3),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": n_cold,
        "warmup": warmup,
        "ms_per_step": round(ms_cold, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "argmax_f32_r16_n248320", "R": ARGMAX_R, "N": ARGMAX_N, "rotation_copies": R,
                   "timing": "HIP graph of launches over rotated inputs; HIP events on the launch stream"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": profiled_traffic("argmax_kernel", "argmax_f32_r16_n248320"), "kernel": "argmax_kernel",
                     "bytes_per_launch": alg},
        "hot_us": round(ms_hot * 1e3, 3),
        "torch_argmax_us": {"cold": round(ms_torch_cold * 1e3, 3), "hot": round(ms_torch_hot * 1e3, 3)},
    }
    if cpu_seconds > 0:
        threads = os.cpu_count() or 1
        if os.environ.get("OMP_NUM_THREADS", "").isdigit():
            threads = max(1, min(threads, int(os.environ["OMP_NUM_THREADS"])))
        times = []
        t0 = time.perf_counter()
        while True:
            t1 = time.perf_counter()
            oracle.argmax_rows(x0, nthreads=threads)
            times.append(time.perf_counter() - t1)
            if time.perf_counter() - t0 >= cpu_seconds:
                break
        per = sorted(times)[len(times) // 2]
        result["cpu_baseline"] = {"value": round(per * 1e6, 1), "unit": "us/call", "cores": threads, "kind": "oracle",
                                  "sample": f"median of {len(times)} oracle argmax calls on the seeded "
                                            f"[16, 248320] input, {time.perf_counter() - t0:.1f} s"}
    return result


def measure_align_ep(steps, warmup):
    """Times the align alone on M=2048 tokens x (10 routed + 1 shared) ids
    over E' = 513 experts (seeded: distinct routed experts per token, the
    shared expert id 512 in the last column): mr_align over every expert,
    and mr_align_local for rank 0 of 8 (routed experts e with e % 8 == 0,
    the shared expert replicated).  Graph replay, HIP events."""
    import numpy as np
    import torch

    import moe_token_routing_amd as mr
    import oracle

    device = "cuda:0"
    M, k, E, ranks = 2048, 10, 512, 8
    rng = np.random.default_rng(0)
    ids = np.empty((M, k + 1), np.int32)
    for m in range(M):
        ids[m, :k] = rng.choice(E, k, replace=False)
    ids[:, k] = E
    emap = np.full(E + 1, -1, np.int32)
    own = np.arange(0, E, ranks)
    emap[own] = np.arange(own.size, dtype=np.int32)
    emap[E] = own.size
    A = mr.mr_select_alignment(M, k, E)
    t_ids = torch.from_numpy(ids).to(device)
    t_map = torch.from_numpy(emap).to(device)
    ws_full = mr.new_workspace(M, E + 1, k + 1, False, device=device)
    ws_loc = mr.new_workspace(M, own.size + 1, k + 1, False, device=device)
    full = mr.mr_align(t_ids, E + 1, A, workspace=ws_full)
    loc = mr.mr_align_local(t_ids, t_map, own.size + 1, A, workspace=ws_loc)
    torch.cuda.synchronize()
    for (srt, eids, npp), want in ((full, oracle.align(ids, E + 1, A)), (loc, oracle.align_local(ids, emap, own.size + 1, A))):
        n = int(npp.item())
        assert n == want[2] and np.array_equal(srt[:n].cpu().numpy(), want[0]), "align differs from the oracle"
    stream = torch.cuda.Stream(device=device)
    cur = torch.cuda.current_stream(device)

    def timed(fn):
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(32):
                fn()
        for _ in range(max(1, warmup // 32)):
            g.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // 32)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        for _ in range(reps):
            g.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * 32) * 1e3

    us_full = timed(lambda: mr.mr_align(t_ids, E + 1, A, workspace=ws_full, sorted_token_ids=full[0],
                                        expert_ids=full[1], npp=full[2]))
    us_loc = timed(lambda: mr.mr_align_local(t_ids, t_map, own.size + 1, A, workspace=ws_loc,
                                             sorted_token_ids=loc[0], expert_ids=loc[1], npp=loc[2]))
    npp_full, npp_loc = int(full[2].item()), int(loc[2].item())
    nbytes = M * (k + 1) * 4 + 4 * npp_full + 4 * (npp_full // A) + 4
    gbs = nbytes / (us_full * 1e-6) / 1e9
    return {
        "metric": "standalone align us/call at M=2048, E'=513, S=11 (all experts / one of 8 EP ranks)",
        "value": round(us_full, 3), "unit": "us/call", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(us_full * 1e-3, 6), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "int32", "data": "synthetic",
        "config": {"workload": "align_m2048_e513_s11", "A": A, "npp": npp_full, "local_rank_npp": npp_loc,
                   "timing": "HIP graph of 32 launches, HIP events on the launch stream"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "align_kernel",
                     "bytes_per_launch": nbytes},
        "local_rank_us": round(us_loc, 3),
    }


CONSUMER_E, CONSUMER_K, CONSUMER_H, CONSUMER_N = 128, 8, 2048, 512
CONSUMER_M = (6, 128, 512, 1024, 2048)


def zipf_routing(M, E, k, seed=0):
    """Top-k ids [M, k]: k distinct experts per token drawn with
    probabilities proportional to Zipf(1.1) over a seeded permutation of the
    experts (the skew of routing captured from real prefills)."""
    import numpy as np

    rng = np.random.default_rng(seed)
    rank = rng.permutation(E) + 1
    p = rank ** -1.1
    p = p / p.sum()
    return np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(M)]).astype(np.int32)


def measure_consumer(steps, warmup):
    """The padding study: for each token count, align the Zipf routing at
    A = 64 and 128 and time the grouped-expert GEMM (E=128, k=8, H=2048,
    N=512 synthetic bf16 weights) over each; the outputs must be
    bit-identical across A."""
    import numpy as np
    import torch

    import moe_token_routing_amd as mr

    device = "cuda:0"
    E, k, H, N = CONSUMER_E, CONSUMER_K, CONSUMER_H, CONSUMER_N
    g = torch.Generator(device=device)
    g.manual_seed(5)
    w = (torch.randn(E, N, H, generator=g, device=device) * 0.02).to(torch.bfloat16)
    stream = torch.cuda.Stream(device=device)
    cur = torch.cuda.current_stream(device)
    rows = []
    for M in CONSUMER_M:
        ids = zipf_routing(M, E, k, seed=M)
        x = torch.randn(M, H, generator=g, device=device).to(torch.bfloat16)
        t_ids = torch.from_numpy(ids).to(device)
        row = {"M": M, "routed_rows": M * k, "tier_A": mr.mr_select_alignment(M, k, E)}
        ys = {}
        for A in (64, 128):
            ws = mr.new_workspace(M, E, k, False, device=device)
            srt, eids, npp = mr.mr_align(t_ids, E, A, workspace=ws)
            y = mr.mr_grouped_gemm_bf16(x, w, k, srt, eids, npp, A)
            torch.cuda.synchronize()
            ys[A] = y
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=stream):
                for _ in range(8):
                    mr.mr_grouped_gemm_bf16(x, w, k, srt, eids, npp, A, y=y)
            for _ in range(max(1, warmup // 64)):
                gr.replay()
            torch.cuda.synchronize()
            reps = max(2, steps // 64)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(cur)
            for _ in range(reps):
                gr.replay()
            e1.record(cur)
            torch.cuda.synchronize()
            n = int(npp.item())
            us = e0.elapsed_time(e1) / (reps * 8) * 1e3
            row[f"npp_A{A}"] = n
            row[f"padding_ratio_A{A}"] = round(n / (M * k), 2)
            row[f"gemm_us_A{A}"] = round(us, 2)
            row[f"gemm_tflops_A{A}"] = round(2.0 * n * N * H / (us * 1e-6) / 1e12, 1)
        row["bit_identical"] = bool(torch.equal(ys[64].view(torch.int32), ys[128].view(torch.int32)))
        rows.append(row)
    return {"metric": "padding study: grouped-expert GEMM us over the align output at A=64 vs 128 (E=128, k=8, "
                      "H=2048, N=512, Zipf routing)", "rows": rows,
            "timing": "HIP graph of 8 launches, HIP events on the launch stream; tflops counts npp rows (padding "
                      "included, as the consumer computes them)"}


def measure(wl, steps, warmup, A=None):
    """Times `steps` route+align launches on workload `wl`; returns the seeded
    input and the result fields."""
    import torch

    import moe_token_routing_amd as mr

    device = "cuda:0"
    per_copy = (wl.E + int(wl.shared)) * wl.H * 2 + wl.M * wl.H * 2
    R = max(8, math.ceil(ROTATE_BYTES / per_copy))
    d, copies = make_copies(wl, R, device)
    if A is None:
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
    timing = "HIP graph of launches over rotated inputs; HIP events on the launch stream"
    result = result_fields(wl, A, ms_per_step, sum(npps) / len(npps), npps, steps, warmup, timing)
    result["config"].update({"rotation_copies": R, "rotation_bytes": R * per_copy})
    if wl.M > 32:
        result["phases"] = prefill_phases(wl, capture, R)
    elif wl.M <= 4:
        result["phases"] = small_phases(capture, R)
    return d, result


def small_phases(capture, R):
    """Phase times of one small-M launch in the steady state (as
    prefill_phases): when the last and the median block published their gate
    keys, then block 0's tail for its first token row."""
    import torch

    import moe_token_routing_amd as mr

    stamps = torch.zeros(8 * 256, dtype=torch.int64, device="cuda:0")
    mr.mr_debug_set_phase_stamps(stamps)
    try:
        g = capture(R)
    finally:
        mr.mr_debug_set_phase_stamps(None)
    g.replay()
    torch.cuda.synchronize()
    st = stamps.view(256, 8).cpu().numpy()
    st = st[st[:, 0] != 0]
    t0 = st[:, 0].min()
    us = lambda v: round(float((v - t0) * 0.01), 3)  # noqa: E731  (100 MHz clock)
    pub = sorted(st[:, 1])
    tail = st[0] if st[0, 2] != 0 else None
    out = {"blocks": int(len(st)), "unit": "us from the first block's start",
           "last_block_start": us(st[:, 0].max()), "keys_published": [us(pub[-1]), us(pub[len(pub) // 2])]}
    if tail is not None:
        out.update({"block0_keys_arrived": us(tail[2]), "sorted": us(tail[3]), "selected": us(tail[4]),
                    "stored": us(tail[5]), "align_done": us(tail[6])})
    return out


def prefill_phases(wl, capture, R):
    """Per-phase times of one prefill launch in the steady state: a graph of
    the same R rotated launches is captured with phase stamps on (every launch
    overwrites them) and replayed once; the stamps of its last launch give,
    from the first block's start, when the last block finished each phase.
    The gate pass is every block's gate items done, partial tiles stored;
    its rate is the launch's flops over that time."""
    import torch

    import moe_token_routing_amd as mr

    stamps = torch.zeros(8 * 256, dtype=torch.int64, device="cuda:0")
    mr.mr_debug_set_phase_stamps(stamps)
    try:
        g = capture(R)
    finally:
        mr.mr_debug_set_phase_stamps(None)
    g.replay()
    torch.cuda.synchronize()
    st = stamps.view(256, 8).cpu().numpy()
    st = st[st[:, 0] != 0]
    t0 = st[:, 0].min()
    tick_us = 0.01  # s_memrealtime counts at 100 MHz

    def col(i):  # blocks that reached point i (a block with no gate item never stamps 1)
        c = st[:, i]
        return c[c != 0]

    def last(i):
        return round(float((col(i).max() - t0) * tick_us), 3)

    def median(i):
        c = sorted(col(i))
        return round(float((c[len(c) // 2] - t0) * tick_us), 3)

    flops = 2.0 * wl.M * (wl.E + int(wl.shared)) * wl.H
    gate_us = last(2)
    return {"blocks": int(len(st)), "unit": "us from the first block's start (last block / median block)",
            "gate_mfma_loop_done": [last(1), median(1)], "gate_done": [last(2), median(2)],
            "topk_start": [last(3), median(3)], "topk_done": [last(4), median(4)],
            "align_start": [last(5), median(5)], "end": [last(6), median(6)],
            "gate_pass": {"us": gate_us, "tflops": round(flops / (gate_us * 1e-6) / 1e12, 2),
                          "frac_of_bf16_peak": round(flops / (gate_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}}


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
    if args.workload == "argmax":
        import moe_token_routing_amd as mr

        mr._binding.lib()
        torch.cuda.set_device(0)
        print(json.dumps(measure_argmax(args.steps, args.warmup, args.cpu_seconds)), flush=True)
        return
    if args.workload == "consumer":
        import moe_token_routing_amd as mr

        mr._binding.lib()
        torch.cuda.set_device(0)
        print(json.dumps(measure_consumer(args.steps, args.warmup)), flush=True)
        return
    if args.workload == "align_ep":
        import moe_token_routing_amd as mr

        mr._binding.lib()
        torch.cuda.set_device(0)
        print(json.dumps(measure_align_ep(args.steps, args.warmup)), flush=True)
        return
    wl = workload(args.workload)
    if args.cpu_only:
        from moe_token_routing_amd import workloads as W

        d = W.workload_inputs(wl)
        base = cpu_baseline(d, wl, args.cpu_seconds if args.cpu_seconds > 0 else 10.0, args.cpu_threads, args.align)
        print(json.dumps({"workload": wl.name, "cpu_baseline": base}), flush=True)
        return
    import moe_token_routing_amd as mr

    mr._binding.lib()
    torch.cuda.set_device(0)
    if args.stream_read:
        print(json.dumps(stream_read()), flush=True)
        return
    if args.method == "memset":
        d, result = measure_memset(wl, 64, max(3, min(args.steps // 64, 15)), args.align)
    else:
        d, result = measure(wl, args.steps, args.warmup, args.align)
    result = {"metric": METRIC, **result}
    if args.secondary_steps > 0 and args.workload == "m4" and args.method == "rotate" and args.align is None:
        _, sec = measure(workload("m2048"), args.secondary_steps, min(args.warmup, 256))
        result["secondary"] = {kk: sec[kk] for kk in ["value", "unit", "ms_per_step", "steps", "config", "roofline",
                                                      "phases"] if kk in sec}
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(d, wl, args.cpu_seconds, args.cpu_threads, args.align)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
