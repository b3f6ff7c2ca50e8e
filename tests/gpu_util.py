"""Helpers for the GPU tests: upload the seeded bf16 inputs, run the HIP
path through the C ABI, bring results back."""
from __future__ import annotations

import numpy as np


def to_dev(bits):
    import torch

    if bits is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda")


def route_align_gpu(d, k, scale=1.0, A=None, ws=None, M_max=None):
    import moe_token_routing_amd as mr

    x, w, s = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["ws"])
    M, E = d["x"].shape[0], d["w"].shape[0]
    if ws is None:
        ws = mr.new_workspace(M_max or M, E, k, s is not None)
    out = mr.mr_route_align(x, w, s, k, scale, A, workspace=ws)
    return {key: (v.cpu().numpy() if hasattr(v, "cpu") else v) for key, v in out.items()}


def logits_gpu(d, ws=None):
    import moe_token_routing_amd as mr

    x, w, s = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["ws"])
    M, E = d["x"].shape[0], d["w"].shape[0]
    if ws is None:
        ws = mr.new_workspace(M, E, 1, s is not None)
    return mr.mr_debug_gate_logits(x, w, s, workspace=ws).cpu().numpy()


def lane_heavy_inputs(M, E, H, favored, seed, alt=None):
    """Exactly representable inputs (integers in [-3, 3] times 2^-4) whose
    largest routed logits sit on chosen experts: x[m, 0] = 1 and
    w[e, 0] = 16 for e in `favored` (0 for the other experts), so those
    experts lead every row by far.  With `alt`, tokens m with (m // 4) odd
    use column 1 and the experts in `alt` instead.  The selection rounds see
    the favored experts together when they share a lane of the wave that
    holds a token's keys."""
    from moe_token_routing_amd import workloads

    rng = np.random.default_rng(seed)
    x = rng.integers(-3, 4, size=(M, H)).astype(np.float64) * 2.0 ** -4
    w = rng.integers(-3, 4, size=(E, H)).astype(np.float64) * 2.0 ** -4
    ws = rng.integers(-3, 4, size=H).astype(np.float64) * 2.0 ** -4
    x[:, :2] = 0.0
    w[:, :2] = 0.0
    ws[:2] = 0.0
    odd = (np.arange(M) // 4) % 2 == 1 if alt is not None else np.zeros(M, dtype=bool)
    x[~odd, 0] = 1.0
    x[odd, 1] = 1.0
    w[list(favored), 0] = 16.0
    if alt is not None:
        w[list(alt), 1] = 16.0
    return {"x": workloads.to_bf16_bits(x), "w": workloads.to_bf16_bits(w), "ws": workloads.to_bf16_bits(ws)}
