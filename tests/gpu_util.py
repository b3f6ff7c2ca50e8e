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
