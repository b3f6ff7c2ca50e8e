"""The route + align entry point that allocates nothing (needs a gfx950 GPU).

mr_route_align_noalloc takes no workspace: it uses the library's static
per-GPU scratch array.  Its outputs must equal those of mr_route_align with a
caller workspace bit for bit (same kernels, same summation order), on calls
in a row whose shapes shrink, so that each call runs on whatever the one
before it left in the shared array.  Every case prints its name and shape
before it runs.
"""
import ctypes

import numpy as np
import pytest

import moe_token_routing_amd as mr
from moe_token_routing_amd import workloads
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mr._binding.lib()


def _say(*a):
    print("[case]", *a, flush=True)


def _outputs(M, S, Ep, A):
    import torch

    cap = mr.mr_align_capacity(M, S, Ep, A)
    return {"topk_ids": torch.full((M, S), -3, dtype=torch.int32, device="cuda"),
            "topk_weights": torch.full((M, S), -3.0, dtype=torch.float32, device="cuda"),
            "sorted_token_ids": torch.full((cap,), -3, dtype=torch.int32, device="cuda"),
            "expert_ids": torch.full((cap // A,), -3, dtype=torch.int32, device="cuda"),
            "npp": torch.full((1,), -3, dtype=torch.int32, device="cuda")}


def _noalloc_via_abi(x, w, s, M, H, E, k, A, o):
    """One call straight through the C ABI (ctypes), on the current stream."""
    import torch

    lib = mr._binding.lib()
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    rc = lib.mr_route_align_noalloc(p(x), p(w), p(s), M, H, E, k, 1.0, A, p(o["topk_ids"]), p(o["topk_weights"]),
                                    p(o["sorted_token_ids"]), o["sorted_token_ids"].numel(), p(o["expert_ids"]),
                                    o["expert_ids"].numel(), p(o["npp"]),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == mr.MR_OK, mr.mr_last_error()


def _same(a, b, A):
    import torch

    torch.cuda.synchronize()
    assert torch.equal(a["topk_ids"], b["topk_ids"]), "ids differ"
    assert torch.equal(a["topk_weights"].view(torch.int32), b["topk_weights"].view(torch.int32)), "weights differ"
    n = int(a["npp"].item())
    assert n == int(b["npp"].item()) and n > 0 and n % A == 0, (n, int(b["npp"].item()))
    assert torch.equal(a["sorted_token_ids"][:n], b["sorted_token_ids"][:n]), "sorted_token_ids differ"
    assert torch.equal(a["expert_ids"][: n // A], b["expert_ids"][: n // A]), "expert_ids differ"


# Shapes in the order they run: each call is smaller than the one before it,
# and they alternate between the prefill and the small-M launches.
SEQUENCE = [
    (2048, 512, 4096, 10, True, "normal"),   # prefill launch, tile waits
    (4, 512, 4096, 10, True, "normal"),      # small-M launch, block 0's tail
    (300, 128, 2048, 8, False, "int"),       # prefill launch, one expert tile, no shared expert
    (12, 100, 200, 7, True, "normal"),       # small-M launch with tail blocks, ragged E and H
]


def test_noalloc_matches_route_align_on_shrinking_calls():
    import torch

    for it, (M, E, H, k, shared, dist) in enumerate(SEQUENCE):
        _say("noalloc", it, M, E, H, k, shared)
        d = workloads.make_inputs(M, E, H, shared, dist, seed=500 + it)
        x, w, s = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["ws"])
        S, Ep = k + shared, E + shared
        A = mr.mr_select_alignment(M, k, E)
        ws = mr.new_workspace(M, E, k, shared)
        ref = mr.mr_route_align(x, w, s, k, 1.0, A, workspace=ws, **_outputs(M, S, Ep, A))
        # twice in a row on the shared array: the second call sees the first
        # call's leftovers of the same shape
        for rep in range(2):
            o = _outputs(M, S, Ep, A)
            if rep == 0:
                _noalloc_via_abi(x, w, s, M, H, E, k, A, o)
                got = dict(o, A=A)
            else:
                got = mr.mr_route_align_noalloc(x, w, s, k, 1.0, A, **o)
            _same(got, ref, A)
        torch.cuda.synchronize()


def test_noalloc_in_a_graph():
    """Captured into a graph and replayed: each replay equals the eager call."""
    import torch

    _say("noalloc graph, M=40")
    d = workloads.make_inputs(40, 512, 4096, True, "normal", seed=77)
    x, w, s = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["ws"])
    A = mr.mr_select_alignment(40, 10, 512)
    ref = mr.mr_route_align_noalloc(x, w, s, 10, 1.0, A, **_outputs(40, 11, 513, A))
    torch.cuda.synchronize()
    ref = {kk: (v.clone() if hasattr(v, "clone") else v) for kk, v in ref.items()}
    o = _outputs(40, 11, 513, A)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        mr.mr_route_align_noalloc(x, w, s, 10, 1.0, A, **o)
    for rep in range(3):
        _say("replay", rep)
        for v in o.values():
            v.fill_(-3)
        g.replay()
        _same(dict(o, A=A), ref, A)


def test_noalloc_refuses_oversized_calls():
    _say("noalloc refusal")
    import torch

    x = torch.zeros(16384, 4096, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(512, 4096, dtype=torch.bfloat16, device="cuda")
    o = _outputs(1, 11, 513, 64)
    with pytest.raises(mr.MoeRouteError) as ei:
        mr._binding.lib()
        rc = mr._binding.lib().mr_route_align_noalloc(
            ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.data_ptr()), None, 16384, 4096, 512, 10, 1.0, 64,
            ctypes.c_void_p(o["topk_ids"].data_ptr()), ctypes.c_void_p(o["topk_weights"].data_ptr()),
            ctypes.c_void_p(o["sorted_token_ids"].data_ptr()), 1, ctypes.c_void_p(o["expert_ids"].data_ptr()), 1,
            ctypes.c_void_p(o["npp"].data_ptr()), None)
        mr._binding._check(rc)
    assert ei.value.code == mr.MR_ECAPACITY and "static scratch array" in ei.value.message
