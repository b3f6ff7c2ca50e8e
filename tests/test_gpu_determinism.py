"""Run-to-run determinism of the prefill route + align launch (needs a gfx950
GPU).

The launch's split-K partial sums are added in a fixed split order and its
grid barriers alternate between two counter sets by the parity of a launch
count, so every launch on the same inputs must produce the same bytes: ids,
weights, npp and the defined part of sorted_token_ids and expert_ids.  A
graph of 20 launches on one workspace, each writing its own set of output
buffers, is replayed 10 times (200 launches, both barrier parities many
times over), and every output set is compared byte for byte with the first.
The test stops at the first mismatch.  Every case prints its name and shape
before it runs.
"""
import pytest

import moe_token_routing_amd as mr
from moe_token_routing_amd import workloads
from gpu_util import to_dev

pytestmark = pytest.mark.gpu

PER_GRAPH, REPLAYS = 20, 10


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mr._binding.lib()


def _outputs(M, S, Ep, A):
    import torch

    cap = mr.mr_align_capacity(M, S, Ep, A)
    return {"topk_ids": torch.full((M, S), -1, dtype=torch.int32, device="cuda"),
            "topk_weights": torch.full((M, S), -1.0, dtype=torch.float32, device="cuda"),
            "sorted_token_ids": torch.full((cap,), -1, dtype=torch.int32, device="cuda"),
            "expert_ids": torch.full((cap // A,), -1, dtype=torch.int32, device="cuda"),
            "npp": torch.full((1,), -1, dtype=torch.int32, device="cuda")}


@pytest.mark.parametrize("wl", [workloads.sweep_workload(2048), workloads.PREFILL_E128_M2048_ZIPF],
                         ids=lambda wl: wl.name)
def test_prefill_launches_are_bytewise_repeatable(wl):
    import torch

    print("[case] determinism", wl.name, flush=True)
    d = workloads.workload_inputs(wl)
    x, w, s = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["ws"])
    A = mr.mr_select_alignment(wl.M, wl.k, wl.E)
    S, Ep = wl.k + int(wl.shared), wl.E + int(wl.shared)
    ws = mr.new_workspace(wl.M, wl.E, wl.k, wl.shared)
    ref = mr.mr_route_align(x, w, s, wl.k, wl.scale, A, workspace=ws, **_outputs(wl.M, S, Ep, A))
    torch.cuda.synchronize()
    n = int(ref["npp"].item())
    assert n > 0 and n % A == 0
    sets = [_outputs(wl.M, S, Ep, A) for _ in range(PER_GRAPH)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        for o in sets:
            mr.mr_route_align(x, w, s, wl.k, wl.scale, A, workspace=ws, **o)
    for rep in range(REPLAYS):
        for o in sets:
            for v in o.values():
                v.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(sets):
            where = f"replay {rep}, launch {i}"
            assert int(o["npp"].item()) == n, where
            assert torch.equal(o["topk_ids"], ref["topk_ids"]), where
            assert torch.equal(o["topk_weights"].view(torch.int32), ref["topk_weights"].view(torch.int32)), where
            assert torch.equal(o["sorted_token_ids"][:n], ref["sorted_token_ids"][:n]), where
            assert torch.equal(o["expert_ids"][: n // A], ref["expert_ids"][: n // A]), where
        print(f"[replay] {rep}: {PER_GRAPH} launches identical", flush=True)
    st = mr.mr_workspace_status(ws)
    torch.cuda.synchronize()
    assert int(st.item()) == mr.MR_STATUS_OK
