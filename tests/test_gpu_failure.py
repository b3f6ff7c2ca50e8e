"""Failure signalling of the route launches (needs a gfx950 GPU).

The host sets the wait limit to 0, so every bounded wait of a launch gives
up at once without polling: no kernel waits for anything, and every launch
runs to its end.  The status word must then name each kind of wait the
launch has, an align launch must write npp = -1, and after
mr_workspace_reset (with the kernels' own bounds back) the next launch on
the same workspace must match the oracle again with a clear status.  Every
case prints its name and shape before it runs.
"""
import numpy as np
import pytest

import oracle
import moe_token_routing_amd as mr
from moe_token_routing_amd import workloads
from gpu_util import to_dev
from parity_util import check_align

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mr._binding.lib()


@pytest.fixture
def no_waits():
    mr.mr_debug_set_wait_limit(0)
    try:
        yield
    finally:
        mr.mr_debug_set_wait_limit(-1)


def _say(*a):
    print("[case]", *a, flush=True)


def _status(ws):
    import torch

    st = mr.mr_workspace_status(ws)
    torch.cuda.synchronize()
    return int(st.item())


# (M, E, H, k, shared, status bits every such launch sets when no wait polls)
CASES = [
    (4, 512, 4096, 10, True, mr.MR_STATUS_KEY_WAIT),                              # block 0 alone runs the tail
    (12, 512, 4096, 10, True, mr.MR_STATUS_KEY_WAIT | mr.MR_STATUS_ID_WAIT),      # three tail blocks hand off ids
    (128, 128, 2048, 8, False, mr.MR_STATUS_KEY_WAIT | mr.MR_STATUS_ID_WAIT),     # 32 tail blocks, the flat id poll
    (120, 512, 4096, 10, True, mr.MR_STATUS_GRID_WAIT),                           # prefill, one token tile: two grid barriers
    (2048, 512, 4096, 10, True, mr.MR_STATUS_TILE_WAIT | mr.MR_STATUS_GRID_WAIT), # token-tile waits + the align barrier
]


@pytest.mark.parametrize("M,E,H,k,shared,bits", CASES)
def test_given_up_waits_are_reported_and_reset_recovers(M, E, H, k, shared, bits):
    import torch

    _say("failure", M, E, H, k, shared)
    d = workloads.make_inputs(M, E, H, shared, "int", seed=900 + M)
    x, w, s = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["ws"])
    ws = mr.new_workspace(M, E, k, shared)
    assert _status(ws) == mr.MR_STATUS_OK

    mr.mr_debug_set_wait_limit(0)
    try:
        out = mr.mr_route_align(x, w, s, k, 1.0, workspace=ws)
        st = _status(ws)
        npp = int(out["npp"].item())
        # a second launch on the unreset workspace also completes, and the
        # word stays set (sticky)
        mr.mr_route(x, w, s, k, 1.0, workspace=ws)
        st2 = _status(ws)
    finally:
        mr.mr_debug_set_wait_limit(-1)
    print(f"[status] {st:#x} npp={npp}", flush=True)
    assert st & bits == bits, (st, bits)
    assert st & ~15 == 0, st
    assert npp == -1
    assert st2 & bits == bits

    mr.mr_workspace_reset(ws)
    assert _status(ws) == mr.MR_STATUS_OK
    ref = oracle.route(d["x"], d["w"], d["ws"], k, 1.0)
    for rep in range(2):
        _say("after reset", rep)
        out = mr.mr_route_align(x, w, s, k, 1.0, workspace=ws)
        torch.cuda.synchronize()
        ids = out["topk_ids"].cpu().numpy()
        assert np.array_equal(ids, ref["ids"]), "ids differ after the reset"
        check_align(ids, E + shared, out["A"], out["sorted_token_ids"].cpu().numpy(),
                    out["expert_ids"].cpu().numpy(), out["npp"].cpu().numpy()[0])
        assert _status(ws) == mr.MR_STATUS_OK


def test_route_only_reports_too(no_waits):
    """mr_route writes no npp; the status word alone reports the failure."""
    _say("route only, M=300")
    d = workloads.make_inputs(300, 512, 1024, True, "int", seed=5)
    x, w, s = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["ws"])
    ws = mr.new_workspace(300, 512, 10, True)
    mr.mr_route(x, w, s, 10, 1.0, workspace=ws)
    assert _status(ws) & mr.MR_STATUS_GRID_WAIT


def test_status_in_a_graph():
    """The status read is an ordinary stream operation: captured after a
    launch, each replay reads the word as that launch left it."""
    import torch

    _say("status in a graph, M=4")
    d = workloads.make_inputs(4, 512, 4096, True, "int", seed=6)
    x, w, s = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["ws"])
    ws = mr.new_workspace(4, 512, 10, True)
    out = mr.mr_route_align(x, w, s, 10, 1.0, workspace=ws)
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        mr.mr_route_align(x, w, s, 10, 1.0, workspace=ws, topk_ids=out["topk_ids"], topk_weights=out["topk_weights"],
                          sorted_token_ids=out["sorted_token_ids"], expert_ids=out["expert_ids"], npp=out["npp"])
        mr.mr_workspace_status(ws, out=st)
    for rep in range(3):
        st.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert int(st.item()) == mr.MR_STATUS_OK, rep
        assert int(out["npp"].item()) > 0
