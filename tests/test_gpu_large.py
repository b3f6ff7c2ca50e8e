"""Parity of the prefill (split-K MFMA) route + align path with the CPU oracle, at the
prefill workloads' full sizes and on ragged and edge shapes (needs a gfx950
GPU).  Every case prints its name and shape before it runs."""
import numpy as np
import pytest

import oracle
from moe_token_routing_amd import workloads
from parity_util import (check_align, check_backstop, check_exemptions, check_ids_random, check_weights,
                         same_rounding_rows)
from gpu_util import lane_heavy_inputs, logits_gpu, route_align_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_token_routing_amd as mr

    mr._binding.lib()


def _say(*a):
    print("[case]", *a, flush=True)


def _counters_ready(ws):
    """Checks the counter words as a prefill launch leaves them and returns
    the launch count (word 16): every word is zero except that count and the
    grid-barrier counter set the last launch used (top word 0 or 32, lane
    words 64 + 64 r + 32 set and their release words 8 further); the set the
    next launch takes is zero."""
    import torch

    c = ws[:4352].view(torch.int32).cpu().numpy().astype(np.int64)
    count = int(c[16])
    last = (count - 1) & 1
    keep = {16, 32 * last} | {64 + 64 * r + 32 * last + d for r in range(16) for d in (0, 8)}
    others = np.array([i for i in range(c.size) if i not in keep])
    assert not c[others].any(), np.nonzero(c[others])
    return count


def _run(d, k, scale=1.0, A=None, exact=False, backstop=True):
    M, E = d["x"].shape[0], d["w"].shape[0]
    has_shared = d["ws"] is not None
    ref = oracle.route(d["x"], d["w"], d["ws"], k, scale)
    g = route_align_gpu(d, k, scale, A)
    lg = logits_gpu(d) if (backstop or not exact) else None
    if backstop:
        check_backstop(d["x"], d["w"], d["ws"], lg, g["topk_ids"], g["topk_weights"], k, scale, ref)
    if exact:
        assert np.array_equal(g["topk_ids"], ref["ids"]), "ids differ on exact inputs"
        check_weights(g["topk_weights"], g["topk_ids"], ref["weights"], ref["ids"])
        exempt = 0
    else:
        exempt = check_ids_random(g["topk_ids"], ref, k)
        rows = same_rounding_rows(lg, ref, g["topk_ids"], k)
        same_set = [sorted(g["topk_ids"][m].tolist()) == sorted(ref["ids"][m].tolist()) for m in range(M)]
        same = [m for m in rows if same_set[m]]
        check_weights(g["topk_weights"], g["topk_ids"], ref["weights"], ref["ids"], same)
        check_exemptions(M, exempt, M - sum(same_set), M - len(rows))
    check_align(g["topk_ids"], E + has_shared, g["A"], g["sorted_token_ids"], g["expert_ids"], g["npp"][0])
    return exempt, g


def test_prefill_e128_m128():
    wl = workloads.PREFILL_E128_M128
    _say(wl)
    d = workloads.workload_inputs(wl)
    _run(d, wl.k)                # tier A = 64
    _run(d, wl.k, A=128)


def test_prefill_e128_m2048_zipf_tier128():
    wl = workloads.PREFILL_E128_M2048_ZIPF
    _say(wl)
    d = workloads.workload_inputs(wl)
    exempt, g = _run(d, wl.k)
    assert g["A"] == 128
    print("exempt rows", exempt)


@pytest.mark.parametrize("M", [m for m in workloads.SWEEP_M if m > 16])
def test_router_sweep_large_m(M):
    wl = workloads.sweep_workload(M)
    _say(wl)
    exempt, g = _run(workloads.workload_inputs(wl), wl.k)
    assert g["A"] == 64


@pytest.mark.parametrize("M", [17, 64, 200])
def test_exact_inputs_large_m(M):
    _say("exact", M)
    d = workloads.make_inputs(M, 512, 4096, True, "int", seed=300 + M)
    _run(d, 10, exact=True)


@pytest.mark.parametrize("E,k,H,shared,M,scale", [
    (1024, 32, 512, True, 100, 0.5),   # largest E and k
    (100, 7, 200, True, 50, 1.0),      # ragged E, H % 32 != 0
    (16, 16, 64, False, 33, 1.0),      # k = E
    (130, 3, 96, True, 257, 2.0),      # two expert tiles, second nearly empty
    (512, 10, 8, True, 70, 1.0),       # H smaller than one MFMA step
    (256, 8, 1024, False, 1000, 1.0),
    (128, 31, 256, True, 300, 1.0),    # E <= 128, S = 32: two tokens per wave side by side, shared slot in lane 31
    (128, 32, 256, True, 300, 1.0),    # E <= 128 but S = 33: the full-wave selection
    (64, 1, 512, False, 300, 1.0),     # S = 1
    (513, 1, 1024, False, 40, 1.0),    # S = 1, E > 512
])
def test_large_shapes(E, k, H, shared, M, scale):
    _say("shape", E, k, H, shared, M, scale)
    d = workloads.make_inputs(M, E, H, shared, "normal", seed=E * 7 + k)
    _run(d, k, scale)


@pytest.mark.parametrize("M", [300, 1100])
def test_selection_e128_lanes_full(M):
    """E = 128: a token's keys fill 32 lanes of 4, and its eight chosen
    experts (0..7) fill lanes 0 and 1 of its half-wave completely, so every
    key of those lanes is taken before any other lane's."""
    _say("e128 lanes full", M)
    d = lane_heavy_inputs(M, 128, 512, list(range(8)), seed=80 + M)
    _run(d, 8, exact=True)


@pytest.mark.parametrize("M,pairs", [(64, False), (1100, True)])
def test_selection_one_lane_holds_many_large(M, pairs):
    """Eight chosen experts (2l, 2l + 1 + 128 j for l = 0) share lane 0 of
    the top-k wave: the rounds over each lane's first keys run out and the
    full rounds take over.  At M = 1100 a wave selects two tokens at once,
    and only the first of each pair has the crowded lane (the second favours
    ten experts in ten different lanes)."""
    _say("lane-heavy", M, pairs)
    fav = [0, 1, 128, 129, 256, 257, 384, 385]
    alt = [10, 30, 50, 70, 90, 110, 150, 170, 190, 210] if pairs else None
    d = lane_heavy_inputs(M, 512, 512, fav, seed=60 + M, alt=alt)
    _run(d, 10, exact=True)


def test_partial_rows_not_line_multiples_two_inputs():
    """Tile waits with many K splits and E % 32 != 0 (E = 202, k = 8,
    M = 1100: 9 token tiles, 13 splits of 5 stages): a partial row's stride
    is padded to whole 128-byte lines, so no line holds the end of one token
    tile's row and the start of the next tile's, which a group reading one
    tile could otherwise pull into its L2 before the other tile's items have
    written it.  Two different inputs run on one workspace, twice each, and
    every run must match the oracle bit-exactly."""
    import moe_token_routing_amd as mr

    M, E, k, H = 1100, 202, 8, 4096
    ws = mr.new_workspace(M, E, k, True)
    for rep in range(2):
        for seed in (71, 72):
            _say("stride", rep, seed, M, E, k, H)
            d = workloads.make_inputs(M, E, H, True, "int", seed=seed)
            ref = oracle.route(d["x"], d["w"], d["ws"], k, 1.0)
            g = route_align_gpu(d, k, 1.0, ws=ws)
            assert np.array_equal(g["topk_ids"], ref["ids"]), "ids differ on exact inputs"
            check_weights(g["topk_weights"], g["topk_ids"], ref["weights"], ref["ids"])
            check_align(g["topk_ids"], E + 1, g["A"], g["sorted_token_ids"], g["expert_ids"], g["npp"][0])


def test_exact_large_alignment_variants():
    d = workloads.make_inputs(96, 512, 4096, True, "int", seed=5)
    for A in [16, 32, 256]:
        _say("A", A)
        _run(d, 10, A=A, exact=True, backstop=False)


def test_grid_larger_than_gpu():
    """More gate items than blocks of the persistent launch (157 token tiles x
    4 expert tiles): every block computes several items."""
    _say("M=20000 E=512")
    d = workloads.make_inputs(20000, 512, 256, True, "normal", seed=21)
    _run(d, 10)


@pytest.mark.parametrize("M,E,H,k,shared", [
    (32768, 128, 64, 8, False),    # 256 token tiles: the most that tile waits take, one group per block
    (33000, 128, 128, 8, True),    # 258 tiles: grid barrier instead of tile waits; two blocks own 2 groups
    (40000, 512, 256, 10, True),   # 313 groups of 128 tokens on 256 blocks
    (100000, 16, 64, 4, False),    # 782 groups: most blocks own 3 or 4
])
def test_more_token_groups_than_blocks(M, E, H, k, shared):
    """Past 256 groups of 128 tokens a block owns several groups: it selects
    them one after another, keeps only the last group's ids in LDS and
    reloads each group's ids for the align.  Exact inputs: ids bit-exact."""
    _say("groups", M, E, H, k, shared)
    d = workloads.make_inputs(M, E, H, shared, "int", seed=M + E)
    _run(d, k, exact=True)


def test_large_consecutive_and_graph():
    import torch
    import moe_token_routing_amd as mr

    ws = mr.new_workspace(2048, 512, 10, True)
    # M = 40 and 17 run the small-M launch on the same workspace between
    # prefill launches (M = 100 and 120 are one-tile prefill launches)
    for it, (M, seed) in enumerate([(512, 1), (2048, 2), (40, 3), (17, 4), (100, 5), (120, 6), (512, 1)]):
        _say("consecutive", it, M)
        d = workloads.make_inputs(M, 512, 4096, True, "int", seed=seed)
        ref = oracle.route(d["x"], d["w"], d["ws"], 10, 1.0)
        g = route_align_gpu(d, 10, 1.0, ws=ws)
        assert np.array_equal(g["topk_ids"], ref["ids"])
        check_align(g["topk_ids"], 513, g["A"], g["sorted_token_ids"], g["expert_ids"], g["npp"][0])
    assert _counters_ready(ws) == 5  # five prefill launches

    d = workloads.make_inputs(512, 512, 4096, True, "normal", seed=8)
    x, w, s = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["ws"])
    eager = mr.mr_route_align(x, w, s, 10, 1.0, workspace=ws)
    torch.cuda.synchronize()
    ref = {kk: v.clone() for kk, v in eager.items() if hasattr(v, "clone")}
    bufs = {kk: torch.full_like(v, -5) for kk, v in ref.items()}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        mr.mr_route_align(x, w, s, 10, 1.0, workspace=ws, topk_ids=bufs["topk_ids"],
                          topk_weights=bufs["topk_weights"], sorted_token_ids=bufs["sorted_token_ids"],
                          expert_ids=bufs["expert_ids"], npp=bufs["npp"])
    npp = int(ref["npp"].item())
    for rep in range(4):
        _say("graph replay", rep)
        for v in bufs.values():
            v.fill_(-5)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs["topk_ids"], ref["topk_ids"])
        assert torch.equal(bufs["topk_weights"], ref["topk_weights"])
        assert int(bufs["npp"].item()) == npp
        assert torch.equal(bufs["sorted_token_ids"][:npp], ref["sorted_token_ids"][:npp])
        assert torch.equal(bufs["expert_ids"][: npp // 64], ref["expert_ids"][: npp // 64])


def test_large_route_only_matches_route_align():
    import moe_token_routing_amd as mr

    d = workloads.make_inputs(300, 512, 4096, True, "normal", seed=9)
    x, w, s = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["ws"])
    ws = mr.new_workspace(300, 512, 10, True)
    ids, wts = mr.mr_route(x, w, s, 10, 1.0, workspace=ws)
    g = mr.mr_route_align(x, w, s, 10, 1.0, workspace=ws)
    assert np.array_equal(ids.cpu().numpy(), g["topk_ids"].cpu().numpy())
    assert np.array_equal(wts.cpu().numpy(), g["topk_weights"].cpu().numpy())


def test_large_debug_logits_exact():
    d = workloads.make_inputs(100, 512, 4096, True, "int", seed=12)
    z, s = oracle.gate(d["x"], d["w"], d["ws"])
    lg = logits_gpu(d)
    assert np.array_equal(lg[:, :512].astype(np.float64), z)
    assert np.array_equal(lg[:, 512].astype(np.float64), s)


_FIRST_CALL_IN_CAPTURE = r"""
import sys, torch
sys.path.insert(0, {root!r})
import moe_token_routing_amd as mr
from moe_token_routing_amd import workloads
from gpu_util import to_dev
if {init}:
    mr.mr_init()
d = workloads.make_inputs(512, 512, 4096, True, "int", seed=31)
x, w, s = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["ws"])
ws = mr.new_workspace(512, 512, 10, True)
A = mr.mr_select_alignment(512, 10, 512)
ids = torch.empty(512, 11, dtype=torch.int32, device="cuda")
wts = torch.empty(512, 11, dtype=torch.float32, device="cuda")
cap = mr.mr_align_capacity(512, 11, 513, A)
srt = torch.empty(cap, dtype=torch.int32, device="cuda")
eids = torch.empty(cap // A, dtype=torch.int32, device="cuda")
npp = torch.empty(1, dtype=torch.int32, device="cuda")
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g, stream=torch.cuda.Stream()):
    mr.mr_route_align(x, w, s, 10, 1.0, A, workspace=ws, topk_ids=ids, topk_weights=wts,
                      sorted_token_ids=srt, expert_ids=eids, npp=npp)
ref = mr.mr_route_align(x, w, s, 10, 1.0, A, workspace=ws)
torch.cuda.synchronize()
n = int(ref["npp"].item())
for rep in range(3):
    ids.fill_(-1); npp.fill_(-1)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(ids, ref["topk_ids"]) and int(npp.item()) == n, rep
    assert torch.equal(srt[:n], ref["sorted_token_ids"][:n])
print("first call in capture ok", {init})
"""


@pytest.mark.parametrize("init", [True, False])
def test_first_prefill_call_inside_graph_capture(init):
    """A fresh process whose very first prefill call is made inside graph
    capture (its one-time set-up queries then run during capture), after
    mr_init and without it; the replays must equal an eager launch."""
    import os
    import subprocess
    import sys

    _say("first call in capture, init", init)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = _FIRST_CALL_IN_CAPTURE.format(root=root, init=init)
    env = dict(os.environ, PYTHONPATH=os.path.join(root, "tests") + os.pathsep + root)
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=240, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
