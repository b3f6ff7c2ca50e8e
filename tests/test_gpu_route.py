"""Parity of the HIP route + align path with the CPU oracle (needs a gfx950
GPU).  Every case prints its name, seed and shape before it runs."""
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

    mr._binding.lib()  # loud failure if the library is missing


def _say(*a):
    print("[case]", *a, flush=True)


def _run_and_check(d, k, scale, A=None, exact=False):
    M, E = d["x"].shape[0], d["w"].shape[0]
    has_shared = d["ws"] is not None
    ref = oracle.route(d["x"], d["w"], d["ws"], k, scale)
    g = route_align_gpu(d, k, scale, A)
    A = g["A"]
    lg = logits_gpu(d)
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
    check_align(g["topk_ids"], E + has_shared, A, g["sorted_token_ids"], g["expert_ids"], g["npp"][0])
    return exempt


@pytest.mark.parametrize("M", [4, 16])
def test_selection_one_lane_holds_many(M):
    """Six of the chosen experts (0, 64, ..., 320) sit in lane 0 of the wave
    that selects a row's top-k, so the rounds over each lane's first keys
    run out in that lane and the selection is redone on the full lists."""
    _say("lane-heavy", M)
    d = lane_heavy_inputs(M, 512, 4096, [0, 64, 128, 192, 256, 320], seed=40 + M)
    _run_and_check(d, 10, 1.0, exact=True)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_selection_two_lanes_hold_the_lead(M):
    """Sixteen experts far ahead of the rest sit in lanes 0 and 1 (all eight
    keys of each), so the rounds' short lists run out in both lanes and the
    selection is redone on the full lists."""
    _say("two lanes lead", M)
    lead = [64 * i for i in range(8)] + [64 * i + 1 for i in range(8)]
    d = lane_heavy_inputs(M, 512, 4096, lead, seed=70 + M)
    _run_and_check(d, 10, 1.0, exact=True)


def test_exact_inputs_m8_bit_exact():
    wl = workloads.ROUTER_E512_M8_EXACT
    _say(wl)
    d = workloads.workload_inputs(wl)
    _run_and_check(d, wl.k, wl.scale, exact=True)


@pytest.mark.parametrize("M", [1, 3, 4, 8, 16])
def test_exact_inputs_small_m(M):
    _say("exact", M)
    d = workloads.make_inputs(M, 512, 4096, True, "int", seed=100 + M)
    _run_and_check(d, 10, 1.0, exact=True)


def test_router_m4_full_size():
    wl = workloads.ROUTER_E512_M4
    _say(wl)
    d = workloads.workload_inputs(wl)
    _run_and_check(d, wl.k, wl.scale)


@pytest.mark.parametrize("M", [m for m in workloads.SWEEP_M if m <= 16])
def test_router_sweep_small_m(M):
    wl = workloads.sweep_workload(M)
    _say(wl)
    _run_and_check(workloads.workload_inputs(wl), wl.k, wl.scale)


@pytest.mark.parametrize("E,k,H,shared,M,scale", [
    (16, 4, 64, False, 5, 1.0),
    (64, 1, 128, True, 2, 2.5),
    (128, 8, 2048, False, 16, 1.0),
    (1024, 32, 512, True, 7, 0.5),
    (100, 7, 200, True, 9, 1.0),     # ragged: E and H not multiples of the wave
    (32, 32, 8, False, 3, 1.0),      # k = E: every expert chosen
    (3, 2, 8, True, 12, 1.0),        # shared-chunk layout with one chunk per row, odd E'
    (32, 32, 24, False, 6, 1.0),     # shared-chunk layout, k = E, H not a multiple of 64
    (512, 10, 4096, True, 12, 1.0),  # 12-row gate loads (9 <= M <= 12), full router shape
    (257, 9, 136, True, 11, 1.0),    # 12-row gate loads, ragged E and H
    (512, 10, 4096, True, 13, 1.0),  # 16-row gate loads from M = 13
    (512, 10, 4096, True, 17, 1.0),  # 32-row gate layout (17 <= M <= 32), 5 tail blocks
    (512, 10, 4096, True, 32, 1.0),  # 32-row gate layout, 8 tail blocks
    (3, 2, 8, True, 32, 1.0),        # 8 tail blocks but E' = 4: the grid is raised to cover them
    (100, 7, 200, False, 24, 2.0),   # ragged E and H, no shared expert
    (512, 10, 4096, True, 10, 1.0),  # 10-row loads
    (64, 4, 520, False, 14, 1.0),    # 14-row loads, H not a multiple of 64
    (512, 10, 4096, True, 21, 1.0),  # 24-row loads
    (512, 10, 4096, True, 28, 1.0),  # 28-row loads
    (512, 10, 4096, True, 29, 1.0),  # 32-row loads
    (128, 8, 4096, False, 3, 1.0),   # one gate row per block (E' <= 256) at M <= 4, H > 2048: two chunks a thread
    (191, 23, 3808, False, 4, 1.0),  # the same with a ragged last pass and k > 16
    (255, 6, 2056, True, 1, 1.0),    # E' = 256, one 16-byte chunk past the two-chunk passes
    (14, 1, 256, False, 15, 1.0),    # S = 1 (k = 1, no shared expert): a pair's token row is its index
    (512, 1, 4096, False, 4, 1.0),   # S = 1 in block 0's own tail
])
def test_router_shapes(E, k, H, shared, M, scale):
    _say("shape", E, k, H, shared, M, scale)
    d = workloads.make_inputs(M, E, H, shared, "normal", seed=E + k)
    _run_and_check(d, k, scale)


@pytest.mark.parametrize("A", [16, 64, 128, 256])
def test_router_forced_alignment(A):
    _say("A", A)
    d = workloads.make_inputs(8, 512, 4096, True, "int", seed=7)
    _run_and_check(d, 10, 1.0, A=A, exact=True)


@pytest.mark.parametrize("M,A", [(32, 32), (20, 16), (32, 16)])
def test_router_forced_alignment_17_to_32(M, A):
    # M <= A stays on the small-M launch; A < M goes to the prefill launch
    _say("M", M, "A", A)
    d = workloads.make_inputs(M, 512, 4096, True, "int", seed=M + A)
    _run_and_check(d, 10, 1.0, A=A, exact=True)


@pytest.mark.parametrize("M,E,k,A", [(15, 14, 10, 128), (9, 15, 4, 128), (12, 20, 8, 64)])
def test_fill_slices_only_from_live_row_groups(M, E, k, A):
    """Small E' at 9 <= M <= 20: the grid rounds the gate's row groups up to
    whole XCDs, so some of the first blocks hold no live gate row and are not
    tail blocks either.  Such a block publishes nothing and no block waits
    for it, so it must not take a slice of the sorted_token_ids pre-fill (its
    sentinels could land after block 0's placements).  20 launches on one
    workspace, each checked against the oracle's align."""
    import moe_token_routing_amd as mr

    _say("fill slices", M, E, k, "A", A)
    ws = mr.new_workspace(M, E, k, False)
    for it in range(20):
        d = workloads.make_inputs(M, E, 64, False, "int", seed=100 * M + it)
        ref = oracle.route(d["x"], d["w"], d["ws"], k, 1.0)
        g = route_align_gpu(d, k, 1.0, A, ws=ws)
        assert np.array_equal(g["topk_ids"], ref["ids"]), it
        check_align(g["topk_ids"], E, A, g["sorted_token_ids"], g["expert_ids"], g["npp"][0])


def test_route_only_matches_route_align():
    import moe_token_routing_amd as mr

    d = workloads.workload_inputs(workloads.ROUTER_E512_M4)
    _say("route vs route_align")
    x, w, s = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["ws"])
    ws = mr.new_workspace(4, 512, 10, True)
    ids, wts = mr.mr_route(x, w, s, 10, 1.0, workspace=ws)
    g = mr.mr_route_align(x, w, s, 10, 1.0, workspace=ws)
    assert np.array_equal(ids.cpu().numpy(), g["topk_ids"].cpu().numpy())
    assert np.array_equal(wts.cpu().numpy(), g["topk_weights"].cpu().numpy())


@pytest.mark.parametrize("M,E,H,A", [(17, 512, 4096, 16), (20, 512, 4096, 16), (24, 512, 4096, 16),
                                     (32, 512, 4096, 16), (40, 512, 4096, 16), (64, 512, 4096, 32),
                                     (100, 512, 4096, 16), (128, 128, 2048, 16)])
def test_route_only_and_logits_match_route_align_any_alignment(M, E, H, A):
    """The launch and its token tiling depend on M, E and H only, never on A
    or on whether the align runs: on random inputs (no exact sums), route-only
    ids and weights equal route+align's bit for bit at a forced A below M, and
    the logits hook's fp32 logits reproduce those ids through the oracle's
    rounding and selection."""
    import moe_token_routing_amd as mr

    _say("route vs route_align vs logits", M, E, H, "A", A)
    d = workloads.make_inputs(M, E, H, True, "normal", seed=M * 3 + A)
    x, w, s = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["ws"])
    ws = mr.new_workspace(M, E, 10, True)
    ids, wts = mr.mr_route(x, w, s, 10, 1.0, workspace=ws)
    g = mr.mr_route_align(x, w, s, 10, 1.0, A, workspace=ws)
    assert np.array_equal(ids.cpu().numpy(), g["topk_ids"].cpu().numpy())
    assert np.array_equal(wts.cpu().numpy(), g["topk_weights"].cpu().numpy())
    ref = oracle.route(d["x"], d["w"], d["ws"], 10, 1.0)
    check_backstop(d["x"], d["w"], d["ws"], logits_gpu(d), g["topk_ids"].cpu().numpy(),
                   g["topk_weights"].cpu().numpy(), 10, 1.0, ref)


def test_consecutive_launches_reuse_workspace():
    """The ticket resets itself: back-to-back launches on one workspace, with
    different inputs and sizes, each match the oracle."""
    import moe_token_routing_amd as mr

    ws = mr.new_workspace(16, 512, 10, True)
    for it, (M, seed) in enumerate([(4, 1), (16, 2), (1, 3), (8, 4), (4, 1)]):
        _say("consecutive", it, M, seed)
        d = workloads.make_inputs(M, 512, 4096, True, "int", seed=seed)
        ref = oracle.route(d["x"], d["w"], d["ws"], 10, 1.0)
        g = route_align_gpu(d, 10, 1.0, ws=ws)
        assert np.array_equal(g["topk_ids"], ref["ids"])
        check_align(g["topk_ids"], 513, g["A"], g["sorted_token_ids"], g["expert_ids"], g["npp"][0])
    import torch

    assert int(ws[:256].view(torch.int32).abs().sum().item()) == 0


def test_deterministic_bytes():
    import torch
    import moe_token_routing_amd as mr

    d = workloads.workload_inputs(workloads.ROUTER_E512_M4)
    x, w, s = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["ws"])
    ws = mr.new_workspace(4, 512, 10, True)
    first = None
    for _ in range(50):
        g = mr.mr_route_align(x, w, s, 10, 1.0, workspace=ws)
        npp = int(g["npp"].item())
        cur = [g["topk_ids"].clone(), g["topk_weights"].clone(), g["sorted_token_ids"][:npp].clone(),
               g["expert_ids"][: npp // g["A"]].clone()]
        if first is None:
            first = cur
        else:
            for a, b in zip(first, cur):
                assert torch.equal(a, b)


def test_graph_replay_matches_eager():
    import torch
    import moe_token_routing_amd as mr

    d = workloads.workload_inputs(workloads.ROUTER_E512_M4)
    x, w, s = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["ws"])
    ws = mr.new_workspace(4, 512, 10, True)
    eager = mr.mr_route_align(x, w, s, 10, 1.0, workspace=ws)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in eager.items() if hasattr(v, "clone")}
    stream = torch.cuda.Stream()
    bufs = {k: torch.full_like(v, -5) for k, v in ref.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        mr.mr_route_align(x, w, s, 10, 1.0, workspace=ws, topk_ids=bufs["topk_ids"],
                          topk_weights=bufs["topk_weights"], sorted_token_ids=bufs["sorted_token_ids"],
                          expert_ids=bufs["expert_ids"], npp=bufs["npp"])
    npp = int(ref["npp"].item())
    for rep in range(5):
        for v in bufs.values():
            v.fill_(-5)
        g.replay()
        torch.cuda.synchronize()
        _ = (x.float() * 2).sum().item()  # unrelated eager work between replays
        assert torch.equal(bufs["topk_ids"], ref["topk_ids"]), rep
        assert torch.equal(bufs["topk_weights"], ref["topk_weights"]), rep
        assert int(bufs["npp"].item()) == npp
        assert torch.equal(bufs["sorted_token_ids"][:npp], ref["sorted_token_ids"][:npp])
        assert torch.equal(bufs["expert_ids"][: npp // 64], ref["expert_ids"][: npp // 64])


def test_workspace_reset_recovers_aborted_state():
    import torch
    import moe_token_routing_amd as mr

    d = workloads.make_inputs(4, 512, 4096, True, "int", seed=9)
    ref = oracle.route(d["x"], d["w"], d["ws"], 10, 1.0)
    ws = mr.new_workspace(4, 512, 10, True)
    ws[:64].fill_(7)  # counters left non-zero, as after an aborted launch
    mr.mr_workspace_reset(ws)
    g = route_align_gpu(d, 10, 1.0, ws=ws)
    assert np.array_equal(g["topk_ids"], ref["ids"])
    assert int(ws[:256].view(torch.int32).abs().sum().item()) == 0


def test_empty_batch():
    import torch
    import moe_token_routing_amd as mr

    _say("M=0")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    ws = mr.new_workspace(1, 16, 4, False)
    npp = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    out = mr.mr_route_align(x, w, None, 4, 1.0, 64, workspace=ws, npp=npp)
    assert int(out["npp"].item()) == 0
    ids, wts = mr.mr_route(x, w, None, 4, workspace=ws)
    assert ids.shape == (0, 4)


def test_debug_logits_exact_on_integer_inputs():
    d = workloads.make_inputs(8, 512, 4096, True, "int", seed=11)
    z, s = oracle.gate(d["x"], d["w"], d["ws"])
    lg = logits_gpu(d)
    assert np.array_equal(lg[:, :512].astype(np.float64), z)
    assert np.array_equal(lg[:, 512].astype(np.float64), s)


# ------------------------------------------------------------- align only --

def _align_case(ids, Ep, A):
    import torch
    import moe_token_routing_amd as mr

    M, S = ids.shape
    t = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
    ws = mr.new_workspace(max(M, 1), Ep, S, False)
    srt, eids, npp = mr.mr_align(t, Ep, A, workspace=ws)
    check_align(ids, Ep, A, srt.cpu().numpy(), eids.cpu().numpy(), int(npp.item()))


@pytest.mark.parametrize("M,S,Ep,A,kind,seed", [
    (4, 11, 513, 64, "uniform", 1),
    (128, 8, 128, 64, "uniform", 2),
    (128, 8, 128, 128, "uniform", 3),
    (2048, 8, 128, 128, "zipf", 4),
    (2048, 11, 513, 64, "uniform", 5),
    (1000, 3, 7, 16, "uniform", 6),      # few experts, many repeats per chunk
    (333, 5, 4096, 256, "uniform", 7),   # many experts, ragged chunk tail
    (50, 4, 9, 32, "one_expert", 8),
    (1, 1, 1, 16, "uniform", 9),
    (257, 2, 64, 64, "out_of_range", 10),
    (4096, 9, 257, 64, "zipf", 11),
])
def test_align_only(M, S, Ep, A, kind, seed):
    _say("align", M, S, Ep, A, kind, seed)
    rng = np.random.default_rng(seed)
    if kind == "uniform":
        ids = rng.integers(0, Ep, size=(M, S))
    elif kind == "zipf":
        ids = (rng.zipf(1.3, size=(M, S)) - 1) % Ep
    elif kind == "one_expert":
        ids = np.full((M, S), Ep - 1)
    else:
        ids = rng.integers(-3, Ep + 3, size=(M, S))
    _align_case(ids.astype(np.int32), Ep, A)


def test_align_every_expert_once():
    _say("align every expert once")
    ids = np.random.default_rng(12).permutation(640).astype(np.int32).reshape(64, 10)
    _align_case(ids, 640, 64)


def test_align_repeated_launches():
    import torch
    import moe_token_routing_amd as mr

    rng = np.random.default_rng(13)
    ws = mr.new_workspace(3000, 600, 9, False)
    for it, M in enumerate([3000, 10, 1777, 3000]):
        _say("align repeat", it, M)
        ids = rng.integers(0, 600, size=(M, 9)).astype(np.int32)
        t = torch.from_numpy(ids).cuda()
        srt, eids, npp = mr.mr_align(t, 600, 64, workspace=ws)
        check_align(ids, 600, 64, srt.cpu().numpy(), eids.cpu().numpy(), int(npp.item()))
    assert int(ws[:256].view(torch.int32).abs().sum().item()) == 0
