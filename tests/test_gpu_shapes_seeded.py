"""Parity over seeded draws of the whole supported shape space (needs a gfx950
GPU): route + align on exactly representable and on random-normal inputs,
one workspace reused over a sequence of token counts, the standalone and the
expert-parallel align on random ids, and the row-wise argmax.

The hand-picked shapes elsewhere aim at known boundaries (tile edges, lane
layouts, row-load variants); these draws are meant to land where nobody
thought to look: ragged E, H and M together, every k, with and without the
shared expert, the tier or a forced alignment.  The inputs are integers in
[-3, 3] times 2^-4, so every gate sum is exact in fp32 whatever the order
of accumulation: ids must equal the oracle's bit for bit (ties, which such
inputs make common, go to the lower id), and the align outputs must equal
the oracle's align of those ids.  Every case prints its draw before it
runs."""
import numpy as np
import pytest

import oracle
from moe_token_routing_amd import workloads
from parity_util import check_align, check_backstop, check_weights
from gpu_util import logits_gpu, route_align_gpu

pytestmark = pytest.mark.gpu

# Oracle work per case (M * E * H multiply-adds in fp64) is kept under this,
# so the whole file's oracle calls take seconds on a few host cores.
_MAX_MACS = 6e8


def _route_draws(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        band = i % 3  # few, middling and many experts in turn
        E = int(rng.integers(1, 17)) if band == 0 else int(rng.integers(17, 300)) if band == 1 \
            else int(rng.integers(300, 1025))
        k = int(rng.integers(1, min(32, E) + 1))
        H = 8 * int(np.clip(np.round(np.exp(rng.uniform(0.0, np.log(512)))), 1, 512))
        M = int(np.round(np.exp(rng.uniform(0.0, np.log(3000)))))
        while M > 1 and M * E * H > _MAX_MACS:
            M //= 2
        shared = bool(rng.random() < 0.5)
        scale = float(rng.choice([0.5, 1.0, 2.5]))
        A = None if rng.random() < 0.6 else int(rng.choice([16, 32, 64, 128, 256]))
        out.append((i, E, k, H, M, shared, scale, A))
    return out


ROUTE_DRAWS = _route_draws(96, 20261202)


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_token_routing_amd as mr

    mr._binding.lib()


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("i,E,k,H,M,shared,scale,A", ROUTE_DRAWS)
def test_route_align_seeded_shape(i, E, k, H, M, shared, scale, A):
    _say("draw", i, "E", E, "k", k, "H", H, "M", M, "shared", shared, "scale", scale, "A", A)
    d = workloads.make_inputs(M, E, H, shared, "int", seed=1000 + i)
    ref = oracle.route(d["x"], d["w"], d["ws"], k, scale)
    g = route_align_gpu(d, k, scale, A)
    if A is not None:
        assert g["A"] == A
    else:
        assert g["A"] == oracle.select_alignment(M, k, E)
    assert np.array_equal(g["topk_ids"], ref["ids"]), "ids differ on exact inputs"
    check_weights(g["topk_weights"], g["topk_ids"], ref["weights"], ref["ids"])
    lg = logits_gpu(d)
    check_backstop(d["x"], d["w"], d["ws"], lg, g["topk_ids"], g["topk_weights"], k, scale, ref)
    check_align(g["topk_ids"], E + shared, g["A"], g["sorted_token_ids"], g["expert_ids"], g["npp"][0])


def _align_draws(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Ep = int(np.round(np.exp(rng.uniform(0.0, np.log(4096)))))
        S = int(rng.integers(1, 34))
        M = int(np.round(np.exp(rng.uniform(0.0, np.log(8192)))))
        A = int(rng.choice([16, 32, 64, 128, 256]))
        kind = str(rng.choice(["uniform", "zipf", "out_of_range"]))
        out.append((i, M, S, Ep, A, kind))
    return out


ALIGN_DRAWS = _align_draws(32, 20261203)


@pytest.mark.parametrize("i,M,S,Ep,A,kind", ALIGN_DRAWS)
def test_align_seeded_shape(i, M, S, Ep, A, kind):
    import torch
    import moe_token_routing_amd as mr

    _say("align draw", i, "M", M, "S", S, "Ep", Ep, "A", A, kind)
    rng = np.random.default_rng(2000 + i)
    if kind == "uniform":
        ids = rng.integers(0, Ep, size=(M, S))
    elif kind == "zipf":
        ids = (rng.zipf(1.3, size=(M, S)) - 1) % Ep
    else:
        ids = rng.integers(-3, Ep + 3, size=(M, S))
    ids = ids.astype(np.int32)
    t = torch.from_numpy(ids).cuda()
    ws = mr.new_workspace(M, Ep, S, False)
    srt, eids, npp = mr.mr_align(t, Ep, A, workspace=ws)
    check_align(ids, Ep, A, srt.cpu().numpy(), eids.cpu().numpy(), int(npp.item()))


NORMAL_DRAWS = _route_draws(32, 20261204)


@pytest.mark.parametrize("i,E,k,H,M,shared,scale,A", NORMAL_DRAWS)
def test_route_align_seeded_normal(i, E, k, H, M, shared, scale, A):
    """Random-normal inputs: the ids and weights must be what the oracle's
    rounding and selection give on the kernel's own fp32 logits, each logit
    within the fp32 accumulation bound, and the align exact."""
    _say("normal draw", i, "E", E, "k", k, "H", H, "M", M, "shared", shared, "scale", scale, "A", A)
    d = workloads.make_inputs(M, E, H, shared, "normal", seed=3000 + i)
    ref = oracle.route(d["x"], d["w"], d["ws"], k, scale)
    g = route_align_gpu(d, k, scale, A)
    lg = logits_gpu(d)
    check_backstop(d["x"], d["w"], d["ws"], lg, g["topk_ids"], g["topk_weights"], k, scale, ref)
    check_align(g["topk_ids"], E + shared, g["A"], g["sorted_token_ids"], g["expert_ids"], g["npp"][0])


def _local_draws(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.integers(1, 1025))
        S = int(rng.integers(1, 34))
        M = int(np.round(np.exp(rng.uniform(0.0, np.log(20000)))))
        A = int(rng.choice([16, 32, 64, 128, 256]))
        ranks = int(rng.choice([1, 2, 4, 8, 16]))
        out.append((i, M, S, E, ranks, int(rng.integers(0, ranks)), A))
    return out


@pytest.mark.parametrize("i,M,S,E,ranks,r,A", _local_draws(24, 20261205))
def test_align_local_seeded_shape(i, M, S, E, ranks, r, A):
    """Expert-parallel align of rank r: experts dealt round-robin, ids two
    past either end of [0, E) skipped."""
    import torch
    import moe_token_routing_amd as mr

    _say("align_local draw", i, "M", M, "S", S, "E", E, "rank", r, "of", ranks, "A", A)
    rng = np.random.default_rng(4000 + i)
    ids = rng.integers(-2, E + 2, size=(M, S)).astype(np.int32)
    emap = np.full(E, -1, np.int32)
    mine = np.arange(r, E, ranks)
    emap[mine] = np.arange(mine.size, dtype=np.int32)
    nl = max(1, int(mine.size))
    ws = mr.new_workspace(M, nl, S, False)
    srt, eids, npp = mr.mr_align_local(torch.from_numpy(ids).cuda(), torch.from_numpy(emap).cuda(), nl, A,
                                       workspace=ws)
    n = int(npp.item())
    want = oracle.align_local(ids, emap, nl, A)
    assert n == want[2], (n, want[2])
    assert np.array_equal(srt[:n].cpu().numpy(), want[0])
    assert np.array_equal(eids[: n // A].cpu().numpy(), want[1])


def _reuse_draws(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        band = i % 4  # tiny, small, middling and many experts in turn
        E = int(rng.integers(2, 17)) if band == 0 else int(rng.integers(17, 64)) if band == 1 \
            else int(rng.integers(64, 300)) if band == 2 else int(rng.integers(300, 1025))
        k = int(rng.integers(1, min(32, E) + 1))
        H = 8 * int(rng.integers(1, 129))
        top = int(rng.integers(9, 161))
        Ms = sorted({top} | {int(rng.integers(1, top + 1)) for _ in range(3)} | {int(rng.integers(1, 9))},
                    reverse=bool(rng.random() < 0.5))
        shared = bool(rng.random() < 0.5)
        A = None if rng.random() < 0.5 else int(rng.choice([16, 32, 64, 128, 256]))
        out.append((i, E, k, H, Ms, shared, A))
    return out


@pytest.mark.parametrize("i,E,k,H,Ms,shared,A", _reuse_draws(32, 20261207))
def test_workspace_reuse_seeded(i, E, k, H, Ms, shared, A):
    """One workspace over a seeded sequence of token counts (the small-M
    launch with and without token tiles, and the prefill launch past its
    range), route + align and route-only in turn, twice over: every call's
    ids equal the oracle's, every align equals the oracle's align of those
    ids, and the status word stays 0.  Exact inputs."""
    import moe_token_routing_amd as mr

    _say("reuse draw", i, "E", E, "k", k, "H", H, "Ms", Ms, "shared", shared, "A", A)
    ws = mr.new_workspace(max(Ms), E, k, shared)
    for j, M in enumerate(Ms + Ms):
        d = workloads.make_inputs(M, E, H, shared, "int", seed=7000 + 10 * i + j)
        ref = oracle.route(d["x"], d["w"], d["ws"], k, 1.0)
        Am = A if A is not None else oracle.select_alignment(M, k, E)
        if j % 2 == 0:
            g = route_align_gpu(d, k, 1.0, Am, ws=ws)
            assert np.array_equal(g["topk_ids"], ref["ids"]), ("ids", j, M)
            check_align(g["topk_ids"], E + shared, Am, g["sorted_token_ids"], g["expert_ids"], g["npp"][0])
        else:
            from gpu_util import to_dev

            ids, _ = mr.mr_route(to_dev(d["x"]), to_dev(d["w"]), to_dev(d["ws"]), k, 1.0, workspace=ws)
            assert np.array_equal(ids.cpu().numpy(), ref["ids"]), ("route ids", j, M)
    assert int(mr.mr_workspace_status(ws).item()) == 0


def _argmax_draws(n, seed):
    rng = np.random.default_rng(seed)
    return [(i, int(rng.integers(1, 65)), int(np.round(np.exp(rng.uniform(0.0, np.log(300000))))),
             str(rng.choice(["normal", "ties", "nan"]))) for i in range(n)]


@pytest.mark.parametrize("i,R,N,kind", _argmax_draws(24, 20261206))
def test_argmax_seeded_shape(i, R, N, kind):
    """Row-wise argmax of [R, N] rows padded to a multiple of 4 values with a
    value larger than any in the rows, which must never be read."""
    import torch
    import moe_token_routing_amd as mr

    _say("argmax draw", i, "R", R, "N", N, kind)
    rng = np.random.default_rng(5000 + i)
    x = rng.standard_normal((R, N)).astype(np.float32)
    if kind == "ties":
        x = np.round(x * 2).astype(np.float32)
    elif kind == "nan":
        x.reshape(-1)[rng.choice(R * N, max(1, R * N // 1000), replace=False)] = np.nan
    ld = N + (-N) % 4
    xp = np.full((R, ld), 7.0e30, np.float32)
    xp[:, :N] = x
    ws = mr.new_argmax_workspace(R, N)
    got = mr.mr_argmax_rows_f32(torch.from_numpy(xp).cuda(), workspace=ws, n=N).cpu().numpy()
    assert np.array_equal(got, oracle.argmax_rows(x))
