"""Parity over seeded draws of the whole supported shape space (needs a gfx950
GPU): route + align on exactly representable inputs, and the standalone
align on random ids.

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


ROUTE_DRAWS = _route_draws(48, 20261202)


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
