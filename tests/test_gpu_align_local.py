"""Parity of the expert-parallel-rank align (mr_align_local) with the CPU
oracle (needs a gfx950 GPU): bit-exact sorted_token_ids[:npp],
expert_ids[:npp/A] and npp.  Every case prints its name and shape first."""
import numpy as np
import pytest

import oracle

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


def _gpu(ids, emap, num_local, A):
    import torch

    import moe_token_routing_amd as mr

    M, S = ids.shape
    ws = mr.new_workspace(max(M, 1), num_local, S, False)
    srt, eids, npp = mr.mr_align_local(torch.from_numpy(ids).cuda(), torch.from_numpy(emap).cuda(), num_local, A,
                                       workspace=ws)
    torch.cuda.synchronize()
    n = int(npp.item())
    return srt[:n].cpu().numpy(), eids[: n // A].cpu().numpy(), n


def _check(ids, emap, num_local, A):
    got = _gpu(ids, emap, num_local, A)
    want = oracle.align_local(ids, emap, num_local, A)
    assert got[2] == want[2], (got[2], want[2])
    assert np.array_equal(got[0], want[0])
    assert np.array_equal(got[1], want[1])


@pytest.mark.parametrize("M,S,E,ranks,A", [(4, 11, 513, 8, 64), (16, 11, 513, 8, 64), (128, 8, 128, 4, 64),
                                           (2048, 8, 128, 8, 128), (2048, 11, 513, 8, 64), (3, 5, 9, 2, 16)])
def test_align_local_ranks(M, S, E, ranks, A):
    # experts dealt round-robin to the ranks (local id e // ranks); the last
    # id (a shared expert when E is odd) is replicated on every rank; a few
    # ids are out of range and must be skipped
    rng = np.random.default_rng(M * 7 + E)
    ids = rng.integers(0, E, size=(M, S)).astype(np.int32)
    ids.reshape(-1)[rng.choice(M * S, max(1, M * S // 50), replace=False)] = -3
    for r in range(ranks):
        _say("align_local", M, S, E, "rank", r, "of", ranks, "A", A)
        emap = np.full(E, -1, np.int32)
        own = np.arange(r, E - 1, ranks)
        emap[own] = np.arange(own.size, dtype=np.int32)
        emap[E - 1] = own.size
        _check(ids, emap, own.size + 1, A)


def test_align_local_identity_matches_align():
    import torch

    import moe_token_routing_amd as mr

    rng = np.random.default_rng(2)
    M, S, E, A = 300, 11, 257, 64
    _say("identity map", M, S, E)
    ids = rng.integers(0, E, size=(M, S)).astype(np.int32)
    got = _gpu(ids, np.arange(E, dtype=np.int32), E, A)
    ws = mr.new_workspace(M, E, S, False)
    srt, eids, npp = mr.mr_align(torch.from_numpy(ids).cuda(), E, A, workspace=ws)
    torch.cuda.synchronize()
    n = int(npp.item())
    assert got[2] == n
    assert np.array_equal(got[0], srt[:n].cpu().numpy()) and np.array_equal(got[1], eids[: n // A].cpu().numpy())


def test_align_local_nothing_local_and_empty():
    _say("nothing local")
    ids = (np.arange(40, dtype=np.int32).reshape(8, 5) % 7)
    got = _gpu(ids, np.full(7, -1, np.int32), 3, 64)
    assert got[2] == 0
    _say("empty")
    got = _gpu(np.zeros((0, 5), np.int32), np.zeros(7, np.int32), 3, 64)
    assert got[2] == 0
