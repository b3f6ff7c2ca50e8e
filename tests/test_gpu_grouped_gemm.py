"""Parity of the grouped-expert GEMM over the align output
(mr_grouped_gemm_bf16) with the CPU oracle (needs a gfx950 GPU): every
placed pair's row within the fp32-accumulation bound, the rows of pairs that
take no slot untouched, and the output bit-identical for A = 64 and 128.
Every case prints its name and shape first."""
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


def _case(M, S, E, N, H, seed, foreign=0):
    rng = np.random.default_rng(seed)
    x = oracle.round_bf16(rng.standard_normal((M, H)))
    w = oracle.round_bf16(rng.standard_normal((E, N, H)) * 0.05)
    ids = np.stack([rng.choice(E, S, replace=False) for _ in range(M)]).astype(np.int32)
    if foreign:
        ids.reshape(-1)[rng.choice(M * S, foreign, replace=False)] = E + 3  # not an expert here
    return x, w, ids


def _dev_bf16(bits):
    import torch

    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def _run(x, w, ids, A):
    import torch

    import moe_token_routing_amd as mr

    M, S = ids.shape
    E = w.shape[0]
    ws = mr.new_workspace(M, E, S, False)
    srt, eids, npp = mr.mr_align(torch.from_numpy(ids).cuda(), E, A, workspace=ws)
    y = mr.mr_grouped_gemm_bf16(_dev_bf16(x), _dev_bf16(w), S, srt, eids, npp, A)
    torch.cuda.synchronize()
    n = int(npp.item())
    return y.cpu().numpy(), srt[:n].cpu().numpy(), eids[: n // A].cpu().numpy(), n


@pytest.mark.parametrize("M,S,E,N,H,A,foreign", [(3, 2, 5, 64, 64, 64, 0), (100, 9, 33, 128, 256, 64, 5),
                                                 (100, 9, 33, 128, 256, 128, 5), (512, 8, 128, 128, 2048, 64, 0),
                                                 (512, 8, 128, 128, 2048, 128, 0)])
def test_grouped_gemm_matches_oracle(M, S, E, N, H, A, foreign):
    _say("grouped gemm", M, S, E, N, H, "A", A)
    x, w, ids = _case(M, S, E, N, H, seed=M + E + A, foreign=foreign)
    y, srt, eids, npp = _run(x, w, ids, A)
    want = oracle.grouped_gemm(x, w, srt, eids, npp, S, A)
    absx = x & np.uint16(0x7FFF)
    absw = w & np.uint16(0x7FFF)
    bound = oracle.grouped_gemm(absx, absw, srt, eids, npp, S, A) * 2.0 ** -16 + 1e-30
    placed = ~np.isnan(want[:, 0])
    assert np.array_equal(placed, ~np.isnan(y[:, 0])), "rows written differ from the pairs placed below npp"
    err = np.abs(y[placed] - want[placed])
    assert (err <= bound[placed]).all(), float((err / bound[placed]).max())


def test_grouped_gemm_bit_identical_across_alignment():
    M, S, E, N, H = 300, 8, 64, 128, 512
    _say("A invariance", M, S, E, N, H)
    x, w, ids = _case(M, S, E, N, H, seed=21)
    y64 = _run(x, w, ids, 64)[0]
    y128 = _run(x, w, ids, 128)[0]
    assert np.array_equal(y64.view(np.uint32), y128.view(np.uint32))
