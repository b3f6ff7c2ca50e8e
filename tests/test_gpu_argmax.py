"""Parity of the HIP row-wise argmax (mr_argmax_rows_f32) with the CPU oracle
(needs a gfx950 GPU).  Integer results: every index must match exactly.
Every case prints its name and shape before it runs."""
import json
import os

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

CHUNK = 4096  # values per block of the kernel


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_token_routing_amd as mr

    mr._binding.lib()  # loud failure if the library is missing


def _say(*a):
    print("[case]", *a, flush=True)


def _gpu_argmax(x, ws=None):
    """x: float32 numpy [R, N]; the device copy has rows padded to a multiple
    of 4 values (the padding holds a NaN that must never be read)."""
    import torch

    import moe_token_routing_amd as mr

    R, N = x.shape
    ld = N + (-N) % 4
    dev = torch.full((R, ld), float("nan"), dtype=torch.float32, device="cuda")
    dev[:, :N] = torch.from_numpy(x).cuda()
    if ws is None:
        ws = mr.new_argmax_workspace(R, N)
    out = mr.mr_argmax_rows_f32(dev[:, :N], workspace=ws) if R != 1 else mr.mr_argmax_rows_f32(dev, workspace=ws, n=N)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ws


def _adversarial(R, N, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((R, N)).astype(np.float32)
    pool = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1.5, -1.5, 4.0], dtype=np.float32)
    for r in range(R):
        kind = r % 7
        if kind == 1:
            x[r, rng.choice(N, min(N, 3), replace=False)] = np.nan
        elif kind == 2:
            x[r, rng.choice(N, min(N, 50), replace=False)] = 9.0
        elif kind == 3:
            x[r] = rng.choice(np.array([0.0, -0.0, -np.inf], dtype=np.float32), N)
        elif kind == 4:
            x[r] = rng.choice(pool, N)
        elif kind == 5:
            x[r] = rng.integers(-3, 4, N).astype(np.float32)
        elif kind == 6:
            x[r] = -np.inf
    return x


def test_argmax_hand_cases(golden_dir):
    with open(os.path.join(golden_dir, "argmax_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        row = np.array([float(v) for v in c["row"]], dtype=np.float32)[None, :]
        _say("hand", c["row"])
        got, _ = _gpu_argmax(row)
        assert got[0] == c["want"], (c, got)


@pytest.mark.parametrize("R,N", [(1, 1), (3, 3), (5, 4), (7, 5), (24, 3001), (4, CHUNK - 1), (4, CHUNK),
                                 (4, CHUNK + 1), (6, 2 * CHUNK + 2), (2, 5 * CHUNK + 3), (1000, 100), (300, 1)])
def test_argmax_adversarial(R, N):
    _say("adversarial", R, N)
    x = _adversarial(R, N, seed=R * 100003 + N)
    got, _ = _gpu_argmax(x)
    assert np.array_equal(got, oracle.argmax_rows(x))


def test_argmax_chunk_boundaries():
    # the winner or a tie sits on either side of every chunk boundary, and
    # NaNs appear only in later chunks
    R, N = 12, 6 * CHUNK + 7
    _say("chunk boundaries", R, N)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((R, N)).astype(np.float32)
    for r in range(R):
        b = CHUNK * (1 + r % 5)
        if r % 4 == 0:
            x[r, b - 1] = x[r, b] = 50.0  # tie across a boundary: the lower index
        elif r % 4 == 1:
            x[r, b] = x[r, N - 1] = 60.0
        elif r % 4 == 2:
            x[r, b + 3] = np.nan
            x[r, N - 2] = np.nan
            x[r, 0] = np.inf
        else:
            x[r, N - 1] = np.nan  # the last value, in the 1..3-value tail
    got, _ = _gpu_argmax(x)
    want = oracle.argmax_rows(x)
    assert np.array_equal(got, want)


def test_argmax_full_size_and_relaunch():
    # the sampling shape, three launches on one workspace (each must leave
    # the row tickets clean for the next), new inputs each time
    R, N = 16, 248320
    ws = None
    for seed in range(3):
        _say("full size", R, N, "seed", seed)
        x = _adversarial(R, N, seed=seed)
        got, ws = _gpu_argmax(x, ws)
        assert np.array_equal(got, oracle.argmax_rows(x))
    import torch

    tickets = ws[: 256 * R].view(torch.int32)  # the block keys may stay; the ticket slots must be zero
    assert int(tickets.abs().sum().item()) == 0


def test_argmax_graph_replay():
    import torch

    import moe_token_routing_amd as mr

    R, N = 16, 248320
    _say("graph replay", R, N)
    xs = [_adversarial(R, N, seed=10 + i) for i in range(3)]
    dev = torch.from_numpy(xs[0]).cuda()
    ws = mr.new_argmax_workspace(R, N)
    out = torch.empty(R, dtype=torch.int64, device="cuda")
    mr.mr_argmax_rows_f32(dev, workspace=ws, out=out)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        mr.mr_argmax_rows_f32(dev, workspace=ws, out=out)
    for i, x in enumerate(xs):
        dev.copy_(torch.from_numpy(x))
        out.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), oracle.argmax_rows(x)), f"replay {i}"


def test_argmax_empty_rows():
    import torch

    import moe_token_routing_amd as mr

    _say("R = 0")
    x = torch.empty((0, 64), dtype=torch.float32, device="cuda")
    out = mr.mr_argmax_rows_f32(x, workspace=mr.new_argmax_workspace(0, 64))
    torch.cuda.synchronize()
    assert out.numel() == 0
