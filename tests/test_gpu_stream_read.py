"""The streaming-read yardstick kernel reads every word it is given: the XOR
of its per-block words matches numpy's XOR of the data for full buffers, a
prefix, and sizes that leave a ragged grid-stride tail (needs a gfx950 GPU)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_token_routing_amd as mr

    mr._binding.lib()


@pytest.mark.parametrize("nwords,prefix", [(4, None), (4 * 1000 + 4, None), (1 << 20, None),
                                           (1 << 20, 4 * 12345), ((1 << 24) + 4 * 77, None)])
def test_stream_read_xor(nwords, prefix):
    import torch

    import moe_token_routing_amd as mr

    print("[case] stream_read", nwords, prefix, flush=True)
    rng = np.random.default_rng(nwords)
    host = rng.integers(0, 1 << 32, size=nwords, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    out = torch.zeros(mr.MR_STREAM_READ_OUT_WORDS, dtype=torch.int32, device="cuda")
    nbytes = None if prefix is None else prefix * 4
    mr.mr_debug_stream_read(src, out, nbytes)
    torch.cuda.synchronize()
    words = host if prefix is None else host[:prefix]
    want = np.bitwise_xor.reduce(words)
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == want
