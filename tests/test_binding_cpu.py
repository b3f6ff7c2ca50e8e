"""The Python binding refuses mismatched tensors before any pointer reaches
the library (CPU only, no GPU needed).

The library cannot see shapes, dtypes or devices: a gate matrix with the
wrong hidden size, a shared row of the wrong length, an int64 output buffer
or a host tensor would become an out-of-bounds access on the GPU.  Each case
below breaks exactly one condition and must raise ValueError.  The device
predicate is swapped for a plain same-device check, so CPU tensors can stand
in for GPU ones; one test keeps the real predicate and checks that host
tensors are refused outright.
"""
import pytest
import torch

import moe_token_routing_amd as mr
from moe_token_routing_amd import _binding



@pytest.fixture
def same_device(monkeypatch):
    def on(t, name, device):
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
        return t

    monkeypatch.setattr(_binding, "_on", on)
    real = _binding.lib()

    def no_call(*a, **k):  # every case must be refused before the library is called
        raise AssertionError("the library was called")

    class NoLib:
        def __getattr__(self, name):
            if name in ("mr_align_capacity", "mr_select_alignment", "mr_last_error"):
                return getattr(real, name)
            return no_call

    monkeypatch.setattr(_binding, "lib", lambda: NoLib())


def inputs(M=4, H=64, E=16, shared=True):
    x = torch.zeros(M, H, dtype=torch.bfloat16)
    w = torch.zeros(E, H, dtype=torch.bfloat16)
    s = torch.zeros(1, H, dtype=torch.bfloat16) if shared else None
    ws = torch.zeros(4096, dtype=torch.uint8)
    return x, w, s, ws


def refuses(fn, needle):
    with pytest.raises(ValueError) as ei:
        fn()
    assert needle in str(ei.value), str(ei.value)


def test_gate_width_mismatch(same_device):
    x, w, s, ws = inputs()
    w = torch.zeros(16, 32, dtype=torch.bfloat16)
    for fn in (mr.mr_route, mr.mr_route_align):
        refuses(lambda: fn(x, w, s, 4, workspace=ws), "gate_w is [16, 32]")
    refuses(lambda: mr.mr_debug_gate_logits(x, w, s, workspace=ws), "gate_w is [16, 32]")


@pytest.mark.parametrize("bad", ["dtype", "length", "stride"])
def test_shared_row(same_device, bad):
    x, w, s, ws = inputs()
    if bad == "dtype":
        s = torch.zeros(1, 64, dtype=torch.float32)
    elif bad == "length":
        s = torch.zeros(1, 32, dtype=torch.bfloat16)
    else:
        s = torch.zeros(64, 2, dtype=torch.bfloat16)[:, 0]
    for fn in (mr.mr_route, mr.mr_route_align):
        refuses(lambda: fn(x, w, s, 4, workspace=ws), "shared_w must be")
    refuses(lambda: mr.mr_debug_gate_logits(x, w, s, workspace=ws), "shared_w must be")


def test_inputs_on_different_devices(same_device):
    x, w, s, ws = inputs()
    meta_w = torch.empty(16, 64, dtype=torch.bfloat16, device="meta")
    refuses(lambda: mr.mr_route(x, meta_w, s, 4, workspace=ws), "gate_w is on meta")
    meta_s = torch.empty(64, dtype=torch.bfloat16, device="meta")
    refuses(lambda: mr.mr_route_align(x, w, meta_s, 4, workspace=ws), "shared_w is on meta")
    meta_ws = torch.empty(4096, dtype=torch.uint8, device="meta")
    refuses(lambda: mr.mr_route(x, w, s, 4, workspace=meta_ws), "workspace is on meta")


@pytest.mark.parametrize("which,tensor,needle", [
    ("topk_ids", torch.zeros(4, 5, dtype=torch.int64), "topk_ids must be a contiguous torch.int32"),
    ("topk_ids", torch.zeros(4, 4, dtype=torch.int32), "topk_ids has 16 elements, expected 20"),
    ("topk_weights", torch.zeros(4, 5, dtype=torch.float64), "topk_weights must be a contiguous torch.float32"),
    ("topk_weights", torch.zeros(5, 4, dtype=torch.float32).t(), "topk_weights must be a contiguous"),
    ("sorted_token_ids", torch.zeros(4096, dtype=torch.int64), "sorted_token_ids must be"),
    ("expert_ids", torch.zeros(64, dtype=torch.float32), "expert_ids must be"),
    ("npp", torch.zeros(0, dtype=torch.int32), "npp has 0 elements"),
    ("npp", torch.zeros(1, dtype=torch.int64), "npp must be"),
])
def test_route_align_outputs(same_device, which, tensor, needle):
    x, w, s, ws = inputs()
    if which.startswith("topk"):
        refuses(lambda: mr.mr_route(x, w, s, 4, workspace=ws, **{which: tensor}), needle)
    refuses(lambda: mr.mr_route_align(x, w, s, 4, workspace=ws, **{which: tensor}), needle)


def test_debug_logits_buffer(same_device):
    x, w, s, ws = inputs()
    refuses(lambda: mr.mr_debug_gate_logits(x, w, s, workspace=ws, logits=torch.zeros(4, 16)),
            "logits has 64 elements, expected 68")
    refuses(lambda: mr.mr_debug_gate_logits(x, w, s, workspace=ws, logits=torch.zeros(4, 17, dtype=torch.float16)),
            "logits must be")


def test_workspace_not_contiguous(same_device):
    x, w, s, _ = inputs()
    ws = torch.zeros(8192, dtype=torch.uint8)[::2]
    refuses(lambda: mr.mr_route_align(x, w, s, 4, workspace=ws), "workspace must be contiguous")
    refuses(lambda: mr.mr_workspace_reset(ws), "workspace must be contiguous")


def test_align_buffers(same_device):
    _, _, _, ws = inputs()
    ids = torch.zeros(8, 3, dtype=torch.int32)
    refuses(lambda: mr.mr_align(ids, 5, 64, workspace=ws, npp=torch.zeros(1, dtype=torch.float32)), "npp must be")
    emap = torch.zeros(5, dtype=torch.int32, device="meta")
    refuses(lambda: mr.mr_align_local(ids, emap, 2, 64, workspace=ws), "expert_map is on meta")


def test_argmax_and_gemm_buffers(same_device):
    x = torch.zeros(4, 100)
    ws = torch.zeros(4096, dtype=torch.uint8)
    refuses(lambda: mr.mr_argmax_rows_f32(x, workspace=ws, out=torch.zeros(4, dtype=torch.int32)), "out must be")
    refuses(lambda: mr.mr_argmax_rows_f32(x, workspace=ws, n=101), "n=101 is outside")
    xb = torch.zeros(4, 64, dtype=torch.bfloat16)
    w = torch.zeros(3, 64, 64, dtype=torch.bfloat16)
    srt = torch.zeros(256, dtype=torch.int32)
    eids = torch.zeros(4, dtype=torch.int32)
    npp = torch.zeros(1, dtype=torch.int32)
    refuses(lambda: mr.mr_grouped_gemm_bf16(xb, w, 2, srt, eids[:1], npp, 64), "expert_ids has 1 elements")
    refuses(lambda: mr.mr_grouped_gemm_bf16(xb, w, 2, srt, eids, npp, 64, y=torch.zeros(8, 32)), "y has 256")


def test_host_tensors_refused():
    """With the real predicate, tensors that are not on a GPU never reach
    the library."""
    x, w, s, ws = inputs()
    refuses(lambda: mr.mr_route_align(x, w, s, 4, workspace=ws), "(a GPU device)")
    refuses(lambda: mr.mr_align(torch.zeros(4, 5, dtype=torch.int32), 5, 64, workspace=ws), "(a GPU device)")
