"""ctypes binding of libmoeroute.so (include/moeroute.h): argument marshalling
only.  Torch tensors provide device memory and streams; every step of the
route and align runs in the library's HIP kernels.  There is no fallback: if
the library is missing or refuses a call, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libmoeroute.so")
_lib = None

MR_OK = 0
MR_EINVAL = -1
MR_EUNSUPPORTED = -2
MR_ECAPACITY = -3
MR_ELAUNCH = -4
MR_STREAM_READ_OUT_WORDS = 4096
MR_STATUS_OK = 0
MR_STATUS_KEY_WAIT = 1
MR_STATUS_ID_WAIT = 2
MR_STATUS_GRID_WAIT = 4
MR_STATUS_TILE_WAIT = 8

# Every symbol include/moeroute.h declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F32 = ctypes.c_float
SIGNATURES = {
    "mr_abi_version": (ctypes.c_int, []),
    "mr_init": (ctypes.c_int, []),
    "mr_last_error": (ctypes.c_char_p, []),
    "mr_select_alignment": (_I32, [_I32, _I32, _I32]),
    "mr_align_capacity": (_I64, [_I32, _I32, _I32, _I32]),
    "mr_expert_ids_capacity": (_I64, [_I32, _I32, _I32, _I32]),
    "mr_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "mr_workspace_reset": (ctypes.c_int, [_P, _SZ, _P]),
    "mr_workspace_status": (ctypes.c_int, [_P, _SZ, _P, _P]),
    "mr_debug_set_wait_limit": (ctypes.c_int, [_I32]),
    "mr_debug_set_phase_stamps": (ctypes.c_int, [_P, _SZ]),
    "mr_route": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, _F32, _P, _P, _P, _SZ, _P]),
    "mr_align": (ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _P, _I64, _P, _I64, _P, _P, _SZ, _P]),
    "mr_align_local": (ctypes.c_int, [_P, _I32, _I32, _I32, _P, _I32, _I32, _P, _I64, _P, _I64, _P, _P, _SZ,
                                      _P]),
    "mr_route_align": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, _F32, _I32, _P, _P, _P, _I64,
                                      _P, _I64, _P, _P, _SZ, _P]),
    "mr_route_align_noalloc": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, _F32, _I32, _P, _P, _P, _I64,
                                              _P, _I64, _P, _P]),
    "mr_debug_gate_logits": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _P, _P, _SZ, _P]),
    "mr_debug_stream_read": (ctypes.c_int, [_P, _SZ, _P, _P]),
    "mr_argmax_workspace_bytes": (_SZ, [_I32, _I64]),
    "mr_grouped_gemm_bf16": (ctypes.c_int, [_P, _I32, _I32, _P, _I32, _I32, _I32, _P, _I64, _P, _P, _I32, _P, _P]),
    "mr_argmax_rows_f32": (ctypes.c_int, [_P, _I32, _I64, _I64, _P, _P, _SZ, _P]),
}


class MoeRouteError(RuntimeError):
    """A refused or failed library call (code is the MR_E* value)."""

    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code
        self.message = message


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise MoeRouteError(MR_ELAUNCH, f"{_LIB_PATH} is missing: build it with "
                                "`python -m moe_token_routing_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != MR_OK:
        raise MoeRouteError(rc, lib().mr_last_error().decode())


def _stream(stream, device):
    import torch

    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _bf16_2d(t, name):
    import torch

    if t.dtype != torch.bfloat16 or t.dim() != 2 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 2-D bfloat16 tensor")
    return t


def _on(t, name, device):
    """t must be a tensor on `device` (a GPU): the library dereferences every
    pointer on that device, so a host tensor or another GPU's memory would be
    read or written out of bounds instead of refused."""
    if t.device != device or device.type != "cuda":
        raise ValueError(f"{name} is on {t.device}, expected {device} (a GPU device)")
    return t


def _out(t, name, dtype, device, numel=None, min_numel=None):
    """A caller-supplied buffer: dtype, contiguity, device and size."""
    if t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor")
    _on(t, name, device)
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected at least {min_numel}")
    return t


def _ws_bytes(workspace, device):
    """Byte size of a workspace tensor (contiguous, on `device`)."""
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _on(workspace, "workspace", device)
    return workspace.numel() * workspace.element_size()


def _gate_inputs(x, gate_w, shared_w):
    """Checks the router inputs; returns (M, H, E, device)."""
    import torch

    _bf16_2d(x, "x")
    _bf16_2d(gate_w, "gate_w")
    M, H = x.shape
    E, H2 = gate_w.shape
    if H2 != H:
        raise ValueError(f"gate_w is [{E}, {H2}], expected [E, {H}] (x is [{M}, {H}])")
    dev = x.device
    _on(x, "x", dev)
    _on(gate_w, "gate_w", dev)
    if shared_w is not None:
        if shared_w.dtype != torch.bfloat16 or not shared_w.is_contiguous() or shared_w.numel() != H:
            raise ValueError(f"shared_w must be a contiguous bfloat16 tensor of {H} elements")
        _on(shared_w, "shared_w", dev)
    return M, H, E, dev


# --------------------------------------------------------------- host-only --

def mr_abi_version() -> int:
    return int(lib().mr_abi_version())


def mr_init(device=None) -> None:
    """Per-device set-up (see include/moeroute.h) on `device` (default: the
    current one)."""
    import torch

    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        _check(lib().mr_init())


def mr_last_error() -> str:
    return lib().mr_last_error().decode()


def mr_select_alignment(M: int, k: int, E: int) -> int:
    return int(lib().mr_select_alignment(M, k, E))


def mr_align_capacity(M: int, S: int, num_experts: int, A: int) -> int:
    return int(lib().mr_align_capacity(M, S, num_experts, A))


def mr_expert_ids_capacity(M: int, S: int, num_experts: int, A: int) -> int:
    return int(lib().mr_expert_ids_capacity(M, S, num_experts, A))


def mr_workspace_bytes(M_max: int, E: int, k: int, has_shared: bool) -> int:
    return int(lib().mr_workspace_bytes(M_max, E, k, int(bool(has_shared))))


# ----------------------------------------------------------------- device --

def new_workspace(M_max: int, E: int, k: int, has_shared: bool, device="cuda"):
    """A zeroed workspace tensor (uint8) big enough for M <= M_max."""
    import torch

    nbytes = mr_workspace_bytes(M_max, E, k, has_shared)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def mr_workspace_reset(workspace, stream=None) -> None:
    nbytes = _ws_bytes(workspace, workspace.device)
    _check(lib().mr_workspace_reset(_ptr(workspace), nbytes, _stream(stream, workspace.device)))


def mr_workspace_status(workspace, out=None, stream=None):
    """The workspace's sticky status word (MR_STATUS_* bits of the bounded
    waits that gave up since the last reset), copied on the stream into a
    device int32 tensor [1] (returned; `out` if given)."""
    import torch

    dev = workspace.device
    nbytes = _ws_bytes(workspace, dev)
    if out is None:
        out = torch.empty(1, dtype=torch.int32, device=dev)
    _out(out, "out", torch.int32, dev, min_numel=1)
    _check(lib().mr_workspace_status(_ptr(workspace), nbytes, _ptr(out), _stream(stream, dev)))
    return out


def mr_debug_set_wait_limit(polls: int) -> None:
    """Test hook: polls every bounded wait of later launches makes before
    giving up (0: at once; negative: the kernels' own bounds)."""
    _check(lib().mr_debug_set_wait_limit(int(polls)))


def mr_debug_set_phase_stamps(stamps=None) -> None:
    """Measurement hook: later prefill launches record per-block phase
    times (100 MHz clock) into `stamps`, an int64 device tensor of at least
    8 * 256 elements; None turns it off."""
    import torch

    if stamps is None:
        _check(lib().mr_debug_set_phase_stamps(None, 0))
        return
    _out(stamps, "stamps", torch.int64, stamps.device)
    _on(stamps, "stamps", stamps.device)
    _check(lib().mr_debug_set_phase_stamps(_ptr(stamps), stamps.numel()))


def mr_route(x, gate_w, shared_w, k: int, scale: float = 1.0, *, workspace,
             topk_ids=None, topk_weights=None, stream=None):
    """Returns (topk_ids [M, S] int32, topk_weights [M, S] float32)."""
    import torch

    M, H, E, dev = _gate_inputs(x, gate_w, shared_w)
    S = k + (shared_w is not None)
    if topk_ids is None:
        topk_ids = torch.empty((M, S), dtype=torch.int32, device=dev)
    if topk_weights is None:
        topk_weights = torch.empty((M, S), dtype=torch.float32, device=dev)
    _out(topk_ids, "topk_ids", torch.int32, dev, numel=M * S)
    _out(topk_weights, "topk_weights", torch.float32, dev, numel=M * S)
    nbytes = _ws_bytes(workspace, dev)
    _check(lib().mr_route(_ptr(x), _ptr(gate_w), _ptr(shared_w), M, H, E, k, float(scale),
                          _ptr(topk_ids), _ptr(topk_weights), _ptr(workspace), nbytes, _stream(stream, dev)))
    return topk_ids, topk_weights


def _align_outputs(M, S, num_experts, A, device, sorted_token_ids, expert_ids, npp):
    import torch

    cap = mr_align_capacity(M, S, num_experts, A)
    if sorted_token_ids is None:
        sorted_token_ids = torch.empty(max(cap, 1), dtype=torch.int32, device=device)
    if expert_ids is None:
        expert_ids = torch.empty(max(cap // A, 1), dtype=torch.int32, device=device)
    if npp is None:
        npp = torch.empty(1, dtype=torch.int32, device=device)
    # capacities are checked by the library against the lengths passed
    _out(sorted_token_ids, "sorted_token_ids", torch.int32, device)
    _out(expert_ids, "expert_ids", torch.int32, device)
    _out(npp, "npp", torch.int32, device, min_numel=1)
    return sorted_token_ids, expert_ids, npp


def mr_align(topk_ids, num_experts: int, A: int, *, workspace, sorted_token_ids=None,
             expert_ids=None, npp=None, stream=None):
    """Returns (sorted_token_ids, expert_ids, npp) as device tensors; entries
    at or past npp are unspecified."""
    import torch

    if topk_ids.dtype != torch.int32 or not topk_ids.is_contiguous():
        raise ValueError("topk_ids must be a contiguous int32 tensor")
    dev = topk_ids.device
    _on(topk_ids, "topk_ids", dev)
    ids2 = topk_ids.view(topk_ids.shape[0], -1) if topk_ids.dim() >= 1 and topk_ids.numel() else topk_ids
    M = topk_ids.shape[0] if topk_ids.dim() else 0
    S = ids2.shape[1] if ids2.dim() == 2 else 1
    sorted_token_ids, expert_ids, npp = _align_outputs(M, S, num_experts, A, dev, sorted_token_ids, expert_ids, npp)
    nbytes = _ws_bytes(workspace, dev)
    _check(lib().mr_align(_ptr(topk_ids), M, S, num_experts, A, _ptr(sorted_token_ids),
                          sorted_token_ids.numel(), _ptr(expert_ids), expert_ids.numel(), _ptr(npp),
                          _ptr(workspace), nbytes, _stream(stream, dev)))
    return sorted_token_ids, expert_ids, npp


def mr_align_local(topk_ids, expert_map, num_local_experts: int, A: int, *, workspace, sorted_token_ids=None,
                   expert_ids=None, npp=None, stream=None):
    """The align of one expert-parallel rank: expert_map (int32 device tensor
    [E'], local id or -1 per global expert) selects and renumbers the pairs.
    Returns (sorted_token_ids, expert_ids, npp) as device tensors; entries at
    or past npp are unspecified."""
    import torch

    if topk_ids.dtype != torch.int32 or not topk_ids.is_contiguous():
        raise ValueError("topk_ids must be a contiguous int32 tensor")
    if expert_map.dtype != torch.int32 or not expert_map.is_contiguous():
        raise ValueError("expert_map must be a contiguous int32 tensor")
    dev = topk_ids.device
    _on(topk_ids, "topk_ids", dev)
    _on(expert_map, "expert_map", dev)
    ids2 = topk_ids.view(topk_ids.shape[0], -1) if topk_ids.dim() >= 1 and topk_ids.numel() else topk_ids
    M = topk_ids.shape[0] if topk_ids.dim() else 0
    S = ids2.shape[1] if ids2.dim() == 2 else 1
    sorted_token_ids, expert_ids, npp = _align_outputs(M, S, num_local_experts, A, dev, sorted_token_ids,
                                                       expert_ids, npp)
    nbytes = _ws_bytes(workspace, dev)
    _check(lib().mr_align_local(_ptr(topk_ids), M, S, expert_map.numel(), _ptr(expert_map), num_local_experts, A,
                                _ptr(sorted_token_ids), sorted_token_ids.numel(), _ptr(expert_ids),
                                expert_ids.numel(), _ptr(npp), _ptr(workspace), nbytes, _stream(stream, dev)))
    return sorted_token_ids, expert_ids, npp


def mr_route_align(x, gate_w, shared_w, k: int, scale: float = 1.0, A: int | None = None, *,
                   workspace, topk_ids=None, topk_weights=None, sorted_token_ids=None,
                   expert_ids=None, npp=None, stream=None):
    """Route + align in one launch.  A defaults to the M-aware tier.
    Returns dict(topk_ids, topk_weights, sorted_token_ids, expert_ids, npp, A)."""
    import torch

    M, H, E, dev = _gate_inputs(x, gate_w, shared_w)
    sh = shared_w is not None
    S = k + sh
    if A is None:
        A = mr_select_alignment(M, k, E)
    if topk_ids is None:
        topk_ids = torch.empty((M, S), dtype=torch.int32, device=dev)
    if topk_weights is None:
        topk_weights = torch.empty((M, S), dtype=torch.float32, device=dev)
    _out(topk_ids, "topk_ids", torch.int32, dev, numel=M * S)
    _out(topk_weights, "topk_weights", torch.float32, dev, numel=M * S)
    sorted_token_ids, expert_ids, npp = _align_outputs(M, S, E + sh, A, dev, sorted_token_ids, expert_ids, npp)
    nbytes = _ws_bytes(workspace, dev)
    _check(lib().mr_route_align(_ptr(x), _ptr(gate_w), _ptr(shared_w), M, H, E, k, float(scale), A,
                                _ptr(topk_ids), _ptr(topk_weights), _ptr(sorted_token_ids),
                                sorted_token_ids.numel(), _ptr(expert_ids), expert_ids.numel(), _ptr(npp),
                                _ptr(workspace), nbytes, _stream(stream, dev)))
    return {"topk_ids": topk_ids, "topk_weights": topk_weights, "sorted_token_ids": sorted_token_ids,
            "expert_ids": expert_ids, "npp": npp, "A": A}


def mr_route_align_noalloc(x, gate_w, shared_w, k: int, scale: float = 1.0, A: int | None = None, *,
                           topk_ids, topk_weights, sorted_token_ids, expert_ids, npp, stream=None):
    """mr_route_align without a workspace (the library's static per-GPU
    scratch array) and without allocating: every output buffer is the
    caller's.  Returns dict(topk_ids, topk_weights, sorted_token_ids,
    expert_ids, npp, A)."""
    import torch

    M, H, E, dev = _gate_inputs(x, gate_w, shared_w)
    sh = shared_w is not None
    S = k + sh
    if A is None:
        A = mr_select_alignment(M, k, E)
    _out(topk_ids, "topk_ids", torch.int32, dev, numel=M * S)
    _out(topk_weights, "topk_weights", torch.float32, dev, numel=M * S)
    _out(sorted_token_ids, "sorted_token_ids", torch.int32, dev)
    _out(expert_ids, "expert_ids", torch.int32, dev)
    _out(npp, "npp", torch.int32, dev, min_numel=1)
    _check(lib().mr_route_align_noalloc(_ptr(x), _ptr(gate_w), _ptr(shared_w), M, H, E, k, float(scale), A,
                                        _ptr(topk_ids), _ptr(topk_weights), _ptr(sorted_token_ids),
                                        sorted_token_ids.numel(), _ptr(expert_ids), expert_ids.numel(), _ptr(npp),
                                        _stream(stream, dev)))
    return {"topk_ids": topk_ids, "topk_weights": topk_weights, "sorted_token_ids": sorted_token_ids,
            "expert_ids": expert_ids, "npp": npp, "A": A}


def mr_debug_gate_logits(x, gate_w, shared_w, *, workspace, logits=None, stream=None):
    """Test hook: the fp32 logits [M, E + shared] the route kernels compute."""
    import torch

    M, H, E, dev = _gate_inputs(x, gate_w, shared_w)
    Ep = E + (shared_w is not None)
    if logits is None:
        logits = torch.empty((M, Ep), dtype=torch.float32, device=dev)
    _out(logits, "logits", torch.float32, dev, numel=M * Ep)
    nbytes = _ws_bytes(workspace, dev)
    _check(lib().mr_debug_gate_logits(_ptr(x), _ptr(gate_w), _ptr(shared_w), M, H, E, _ptr(logits),
                                      _ptr(workspace), nbytes, _stream(stream, dev)))
    return logits


def mr_debug_stream_read(src, out, nbytes=None, stream=None):
    """Measurement hook: one plain streaming-read launch over the first
    nbytes of src (default: all of it).  out: MR_STREAM_READ_OUT_WORDS int32
    words on the device; block b stores the XOR of what it read in out[b]."""
    if not src.is_contiguous() or not out.is_contiguous():
        raise ValueError("src and out must be contiguous")
    _on(src, "src", src.device)
    _on(out, "out", src.device)
    if out.numel() * out.element_size() < 4 * MR_STREAM_READ_OUT_WORDS:
        raise ValueError(f"out must hold {MR_STREAM_READ_OUT_WORDS} 32-bit words")
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if n < 0 or n > src.numel() * src.element_size():
        raise ValueError(f"nbytes={n} is outside src ({src.numel() * src.element_size()} bytes)")
    _check(lib().mr_debug_stream_read(_ptr(src), n, _ptr(out), _stream(stream, src.device)))


def mr_argmax_workspace_bytes(R: int, N: int) -> int:
    return int(lib().mr_argmax_workspace_bytes(R, N))


def new_argmax_workspace(R: int, N: int, device="cuda"):
    """A zeroed workspace for mr_argmax_rows_f32 on R rows of N values."""
    import torch

    return torch.zeros(max(mr_argmax_workspace_bytes(R, N), 16), dtype=torch.uint8, device=device)


def mr_argmax_rows_f32(x, *, workspace, out=None, n=None, stream=None):
    """Row-wise argmax (PyTorch semantics) of a 2-D float32 CUDA tensor whose
    rows are contiguous; reads the first n (default: all) values of each row.
    Returns int64 [R]."""
    import torch

    if x.dtype != torch.float32 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D float32 tensor with contiguous rows")
    dev = x.device
    _on(x, "x", dev)
    R, N = x.shape
    if n is not None and not 1 <= int(n) <= N:
        raise ValueError(f"n={n} is outside [1, {N}]")
    N = N if n is None else int(n)
    if out is None:
        out = torch.empty(R, dtype=torch.int64, device=dev)
    _out(out, "out", torch.int64, dev, min_numel=R)
    # a single row's stride is never used: pass N rounded up to 4
    ld = x.stride(0) if R > 1 else N + (-N) % 4
    nbytes = _ws_bytes(workspace, dev)
    _check(lib().mr_argmax_rows_f32(_ptr(x), R, N, ld, _ptr(out), _ptr(workspace), nbytes, _stream(stream, dev)))
    return out


def mr_grouped_gemm_bf16(x, w_experts, S: int, sorted_token_ids, expert_ids, npp, A: int, *, y=None, stream=None):
    """Grouped-expert GEMM over the align output: x bf16 [M, H], w_experts
    bf16 [E', N, H]; returns y fp32 [M*S, N] (rows of pairs not placed below
    npp keep y's previous contents; a new y starts as NaN)."""
    import torch

    _bf16_2d(x, "x")
    if w_experts.dtype != torch.bfloat16 or w_experts.dim() != 3 or not w_experts.is_contiguous():
        raise ValueError("w_experts must be a contiguous bf16 tensor [E', N, H]")
    M, H = x.shape
    Ep, N, H2 = w_experts.shape
    if H2 != H:
        raise ValueError("w_experts hidden size differs from x")
    dev = x.device
    _on(x, "x", dev)
    _on(w_experts, "w_experts", dev)
    _out(sorted_token_ids, "sorted_token_ids", torch.int32, dev)
    # the kernel reads expert_ids for every block below npp / A, and npp can
    # reach sorted_cap
    _out(expert_ids, "expert_ids", torch.int32, dev, min_numel=sorted_token_ids.numel() // A)
    _out(npp, "npp", torch.int32, dev, min_numel=1)
    if y is None:
        y = torch.full((M * S, N), float("nan"), dtype=torch.float32, device=dev)
    _out(y, "y", torch.float32, dev, numel=M * S * N)
    _check(lib().mr_grouped_gemm_bf16(_ptr(x), M, H, _ptr(w_experts), Ep, N, S, _ptr(sorted_token_ids),
                                      sorted_token_ids.numel(), _ptr(expert_ids), _ptr(npp), A, _ptr(y),
                                      _stream(stream, dev)))
    return y
