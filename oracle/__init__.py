"""CPU oracle for MoE token routing + moe_align_block_size (plain C, fp64).

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module; the product path (the
HIP library and its binding) never does.  The C source, ``oracle.c``, shares
no code with the HIP library.

Each function wraps the C function of the same name (``or_*``); the passages
each one follows are cited in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared",
          "-fPIC", "-std=c11", "-Wall", "-Wextra"]


def build() -> str:
    """Compile oracle.c into liboracle.so with the system C compiler."""
    cmd = ["gcc", *CFLAGS, _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.or_bf16_value.argtypes = [ctypes.c_uint16]
    lib.or_bf16_value.restype = f64
    lib.or_round_bf16.argtypes = [f64]
    lib.or_round_bf16.restype = ctypes.c_uint16
    lib.or_gate.argtypes = [P, P, P, i32, i32, i32, P, P, i32]
    lib.or_gate.restype = None
    lib.or_select.argtypes = [P, P, i32, i32, i32, i32, f64, i32, P, P, P, i32]
    lib.or_select.restype = i32
    lib.or_route.argtypes = [P, P, P, i32, i32, i32, i32, f64, i32, P, P, P, P, i32]
    lib.or_route.restype = i32
    lib.or_select_alignment.argtypes = [i32, i32, i32]
    lib.or_select_alignment.restype = i32
    lib.or_align_capacity.argtypes = [i32, i32, i32, i32, i32]
    lib.or_align_capacity.restype = i64
    lib.or_align.argtypes = [P, i32, i32, i32, i32, P, i64, P, i64, P]
    lib.or_align.restype = i32
    lib.or_round_bf16_array.argtypes = [P, P, i64]
    lib.or_round_bf16_array.restype = None
    lib.or_bf16_value_array.argtypes = [P, P, i64]
    lib.or_bf16_value_array.restype = None
    lib.or_align_local.argtypes = [P, i32, i32, i32, P, i32, i32, P, i64, P, i64, P]
    lib.or_align_local.restype = i32
    lib.or_grouped_gemm.argtypes = [P, i32, i32, P, i32, i32, i32, P, P, i64, i32, P, i32]
    lib.or_grouped_gemm.restype = i32
    lib.or_argmax_rows.argtypes = [P, i64, i64, i64, P, i32]
    lib.or_argmax_rows.restype = i32
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _bits(a, shape=None):
    a = np.ascontiguousarray(a, dtype=np.uint16)
    if shape is not None:
        a = a.reshape(shape)
    return a


def round_bf16(z) -> np.ndarray:
    """double -> bf16 bit patterns, nearest-even, one rounding."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    out = np.empty(z.shape, dtype=np.uint16)
    _load().or_round_bf16_array(_ptr(z), _ptr(out), z.size)
    return out


def bf16_value(bits) -> np.ndarray:
    """bf16 bit patterns -> exact double values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    _load().or_bf16_value_array(_ptr(b), _ptr(out), b.size)
    return out


def gate(x_bits, w_bits, ws_bits=None, nthreads: int = 0):
    """Double-precision gate logits: (z [M, E], s [M] or None)."""
    x = _bits(x_bits)
    w = _bits(w_bits)
    M, H = x.shape
    E = w.shape[0]
    assert w.shape[1] == H
    ws = None if ws_bits is None else _bits(ws_bits).reshape(-1)
    if ws is not None:
        assert ws.size == H
    z = np.empty((M, E), dtype=np.float64)
    s = np.empty(M, dtype=np.float64) if ws is not None else None
    _load().or_gate(_ptr(x), _ptr(w), _ptr(ws), M, H, E, _ptr(z), _ptr(s), nthreads)
    return z, s


def select(z, s, k: int, scale: float = 1.0, round_shared: bool = False,
           nthreads: int = 0):
    """Rounding, top-k, softmax + renormalise and the shared slot, from
    double logits z [M, E] (and s [M] or None).  Returns (ids [M, S] int32,
    weights [M, S] float32, r_bits [M, E] uint16)."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    M, E = z.shape
    has_shared = s is not None
    sv = None if s is None else np.ascontiguousarray(s, dtype=np.float64).reshape(M)
    S = k + int(has_shared)
    ids = np.empty((M, S), dtype=np.int32)
    wts = np.empty((M, S), dtype=np.float32)
    rb = np.empty((M, E), dtype=np.uint16)
    rc = _load().or_select(_ptr(z), _ptr(sv), M, E, k, int(has_shared), float(scale),
                           int(round_shared), _ptr(ids), _ptr(wts), _ptr(rb), nthreads)
    if rc != 0:
        raise ValueError(f"or_select failed ({rc})")
    return ids, wts, rb


def route(x_bits, w_bits, ws_bits, k: int, scale: float = 1.0,
          round_shared: bool = False, nthreads: int = 0):
    """Whole route.  Returns dict(ids, weights, z, s)."""
    x = _bits(x_bits)
    w = _bits(w_bits)
    M, H = x.shape
    E = w.shape[0]
    ws = None if ws_bits is None else _bits(ws_bits).reshape(-1)
    S = k + int(ws is not None)
    ids = np.empty((M, S), dtype=np.int32)
    wts = np.empty((M, S), dtype=np.float32)
    z = np.empty((M, E), dtype=np.float64)
    s = np.empty(M, dtype=np.float64) if ws is not None else None
    rc = _load().or_route(_ptr(x), _ptr(w), _ptr(ws), M, H, E, k, float(scale),
                          int(round_shared), _ptr(ids), _ptr(wts), _ptr(z), _ptr(s),
                          nthreads)
    if rc != 0:
        raise ValueError(f"or_route failed ({rc})")
    return {"ids": ids, "weights": wts, "z": z, "s": s}


def select_alignment(M: int, k: int, E: int) -> int:
    return int(_load().or_select_alignment(M, k, E))


def align_capacity(M: int, S: int, num_experts: int, A: int, loose: bool = False) -> int:
    return int(_load().or_align_capacity(M, S, num_experts, A, int(loose)))


def align(topk_ids, num_experts: int, A: int, sorted_cap: int | None = None,
          expert_cap: int | None = None):
    """moe_align_block_size on ids [M, S].  Returns (sorted_token_ids[:npp],
    expert_ids[:npp // A], npp)."""
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    if ids.ndim == 1:
        ids = ids.reshape(-1, 1)
    M, S = ids.shape
    if sorted_cap is None:
        sorted_cap = align_capacity(M, S, num_experts, A)
    if expert_cap is None:
        expert_cap = max(1, sorted_cap // A)
    srt = np.full(max(1, sorted_cap), -7, dtype=np.int32)
    eids = np.full(max(1, expert_cap), -7, dtype=np.int32)
    npp = np.zeros(1, dtype=np.int32)
    rc = _load().or_align(_ptr(ids), M, S, num_experts, A, _ptr(srt), sorted_cap,
                          _ptr(eids), expert_cap, _ptr(npp))
    if rc != 0:
        raise ValueError(f"or_align failed ({rc})")
    n = int(npp[0])
    return srt[:n].copy(), eids[: n // A].copy(), n


def align_local(topk_ids, expert_map, num_local: int, A: int):
    """Align of one expert-parallel rank: expert_map [E'] gives each global
    expert's local id or -1; returns (sorted_token_ids[:npp],
    expert_ids[:npp // A] as local ids, npp)."""
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    if ids.ndim == 1:
        ids = ids.reshape(-1, 1)
    emap = np.ascontiguousarray(expert_map, dtype=np.int32)
    M, S = ids.shape
    cap = align_capacity(M, S, num_local, A)
    srt = np.full(max(1, cap), -7, dtype=np.int32)
    eids = np.full(max(1, cap // A), -7, dtype=np.int32)
    npp = np.zeros(1, dtype=np.int32)
    rc = _load().or_align_local(_ptr(ids), M, S, emap.size, _ptr(emap), num_local, A, _ptr(srt), cap,
                                _ptr(eids), max(1, cap // A), _ptr(npp))
    if rc != 0:
        raise ValueError(f"or_align_local failed ({rc})")
    n = int(npp[0])
    return srt[:n].copy(), eids[: n // A].copy(), n


def grouped_gemm(x_bits, w_bits, sorted_ids, expert_ids, npp: int, S: int, A: int, nthreads: int = 0):
    """Consumer of the align output: x bf16 bits [M, H], w bf16 bits
    [E', N, H]; returns y [M*S, N] float64 with NaN in the rows of pairs that
    no slot below npp holds."""
    x = _bits(x_bits)
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    Ep, N, H = w.shape
    M = x.shape[0]
    srt = np.ascontiguousarray(sorted_ids, dtype=np.int32)
    eids = np.ascontiguousarray(expert_ids, dtype=np.int32)
    if srt.size < npp or eids.size < npp // A:
        raise ValueError("sorted_ids / expert_ids shorter than npp")
    y = np.full((M * S, N), np.nan)
    rc = _load().or_grouped_gemm(_ptr(x), M, H, _ptr(w), Ep, N, S, _ptr(srt), _ptr(eids), npp, A, _ptr(y),
                                 nthreads)
    if rc != 0:
        raise ValueError(f"or_grouped_gemm failed ({rc})")
    return y


def argmax_rows(x, nthreads: int = 0) -> np.ndarray:
    """Row-wise argmax of a 2-D float32 array with PyTorch's semantics (NaN
    first, lowest index on ties, -0 == +0); int64 [R]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] < 1:
        raise ValueError("x must be [R, N] with N >= 1")
    out = np.empty(x.shape[0], dtype=np.int64)
    rc = _load().or_argmax_rows(_ptr(x), x.shape[0], x.shape[1], x.shape[1], _ptr(out), nthreads)
    if rc != 0:
        raise ValueError(f"or_argmax_rows failed ({rc})")
    return out


class use_library:
    """Context manager that points this module at another build of oracle.c
    (the mutation tests use it to check that the pins catch planted
    mistakes)."""

    def __init__(self, path: str):
        self.path = path
        self.saved = None

    def __enter__(self):
        global _lib, _LIB_PATH
        self.saved = (_lib, _LIB_PATH)
        _lib, _LIB_PATH = None, self.path
        _load()
        return self

    def __exit__(self, *exc):
        global _lib, _LIB_PATH
        _lib, _LIB_PATH = self.saved
        return False


def build_variant(source_text: str, out_path: str) -> str:
    """Compile a modified copy of oracle.c (same flags) to out_path."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(source_text)
    subprocess.run(["gcc", *CFLAGS, src, "-o", out_path, "-lm"], check=True)
    return out_path


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()
