"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every symbol include/moeroute.h declares, and its host-only logic (tier,
capacities, workspace sizing, refusals that list every failed check) behaves
as documented.  No kernel is launched here."""
import ctypes
import os
import re

import pytest

import oracle
import moe_token_routing_amd as mr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    with open(os.path.join(ROOT, "include", "moeroute.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(mr_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mr.library_path()):
        pytest.skip("libmoeroute.so not built (python -m moe_token_routing_amd.build)")
    return mr._binding.lib()


def test_exports_every_declared_symbol(lib):
    declared = _declared_symbols()
    assert declared, "no declarations found"
    assert set(declared) == set(mr.SIGNATURES), (declared, sorted(mr.SIGNATURES))
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version(lib):
    assert mr.mr_abi_version() == 1


def test_tier_matches_oracle(lib):
    for M in [0, 1, 4, 6, 128, 1024, 2047, 2048, 6553, 6554, 100000]:
        for k, E in [(8, 128), (10, 512), (1, 1), (4, 16)]:
            assert mr.mr_select_alignment(M, k, E) == oracle.select_alignment(M, k, E)
    assert mr.mr_select_alignment(-1, 8, 128) < 0
    assert mr.mr_select_alignment(4, 0, 128) < 0


def test_capacity_matches_oracle(lib):
    for M, S, Ep, A in [(4, 11, 513, 64), (2048, 8, 128, 128), (1, 1, 1, 16), (3, 5, 1000, 256)]:
        assert mr.mr_align_capacity(M, S, Ep, A) == oracle.align_capacity(M, S, Ep, A)
        assert mr.mr_expert_ids_capacity(M, S, Ep, A) == oracle.align_capacity(M, S, Ep, A) // A


def test_workspace_bytes_monotone(lib):
    prev = 0
    for M in [1, 4, 16, 17, 128, 2048, 4096]:
        b = mr.mr_workspace_bytes(M, 512, 10, True)
        assert b >= prev and b % 256 == 0
        prev = b
    assert mr.mr_workspace_bytes(-1, 512, 10, True) == 0


def _err(lib):
    return lib.mr_last_error().decode()


def test_route_refusal_lists_every_reason(lib):
    rc = lib.mr_route(None, None, None, -1, 7, 0, 0, 1.0, None, None, None, 0, None)
    assert rc == mr.MR_EINVAL
    msg = _err(lib)
    for needle in ["gate_w is NULL", "M=-1", "H=7", "E=0", "k=0", "ws is NULL", "ws_bytes=0"]:
        assert needle in msg, (needle, msg)


def test_route_refusal_unsupported(lib):
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: refused before launch
    rc = lib.mr_route(fake, fake, None, 4, 4100, 2000, 40, 1.0, fake, fake, fake, 1 << 30, None)
    assert rc == mr.MR_EUNSUPPORTED
    msg = _err(lib)
    for needle in ["H=4100 is not a multiple of 8", "E=2000 > 1024", "k=40 > 32"]:
        assert needle in msg, (needle, msg)


def test_route_refusal_misaligned(lib):
    ok = ctypes.c_void_p(1 << 20)
    bad = ctypes.c_void_p((1 << 20) + 2)
    rc = lib.mr_route(bad, ok, bad, 4, 64, 16, 4, 1.0, ok, ok, ok, 1 << 30, None)
    assert rc == mr.MR_EUNSUPPORTED
    assert "x is not 16-byte aligned" in _err(lib) and "shared_w is not 16-byte aligned" in _err(lib)


def test_route_align_refusal_capacity(lib):
    p = ctypes.c_void_p(1 << 20)
    need = mr.mr_align_capacity(4, 11, 513, 64)
    rc = lib.mr_route_align(p, p, p, 4, 4096, 512, 10, 1.0, 64, p, p, p, need - 1, p, need // 64 - 1, p,
                            p, 16, None)
    assert rc == mr.MR_ECAPACITY
    msg = _err(lib)
    assert f"sorted_cap={need - 1} < {need}" in msg
    assert f"expert_cap={need // 64 - 1} < {need // 64}" in msg
    assert "ws_bytes=16" in msg


def test_route_align_refusal_alignment(lib):
    p = ctypes.c_void_p(1 << 20)
    for A in [0, 8, 48, 512]:
        rc = lib.mr_route_align(p, p, p, 4, 4096, 512, 10, 1.0, A, p, p, p, 1 << 20, p, 1 << 20, p,
                                p, 1 << 30, None)
        assert rc == mr.MR_EUNSUPPORTED and f"A={A} is not a power of two" in _err(lib)


def test_align_refusals(lib):
    p = ctypes.c_void_p(1 << 20)
    rc = lib.mr_align(None, 4, 0, 0, 64, None, 0, None, 0, None, None, 0, None)
    assert rc == mr.MR_EINVAL
    msg = _err(lib)
    for needle in ["topk_ids is NULL", "S=0", "num_experts=0", "sorted_token_ids is NULL",
                   "expert_ids is NULL", "npp is NULL", "ws is NULL"]:
        assert needle in msg, (needle, msg)
    rc = lib.mr_align(p, 4, 2, 5000, 64, p, 1 << 20, p, 1 << 20, p, p, 1 << 30, None)
    assert rc == mr.MR_EUNSUPPORTED and "num_experts=5000 > 4096" in _err(lib)


def test_stream_read_refusals(lib):
    rc = lib.mr_debug_stream_read(None, 16, None, None)
    assert rc == mr.MR_EINVAL
    msg = _err(lib)
    assert "src is NULL" in msg and "out is NULL" in msg, msg
    rc = lib.mr_debug_stream_read(ctypes.c_void_p((1 << 20) + 8), 24, ctypes.c_void_p((1 << 20) + 2), None)
    assert rc == mr.MR_EUNSUPPORTED
    msg = _err(lib)
    for needle in ["src is not 16-byte aligned", "out is not 4-byte aligned", "nbytes=24 is not a multiple of 16"]:
        assert needle in msg, (needle, msg)
    with open(os.path.join(ROOT, "include", "moeroute.h")) as f:
        words = re.search(r"#define MR_STREAM_READ_OUT_WORDS (\d+)", f.read())
    assert words and int(words.group(1)) == mr.MR_STREAM_READ_OUT_WORDS


def test_argmax_refusals(lib):
    p = ctypes.c_void_p(1 << 20)
    rc = lib.mr_argmax_rows_f32(None, 2, 0, 2, None, None, 0, None)
    assert rc == mr.MR_EINVAL
    msg = _err(lib)
    for needle in ["N=0 < 1", "x is NULL", "out is NULL", "ws is NULL", "ld=2 is not a multiple of 4"]:
        assert needle in msg, (needle, msg)
    rc = lib.mr_argmax_rows_f32(ctypes.c_void_p((1 << 20) + 4), 2, 10, 8, p, p, 16, None)
    assert rc == mr.MR_EINVAL
    msg = _err(lib)
    for needle in ["ld=8 < N=10", "x is not 16-byte aligned"]:
        assert needle in msg, (needle, msg)
    need = lib.mr_argmax_workspace_bytes(16, 248320)
    assert need == 16 * 256 + 16 * 61 * 8
    rc = lib.mr_argmax_rows_f32(p, 16, 248320, 248320, p, p, need - 8, None)
    assert rc == mr.MR_ECAPACITY and f"< {need}" in _err(lib)
    rc = lib.mr_argmax_rows_f32(p, 1, 1 << 31, 1 << 31, p, p, 1 << 40, None)
    assert rc == mr.MR_EUNSUPPORTED and ">= 2^31" in _err(lib)
    assert lib.mr_argmax_rows_f32(None, 0, 5, 8, None, None, 0, None) == mr.MR_OK  # R == 0: nothing to do
    assert lib.mr_argmax_workspace_bytes(-1, 5) == 0 and lib.mr_argmax_workspace_bytes(3, 0) == 0


def test_align_local_refusals(lib):
    p = ctypes.c_void_p(1 << 20)
    rc = lib.mr_align_local(p, 4, 2, 0, None, 3, 64, p, 1 << 20, p, 1 << 20, p, p, 1 << 30, None)
    assert rc == mr.MR_EINVAL
    msg = _err(lib)
    assert "expert_map is NULL" in msg and "num_experts_global=0 < 1" in msg, msg
    rc = lib.mr_align_local(p, 4, 2, 8, p, 0, 64, p, 1 << 20, p, 1 << 20, p, p, 1 << 30, None)
    assert rc == mr.MR_EINVAL and "num_experts=0 < 1" in _err(lib)


def test_error_cleared_after_success_path(lib):
    lib.mr_route(None, None, None, -1, 7, 0, 0, 1.0, None, None, None, 0, None)
    assert _err(lib)
    lib.mr_workspace_reset(None, 0, None)
    assert "ws is NULL" in _err(lib)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(mr._binding, "_lib", None)
    monkeypatch.setattr(mr._binding, "_LIB_PATH", str(tmp_path / "libmoeroute.so"))
    with pytest.raises(mr.MoeRouteError, match="is missing"):
        mr.mr_abi_version()


def test_status_refusals(lib):
    """mr_workspace_status refuses, listing every reason, before any launch."""
    rc = lib.mr_workspace_status(None, 0, None, None)
    assert rc == mr.MR_EINVAL
    msg = _err(lib)
    for needle in ["ws is NULL", "ws_bytes=0", "status is NULL"]:
        assert needle in msg, (needle, msg)
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: refused before launch
    rc = lib.mr_workspace_status(ctypes.c_void_p((1 << 20) + 16), 1 << 20, ctypes.c_void_p((1 << 20) + 2), None)
    assert rc == mr.MR_EUNSUPPORTED
    msg = _err(lib)
    assert "ws is not 256-byte aligned" in msg and "status is not 4-byte aligned" in msg, msg
    rc = lib.mr_workspace_status(fake, 64, fake, None)
    assert rc == mr.MR_ECAPACITY and "ws_bytes=64 <" in _err(lib)


def test_workspace_must_be_256_byte_aligned(lib):
    """The prefill launch's partial rows start on 128-byte lines only when
    the workspace base is 256-byte aligned."""
    fake = ctypes.c_void_p(1 << 20)
    ws = ctypes.c_void_p((1 << 20) + 128)
    rc = lib.mr_route_align(fake, fake, None, 4, 64, 16, 4, 1.0, 64, fake, fake, fake, 1 << 20, fake, 1 << 20,
                            fake, ws, 1 << 30, None)
    assert rc == mr.MR_EUNSUPPORTED and "ws is not 256-byte aligned" in _err(lib), _err(lib)


def test_wait_limit_hook(lib):
    for v in (0, 5, -3, -1):
        assert lib.mr_debug_set_wait_limit(v) == mr.MR_OK
    assert mr.MR_STATUS_KEY_WAIT | mr.MR_STATUS_ID_WAIT | mr.MR_STATUS_GRID_WAIT | mr.MR_STATUS_TILE_WAIT == 15
