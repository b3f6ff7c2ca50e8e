"""Pins for the CPU oracle: every check here compares the oracle with something
other than itself -- values the pages print, hand-worked cases, closed forms,
library routines (torch's bf16 cast, math.fsum, math.tanh, numpy exp, sorted())
and brute force on tiny inputs.  No GPU needed.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from moe_token_routing_amd import workloads


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ----------------------------------------------------------- bf16 rounding --

def test_round_hand_cases(golden_dir):
    g = _load(golden_dir, "bf16_rounding_cases.json")
    for c in g["cases"]:
        v = float(eval(c["value"]))  # fixture expressions are plain arithmetic
        got = int(oracle.round_bf16(np.array([v]))[0])
        assert got == int(c["bits"], 16), (c, hex(got))


def test_round_matches_torch_on_binary32_values():
    """On values a binary32 holds exactly, one rounding from double equals
    torch's float32 -> bfloat16 cast (round to nearest even)."""
    import torch

    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f32 = bits.view(np.float32)
    f32 = f32[np.isfinite(f32)]
    # add values near bf16 half-way points and binary32 subnormals
    extra = np.uint32(0x3F000000) + (np.arange(0, 4000, dtype=np.uint32) << np.uint32(15))
    sub = rng.integers(1, 2 ** 23, size=5000, dtype=np.uint64).astype(np.uint32)
    f32 = np.concatenate([f32, extra.view(np.float32), sub.view(np.float32),
                          -sub.view(np.float32), np.array([0.0, -0.0], np.float32)])
    want = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bf16(f32.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(f32[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def _bf16_exact(bits: int) -> Fraction:
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0:
        return sign * Fraction(m, 2 ** 133)
    return sign * Fraction(128 + m, 128) * Fraction(2) ** (e - 127)


def _nearest_even_by_search(z: float) -> int:
    """Brute force: among all finite bf16 patterns near z, the closest one by
    exact rational distance; equal distance -> even last bit."""
    zf = Fraction(z)
    approx = int(np.array([z], np.float32).view(np.uint32)[0] >> 16)
    sign = 0x8000 if math.copysign(1.0, z) < 0 else 0  # rounding keeps the sign
    cands = [b | sign for b in range(max(0, (approx & 0x7FFF) - 3),
                                     min(0x7F7F, (approx & 0x7FFF) + 3) + 1)]
    best = min(cands, key=lambda b: (abs(_bf16_exact(b) - zf), b & 1))
    return best


def test_round_direct_from_double_by_exact_search():
    """Doubles that binary32 cannot hold (where rounding through binary32 would
    round twice): the oracle's result is the nearest bf16 by exact rational
    distance, ties to even."""
    rng = np.random.default_rng(2)
    vals = []
    for _ in range(3000):
        base = float(rng.uniform(-300, 300))
        b = int(np.array([base], np.float32).view(np.uint32)[0] >> 16) & 0xFFFF
        lo = _bf16_exact(b & 0x7FFF) * (1 if base >= 0 else -1)
        nxt = _bf16_exact((b & 0x7FFF) + 1) * (1 if base >= 0 else -1)
        mid = (lo + nxt) / 2
        off = Fraction(int(rng.integers(-5, 6)), 2 ** int(rng.integers(30, 60)))
        vals.append(float(mid + off))
    vals += [float(rng.normal()) * 2.0 ** int(rng.integers(-140, -120)) for _ in range(300)]
    got = oracle.round_bf16(np.array(vals))
    for v, g in zip(vals, got):
        assert int(g) == _nearest_even_by_search(v), (v, hex(g))


def test_bf16_value_roundtrip():
    bits = np.arange(0, 2 ** 16, dtype=np.uint16)
    vals = oracle.bf16_value(bits)
    fin = np.isfinite(vals)
    # every finite pattern maps to itself (except -0 vs +0 which both keep sign)
    assert np.array_equal(oracle.round_bf16(vals[fin]), bits[fin])
    # exact decode against the rational definition on a sample
    for b in list(range(0, 300)) + list(range(0x3F00, 0x4100, 7)) + [0x7F7F, 0xFF7F, 0x8001]:
        assert Fraction(float(vals[b])) == _bf16_exact(b)


# ------------------------------------------------------------------- gate --

def test_gate_exact_on_integer_inputs():
    """Integer inputs times 2^-4: the logit is an exact integer sum times
    2^-8.  Non-square shapes catch a transposed operand."""
    d = workloads.make_inputs(5, 7, 96, True, "int", seed=3)
    z, s = oracle.gate(d["x"], d["w"], d["ws"])
    xi = np.rint(oracle.bf16_value(d["x"]) * 16).astype(np.int64)
    wi = np.rint(oracle.bf16_value(d["w"]) * 16).astype(np.int64)
    si = np.rint(oracle.bf16_value(d["ws"]) * 16).astype(np.int64)
    assert np.array_equal(z * 256, (xi @ wi.T).astype(np.float64))
    assert np.array_equal(s * 256, (xi @ si).astype(np.float64))


def test_gate_one_hot_rows():
    H, E = 64, 9
    d = workloads.make_inputs(3, E, H, True, "normal", seed=4)
    x = np.zeros((3, H), np.uint16)
    one = 0x3F80
    for m, h in enumerate([0, 17, 63]):
        x[m, h] = one
    z, s = oracle.gate(x, d["w"], d["ws"])
    wv = oracle.bf16_value(d["w"])
    wsv = oracle.bf16_value(d["ws"])
    for m, h in enumerate([0, 17, 63]):
        assert np.array_equal(z[m], wv[:, h])
        assert s[m] == wsv[h]


def test_gate_matches_exactly_rounded_sum():
    """Random bf16 inputs: bf16 x bf16 products are exact in double, so
    math.fsum gives the exactly rounded logit.  The oracle's sequential sum
    must lie within the recursive-summation bound H * 2^-53 * sum|terms|."""
    d = workloads.make_inputs(3, 11, 512, True, "normal", seed=5)
    z, s = oracle.gate(d["x"], d["w"], d["ws"])
    xv = oracle.bf16_value(d["x"])
    wv = oracle.bf16_value(d["w"])
    for m in range(3):
        for e in range(11):
            terms = xv[m] * wv[e]
            exact = math.fsum(terms.tolist())
            bound = 512 * 2.0 ** -53 * float(np.abs(terms).sum())
            assert abs(z[m, e] - exact) <= bound
        terms = xv[m] * oracle.bf16_value(d["ws"])
        assert abs(s[m] - math.fsum(terms.tolist())) <= 512 * 2.0 ** -53 * float(np.abs(terms).sum())


# ----------------------------------------------------------------- select --

def _beats(r, a, b):
    """a precedes b: larger value, or equal value (-0 == +0) and lower id."""
    return r[a] > r[b] or (r[a] == r[b] and a < b)


def _brute_topk(r, k):
    E = len(r)
    winners = [c for c in itertools.combinations(range(E), k)
               if all(_beats(r, a, b) for a in c for b in range(E) if b not in c)]
    assert len(winners) == 1
    chosen = winners[0]
    orders = [p for p in itertools.permutations(chosen)
              if all(_beats(r, p[i], p[i + 1]) for i in range(k - 1))]
    assert len(orders) == 1
    return list(orders[0])


def test_topk_hand_cases(golden_dir):
    g = _load(golden_dir, "topk_tie_cases.json")
    for c in g["cases"]:
        z = np.array([c["r"]], dtype=np.float64)
        ids, w, _ = oracle.select(z, None, c["k"])
        assert ids[0].tolist() == c["ids"], c["name"]
    c = g["rounding_creates_tie"]
    z = np.array([[float(eval(v)) for v in c["z"]]])
    ids, _, _ = oracle.select(z, None, c["k"])
    assert ids[0].tolist() == c["ids"]


def test_topk_brute_force_tiny():
    rng = np.random.default_rng(6)
    pool = np.array([-1.0, -0.0, 0.0, 0.5, 1.0, 1.5, -0.5])
    for _ in range(400):
        E = int(rng.integers(1, 8))
        k = int(rng.integers(1, min(E, 4) + 1))
        r = rng.choice(pool, size=E)
        ids, _, _ = oracle.select(r[None, :], None, k)
        assert ids[0].tolist() == _brute_topk(r, k), (r, k)


def test_topk_selects_on_rounded_logits():
    """Random double logits: the chosen experts are the brute-force top-k of
    the bf16-rounded values (torch's cast on binary32 inputs gives them)."""
    import torch

    rng = np.random.default_rng(7)
    for _ in range(200):
        E, k = 7, 3
        z32 = (rng.normal(size=E) * 0.05).astype(np.float32)
        z32[rng.integers(0, E)] = z32[0]  # force some ties
        rb = torch.from_numpy(z32).to(torch.bfloat16).to(torch.float64).numpy()
        ids, _, rbits = oracle.select(z32.astype(np.float64)[None], None, k)
        assert ids[0].tolist() == _brute_topk(rb, k)
        assert np.array_equal(oracle.bf16_value(rbits[0]), rb)


def test_softmax_closed_forms():
    # equal logits -> 1/k each
    ids, w, _ = oracle.select(np.full((1, 9), 0.75), None, 4)
    assert np.allclose(w, 0.25, rtol=0, atol=1e-7)
    # two chosen experts with gap d: w0 = (1 + tanh(d/2)) / 2
    for d in [0.0, 0.125, 1.0, 3.5, 10.0]:
        z = np.array([[0.5, 0.5 + d, -4.0, -7.0]])
        ids, w, _ = oracle.select(z, None, 2)
        assert ids[0].tolist() == ([0, 1] if d == 0 else [1, 0])
        assert abs(w[0, 0] - 0.5 * (1 + math.tanh(d / 2))) <= 1e-7
        assert abs(w[0, 1] - 0.5 * (1 - math.tanh(d / 2))) <= 1e-7


def test_softmax_invariants_random():
    rng = np.random.default_rng(8)
    z = rng.normal(size=(50, 64))
    ids, w, rbits = oracle.select(z, None, 10)
    r = oracle.bf16_value(rbits)
    for m in range(50):
        assert abs(float(w[m].astype(np.float64).sum()) - 1.0) <= 1e-6
        assert np.all(np.diff(w[m]) <= 0)
        sel = r[m, ids[m]]
        ratio = w[m].astype(np.float64) / w[m, 0]
        assert np.allclose(ratio, np.exp(sel - sel[0]), rtol=1e-6, atol=0)


def test_shared_slot():
    H, E, k = 32, 6, 2
    d = workloads.make_inputs(4, E, H, True, "normal", seed=9)
    zero = np.zeros(H, np.uint16)
    out = oracle.route(d["x"], d["w"], zero, k, scale=2.5)
    assert out["ids"][:, k].tolist() == [E] * 4
    assert np.all(out["weights"][:, k] == np.float32(1.25))
    # nonzero shared row: sigmoid(s) = (1 + tanh(s/2)) / 2, and s from fsum
    out = oracle.route(d["x"], d["w"], d["ws"], k, scale=0.75)
    xv = oracle.bf16_value(d["x"])
    wsv = oracle.bf16_value(d["ws"])
    for m in range(4):
        s = math.fsum((xv[m] * wsv).tolist())
        want = 0.75 * 0.5 * (1 + math.tanh(s / 2))
        assert abs(out["weights"][m, k] - want) <= 1e-7 * max(1.0, want)
        assert abs(out["s"][m] - s) <= 1e-12
    # sign: negating the shared row gives scale - w
    neg = d["ws"] ^ np.uint16(0x8000)
    out2 = oracle.route(d["x"], d["w"], neg, k, scale=0.75)
    assert np.allclose(out2["weights"][:, k] + out["weights"][:, k], 0.75, atol=1e-7)


def test_shared_logit_not_rounded_by_default():
    # s = 1 + 2^-8 exactly: rounding it to bf16 would give 1.0
    H = 16
    x = np.zeros((1, H), np.uint16)
    x[0, 0] = 0x3F80
    x[0, 1] = 0x3B80  # 2^-8
    ws = np.zeros(H, np.uint16)
    ws[0] = 0x3F80
    ws[1] = 0x3F80
    w = np.zeros((3, H), np.uint16)
    a = oracle.route(x, w, ws, 1, 1.0)
    b = oracle.route(x, w, ws, 1, 1.0, round_shared=True)
    s = 1 + 2 ** -8
    assert abs(a["weights"][0, 1] - 0.5 * (1 + math.tanh(s / 2))) <= 1e-7
    assert abs(b["weights"][0, 1] - 0.5 * (1 + math.tanh(0.5))) <= 1e-7


# ------------------------------------------------------------------ align --

def _brute_align(ids, E_prime, A):
    """Comparison sort of the flat indices by (expert, index), then padding
    built segment by segment."""
    flat = ids.reshape(-1).tolist()
    n = len(flat)
    valid = [i for i in range(n) if 0 <= flat[i] < E_prime]
    order = sorted(valid, key=lambda i: (flat[i], i))
    out, blocks = [], []
    pos = 0
    while pos < len(order):
        e = flat[order[pos]]
        seg = []
        while pos < len(order) and flat[order[pos]] == e:
            seg.append(order[pos])
            pos += 1
        while len(seg) % A:
            seg.append(n)
        out += seg
        blocks += [e] * (len(seg) // A)
    return out, blocks, len(out)


def _check_align_invariants(ids, E_prime, A, srt, eids, npp):
    flat = ids.reshape(-1)
    n = flat.size
    assert npp % A == 0
    assert len(srt) == npp and len(eids) == npp // A
    valid = [i for i in range(n) if 0 <= flat[i] < E_prime]
    real = [int(v) for v in srt if v != n]
    assert sorted(real) == valid  # each valid flat index exactly once
    assert all(a <= b for a, b in zip(eids[:-1], eids[1:]))  # non-decreasing
    for b, e in enumerate(eids):
        blk = srt[b * A:(b + 1) * A]
        toks = [int(t) for t in blk if t != n]
        assert all(flat[t] == e for t in toks)
        assert toks == sorted(toks)
    touched = len(set(int(flat[i]) for i in valid))
    assert A * touched <= npp <= len(valid) + touched * (A - 1)


def test_align_npp_page_row_6_tokens(golden_dir):
    """6 tokens x top-8 = 48 routed rows over 33 touched experts of 128 give
    npp 2112 at A=64 and 4224 at A=128 (88.0x the routed rows)."""
    g = _load(golden_dir, "npp_table_e128_k8.json")
    tokens, touched, n64, n128, ratio = g["rows"][0]
    rng = np.random.default_rng(10)
    experts = rng.permutation(128)[:touched]
    # 48 slots: the 33 experts once each, then the first 15 again; rows of 8
    # consecutive slots never repeat an expert
    slots = list(experts) + list(experts[:tokens * 8 - touched])
    ids = np.array(slots, dtype=np.int32).reshape(tokens, 8)
    assert all(len(set(r.tolist())) == 8 for r in ids)
    assert len(set(ids.reshape(-1).tolist())) == touched
    for A, want in ((64, n64), (128, n128)):
        srt, eids, npp = oracle.align(ids, 128, A)
        assert npp == want
        _check_align_invariants(ids, 128, A, srt, eids, npp)
    assert round(n128 / (tokens * 8), 1) == ratio


def test_align_npp_page_row_128_tokens_a128(golden_dir):
    """128 tokens x top-8 over 110 touched experts, none above 128 rows: npp
    at A=128 is 110 x 128 = 14080 (13.75x, printed as 13.8x)."""
    g = _load(golden_dir, "npp_table_e128_k8.json")
    tokens, touched, _, n128, ratio = g["rows"][1]
    rng = np.random.default_rng(11)
    experts = rng.permutation(128)[:touched]
    # the first 14 rows cover all 110 experts, the rest pick 8 of them at random
    cover = list(experts) + list(experts[:14 * 8 - touched])
    head = np.array(cover, dtype=np.int32).reshape(14, 8)
    tail = np.stack([rng.choice(experts, size=8, replace=False) for _ in range(tokens - 14)])
    ids = np.concatenate([head, tail.astype(np.int32)])
    assert all(len(set(r.tolist())) == 8 for r in ids)
    assert np.bincount(ids.reshape(-1), minlength=128).max() <= 128
    assert len(set(ids.reshape(-1).tolist())) == touched
    srt, eids, npp = oracle.align(ids, 128, 128)
    assert npp == n128
    assert round(npp / (tokens * 8), 1) == ratio
    _check_align_invariants(ids, 128, 128, srt, eids, npp)


def test_align_npp_page_rows_bounds(golden_dir):
    """Rows that are layer averages still obey npp@64 <= npp@128 and
    A * touched <= npp <= rows + touched * (A - 1)."""
    g = _load(golden_dir, "npp_table_e128_k8.json")
    for tokens, touched, n64, n128, ratio in g["rows"]:
        rows = tokens * 8
        assert n64 <= n128
        for A, n in ((64, n64), (128, n128)):
            assert A * touched <= n <= rows + touched * (A - 1)
        assert abs(n128 / rows - ratio) <= 0.05 + 1e-9  # printed to one decimal


def test_align_capacity_page_numbers(golden_dir):
    g = _load(golden_dir, "align_workspace_slots.json")
    for tokens, A, slots in g["rows"]:
        assert oracle.align_capacity(tokens, 8, 128, A, loose=True) == slots
        assert oracle.align_capacity(tokens, 8, 128, A) <= slots


def test_align_brute_force_random():
    rng = np.random.default_rng(12)
    for trial in range(300):
        M = int(rng.integers(0, 40))
        S = int(rng.integers(1, 6))
        Ep = int(rng.integers(1, 20))
        A = int(rng.choice([1, 2, 4, 16, 64]))
        if trial % 3 == 0:  # skewed
            ids = rng.zipf(1.5, size=(M, S)) % Ep
        else:
            ids = rng.integers(0, Ep, size=(M, S))
        ids = ids.astype(np.int32)
        if trial % 7 == 0 and ids.size:  # out-of-range ids are skipped
            ids.reshape(-1)[:: 5] = Ep + 3
            ids.reshape(-1)[1:: 11] = -1
        srt, eids, npp = oracle.align(ids, Ep, A)
        bs, be, bn = _brute_align(ids, Ep, A)
        assert npp == bn and srt.tolist() == bs and eids.tolist() == be
        _check_align_invariants(ids, Ep, A, srt, eids, npp)


def test_align_edge_cases():
    # empty input
    srt, eids, npp = oracle.align(np.zeros((0, 3), np.int32), 5, 64)
    assert npp == 0
    # all pairs on one expert
    ids = np.full((100, 1), 3, np.int32)
    srt, eids, npp = oracle.align(ids, 5, 64)
    assert npp == 128 and eids.tolist() == [3, 3]
    assert srt[:100].tolist() == list(range(100)) and set(srt[100:].tolist()) == {100}
    # every expert touched once
    ids = np.arange(8, dtype=np.int32).reshape(2, 4)[:, ::-1].copy()
    srt, eids, npp = oracle.align(ids, 8, 16)
    assert npp == 128 and eids.tolist() == list(range(8))
    assert [srt[16 * e] for e in range(8)] == [3, 2, 1, 0, 7, 6, 5, 4]
    # capacity too small is an error
    with pytest.raises(ValueError):
        oracle.align(np.zeros((4, 2), np.int32), 3, 64, sorted_cap=63)


def test_align_shared_segment_closed_form():
    """With a shared column (id E in every row), the shared expert's segment
    is m*S + k for every row m, padded to ceil(M/A)*A."""
    M, k, E, A = 70, 3, 9, 64
    rng = np.random.default_rng(13)
    ids = np.stack([np.append(rng.choice(E, size=k, replace=False), E) for _ in range(M)]).astype(np.int32)
    srt, eids, npp = oracle.align(ids, E + 1, A)
    S = k + 1
    first = int(np.argmax(eids == E)) * A
    seg = srt[first:first + 128]
    assert seg[:M].tolist() == [m * S + k for m in range(M)]
    assert set(seg[M:].tolist()) == {M * S}
    assert (eids == E).sum() == math.ceil(M / A)


# ------------------------------------------------------------------- tier --

def test_tier_staircase():
    # E=128, top-8: the large tier starts at 2048 tokens
    assert oracle.select_alignment(2047, 8, 128) == 64
    assert oracle.select_alignment(2048, 8, 128) == 128
    assert oracle.select_alignment(6, 8, 128) == 64
    assert oracle.select_alignment(1024, 8, 128) == 64
    # E=512, top-10: every M of the sweep stays at 64; 128*512/10 = 6553.6
    for M in workloads.SWEEP_M:
        assert oracle.select_alignment(M, 10, 512) == 64
    assert oracle.select_alignment(6553, 10, 512) == 64
    assert oracle.select_alignment(6554, 10, 512) == 128


# -------------------------------------------------------------- end to end --

def test_route_exact_inputs_consistency():
    """On integer inputs the whole route is exact: the rounded logits are the
    bf16 rounding of exact integer sums, and the ids are the brute-force
    order of those values."""
    d = workloads.make_inputs(3, 12, 64, True, "int", seed=14)
    out = oracle.route(d["x"], d["w"], d["ws"], 3, 1.0)
    import torch

    xi = np.rint(oracle.bf16_value(d["x"]) * 16).astype(np.int64)
    wi = np.rint(oracle.bf16_value(d["w"]) * 16).astype(np.int64)
    zexact = (xi @ wi.T).astype(np.float32) / 256.0  # exact in binary32
    rb = torch.from_numpy(zexact).to(torch.bfloat16).to(torch.float64).numpy()
    for m in range(3):
        assert out["ids"][m, :3].tolist() == _brute_topk(rb[m], 3)
        assert out["ids"][m, 3] == 12


# ---------------------------------------------------------------- argmax --
# [N] Sampling: a NaN beats every number, the first NaN beats later NaNs,
# equal numbers go to the lowest index, -0 equals +0 (PyTorch's argmax).

def test_argmax_hand_cases(golden_dir):
    with open(os.path.join(golden_dir, "argmax_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        row = np.array([float(v) for v in c["row"]], dtype=np.float32)
        got = int(oracle.argmax_rows(row[None, :])[0])
        assert got == c["want"], (c, got)


def test_argmax_brute_force_tiny():
    # every row of length 4 over seven special values, against the rule
    # stated as a set: the first NaN if there is one, else the first index
    # whose value equals the maximum
    vals = [float("nan"), float("-inf"), -1.0, -0.0, 0.0, 1.0, float("inf")]
    rows = np.array(list(itertools.product(vals, repeat=4)), dtype=np.float32)
    got = oracle.argmax_rows(rows)
    for r, g in zip(rows, got):
        nans = [i for i, v in enumerate(r) if math.isnan(v)]
        if nans:
            want = nans[0]
        else:
            mx = max(float(v) for v in r)
            want = min(i for i, v in enumerate(r) if float(v) == mx)
        assert g == want, (r, g, want)


def test_argmax_matches_torch_and_numpy():
    import torch

    rng = np.random.default_rng(7)
    R, N = 24, 3001
    x = rng.standard_normal((R, N)).astype(np.float32)
    pool = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1.5, -1.5, 4.0], dtype=np.float32)
    for r in range(R):
        kind = r % 6
        if kind == 1:  # a few NaNs
            x[r, rng.choice(N, 3, replace=False)] = np.nan
        elif kind == 2:  # many ties at the maximum
            x[r, rng.choice(N, 50, replace=False)] = 9.0
        elif kind == 3:  # only signed zeros and -inf
            x[r] = rng.choice(np.array([0.0, -0.0, -np.inf], dtype=np.float32), N)
        elif kind == 4:  # special values everywhere
            x[r] = rng.choice(pool, N)
        elif kind == 5:  # integer-valued, heavy ties
            x[r] = rng.integers(-3, 4, N).astype(np.float32)
    got = oracle.argmax_rows(x)
    assert np.array_equal(got, torch.from_numpy(x).argmax(dim=1).numpy())
    assert np.array_equal(got, np.argmax(x, axis=1))
    # thread count does not change the result
    assert np.array_equal(got, oracle.argmax_rows(x, nthreads=1))


# ------------------------------------------------------- EP-local align --

def test_align_local_identity_map_is_align():
    # every expert local under its own id: the plain align, already pinned
    rng = np.random.default_rng(11)
    for (M, S, E, A) in [(37, 9, 65, 16), (300, 11, 257, 64), (5, 3, 4, 128)]:
        ids = rng.integers(0, E, size=(M, S)).astype(np.int32)
        got = oracle.align_local(ids, np.arange(E, dtype=np.int32), E, A)
        want = oracle.align(ids, E, A)
        assert got[2] == want[2] and np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def test_align_local_hand_case():
    # 8 global experts, this rank owns 2 -> 0 and 5 -> 1; flat pairs
    # i = 0..5 carry experts 2, 5, 5, 7, 0, 2
    ids = np.array([[2, 5], [5, 7], [0, 2]], np.int32)
    emap = np.full(8, -1, np.int32)
    emap[2], emap[5] = 0, 1
    srt, eids, npp = oracle.align_local(ids, emap, 2, 16)
    assert npp == 32 and eids.tolist() == [0, 1]
    assert srt[:2].tolist() == [0, 5] and set(srt[2:16].tolist()) == {6}
    assert srt[16:18].tolist() == [1, 2] and set(srt[18:].tolist()) == {6}


def test_align_local_nothing_local():
    ids = np.arange(12, dtype=np.int32).reshape(4, 3) % 7
    srt, eids, npp = oracle.align_local(ids, np.full(7, -1, np.int32), 3, 64)
    assert npp == 0 and srt.size == 0 and eids.size == 0


def test_align_local_partition_covers_every_pair():
    # split E' experts over 4 ranks: every flat index lands on exactly one
    # rank, and each rank's npp is its own closed form
    rng = np.random.default_rng(3)
    M, S, E, A, ranks = 64, 9, 33, 16, 4
    ids = rng.integers(0, E, size=(M, S)).astype(np.int32)
    owner = rng.integers(0, ranks, size=E)
    seen = []
    for r in range(ranks):
        local = np.flatnonzero(owner == r)
        emap = np.full(E, -1, np.int32)
        emap[local] = np.arange(local.size, dtype=np.int32)
        srt, eids, npp = oracle.align_local(ids, emap, max(1, local.size), A)
        counts = [int((ids == e).sum()) for e in local]
        assert npp == sum(-(-c // A) * A for c in counts if c)
        seen += [int(v) for v in srt if v != M * S]
        assert all(owner[ids.reshape(-1)[v]] == r for v in srt if v != M * S)
    assert sorted(seen) == list(range(M * S))


# ------------------------------------------- grouped GEMM over the align --
# [A] Purpose: the consumer multiplies each block of A slots by its expert's
# weights; alignment only regroups rows, so every pair's output is its own
# row times its own expert, whatever A is.

def _consumer_case(M=37, S=3, E=9, N=8, H=24, seed=4):
    rng = np.random.default_rng(seed)
    x = oracle.round_bf16(rng.standard_normal((M, H)))
    w = oracle.round_bf16(rng.standard_normal((E, N, H)) * 0.1)
    ids = np.stack([rng.choice(E, S, replace=False) for _ in range(M)]).astype(np.int32)
    return x, w, ids


def test_grouped_gemm_is_the_direct_product():
    x, w, ids = _consumer_case()
    M, S = ids.shape
    xv, wv = oracle.bf16_value(x), oracle.bf16_value(w)
    want = np.einsum("ph,pnh->pn", np.repeat(xv, S, axis=0), wv[ids.reshape(-1)])  # library product, float64
    for A in (16, 64, 128):
        srt, eids, npp = oracle.align(ids, w.shape[0], A)
        y = oracle.grouped_gemm(x, w, srt, eids, npp, S, A)
        assert not np.isnan(y).any()
        np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)


def test_grouped_gemm_bit_identical_across_alignment():
    x, w, ids = _consumer_case(M=200, S=5, E=17, seed=9)
    ys = []
    for A in (16, 64, 128):
        srt, eids, npp = oracle.align(ids, w.shape[0], A)
        ys.append(oracle.grouped_gemm(x, w, srt, eids, npp, ids.shape[1], A))
    assert all(np.array_equal(ys[0], y) for y in ys[1:])


def test_grouped_gemm_skips_padding_and_foreign_pairs():
    # ids outside [0, E') take no slot, so their rows stay unwritten
    x, w, ids = _consumer_case(M=10, S=2, E=5, seed=1)
    ids[3, 1] = 7
    ids[6, 0] = -1
    srt, eids, npp = oracle.align(ids, 5, 16)
    y = oracle.grouped_gemm(x, w, srt, eids, npp, 2, 16)
    flat = ids.reshape(-1)
    assert np.isnan(y[flat >= 5]).all() and np.isnan(y[flat < 0]).all()
    assert not np.isnan(y[(flat >= 0) & (flat < 5)]).any()
