"""Comparison rules between the HIP path and the CPU oracle.

* Exact inputs (every logit exact in fp32): ids, sorted_token_ids[:npp],
  expert_ids[:npp/A] and npp bit-exact; weights within 1e-5 relative.
* Random inputs: a row is EXEMPT when the oracle's double-precision gap
  between its weakest chosen expert and its strongest unchosen one is below
  one bf16 ulp (at the larger magnitude of the two): an fp32 accumulation can
  then legitimately round the two logits across each other.  In every other
  row the chosen sets match exactly, and slot order matches for every pair of
  chosen experts whose fp64 gap is at least one bf16 ulp.  Weights are
  compared per expert id, 1e-5 relative.  The align outputs are bit-exact
  against the oracle's align run on the GPU's own ids.
* Weights of a row are compared with the oracle's directly only when the
  kernel's fp32 logits round to the same bf16 values as the oracle's double
  logits for every chosen expert (the rounding of a logit lying within fp32
  error of a bf16 midpoint is decided by the accumulation precision); every
  row's weights are compared through the backstop.
* Backstop for every row (exempt or not): the oracle's rounding, selection,
  softmax and shared slot applied to the kernel's own fp32 logits reproduce
  the GPU ids bit-exactly and the weights within 1e-5; and each fp32 logit is
  within 2^-18 * sum_h |x*W| of the double-precision one.
"""
from __future__ import annotations

import numpy as np

import oracle

RTOL_W = 1e-5
ATOL_W = 1e-7


def bf16_ulp(v):
    v = np.abs(np.asarray(v, dtype=np.float64))
    v = np.maximum(v, 2.0 ** -126)
    return np.exp2(np.floor(np.log2(v)) - 7)


def row_margins(z, ids, k):
    """(gap, ulp) per row: gap = min z over chosen - max z over the rest."""
    M, E = z.shape
    gaps = np.empty(M)
    ulps = np.empty(M)
    for m in range(M):
        chosen = ids[m, :k]
        mask = np.ones(E, bool)
        mask[chosen] = False
        lo = z[m, chosen].min()
        if mask.any():
            hi = z[m, mask].max()
            gaps[m] = lo - hi
            ulps[m] = bf16_ulp(max(abs(lo), abs(hi)))
        else:
            gaps[m] = np.inf
            ulps[m] = 0.0
    return gaps, ulps


def check_weights(w_gpu, ids_gpu, w_ref, ids_ref, rows=None):
    M = w_gpu.shape[0]
    rows = range(M) if rows is None else rows
    for m in rows:
        ref = dict(zip(ids_ref[m].tolist(), w_ref[m].astype(np.float64).tolist()))
        for e, w in zip(ids_gpu[m].tolist(), w_gpu[m].astype(np.float64).tolist()):
            assert e in ref, (m, e)
            assert abs(w - ref[e]) <= RTOL_W * abs(ref[e]) + ATOL_W, (m, e, w, ref[e])


def same_rounding_rows(logits_gpu, ref, ids_gpu, k):
    """Rows whose chosen experts' logits round to the same bf16 on both
    sides (kernel fp32 vs oracle double)."""
    E = ref["z"].shape[1]
    rg = oracle.round_bf16(logits_gpu[:, :E].astype(np.float64))
    ro = oracle.round_bf16(ref["z"])
    rows = []
    for m in range(ids_gpu.shape[0]):
        sel = [e for e in ids_gpu[m, :k].tolist() if 0 <= e < E]
        if np.array_equal(rg[m, sel], ro[m, sel]):
            rows.append(m)
    return rows


def check_ids_random(ids_gpu, ref, k):
    """Returns the number of exempt rows; asserts on every other row."""
    z = ref["z"]
    ids_ref = ref["ids"]
    gaps, ulps = row_margins(z, ids_ref, k)
    exempt = gaps < ulps
    for m in np.nonzero(~exempt)[0]:
        g = ids_gpu[m, :k].tolist()
        o = ids_ref[m, :k].tolist()
        assert sorted(g) == sorted(o), (m, g, o)
        pos = {e: i for i, e in enumerate(g)}
        for i in range(k):
            for j in range(i + 1, k):
                a, b = o[i], o[j]
                if z[m, a] - z[m, b] >= bf16_ulp(max(abs(z[m, a]), abs(z[m, b]))):
                    assert pos[a] < pos[b], (m, a, b)
    # slots after k (the shared slot) always match
    if ids_gpu.shape[1] > k:
        assert np.array_equal(ids_gpu[:, k:], ids_ref[:, k:])
    return int(exempt.sum())


# Bounds on how many rows leave the direct comparisons on random inputs (the
# backstop still covers every row).  Exempt rows depend on the seeded input
# alone; measured with the oracle over this suite's random cases: 5.5%
# (skewed E = 128 prefill) to 26% (E = 512, k = 10) of rows at M >= 50, 42%
# at E = 1024, k = 32, and 4 of 7 rows at that shape with M = 7.  Among
# exempt rows the kernel's fp32 sums pick a different expert set only when
# two logits sit within fp32 error (about 2^-18 relative) of each other
# across a bf16 rounding boundary: rare.  Rounding-excluded rows: a chosen
# logit within fp32 error of a bf16 midpoint (ulp 2^-8 relative) is roughly
# a 2^-9 event per logit.
MAX_EXEMPT_FRAC = 0.6
MAX_FLIPPED_FRAC = 0.01
MAX_ROUNDING_EXCLUDED_FRAC = 0.05


def check_exemptions(M, exempt, flipped, excluded):
    """Prints and bounds the rows left out of the direct id comparison
    (exempt), the exempt rows whose chosen set differs from the oracle's
    (flipped), and the rows left out of the direct weight comparison
    (rounding-excluded)."""
    print(f"[rows] M={M} exempt={exempt} flipped={flipped} rounding_excluded={excluded}", flush=True)
    assert exempt <= max(4, MAX_EXEMPT_FRAC * M), (exempt, M)
    assert flipped <= max(2, MAX_FLIPPED_FRAC * M), (flipped, M)
    assert excluded <= max(2, MAX_ROUNDING_EXCLUDED_FRAC * M), (excluded, M)


def check_align(ids_gpu, num_experts, A, srt_gpu, eids_gpu, npp_gpu):
    srt, eids, npp = oracle.align(ids_gpu, num_experts, A)
    assert int(npp_gpu) == npp, (int(npp_gpu), npp)
    assert np.array_equal(srt_gpu[:npp], srt), "sorted_token_ids differ"
    assert np.array_equal(eids_gpu[: npp // A], eids), "expert_ids differ"
    return npp


def check_backstop(x, w, ws, logits_gpu, ids_gpu, w_gpu, k, scale, z_ref):
    """Oracle steps after the gate, on the kernel's own fp32 logits."""
    E = w.shape[0]
    has_shared = ws is not None
    zg = logits_gpu[:, :E].astype(np.float64)
    sg = logits_gpu[:, E].astype(np.float64) if has_shared else None
    ids_b, w_b, _ = oracle.select(zg, sg, k, scale)
    assert np.array_equal(ids_gpu, ids_b), "GPU ids differ from oracle steps on GPU logits"
    check_weights(w_gpu, ids_gpu, w_b, ids_b)
    # fp32 accumulation error bound per logit
    xv = np.abs(oracle.bf16_value(x))
    wv = np.abs(oracle.bf16_value(w))
    bound = 2.0 ** -18 * (xv @ wv.T)
    assert np.all(np.abs(zg - z_ref["z"]) <= bound + 1e-30)
    if has_shared:
        bs = 2.0 ** -18 * (xv @ np.abs(oracle.bf16_value(ws)))
        assert np.all(np.abs(sg - z_ref["s"]) <= bs + 1e-30)
