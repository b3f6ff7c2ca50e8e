"""The pins in test_oracle.py must catch plausible mistakes.  Each case plants
one mistake in a copy of oracle.c (on the CPU), builds it, points the oracle
at it and runs every pin; at least one pin has to fail."""
import os

import pytest

import oracle
import test_oracle as pins

MUTATIONS = {
    "gate_dropped_first_term": ("for (int h = 0; h < H; ++h)\n                acc += or_bf16_value(x[(size_t)m * H + h]) *",
                                "for (int h = 1; h < H; ++h)\n                acc += or_bf16_value(x[(size_t)m * H + h]) *"),
    "gate_transposed_weight": ("or_bf16_value(W[(size_t)e * H + h])", "or_bf16_value(W[(size_t)h * E + e])"),
    "gate_shared_wrong_row": ("or_bf16_value(x[(size_t)m * H + h]) * or_bf16_value(ws[h])",
                              "or_bf16_value(x[(size_t)h]) * or_bf16_value(ws[h])"),
    "round_one_bit_short": ("int qexp = ex - 8;", "int qexp = ex - 7;"),
    "round_ties_away": ("nearbyint(ldexp(z, -qexp))", "round(ldexp(z, -qexp))"),
    "round_via_binary32": ("double r = ldexp(nearbyint(ldexp(z, -qexp)), qexp);",
                           "double r = ldexp(nearbyint(ldexp((double)(float)z, -qexp)), qexp);"),
    "round_no_subnormal_floor": ("if (qexp < -133)\n        qexp = -133;", ""),
    "tie_highest_id": ("return (a->e < b->e) ? -1 : (a->e > b->e);", "return (a->e > b->e) ? -1 : (a->e < b->e);"),
    "select_ascending": ("if (a->r > b->r)\n        return -1;", "if (a->r < b->r)\n        return -2;"),
    "select_on_unrounded": ("c[e].r = or_bf16_value(b);", "c[e].r = zr[e];"),
    "softmax_sign": ("p[e] = exp(c[e].r - rmax);", "p[e] = exp(rmax - c[e].r);"),
    "softmax_not_renormalised": ("(float)(p[c[j].e] / sel)", "(float)(p[c[j].e])"),
    "sigmoid_sign": ("(float)(scale / (1.0 + exp(-sm)))", "(float)(scale / (1.0 + exp(sm)))"),
    "shared_id_off_by_one": ("ids[(size_t)m * S + k] = E;", "ids[(size_t)m * S + k] = E - 1;"),
    "align_floor_not_ceil": ("total += (cnt[e] + A - 1) / A * A;", "total += cnt[e] / A * A + A;"),
    "align_unstable_scatter": ("for (int64_t i = 0; i < n; ++i) {\n        int32_t e = ids[i];\n        if (e >= 0 && e < Eprime)\n            sorted[off[e]++]",
                               "for (int64_t i = n - 1; i >= 0; --i) {\n        int32_t e = ids[i];\n        if (e >= 0 && e < Eprime)\n            sorted[off[e]++]"),
    "align_sentinel": ("sorted[p] = (int32_t)n;", "sorted[p] = -1;"),
    "align_blocks_shifted": ("for (int64_t b = off[e] / A; b < (off[e] + padded) / A; ++b)",
                             "for (int64_t b = off[e] / A + 1; b <= (off[e] + padded) / A && b < expert_cap; ++b)"),
    "tier_strict": ("((int64_t)M * k >= (int64_t)128 * E)", "((int64_t)M * k > (int64_t)128 * E)"),
    "tier_uses_slots": ("((int64_t)M * k >= (int64_t)128 * E)", "((int64_t)M * (k + 1) >= (int64_t)128 * E)"),
    "align_local_ignores_map": ("const int32_t l = (e >= 0 && e < Eglobal) ? map[e] : -1;", "const int32_t l = (e >= 0 && e < Eglobal) ? e : -1;"),
    "align_local_map_off_by_one": ("const int32_t l = (e >= 0 && e < Eglobal) ? map[e] : -1;", "const int32_t l = (e >= 1 && e < Eglobal) ? map[e - 1] : -1;"),
    "gemm_token_of_pair": ("const uint16_t *xr = x + (size_t)(p / S) * H;", "const uint16_t *xr = x + (size_t)(p % M) * H;"),
    "gemm_expert_of_next_block": ("const int32_t e = expert_ids[j / A];", "const int32_t e = expert_ids[(j + 1) / A];"),
    "gemm_weight_transposed": ("const uint16_t *wr = W + ((size_t)e * N + c) * H;", "const uint16_t *wr = W + ((size_t)c * Ep + e) * H;"),
    "argmax_ties_last": ("if (isnan(v) || v > b)", "if (isnan(v) || v >= b)"),
    "argmax_last_nan": ("            if (isnan(b))\n                break; /* the first NaN has won the row */\n", ""),
    "argmax_nan_loses": ("if (isnan(v) || v > b)", "if (v > b)"),
    "argmax_positive_zero_wins": ("if (isnan(v) || v > b)", "if (isnan(v) || v > b || (v == b && signbit(b) && !signbit(v)))"),
    "capacity_tight_wrong": ("int64_t touched = loose ? Eprime : (Eprime < n ? Eprime : n);",
                             "int64_t touched = loose ? Eprime - 1 : (Eprime < n ? Eprime : n);"),
}

PIN_TESTS = [getattr(pins, n) for n in dir(pins) if n.startswith("test_")]


def _run_pins(golden_dir):
    failed = []
    for t in PIN_TESTS:
        try:
            if "golden_dir" in t.__code__.co_varnames[: t.__code__.co_argcount]:
                t(golden_dir)
            else:
                t()
        except Exception:  # noqa: BLE001 -- any failure counts as caught
            failed.append(t.__name__)
    return failed


def test_unmutated_oracle_passes_all_pins(golden_dir):
    assert _run_pins(golden_dir) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, golden_dir, tmp_path):
    old, new = MUTATIONS[name]
    src = oracle.source_text()
    assert src.count(old) >= 1, f"mutation anchor not found: {name}"
    mutated = src.replace(old, new, 1)
    lib = oracle.build_variant(mutated, os.path.join(str(tmp_path), f"lib_{name}.so"))
    with oracle.use_library(lib):
        failed = _run_pins(golden_dir)
    assert failed, f"no pin caught the planted mistake {name}"
