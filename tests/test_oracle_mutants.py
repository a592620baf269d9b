"""Planted mistakes in the oracle must fail at least one pin.

Each mutant is a copy of oracle.c with one plausible error (a dropped clamp, a
wrong row index, a flipped comparison ...).  It is compiled with gcc into a
temporary library, swapped in for the real one, and the pins are re-run; the
test passes only if some pin rejects the mutant.  Everything runs on the CPU.
"""
import ctypes
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_enumeration as enum_pins
from tests import test_oracle_kv as kv_pins
from tests import test_oracle_margins as margin_pins
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "non_strict_accept": ("int acc = ui < thr;", "int acc = ui <= thr;"),
    "scalar_residual": ("prob_at(draft, dtype, dr, v, md[n], Zd[n], T);",
                        "prob_at(draft, dtype, dr, d[n], md[n], Zd[n], T);"),
    "no_clamp": ("w[v] = diff > 0.0 ? diff : 0.0;", "w[v] = diff;"),
    "residual_uses_previous_draft_row": ("const size_t dr = drow0 + (size_t)n * V;",
                                         "const size_t dr = drow0 + (size_t)(n > 0 ? n - 1 : 1) * V;"),
    "bonus_from_last_draft_position": ("w[v] = prob_at(target, dtype, tr, v, mt[K], Zt[K], T); S += w[v]; }\n    }",
                                       "w[v] = prob_at(target, dtype, tr - (size_t)V, v, mt[K-1], Zt[K-1], T); S += w[v]; }\n    }"),
    "cdf_ge": ("if (C > target_mass) { pick = v; break; }", "if (C >= target_mass) { pick = v; break; }"),
    "temperature_multiplies": ("Z += exp((x - m) / T);", "Z += exp((x - m) * T);"),
    "greedy_last_tie": ("if (x > best) { best = x; arg = v; }\n        }\n        if (!isfinite(best)) faulty = 1;",
                        "if (x >= best) { best = x; arg = v; }\n        }\n        if (!isfinite(best)) faulty = 1;"),
    "last_rejection": ("if (!acc && n == K) n = i;", "if (!acc) n = i;"),
    "emit_draft_at_rejection": ("out[n] = pick;", "out[n] = n < K ? d[n] : pick;"),
    "zero_ratio_accepts": ("double ratio = pd > 0.0 ? pt / pd : INFINITY;",
                           "double ratio = pd > 0.0 ? pt / pd : 0.0;"),
    # tie-band outputs and the rounding fallbacks
    "sample_margin_lower_gap_only": ("margin = (lo < hi ? lo : hi) / S;", "margin = lo / S;"),
    "sample_margin_not_divided_by_mass": ("margin = (lo < hi ? lo : hi) / S;", "margin = (lo < hi ? lo : hi);"),
    "accept_margin_against_ratio": ("accept_margin[(size_t)b * K + i] = fabs(ui - thr);",
                                    "accept_margin[(size_t)b * K + i] = fabs(ui - ratio);"),
    "no_crossing_picks_smallest": ("for (int32_t v = V - 1; v >= 0; --v) if (w[v] > 0.0) { pick = v; break; }",
                                   "for (int32_t v = 0; v < V; ++v) if (w[v] > 0.0) { pick = v; break; }"),
    "no_crossing_picks_last_id": ("for (int32_t v = V - 1; v >= 0; --v) if (w[v] > 0.0) { pick = v; break; }",
                                  "pick = V - 1;"),
    "no_zero_residual_fallback": ("if (!(S > 0.0)) {", "if (0) {"),
    "zero_residual_fallback_uncounted": ("if (fallbacks) fallbacks[b] = 1;", "(void)0;"),
    "probe_interval_without_own_weight": ("const double Cg1 = Cg0 + w[g];", "const double Cg1 = Cg0;"),
    "probe_gap_not_divided_by_mass": ("probe_gap[b] = gap / S;", "probe_gap[b] = gap;"),
    # acceptance probability of one position
    "overlap_takes_max": ("s += pt < pd ? pt : pd;", "s += pt > pd ? pt : pd;"),
    "overlap_draft_normalised_by_target": ("const double pd = prob_at(draft, dtype, row0, v, md, Zd, T);",
                                           "const double pd = prob_at(draft, dtype, row0, v, md, Zt, T);"),
    "kv_commit_off_by_one": ("(size_t)Lmax + (size_t)(len + j)) * (size_t)row_bytes;",
                             "(size_t)Lmax + (size_t)(len + j + 1)) * (size_t)row_bytes;"),
    "kv_commit_includes_rejected": ("for (int32_t j = 0; j < n; ++j) {", "for (int32_t j = 0; j <= n && j < K; ++j) {"),
    "head_w_transposed": ("double wv = logit_at(W, OR_BF16, (size_t)tok * d + (size_t)j);",
                          "double wv = logit_at(W, OR_BF16, (size_t)j * V + (size_t)tok);"),
    "head_tokens_reversed_in_cluster": ("int32_t tok = c * cluster_size + t;",
                                        "int32_t tok = c * cluster_size + (cluster_size - 1 - t);"),
    "head_compact_in_reverse_selection_order": (
        "size_t o = ((size_t)b * K + k) * (size_t)L + (size_t)s * cluster_size + (size_t)t;",
        "size_t o = ((size_t)b * K + k) * (size_t)L + (size_t)(n_sel - 1 - s) * cluster_size + (size_t)t;"),
    "head_absdot_signed": ("aacc += fabs(hv * wv);", "aacc += hv * wv;"),
    "head_dense_zero_fill": ("dense[i] = -INFINITY;", "dense[i] = 0.0;"),
    "kv_commit_no_room_check": ("if (len < 0 || len > Lmax - n) { status[b] = 1; continue; }",
                                "if (len < 0) { status[b] = 1; continue; }"),
}

PINS = [
    pins.test_worked_example_acceptance_by_quadrature,
    pins.test_worked_example_replacements_by_quadrature,
    pins.test_worked_example_output_marginal_is_target,
    lambda: pins.test_row_stats_against_logsumexp(0.8),
    pins.test_identical_draft_accepts_everything_and_samples_bonus,
    pins.test_disjoint_supports_reject_and_sample_target,
    pins.test_zero_draft_probability_means_accept,
    pins.test_greedy_is_argmax_prefix,
    pins.test_accept_comparison_is_strict,
    pins.test_inverse_cdf_skips_zero_weight_tokens,
    pins.test_expected_tokens_closed_form,
    lambda: pins.test_chi_square_output_follows_target(2.0),
    lambda: enum_pins.test_oracle_law_equals_the_exact_law("v4_k3"),
    lambda: enum_pins.test_oracle_law_equals_the_exact_law("v3_k2_t07"),
    margin_pins.test_accept_margin_below_threshold_exact,
    margin_pins.test_accept_margin_above_threshold_exact,
    margin_pins.test_accept_margin_is_measured_against_the_clamped_threshold,
    margin_pins.test_accept_margin_with_zero_draft_probability,
    margin_pins.test_sample_margin_of_a_residual_upper_gap_nearer,
    margin_pins.test_sample_margin_of_a_residual_lower_gap_nearer,
    margin_pins.test_sample_margin_of_a_bonus_token,
    margin_pins.test_probe_gap_of_a_residual,
    margin_pins.test_probe_gap_of_a_bonus_token,
    margin_pins.test_probe_gap_undefined_cases,
    margin_pins.test_zero_residual_falls_back_to_the_target_row,
    margin_pins.test_no_crossing_takes_the_largest_id_of_positive_weight,
    pins.test_overlap_worked_example_is_the_printed_acceptance,
    pins.test_overlap_is_one_minus_total_variation,
    pins.test_overlap_limits,
    pins.test_head_all_clusters_is_dense_matmul_and_permutation_free,
    pins.test_head_one_hot_rows_pick_columns_of_W,
    pins.test_head_absdot_is_the_sum_of_absolute_products,
    kv_pins.test_exercise_prefix_plus_accepted_drafts,
    kv_pins.test_multi_step_cache_holds_the_committed_stream,
    kv_pins.test_status_cases_commit_nothing,
]


def _build_mutant(name, old, new, tmp):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    path = os.path.join(tmp, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    so = os.path.join(tmp, f"lib{name}.so")
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
                           "-o", so, path, "-lm"])
    return so


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    old, new = MUTANTS[name]
    real = oracle._load()
    with tempfile.TemporaryDirectory() as tmp:
        so = _build_mutant(name, old, new, tmp)
        lib = ctypes.CDLL(so)
        for fn in ("oracle_verify", "oracle_row_stats", "oracle_overlap", "oracle_head", "oracle_kv_commit"):
            getattr(lib, fn).argtypes = getattr(real, fn).argtypes
            getattr(lib, fn).restype = getattr(real, fn).restype
        monkeypatch.setattr(oracle, "_lib", lib)
        caught = []
        for pin in PINS:
            try:
                pin()
            except AssertionError:
                caught.append(getattr(pin, "__name__", "pin"))
                break
        assert caught, f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", ["no_clamp", "scalar_residual", "residual_uses_previous_draft_row",
                                  "bonus_from_last_draft_position", "last_rejection",
                                  "emit_draft_at_rejection", "temperature_multiplies"])
def test_enumeration_pin_alone_catches_rule_mutants(name, monkeypatch):
    """The exact-law pin by itself rejects every mutant of the rule's steps.
    (The strictness mutants, <= for < in the accept test and >= for > in the
    inverse CDF, change the output only on boundaries of measure zero; the
    boundary pins catch them, and an infinite ratio concerns only tokens the
    draft gives probability 0, which the enumeration never proposes.)"""
    old, new = MUTANTS[name]
    real = oracle._load()
    with tempfile.TemporaryDirectory() as tmp:
        lib = ctypes.CDLL(_build_mutant(name, old, new, tmp))
        lib.oracle_verify.argtypes = real.oracle_verify.argtypes
        lib.oracle_verify.restype = real.oracle_verify.restype
        monkeypatch.setattr(oracle, "_lib", lib)
        with pytest.raises(AssertionError):
            for case in sorted(enum_pins.CASES):
                enum_pins.test_oracle_law_equals_the_exact_law(case)
