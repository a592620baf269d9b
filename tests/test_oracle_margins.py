"""Pins of the oracle's tie-band outputs and of its two rounding fallbacks.

The parity tests excuse a GPU/oracle disagreement only when the oracle's own
margin for that decision is below 1e-6, so the margins are pinned here on
cases whose every quantity is exact in IEEE double: each row is uniform over a
subset of the vocabulary (logit 0 on the subset, -inf elsewhere), so each
probability is 1/|subset|, a power of two, and every ratio, residual and
cumulative sum the rule forms is a short dyadic number.  The expected values
are worked out with ``fractions.Fraction`` from the definitions:

- accept margin = |u - min(1, P_t(d)/P_d(d))| (Speculative Decoding lesson,
  "Step 1": accept iff u < min(1, ratio));
- sample margin = distance of u*S to the nearer end of the chosen token's
  cumulative interval, divided by S (inverse CDF in token-id order);
- probe gap = mass between u*S and a given token's cumulative interval,
  divided by S.

The two fallbacks (a rejection whose residual mass is zero samples P_t; an
inverse CDF that finds no crossing takes the largest id of positive weight) are
reachable from in-range uniforms only through rounding; a sample uniform of
exactly 1 reaches both branches deterministically, so the pins use it.
"""
from fractions import Fraction as F

import numpy as np

import oracle


def _subset_row(V, support):
    x = np.full(V, -np.inf, np.float32)
    x[list(support)] = 0.0
    return x


def _one(target_rows, draft_rows, tokens, uni, probe=None, T=1.0):
    """A single sequence: target_rows K+1 supports, draft_rows K supports."""
    V = 8
    K = len(draft_rows)
    t = np.stack([_subset_row(V, s) for s in target_rows])[None]
    d = (np.stack([_subset_row(V, s) for s in draft_rows])[None] if K else np.zeros((1, 0, V), np.float32))
    tok = np.asarray(tokens, np.int32).reshape(1, K)
    u = np.asarray(uni, np.float32).reshape(1, K + 1, 2)
    pr = None if probe is None else np.asarray([probe], np.int32)
    return oracle.verify(t, d, tok, u, T, probe_token=pr)


def _f(x):
    return F(float(np.float32(x)))


# --------------------------------------------------------------------------------------
# accept margin
# --------------------------------------------------------------------------------------

def test_accept_margin_below_threshold_exact():
    # P_t = 1/4 on {0..3}, P_d = 1/2 on {0, 1}: ratio at d = 0 is 1/2
    u = 0.5 - 2.0 ** -20
    r = _one([{0, 1, 2, 3}, {0, 1, 2, 3}], [{0, 1}], [0], [[u, 0.5], [0.5, 0.5]])
    assert r["accepted_len"][0] == 1
    assert r["p_target"][0, 0] == 0.25 and r["p_draft"][0, 0] == 0.5
    assert r["accept_margin"][0, 0] == float(abs(_f(u) - F(1, 2))) == 2.0 ** -20


def test_accept_margin_above_threshold_exact():
    u = 0.5 + 3 * 2.0 ** -22
    r = _one([{0, 1, 2, 3}, {0, 1, 2, 3}], [{0, 1}], [0], [[u, 0.5], [0.5, 0.5]])
    assert r["accepted_len"][0] == 0
    assert r["accept_margin"][0, 0] == float(_f(u) - F(1, 2)) == 3 * 2.0 ** -22


def test_accept_margin_is_measured_against_the_clamped_threshold():
    """Ratio 2 > 1: the threshold is min(1, 2) = 1, so u = 0.75 is 0.25 away
    from it (not 1.25 away from the ratio)."""
    r = _one([{0, 1}, {0, 1}], [{0, 1, 2, 3}], [0], [[0.75, 0.5], [0.5, 0.5]])
    assert r["accepted_len"][0] == 1
    assert r["accept_margin"][0, 0] == 0.25


def test_accept_margin_with_zero_draft_probability():
    """P_d(d) = 0: infinite ratio, threshold 1, margin 1 - u."""
    r = _one([{0, 1, 2, 3}, {0}], [{0, 1}], [3], [[0.625, 0.5], [0.5, 0.5]])
    assert r["accepted_len"][0] == 1
    assert r["accept_margin"][0, 0] == 0.375


# --------------------------------------------------------------------------------------
# sample margin and residual mass
# --------------------------------------------------------------------------------------

def _residual_case(u_sample, probe=None):
    # P_t = 1/4 on {0..3}, P_d = 1/4 on {2..5}; the draft proposes 4, which the
    # target gives 0, so it is rejected for every u.  Residual (P_t - P_d)_+ =
    # 1/4 on {0, 1}, 0 elsewhere: S = 1/2, cumulative sums 1/4, 1/2, 1/2, ...
    return _one([{0, 1, 2, 3}, {5}], [{2, 3, 4, 5}], [4], [[0.0, u_sample], [0.5, 0.5]], probe=probe)


def test_sample_margin_of_a_residual_upper_gap_nearer():
    u = 0.3                                   # u*S = 0.15 in [0, 1/4): token 0, upper gap nearer
    r = _residual_case(u)
    assert r["accepted_len"][0] == 0 and r["out_tokens"][0, 0] == 0
    assert r["residual_mass"][0] == 0.5
    S = F(1, 2)
    us = _f(u) * S
    want = min(us - 0, F(1, 4) - us) / S
    assert F(1, 4) - us < us                  # the case is the one described
    assert r["sample_margin"][0] == float(want)


def test_sample_margin_of_a_residual_lower_gap_nearer():
    u = 0.625                                 # u*S = 0.3125 in [1/4, 1/2): token 1, lower gap nearer
    r = _residual_case(u)
    assert r["out_tokens"][0, 0] == 1
    S = F(1, 2)
    us = _f(u) * S
    assert us - F(1, 4) < F(1, 2) - us
    assert r["sample_margin"][0] == float((us - F(1, 4)) / S) == 0.125


def test_sample_margin_of_a_bonus_token():
    # every draft accepted (identical rows); bonus row 1/4 on {1, 2, 5, 6}
    u = 0.4                                   # u*S = 0.4 in [1/4, 1/2): token 2
    r = _one([{0, 1}, {1, 2, 5, 6}], [{0, 1}], [0], [[0.25, 0.5], [0.0, u]])
    assert r["accepted_len"][0] == 1 and r["out_tokens"][0, 1] == 2
    assert r["residual_mass"][0] == 1.0
    us = _f(u)
    assert r["sample_margin"][0] == float(min(us - F(1, 4), F(1, 2) - us))


# --------------------------------------------------------------------------------------
# probe gap: where another implementation's token sits in the oracle's CDF
# --------------------------------------------------------------------------------------

def test_probe_gap_of_a_residual():
    u = 0.3
    us = _f(u) * F(1, 2)
    S = F(1, 2)
    for probe, lo, hi in ((0, F(0), F(1, 4)), (1, F(1, 4), F(1, 2)), (2, F(1, 2), F(1, 2)),
                          (7, F(1, 2), F(1, 2))):
        r = _residual_case(u, probe=probe)
        gap = F(0) if lo <= us <= hi else (lo - us if us < lo else us - hi)
        assert r["probe_gap"][0] == float(gap / S), probe
    assert _residual_case(u, probe=0)["probe_gap"][0] == 0.0       # the oracle's own pick
    assert _residual_case(u, probe=1)["probe_gap"][0] == float((F(1, 4) - us) / S)


def test_probe_gap_of_a_bonus_token():
    u = 0.4
    us = _f(u)
    rows = ([{0, 1}, {1, 2, 5, 6}], [{0, 1}], [0], [[0.25, 0.5], [0.0, u]])
    want = {2: F(0), 1: us - F(1, 4), 0: us, 5: F(1, 2) - us, 6: F(3, 4) - us, 7: F(1) - us}
    for probe, gap in want.items():
        r = _one(*rows, probe=probe)
        assert r["probe_gap"][0] == float(gap), probe


def test_probe_gap_undefined_cases():
    assert np.isnan(_residual_case(0.3, probe=-1)["probe_gap"][0])
    assert np.isnan(_residual_case(0.3, probe=8)["probe_gap"][0])
    # faulty sequence (draft token out of range)
    r = _one([{0, 1, 2, 3}, {5}], [{2, 3, 4, 5}], [9], [[0.0, 0.3], [0.5, 0.5]], probe=0)
    assert r["accepted_len"][0] == -1 and np.isnan(r["probe_gap"][0])


# --------------------------------------------------------------------------------------
# fallbacks
# --------------------------------------------------------------------------------------

def test_zero_residual_falls_back_to_the_target_row():
    """Identical rows and accept uniform 1: ratio 1, threshold 1, and 1 < 1 is
    false, so position 0 is rejected with an all-zero residual.  The oracle
    then samples P_t,0 itself and counts the fallback."""
    u = 0.6                                   # P_t,0 = 1/4 on {0..3}: 0.6 falls in [1/2, 3/4) -> token 2
    r = _one([{0, 1, 2, 3}, {6}], [{0, 1, 2, 3}], [1], [[1.0, u], [0.5, 0.5]])
    assert r["accepted_len"][0] == 0
    assert r["fallbacks"][0] == 1
    assert r["residual_mass"][0] == 1.0
    assert r["out_tokens"][0, 0] == 2
    assert r["sample_margin"][0] == float(min(_f(u) - F(1, 2), F(3, 4) - _f(u)))
    # an ordinary rejection does not count a fallback
    assert _residual_case(0.3)["fallbacks"][0] == 0


def test_no_crossing_takes_the_largest_id_of_positive_weight():
    """Sample uniform 1: u*S = S and no cumulative sum exceeds it.  The pick is
    the largest id of positive weight (3 here, with ids 4..7 of weight 0), at
    margin 0."""
    r = _one([{0, 1}, {1, 3}], [{0, 1}], [0], [[0.25, 0.5], [0.0, 1.0]])
    assert r["accepted_len"][0] == 1
    assert r["out_tokens"][0, 1] == 3
    assert r["sample_margin"][0] == 0.0
    # the same through a residual: weights 1/4 on {0, 1} only
    r = _residual_case(1.0)
    assert r["out_tokens"][0, 0] == 1 and r["sample_margin"][0] == 0.0
