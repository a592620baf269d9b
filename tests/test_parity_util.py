"""The GPU/oracle comparison excuses only true near-ties (CPU only).

Fake "GPU" outputs are compared with oracle results on exact dyadic cases
(rows uniform over subsets, as in the margin pins), so the distance of every
decision from its boundary is known exactly."""
import numpy as np

import oracle
from tests.parity_util import Report, compare, decisions_taken, probe_tokens


def _subset_row(V, support):
    x = np.full(V, -np.inf, np.float32)
    x[list(support)] = 0.0
    return x


def _residual_case(u_accept, u_sample):
    # P_t = 1/4 on {0..3} at position 0, P_d = 1/4 on {2..5}, draft token 2
    # (ratio 1 -> accepted below u = 1) or 4 (ratio 0 -> rejected).
    V = 8
    t = np.stack([_subset_row(V, {0, 1, 2, 3}), _subset_row(V, {5})])[None]
    d = _subset_row(V, {2, 3, 4, 5})[None, None]
    tok = np.array([[4]], np.int32)
    uni = np.array([[[u_accept, u_sample], [0.5, 0.5]]], np.float32)
    return t, d, tok, uni


def _compare_with(gpu_len, gpu_out, case):
    t, d, tok, uni = case
    orc = oracle.verify(t, d, tok, uni, 1.0, probe_token=probe_tokens(gpu_len, gpu_out))
    return compare(np.asarray(gpu_len), np.asarray(gpu_out), orc, 1), orc


def test_neighbour_across_a_near_tie_is_excused():
    # residual 1/4 on {0, 1}: S = 1/2, boundary between tokens 0 and 1 at u*S = 1/4.
    # u = 1/2 - 2^-24: the oracle picks 0, 2^-24 of normalised mass from token 1.
    case = _residual_case(0.0, 0.5 - 2.0 ** -24)
    rep, orc = _compare_with([0], [[1, -1]], case)
    assert orc["out_tokens"][0, 0] == 0
    assert orc["probe_gap"][0] == 2.0 ** -24
    assert rep.excused == 1 and not rep.failures


def test_a_far_token_is_not_excused_even_when_the_oracle_is_near_a_boundary():
    case = _residual_case(0.0, 0.5 - 2.0 ** -24)
    # the oracle's own sample margin is tiny, but token 5 has no residual mass
    # and lies 1/2 of the mass away
    rep, orc = _compare_with([0], [[5, -1]], case)
    assert orc["sample_margin"][0] < 1e-6
    assert rep.excused == 0 and len(rep.failures) == 1


def test_same_output_is_not_a_disagreement():
    case = _residual_case(0.0, 0.3)
    rep, orc = _compare_with([0], [[0, -1]], case)
    assert rep.excused == 0 and not rep.failures


def test_accept_disagreement_near_the_threshold_is_excused_and_far_is_not():
    V = 8
    t = np.stack([_subset_row(V, {0, 1, 2, 3}), _subset_row(V, {0, 1, 2, 3})])[None]
    d = _subset_row(V, {0, 1})[None, None]          # ratio at token 0: 1/2
    tok = np.array([[0]], np.int32)
    for u, excused in ((0.5 + 2.0 ** -23, True), (0.75, False)):
        uni = np.array([[[u, 0.5], [0.5, 0.5]]], np.float32)
        orc = oracle.verify(t, d, tok, uni, 1.0, probe_token=np.array([0], np.int32))
        assert orc["accepted_len"][0] == 0
        rep = compare(np.array([1]), np.array([[0, 2]]), orc, 1)    # the "GPU" accepted
        assert (rep.excused == 1) == excused and (len(rep.failures) == 1) != excused


def test_other_tokens_must_match_exactly():
    case = _residual_case(0.0, 0.5 - 2.0 ** -24)
    t, d, tok, uni = case
    # K = 1: a different padding entry is a failure even with a near-tie sample
    orc = oracle.verify(t, d, tok, uni, 1.0, probe_token=np.array([1], np.int32))
    rep = compare(np.array([0]), np.array([[1, 7]]), orc, 1)
    assert len(rep.failures) == 1


def test_faulty_flag_difference_fails():
    case = _residual_case(0.0, 0.3)
    rep, _ = _compare_with([-1], [[-1, -1]], case)
    assert len(rep.failures) == 1


def test_decisions_taken():
    # K = 3: n = 0 -> 1 accept test + sample; n = 2 -> 3 + 1; n = 3 (all accepted) -> 3 + 1; faulty -> 0
    assert decisions_taken([0, 2, 3, -1], 3) == 2 + 4 + 4 + 0
    assert decisions_taken([0, 0], 0) == 2
    r = Report(decisions=100)
    assert r.allowed_excused() == 1
    r = Report(decisions=57600)
    assert r.allowed_excused() == 5


def test_probe_tokens():
    pt = probe_tokens(np.array([0, 2, -1]), np.array([[5, -1, -1], [1, 2, 9], [-1, -1, -1]]))
    assert pt.tolist() == [5, 9, -1]


def test_probability_error_is_relative_above_the_fp32_normal_range():
    from tests.parity_util import FLT_MIN, prob_rel_error
    assert prob_rel_error([1.0000358], [1.0]) > 3e-5
    assert prob_rel_error([0.5, 1e-20 * (1 + 2e-6)], [0.5, 1e-20]) < 3e-6
    # both below 2^-126 (a subnormal or zero on the fp32 side): equal
    assert prob_rel_error([0.0, 1e-40], [3e-42, 1e-41]) == 0.0
    # the oracle below 2^-126 but the GPU not: counted as a full error
    assert prob_rel_error([2 * FLT_MIN], [1e-41]) == 1.0
    # the oracle above 2^-126 and the GPU flushed to zero: a full relative error
    assert prob_rel_error([0.0], [1e-30]) == 1.0
