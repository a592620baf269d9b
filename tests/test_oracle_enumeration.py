"""Exact law of the verify step on tiny vocabularies, by enumeration.

The rule's defining property (Speculative Decoding lesson, "Step 1": the
output keeps the target's distribution exactly; RuneLab explainer, the
single-position figure and the paragraph after it: accepted drafts plus
replacements give back every target probability) is that each emitted
position follows the target.  With fixed rows per position that reads:
for every position i and every emitted prefix,

    P(out_i = v | position i is emitted, out_0..out_{i-1}) = P_t,i(v).

On V <= 4, K <= 3 with rational probabilities this test

1. derives the exact law of (n, out) from the rule with ``Fraction``
   arithmetic: every draft sequence d (weight prod_i P_d,i(d_i)), accept with
   probability min(1, P_t/P_d) left to right, residual (P_t,n - P_d,n)_+ at
   the first rejection, bonus from P_t,K;
2. checks that this law has the property above, exactly;
3. runs the oracle on one point inside every cell of the uniforms' partition
   (each accept uniform below or above its threshold; the sample uniform in
   each interval between consecutive cumulative-sum breakpoints of every
   distribution that position could sample), weights each output by the
   cell's exact measure, and requires the resulting law to equal the exact
   law, Fraction for Fraction.

The oracle computes in fp64 from float32 logits ln(p), so its probabilities
differ from the rationals by ~1e-7 relative; the points are at least ~1e-3
from any breakpoint, so each lands in the cell the exact rule puts it in.
"""
import itertools
from collections import defaultdict
from fractions import Fraction as F

import numpy as np
import pytest

import oracle


def _rows(spec, den):
    return [[F(a, den) for a in row] for row in spec]


CASES = {
    # V = 4, K = 3: zeros in both models, a ratio above 1, an always-accepted
    # and an always-rejected token, a different row at every position
    "v4_k3": (16,
              [[6, 5, 3, 2], [0, 8, 4, 4], [4, 4, 4, 4], [1, 2, 3, 10]],
              [[3, 6, 5, 2], [8, 0, 4, 4], [1, 1, 1, 13]], 1.0),
    # V = 3, K = 2 at temperature 0.7 (logits are 0.7 * ln p)
    "v3_k2_t07": (8, [[1, 3, 4], [5, 0, 3], [2, 2, 4]], [[4, 3, 1], [1, 6, 1]], 0.7),
    # V = 4, K = 1: the single-position case with one token absent from the draft
    "v4_k1": (8, [[3, 1, 2, 2], [1, 1, 1, 5]], [[1, 4, 3, 0]], 1.0),
    # V = 2, K = 3: identical rows at position 1 (always accepted)
    "v2_k3": (4, [[1, 3], [2, 2], [3, 1], [1, 3]], [[3, 1], [2, 2], [1, 3]], 1.3),
}


def _cdf(w):
    out, c = [], F(0)
    for x in w:
        c += x
        out.append(c)
    return out


def _sampled_dist(Pt, Pd, d, n, K):
    """Distribution sampled at position n (unnormalised) and its total."""
    if n < K:
        w = [max(F(0), a - b) for a, b in zip(Pt[n], Pd[n])]
    else:
        w = list(Pt[K])
    return w, sum(w)


def _threshold(Pt, Pd, d, i):
    pt, pd = Pt[i][d[i]], Pd[i][d[i]]
    return F(1) if pd == 0 else min(F(1), pt / pd)


def exact_law(Pt, Pd):
    K, V = len(Pd), len(Pt[0])
    law = defaultdict(F)
    for d in itertools.product(range(V), repeat=K):
        wd = F(1)
        for i in range(K):
            wd *= Pd[i][d[i]]
        if wd == 0:
            continue
        reach = F(1)                           # probability of accepting positions 0..n-1
        for n in range(K + 1):
            stop = F(1) if n == K else 1 - _threshold(Pt, Pd, d, n)
            if stop > 0 and reach > 0:
                w, S = _sampled_dist(Pt, Pd, d, n, K)
                assert S > 0                   # a rejection leaves positive residual mass exactly
                for v in range(V):
                    if w[v] > 0:
                        out = tuple(d[:n]) + (v,) + (-1,) * (K - n)
                        law[(n, out)] += wd * reach * stop * w[v] / S
            if n < K:
                reach *= _threshold(Pt, Pd, d, n)
    return dict(law)


def check_sequential_marginals(law, Pt):
    """P(out_i = v, emitted, prefix) = P_t,i(v) * P(emitted, prefix) for every i and prefix."""
    K = len(Pt) - 1
    V = len(Pt[0])
    assert sum(law.values()) == 1
    for i in range(K + 1):
        joint = defaultdict(F)
        marg = defaultdict(F)
        for (n, out), p in law.items():
            if n >= i:
                joint[(out[:i], out[i])] += p
                marg[out[:i]] += p
        assert marg, i
        for prefix, pm in marg.items():
            for v in range(V):
                assert joint.get((prefix, v), F(0)) == Pt[i][v] * pm, (i, prefix, v)


def oracle_law(Pt, Pd, T):
    """Law of the oracle's output over the exact partition of the uniforms."""
    K, V = len(Pd), len(Pt[0])
    with np.errstate(divide="ignore"):
        lt = (T * np.log(np.array([[float(p) for p in r] for r in Pt]))).astype(np.float32)
        ld = (T * np.log(np.array([[float(p) for p in r] for r in Pd]))).astype(np.float32)
    seqs = []   # (d, accept uniforms, sample uniform, weight)
    for d in itertools.product(range(V), repeat=K):
        wd = F(1)
        for i in range(K):
            wd *= Pd[i][d[i]]
        if wd == 0:
            continue
        # cells of each accept uniform: [0, thr) and [thr, 1)
        acc_cells = []
        for i in range(K):
            thr = _threshold(Pt, Pd, d, i)
            cells = []
            if thr > 0:
                cells.append((thr / 2, thr))
            if thr < 1:
                cells.append(((1 + thr) / 2, 1 - thr))
            acc_cells.append(cells)
        # breakpoints of every distribution any position could sample
        bps = {F(0), F(1)}
        for n in range(K + 1):
            cand = [list(Pt[n])]
            if n < K:
                cand.append([max(F(0), a - b) for a, b in zip(Pt[n], Pd[n])])
            for w in cand:
                S = sum(w)
                if S > 0:
                    bps.update(c / S for c in _cdf(w))
        bps = sorted(bps)
        smp_cells = [((a + b) / 2, b - a) for a, b in zip(bps, bps[1:]) if b > a]
        for combo in itertools.product(*acc_cells) if K else [()]:
            wa = F(1)
            for _, m in combo:
                wa *= m
            for us, ms in smp_cells:
                seqs.append((d, [u for u, _ in combo], us, wd * wa * ms))
    B = len(seqs)
    tok = np.array([s[0] for s in seqs], np.int32).reshape(B, K)
    uni = np.zeros((B, K + 1, 2), np.float32)
    for b, (_, ua, us, _) in enumerate(seqs):
        for i, u in enumerate(ua):
            uni[b, i, 0] = float(u)
        uni[b, :, 1] = float(us)
    tgt = np.broadcast_to(lt, (B, K + 1, V)).copy()
    dr = np.broadcast_to(ld, (B, K, V)).copy() if K else np.zeros((B, 0, V), np.float32)
    r = oracle.verify(tgt, dr, tok, uni, T)
    law = defaultdict(F)
    for b, s in enumerate(seqs):
        law[(int(r["accepted_len"][b]), tuple(int(x) for x in r["out_tokens"][b]))] += s[3]
    assert np.all(r["fallbacks"] == 0)
    # the probabilities the oracle reports at the draft tokens are the rationals
    # up to the float32 rounding of the logits
    for b, s in enumerate(seqs):
        for i, di in enumerate(s[0]):
            for key, P in (("p_target", Pt), ("p_draft", Pd)):
                got = r[key][b, i]
                if not np.isnan(got):
                    assert abs(got - float(P[i][di])) <= 1e-6 * float(P[i][di]) + 1e-300, (key, b, i)
    return {k: v for k, v in law.items() if v != 0}


@pytest.mark.parametrize("name", sorted(CASES))
def test_exact_law_keeps_the_target_at_every_position(name):
    den, pt, pd, T = CASES[name]
    Pt, Pd = _rows(pt, den), _rows(pd, den)
    for r in Pt + Pd:
        assert sum(r) == 1
    law = exact_law(Pt, Pd)
    check_sequential_marginals(law, Pt)


@pytest.mark.parametrize("name", sorted(CASES))
def test_oracle_law_equals_the_exact_law(name):
    den, pt, pd, T = CASES[name]
    Pt, Pd = _rows(pt, den), _rows(pd, den)
    law = oracle_law(Pt, Pd, T)
    assert law == exact_law(Pt, Pd)
    check_sequential_marginals(law, Pt)


def test_a_wrong_rule_breaks_the_marginals():
    """The property is sharp: the listing's scalar residual (subtracting
    P_d(d) from every entry) loses it on the V = 4, K = 3 case."""
    den, pt, pd, _ = CASES["v4_k3"]
    Pt, Pd = _rows(pt, den), _rows(pd, den)
    law = defaultdict(F)
    K, V = len(Pd), len(Pt[0])
    for d in itertools.product(range(V), repeat=K):
        wd = F(1)
        for i in range(K):
            wd *= Pd[i][d[i]]
        if wd == 0:
            continue
        reach = F(1)
        for n in range(K + 1):
            stop = F(1) if n == K else 1 - _threshold(Pt, Pd, d, n)
            if stop > 0 and reach > 0:
                w = list(Pt[K]) if n == K else [max(F(0), a - Pd[n][d[n]]) for a in Pt[n]]
                S = sum(w)
                for v in range(V):
                    if w[v] > 0:
                        law[(n, tuple(d[:n]) + (v,) + (-1,) * (K - n))] += wd * reach * stop * w[v] / S
            if n < K:
                reach *= _threshold(Pt, Pd, d, n)
    with pytest.raises(AssertionError):
        check_sequential_marginals(dict(law), Pt)
