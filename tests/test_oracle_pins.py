"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: numbers the
pages print, closed forms, library routines (scipy, numpy), or invariants of the
rule.  These run on the CPU.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _logits_from_probs(p):
    """float32 logits ln(p) (-inf for p == 0) so that softmax(logits) = p up to float32 rounding."""
    p = np.asarray(p, np.float64)
    with np.errstate(divide="ignore"):
        return np.log(p).astype(np.float32)


def _single_position_batch(pt, pd, d, u_acc, u_smp):
    """K=1 batch: every sequence has target rows (pt, pt) and draft row pd."""
    V = len(pt)
    B = len(d)
    lt = _logits_from_probs(pt)
    ld = _logits_from_probs(pd)
    target = np.broadcast_to(lt, (B, 2, V)).copy()
    draft = np.broadcast_to(ld, (B, 1, V)).copy()
    uni = np.zeros((B, 2, 2), np.float32)
    uni[:, 0, 0] = u_acc
    uni[:, 0, 1] = u_smp
    uni[:, 1, 1] = u_smp
    return target, draft, np.asarray(d, np.int32).reshape(B, 1), uni


# --------------------------------------------------------------------------------------
# Worked example: RuneLab explainer, single-position figure (five words).
# --------------------------------------------------------------------------------------

def _worked():
    with open(os.path.join(GOLDEN, "worked_example_single_position.json")) as f:
        g = json.load(f)
    pt = np.array(g["p_target_percent"], np.float64) / 100
    pd = np.array(g["p_draft_percent"], np.float64) / 100
    return g, pt, pd


def test_worked_example_acceptance_by_quadrature():
    """Acceptance probability per drafted word and in total (printed: 67 %).

    For each draft word, the accept decision is swept over a midpoint grid of
    N accept-uniforms; the accepted fraction is that word's acceptance
    probability up to 1/N."""
    g, pt, pd = _worked()
    N = 20000
    grid = ((np.arange(N) + 0.5) / N).astype(np.float32)
    acc = np.empty(5)
    for d in range(5):
        t, dr, tok, uni = _single_position_batch(pt, pd, np.full(N, d), grid, 0.5)
        r = oracle.verify(t, dr, tok, uni, 1.0)
        acc[d] = np.mean(r["accepted_len"] == 1)
    total = float(np.dot(pd, acc))
    assert abs(total * 100 - g["printed"]["accept_percent"]) < 0.01
    assert abs((1 - total) * 100 - g["printed"]["reject_percent"]) < 0.01
    # accepted contribution to dalga is printed as 20 points, to tekne as 26
    assert abs(pd[0] * acc[0] * 100 - g["printed"]["dalga_from_accepted_drafts"]) < 0.01
    assert abs(pd[1] * acc[1] * 100 - g["printed"]["tekne_from_accepted_drafts"]) < 0.01


def test_worked_example_replacements_by_quadrature():
    """Replacement (residual) distribution after a rejection (printed: 22, 0, 6, 5; total 33)."""
    g, pt, pd = _worked()
    N = 20000
    grid = ((np.arange(N) + 0.5) / N).astype(np.float32)
    # tekne (id 1) is over-drafted (45 vs 26): with u close to 1 it is always rejected
    t, dr, tok, uni = _single_position_batch(pt, pd, np.full(N, 1), np.float32(0.99999), grid)
    r = oracle.verify(t, dr, tok, uni, 1.0)
    assert np.all(r["accepted_len"] == 0)
    frac = np.bincount(r["out_tokens"][:, 0], minlength=5) / N
    reject_pts = g["printed"]["replacement_points_total"]
    pts = frac * reject_pts
    assert abs(pts[0] - g["printed"]["dalga_from_replacements"]) < 0.01
    assert abs(pts[1] - g["printed"]["tekne_from_replacements"]) < 1e-12
    np.testing.assert_allclose(pts[[0, 2, 3]], g["printed"]["replacement_points_dalga_marti_bulut"], atol=0.01)
    assert pts[4] < 1e-12
    # the residual mass the oracle reports is the rejection probability
    np.testing.assert_allclose(r["residual_mass"], reject_pts / 100, rtol=1e-6)


def test_worked_example_output_marginal_is_target():
    """Accepted drafts plus replacements give back the target's probabilities exactly."""
    g, pt, pd = _worked()
    N = 20000
    grid = ((np.arange(N) + 0.5) / N).astype(np.float32)
    marg = np.zeros(5)
    for d in range(5):
        # 2-D midpoint quadrature, separable: accept depends on u only, the replacement on v only
        t, dr, tok, uni = _single_position_batch(pt, pd, np.full(N, d), grid, 0.5)
        a = np.mean(oracle.verify(t, dr, tok, uni, 1.0)["accepted_len"] == 1)
        t, dr, tok, uni = _single_position_batch(pt, pd, np.full(N, d), np.float32(0.99999), grid)
        r = oracle.verify(t, dr, tok, uni, 1.0)
        if a < 1.0:
            res = np.bincount(r["out_tokens"][:, 0], minlength=5) / N
        else:
            res = np.zeros(5)
        marg += pd[d] * (a * np.eye(5)[d] + (1 - a) * res)
    np.testing.assert_allclose(marg, pt, atol=2e-4)


def test_worked_example_ten_thousand_draws():
    """Monte Carlo as in the figure: 10,000 draws land within about one point of the target."""
    g, pt, pd = _worked()
    rng = np.random.default_rng(20261202)
    N = 10000
    d = rng.choice(5, size=N, p=pd)
    u = rng.random(N, dtype=np.float32)
    v = rng.random(N, dtype=np.float32)
    t, dr, tok, uni = _single_position_batch(pt, pd, d, u, v)
    r = oracle.verify(t, dr, tok, uni, 1.0)
    hist = np.bincount(r["out_tokens"][:, 0], minlength=5) / N
    assert np.max(np.abs(hist - pt)) * 100 < 2 * g["printed"]["empirical_match_points_after_10000_draws"]


# --------------------------------------------------------------------------------------
# Row statistics against a library routine.
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1.0, 0.8, 0.37, 2.5])
def test_row_stats_against_logsumexp(T):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((6, 3001)) * 3).astype(np.float32)
    x[2, ::7] = -np.inf
    m, Z = oracle.row_stats(x, T)
    T32 = float(np.float32(T))
    lse = scipy.special.logsumexp(x.astype(np.float64) / T32, axis=-1)
    np.testing.assert_array_equal(m, x.max(axis=-1).astype(np.float64))
    np.testing.assert_allclose(np.log(Z) + m / T32, lse, rtol=0, atol=1e-12)


def test_bf16_widening_matches_torch():
    import torch
    x = (torch.randn(4, 999, generator=torch.Generator().manual_seed(3)) * 5).to(torch.bfloat16)
    m, Z = oracle.row_stats(x, 1.0)
    xf = x.to(torch.float64).numpy()
    np.testing.assert_array_equal(m, xf.max(axis=-1))
    np.testing.assert_allclose(np.log(Z) + m, scipy.special.logsumexp(xf, axis=-1), atol=1e-12)


# --------------------------------------------------------------------------------------
# Closed form for the expected number of tokens per verify.
# --------------------------------------------------------------------------------------

def test_expected_tokens_closed_form():
    """(1 - a^(K+1)) / (1 - a) tokens per verify under i.i.d. acceptance a; the
    LLMs-from-Scratch lesson ("Expected speedup") prints 3.36 at a = 0.8, K = 4."""
    pt = np.array([0.30, 0.20, 0.15, 0.10, 0.10, 0.05, 0.05, 0.05])
    pd = np.array([0.10, 0.20, 0.15, 0.10, 0.10, 0.05, 0.05, 0.25])
    assert abs(np.minimum(pt, pd).sum() - 0.8) < 1e-12
    K, V = 4, 8
    rng = np.random.default_rng(11)
    lt, ld = _logits_from_probs(pt), _logits_from_probs(pd)
    total, total_sq, count = 0.0, 0.0, 0
    for chunk in range(4):
        B = 50000
        target = np.broadcast_to(lt, (B, K + 1, V)).copy()
        draft = np.broadcast_to(ld, (B, K, V)).copy()
        tok = rng.choice(V, size=(B, K), p=pd).astype(np.int32)
        uni = rng.random((B, K + 1, 2), dtype=np.float32)
        r = oracle.verify(target, draft, tok, uni, 1.0)
        tokens = r["accepted_len"].astype(np.float64) + 1
        total += tokens.sum()
        total_sq += (tokens ** 2).sum()
        count += B
    mean = total / count
    se = math.sqrt((total_sq / count - mean ** 2) / count)
    assert abs(3.36 - round((1 - 0.8 ** 5) / 0.2, 2)) < 1e-12   # the printed value, rounded
    assert abs(mean - 3.3616) < 4 * se, (mean, se)
    assert abs(mean - 3.36) < 0.02


# --------------------------------------------------------------------------------------
# Limit cases that reduce to plain sampling.
# --------------------------------------------------------------------------------------

def _inverse_cdf_numpy(logits_row, T, u):
    p = scipy.special.softmax(logits_row.astype(np.float64) / T)
    c = np.cumsum(p)
    return int(np.searchsorted(c, u * c[-1], side="right")), c


def test_identical_draft_accepts_everything_and_samples_bonus():
    """P_d = P_t: every ratio is 1, so all K drafts are accepted and the bonus
    token is a plain inverse-CDF sample of P_t at position K."""
    import torch
    from workloads import verify_case
    c = verify_case(16, 3, 1000, "bf16", target_std=2.0, zipf_s=0.0, sigma=0.0, temperature=0.9,
                    key=(99, 1))
    assert torch.equal(c.draft, c.target[:, :3])
    r = oracle.verify(c.target, c.draft, c.draft_tokens, c.uniforms, c.temperature)
    assert np.all(r["accepted_len"] == 3)
    np.testing.assert_array_equal(r["out_tokens"][:, :3], c.draft_tokens.numpy())
    x = c.target.to(torch.float64).numpy()
    u = c.uniforms.numpy()
    for b in range(16):
        want, cdf = _inverse_cdf_numpy(x[b, 3], c.temperature, float(u[b, 3, 1]))
        assert r["out_tokens"][b, 3] == want
    np.testing.assert_allclose(r["p_target"], r["p_draft"], rtol=1e-15)


def test_disjoint_supports_reject_and_sample_target():
    """Disjoint supports: acceptance is 0, n = 0 and the residual is P_t itself."""
    rng = np.random.default_rng(5)
    B, K, V, T = 32, 2, 64, 1.0
    x = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    y = (rng.standard_normal((B, K, V)) * 2).astype(np.float32)
    x[..., V // 2:] = -np.inf
    y[..., : V // 2] = -np.inf
    tok = rng.integers(V // 2, V, size=(B, K)).astype(np.int32)
    uni = rng.random((B, K + 1, 2), dtype=np.float32)
    r = oracle.verify(x, y, tok, uni, T)
    assert np.all(r["accepted_len"] == 0)
    for b in range(B):
        want, _ = _inverse_cdf_numpy(x[b, 0], T, float(uni[b, 0, 1]))
        assert r["out_tokens"][b, 0] == want
        assert np.all(r["out_tokens"][b, 1:] == -1)
    np.testing.assert_allclose(r["residual_mass"], 1.0, rtol=1e-12)


def test_zero_draft_probability_means_accept():
    """A draft token the draft model gives probability 0 has an infinite ratio
    (Speculative Decoding lesson, "Step 1") and is accepted."""
    V = 10
    x = np.zeros((1, 2, V), np.float32)
    y = np.zeros((1, 1, V), np.float32)
    y[0, 0, 3] = -np.inf
    uni = np.full((1, 2, 2), 0.999, np.float32)
    r = oracle.verify(x, y, np.array([[3]], np.int32), uni, 1.0)
    assert r["accepted_len"][0] == 1
    assert r["p_draft"][0, 0] == 0.0


# --------------------------------------------------------------------------------------
# Greedy: argmax of the target row (LLMs-from-Scratch lesson 25, "Greedy case").
# --------------------------------------------------------------------------------------

def test_greedy_is_argmax_prefix():
    rng = np.random.default_rng(3)
    B, K, V = 200, 5, 257
    # coarse values make ties common; the first maximal id must win
    x = rng.integers(-6, 6, size=(B, K + 1, V)).astype(np.float32)
    a = np.argmax(x, axis=-1)
    tok = a[:, :K].copy()
    flip = rng.random((B, K)) < 0.25
    tok[flip] = rng.integers(0, V, size=flip.sum())
    r = oracle.verify(x, None, tok.astype(np.int32), None, 1.0, mode=oracle.GREEDY)
    for b in range(B):
        mism = np.nonzero(tok[b] != a[b, :K])[0]
        n = int(mism[0]) if len(mism) else K
        assert r["accepted_len"][b] == n
        np.testing.assert_array_equal(r["out_tokens"][b, :n], tok[b, :n])
        assert r["out_tokens"][b, n] == a[b, n]
        assert np.all(r["out_tokens"][b, n + 1:] == -1)


# --------------------------------------------------------------------------------------
# Distribution of the emitted tokens: chi-square on V = 8, 10^6 trials.
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("sigma", [0.5, 2.0])
def test_chi_square_output_follows_target(sigma):
    """Every emitted position follows P_t (Speculative Decoding lesson, "Step 5";
    exercise 1 asks for a chi-square test).  For position i the sample is the
    trials that reach it (n >= i).  10^6 trials in chunks."""
    rng = np.random.default_rng(1234 + int(sigma * 10))
    V, K, T = 8, 4, 1.0
    xt = (rng.standard_normal((K + 1, V)) * 2).astype(np.float32)
    xd = (xt[:K] + rng.standard_normal((K, V)) * sigma).astype(np.float32)
    pt = scipy.special.softmax(xt.astype(np.float64) / T, axis=-1)
    pd = scipy.special.softmax(xd.astype(np.float64) / T, axis=-1)
    counts = np.zeros((K + 1, V))
    for chunk in range(10):
        B = 100000
        tok = np.stack([rng.choice(V, size=B, p=pd[i]) for i in range(K)], axis=1).astype(np.int32)
        uni = rng.random((B, K + 1, 2), dtype=np.float32)
        r = oracle.verify(np.broadcast_to(xt, (B, K + 1, V)).copy(),
                          np.broadcast_to(xd, (B, K, V)).copy(), tok, uni, T)
        n = r["accepted_len"]
        for i in range(K + 1):
            sel = n >= i
            counts[i] += np.bincount(r["out_tokens"][sel, i], minlength=V)
    alpha = 1e-3 / (K + 1)
    for i in range(K + 1):
        tot = counts[i].sum()
        if tot < 1000:
            continue
        p = scipy.stats.chisquare(counts[i], pt[i] * tot).pvalue
        assert p > alpha, (i, p)
        tv = 0.5 * np.abs(counts[i] / tot - pt[i]).sum()
        assert tv < 0.01


def test_acceptance_falls_as_draft_diverges():
    """Acceptance decreases as the draft moves away from the target (Speculative
    Decoding lesson, "Step 4": inverse monotone relation with KL)."""
    rng = np.random.default_rng(8)
    V, K, T, B = 16, 3, 1.0, 10000
    xt = (rng.standard_normal((K + 1, V)) * 2).astype(np.float32)
    noise = rng.standard_normal((K, V))
    rates, kls = [], []
    for sigma in [0.1, 0.5, 1.0, 2.0, 4.0]:
        xd = (xt[:K] + noise * sigma).astype(np.float32)
        pd = scipy.special.softmax(xd.astype(np.float64), axis=-1)
        pt = scipy.special.softmax(xt[:K].astype(np.float64), axis=-1)
        tok = np.stack([rng.choice(V, size=B, p=pd[i]) for i in range(K)], axis=1).astype(np.int32)
        uni = rng.random((B, K + 1, 2), dtype=np.float32)
        r = oracle.verify(np.broadcast_to(xt, (B, K + 1, V)).copy(),
                          np.broadcast_to(xd, (B, K, V)).copy(), tok, uni, T)
        # accepted fraction per tested position
        rates.append(np.mean(r["accepted_len"]) / K)
        kls.append(float(np.sum(pd * np.log(pd / pt))))
    assert all(np.diff(kls) > 0)
    assert all(np.diff(rates) < 0), rates


# --------------------------------------------------------------------------------------
# Faulty inputs.
# --------------------------------------------------------------------------------------

def test_faulty_sequences_are_flagged():
    rng = np.random.default_rng(2)
    B, K, V = 4, 2, 50
    x = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    y = rng.standard_normal((B, K, V)).astype(np.float32)
    tok = rng.integers(0, V, size=(B, K)).astype(np.int32)
    tok[1, 1] = V            # out of range
    x[2, 0, :] = -np.inf     # a row without a finite maximum
    uni = rng.random((B, K + 1, 2), dtype=np.float32)
    r = oracle.verify(x, y, tok, uni, 1.0)
    assert r["accepted_len"][1] == -1 and np.all(r["out_tokens"][1] == -1)
    assert r["accepted_len"][2] == -1 and np.all(r["out_tokens"][2] == -1)
    assert r["accepted_len"][0] >= 0 and r["accepted_len"][3] >= 0
    g = oracle.verify(x, None, tok, None, 1.0, mode=oracle.GREEDY)
    assert g["accepted_len"][1] == -1 and g["accepted_len"][2] == -1


# --------------------------------------------------------------------------------------
# Shortlisted head (DynaSpec summary, "Model architecture").
# --------------------------------------------------------------------------------------

def test_head_all_clusters_is_dense_matmul_and_permutation_free():
    import torch
    g = torch.Generator().manual_seed(4)
    B, K, d, V, cs = 2, 3, 64, 96, 8
    h = torch.randn(B, K, d, generator=g).to(torch.bfloat16)
    W = (torch.randn(V, d, generator=g) * 0.05).to(torch.bfloat16)
    allc = np.tile(np.arange(V // cs, dtype=np.int32), (B, 1))
    r = oracle.head(h, W, allc, cs, dense=True)
    ref = h.to(torch.float64).numpy() @ W.to(torch.float64).numpy().T
    np.testing.assert_allclose(r["compact"], ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["dense"], ref, rtol=1e-12, atol=1e-12)
    # a token's logit does not depend on which other clusters are selected
    sel_a = np.array([[1, 4, 7], [0, 4, 11]], np.int32)
    ra = oracle.head(h, W, sel_a, cs, dense=True)
    for b in range(B):
        for s, c in enumerate(sel_a[b]):
            np.testing.assert_array_equal(ra["compact"][b, :, s * cs:(s + 1) * cs],
                                          r["compact"][b, :, c * cs:(c + 1) * cs])
        mask = np.zeros(V, bool)
        for c in sel_a[b]:
            mask[c * cs:(c + 1) * cs] = True
        assert np.all(np.isneginf(ra["dense"][b][:, ~mask]))
    with pytest.raises(ValueError):
        oracle.head(h, W, np.array([[4, 1, 7], [0, 4, 11]], np.int32), cs)


def test_head_one_hot_rows_pick_columns_of_W():
    """With h[b, k] the unit vector e_j, the logit of token v is W[v, j]
    exactly (DynaSpec summary, "Model architecture" item 4: logits over the
    selected clusters only).  W holds small integers that encode (v, j), so
    the shortlist layout (entry s, offset t -> token c_s * cs + t), the column
    read, the magnitude sum and the dense scatter are all read off exactly."""
    import torch
    B, K, d, V, cs = 2, 3, 16, 40, 5
    j_of = np.array([[0, 7, 15], [3, 3, 9]])
    h = torch.zeros(B, K, d)
    for b in range(B):
        for k in range(K):
            h[b, k, j_of[b, k]] = 1.0
    Wf = (np.arange(V)[:, None] + 1) + 64.0 * (np.arange(d)[None, :] % 3)   # integers up to 168
    W = torch.from_numpy(Wf).to(torch.bfloat16)
    assert np.array_equal(W.double().numpy(), Wf)                           # exact in bf16
    sel = np.array([[1, 4, 6], [0, 2, 7]], np.int32)
    r = oracle.head(h.to(torch.bfloat16), W, sel, cs, dense=True)
    for b in range(B):
        for k in range(K):
            off = np.ones(V, bool)
            for s, c in enumerate(sel[b]):
                for t in range(cs):
                    tok = c * cs + t
                    want = Wf[tok, j_of[b, k]]
                    assert r["compact"][b, k, s * cs + t] == want
                    assert r["absdot"][b, k, s * cs + t] == abs(want)
                    assert r["dense"][b, k, tok] == want
                    off[tok] = False
            assert np.all(np.isneginf(r["dense"][b, k, off]))


def test_head_absdot_is_the_sum_of_absolute_products():
    """absdot, the magnitude the head's tolerance is relative to, is
    sum_j |h_j W_vj|.  With h = +-1 and W rows (v + 1) * a_j * (-1)^j,
    a_j = 2^j, the logit cancels to -85 (v + 1) times h's sign while absdot
    is 255 (v + 1)."""
    import torch
    B, K, d, V, cs = 1, 2, 8, 6, 3
    h = torch.ones(B, K, d)
    h[0, 1] = -1.0
    a = 2.0 ** np.arange(d)
    Wf = np.stack([(v + 1) * a * (-1.0) ** np.arange(d) for v in range(V)])
    W = torch.from_numpy(Wf).to(torch.bfloat16)
    assert np.array_equal(W.double().numpy(), Wf)
    r = oracle.head(h.to(torch.bfloat16), W, np.array([[0, 1]], np.int32), cs)
    v = np.arange(V)
    np.testing.assert_array_equal(r["compact"][0, 0], -85.0 * (v + 1))
    np.testing.assert_array_equal(r["compact"][0, 1], 85.0 * (v + 1))
    np.testing.assert_array_equal(r["absdot"][0, 0], 255.0 * (v + 1))
    np.testing.assert_array_equal(r["absdot"][0, 1], 255.0 * (v + 1))


# --------------------------------------------------------------------------------------
# Boundary conventions: strict accept comparison and the inverse-CDF boundary.
# --------------------------------------------------------------------------------------

def test_accept_comparison_is_strict():
    """u < min(1, ratio): a draft token the target gives probability 0 is
    rejected even at u = 0 (Speculative Decoding lesson, "Step 1")."""
    V = 6
    x = np.zeros((1, 2, V), np.float32)
    x[0, 0, 2] = -np.inf
    y = np.zeros((1, 1, V), np.float32)
    uni = np.zeros((1, 2, 2), np.float32)
    r = oracle.verify(x, y, np.array([[2]], np.int32), uni, 1.0)
    assert r["accepted_len"][0] == 0
    assert r["p_target"][0, 0] == 0.0


def test_inverse_cdf_skips_zero_weight_tokens():
    """With sample uniform 0 the chosen token is the first one with positive weight."""
    V = 6
    x = np.zeros((1, 2, V), np.float32)
    x[0, :, :3] = -np.inf                      # tokens 0..2 have P_t = 0
    y = np.zeros((1, 1, V), np.float32)
    y[0, 0, 4] = 5.0                            # the draft over-weights token 4
    uni = np.zeros((1, 2, 2), np.float32)
    uni[0, 0, 0] = 0.999                        # reject the draft
    r = oracle.verify(x, y, np.array([[4]], np.int32), uni, 1.0)
    assert r["accepted_len"][0] == 0
    assert r["out_tokens"][0, 0] == 3


# --------------------------------------------------------------------------------------
# Acceptance probability beta = sum_v min(P_t, P_d) of one position.
# --------------------------------------------------------------------------------------

def test_overlap_worked_example_is_the_printed_acceptance():
    """RuneLab explainer, single-position figure: the two rows are accepted
    67 % of the time."""
    g, pt, pd = _worked()
    beta = oracle.overlap(_logits_from_probs(pt)[None], _logits_from_probs(pd)[None], 1.0)
    assert abs(float(beta[0]) - g["printed"]["accept_percent"] / 100) < 1e-6


def test_overlap_is_one_minus_total_variation():
    """sum_v min(p, q) = 1 - (1/2) sum_v |p - q| for two distributions; both
    sides of the identity from an fp64 softmax of the same float32 logits
    (scipy), at two temperatures and with a -inf entry in the draft."""
    rng = np.random.default_rng(7)
    V = 97
    t = rng.normal(0.0, 2.0, (6, V)).astype(np.float32)
    d = (t + rng.normal(0.0, 0.8, (6, V))).astype(np.float32)
    d[2, 5] = -np.inf
    for T in (1.0, 0.6):
        beta = oracle.overlap(t, d, T)
        p = scipy.special.softmax(t.astype(np.float64) / np.float64(np.float32(T)), axis=-1)
        q = scipy.special.softmax(d.astype(np.float64) / np.float64(np.float32(T)), axis=-1)
        want = 1.0 - 0.5 * np.abs(p - q).sum(-1)
        np.testing.assert_allclose(beta, want, rtol=0, atol=1e-12)
        assert np.all((beta > 0) & (beta < 1))


def test_overlap_limits():
    """Identical rows overlap fully; rows with disjoint supports not at all;
    a row with no finite logit has no beta."""
    x = np.array([[0.3, -1.0, 2.0, -np.inf]], np.float32)
    assert abs(float(oracle.overlap(x, x, 1.3)[0]) - 1.0) < 1e-12
    a = np.array([[0.0, 1.0, -np.inf, -np.inf]], np.float32)
    b = np.array([[-np.inf, -np.inf, 0.5, 2.0]], np.float32)
    assert float(oracle.overlap(a, b, 1.0)[0]) == 0.0
    assert np.isnan(oracle.overlap(np.full((1, 4), -np.inf, np.float32), a, 1.0)[0])
