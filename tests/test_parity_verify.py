"""GPU verify (SAMPLE and GREEDY) against the fp64 oracle, element by element.

Sizes here are small enough for the oracle to finish in seconds while still
spanning several tiles and a ragged tail; the full workloads are in
test_parity_workloads.py.
"""
import numpy as np
import pytest
import torch

from tests.parity_util import check_case, compare, run_gpu, run_oracle
from workloads import VerifyCase, verify_case, verify_uniforms

pytestmark = pytest.mark.gpu


def _case(B, K, V, dtype, T=1.0, std=3.0, zipf=1.1, sigma=0.7, key=(7,)):
    return verify_case(B, K, V, dtype, target_std=std, zipf_s=zipf, sigma=sigma, temperature=T, key=key)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [4096, 10000, 20000, 5003, 33, 1])
def test_sample_shapes(dtype, V):
    """Several tiles, a ragged last tile (10000, 20000), rows that are not
    16-byte multiples (5003, 33) and a one-token vocabulary."""
    print(f"case dtype={dtype} V={V}", flush=True)
    c = _case(6, 3, V, dtype, key=(11, V))
    rep, out, orc = check_case(c)
    assert rep.excused <= 1


@pytest.mark.parametrize("T", [0.02, 0.37, 0.8, 2.5, 50.0])
def test_sample_temperatures(T):
    print(f"case T={T}", flush=True)
    c = _case(8, 4, 12345 * 8, "bf16", T=T, key=(12, int(T * 100)))
    check_case(c)


@pytest.mark.parametrize("T", [1e-7, 1e-20, 1e-30])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sample_tiny_temperatures(T, dtype):
    """Temperatures at which |max logit| * log2(e) / T reaches 2^26 and far
    beyond (at 1e-7 only the tiles with the larger maxima do): there the
    exponent references are wide, and each tile whose reference is wide takes
    RN((x - m) * s) instead of the one-FMA form, whose remainder 2^lo would
    leave the fp32 range."""
    print(f"case T={T} {dtype}", flush=True)
    c = _case(8, 4, 12345 * 8, dtype, T=T, key=(19, int(-np.log10(T))))
    rep, out, orc = check_case(c)
    assert np.all(out[0] >= 0)


def test_sample_large_logits_at_small_temperature():
    """Logits shifted by +3000 at T = 1e-5: |m * s| is about 4.3e8, a wide
    reference in every tile."""
    c = _case(8, 4, 20000, "f32", T=1e-5, key=(20,))
    c = VerifyCase(c.target + 3000.0, c.draft + 3000.0, c.draft_tokens, c.uniforms, c.temperature, c.dtype)
    rep, out, orc = check_case(c)
    assert np.all(out[0] >= 0)


@pytest.mark.parametrize("scale", [1e10, 1e37])
def test_sample_scaled_logits(scale):
    """fp32 logits scaled by 1e10 and 1e37: at T = 1 every reference is wide
    (a near-greedy row); at T = scale the softmax is that of the unscaled
    logits, computed from products near the top of the fp32 range."""
    c = _case(8, 4, 20000, "f32", key=(21,))
    for T in (1.0, float(np.float32(scale))):
        print(f"case logits x {scale}, T={T}", flush=True)
        check_case(VerifyCase(c.target * scale, c.draft * scale, c.draft_tokens, c.uniforms, T, c.dtype))


def test_sample_huge_temperature():
    """T = 1e38: s = log2(e)/T is 1.4e-38, next to the smallest normal fp32;
    every exponent's argument is within rounding of 0, and both distributions
    are uniform."""
    rep, out, orc = check_case(_case(8, 4, 20000, "bf16", T=1e38, key=(22,)))
    assert np.all(out[0] == 4)


@pytest.mark.parametrize("mode", ["sample", "greedy"])
def test_very_large_batch_small_vocabulary(mode):
    """B = 100,000 sequences of 33-token rows: grids of hundreds of thousands
    of blocks and one decision block per sequence."""
    c = _case(100000, 4, 33, "bf16", std=2.0, zipf=0.0, key=(23,))
    check_case(c, mode)


def test_sample_large_logit_magnitudes():
    """Logits shifted by +3000 and -3000 (fp32): the softmax does not change,
    but x*s is large, so the exponents' reference offsets (RN(m*s) and its
    exact remainder) are large and must be taken out exactly."""
    for shift in (3000.0, -3000.0):
        print(f"case logits shifted by {shift}", flush=True)
        c = _case(8, 4, 20000, "f32", key=(18, 0 if shift > 0 else 1))
        c = VerifyCase(c.target + shift, c.draft + shift, c.draft_tokens, c.uniforms, c.temperature, c.dtype)
        check_case(c)


def test_sample_k0_only_bonus():
    c = _case(5, 0, 9000, "bf16", key=(13,))
    rep, out, orc = check_case(c)
    assert np.all(out[0] == 0)


def test_sample_identical_draft_accepts_all():
    c = _case(8, 5, 30000, "bf16", sigma=0.0, key=(14,))
    assert torch.equal(c.draft, c.target[:, :5])
    rep, out, orc = check_case(c)
    assert np.all(out[0] == 5)


def test_sample_low_acceptance():
    c = _case(16, 6, 20000, "bf16", sigma=4.0, key=(15,))
    rep, out, orc = check_case(c)
    assert np.mean(out[0]) < 2


def test_faulty_sequences():
    c = _case(6, 3, 8192, "bf16", key=(16,))
    c.draft_tokens[1, 2] = 8192          # out of range
    c.draft_tokens[2, 0] = -5
    c.target[3, 1, :] = float("-inf")    # a row without a finite maximum
    c.draft[4, 2, :] = float("-inf")
    rep, out, orc = check_case(c)
    for b in (1, 2, 3, 4):
        assert out[0][b] == -1 and np.all(out[1][b] == -1)
    assert out[0][0] >= 0 and out[0][5] >= 0


def test_nan_logits_mark_the_sequence_faulty():
    """A NaN in a row the rule reads leaves that row without a finite
    normaliser: the sequence is faulty on both sides, as for a row without a
    finite maximum.  bf16 and fp32; a NaN in target and in draft rows, and a
    NaN in the bonus row (read only when every draft is accepted)."""
    for dtype in ("bf16", "f32"):
        print(f"case NaN logits {dtype}", flush=True)
        c = _case(6, 3, 8192, dtype, sigma=0.05, key=(19,))
        c.target[1, 0, 17] = float("nan")
        c.draft[2, 2, 8000] = float("nan")
        c.target[3, 3, 5] = float("nan")     # bonus row
        rep, out, orc = check_case(c)
        for b in (1, 2):
            assert out[0][b] == -1 and np.all(out[1][b] == -1)
        # greedy ignores a single NaN (it is never the maximum) on both sides
        g = VerifyCase(c.target, None, c.draft_tokens, c.uniforms, 0.0, c.dtype)
        check_case(g, mode="greedy")


def test_small_residual_mass_bf16():
    """A draft within a few bf16 ulps of the target (sigma 0.02 and 0.005)
    and accept uniforms of 1 - 2^-24, so nearly every position with a ratio
    below 1 is rejected and sampled from a residual of small mass."""
    for sigma in (0.02, 0.005):
        print(f"case small residual mass sigma={sigma}", flush=True)
        for seed in range(3):
            c = _case(64, 4, 32000, "bf16", sigma=sigma, key=(22, seed, int(sigma * 1000)))
            c.uniforms[:, :, 0] = 1.0 - 2.0 ** -24
            rep, out, orc = check_case(c)
            assert np.sum(orc["accepted_len"] < c.K) > 40   # the residual path is exercised


def test_constant_rows():
    """Every logit of every row equal: P_t = P_d = 1/V, every draft accepted
    (ratio exactly 1), and the bonus token is the inverse CDF of a uniform
    distribution, a boundary case for every u on the 1/V grid."""
    for dtype, V in (("bf16", 1000), ("f32", 12288)):
        print(f"case constant rows {dtype} V={V}", flush=True)
        c = _case(8, 3, V, dtype, key=(20,))
        c = VerifyCase(torch.full_like(c.target, 0.75), torch.full_like(c.draft, 0.75), c.draft_tokens,
                       c.uniforms, c.temperature, c.dtype)
        rep, out, orc = check_case(c)
        assert np.all(out[0] == 3)


def test_near_one_hot_rows():
    """fp32 logits scaled by 1e4: every row is one-hot to within fp64, so
    almost every probability underflows to exactly zero on both sides."""
    print("case near one-hot rows", flush=True)
    c = _case(8, 4, 9000, "f32", key=(21,))
    c = VerifyCase(c.target * 1e4, c.draft * 1e4, c.draft_tokens, c.uniforms, c.temperature, c.dtype)
    check_case(c)


def test_faulty_bonus_row_only_matters_when_sampled():
    c = _case(4, 2, 4096, "bf16", sigma=0.0, key=(17,))
    c.target[0, 2, :] = float("-inf")    # bonus row of sequence 0; all drafts accepted
    rep, out, orc = check_case(c)
    assert out[0][0] == -1 and orc["accepted_len"][0] == -1


def test_shortlist_draft_rows_with_neg_inf():
    """Draft rows that are -inf off a shortlist (P_d = 0 there)."""
    c = _case(8, 4, 16384, "bf16", key=(18,))
    mask = torch.ones(16384, dtype=torch.bool)
    mask[::3] = False
    c.draft[..., mask] = float("-inf")
    # redraw draft tokens inside the shortlist
    keep = torch.nonzero(~mask).flatten()
    g = torch.Generator().manual_seed(5)
    c.draft_tokens = keep[torch.randint(0, len(keep), (8, 4), generator=g)].to(torch.int32)
    check_case(c)


def test_zero_uniforms_and_near_one():
    c = _case(8, 3, 8192, "bf16", key=(19,))
    c.uniforms[:4] = 0.0
    c.uniforms[4:] = 1.0 - 2.0 ** -24
    check_case(c)


@pytest.mark.parametrize("sigma", [0.0, 0.3])
def test_sample_max_k(sigma):
    """K = SPEC_MAX_K = 64 draft positions: every accept decision, the first
    rejection or the bonus row at position 64 (sigma = 0: identical rows)."""
    print(f"case K=64 sigma={sigma}", flush=True)
    c = _case(3, 64, 3000, "bf16", sigma=sigma, key=(23, int(sigma * 10)))
    rep, out, orc = check_case(c)
    if sigma == 0.0:
        assert np.all(out[0] == 64)


def test_sample_decision_launch_and_prologue_agree():
    """B=1024, K=9, V=16384 takes the separate decision launch (two sampling
    tiles per wave, 18 rows per sequence); the same sequences in batches of 64
    take the decisions in the sampling prologue.  Outputs are bit-identical
    and match the oracle."""
    import speculative_sampling_verification_vocab_amd as sv
    from speculative_sampling_verification_vocab_amd import _native
    lib = _native.load()
    assert lib.spec_verify_launch_count(1024, 9, 16384, 1, 0) == 4
    assert lib.spec_verify_launch_count(64, 9, 16384, 1, 0) == 2    # small grid: fused pick
    c = _case(1024, 9, 16384, "bf16", key=(25,))
    rep, out, orc = check_case(c)
    for s0 in range(0, 1024, 64):
        part = VerifyCase(c.target[s0:s0 + 64], c.draft[s0:s0 + 64], c.draft_tokens[s0:s0 + 64],
                          c.uniforms[s0:s0 + 64], c.temperature, c.dtype)
        o = run_gpu(part)
        for k in range(4):
            np.testing.assert_array_equal(o[k], out[k][s0:s0 + 64])


@pytest.mark.parametrize("V,dtype", [(131072, "bf16"), (131073, "bf16"), (65536, "f32"), (65537, "f32")])
def test_pick_choice_at_64_sampling_tiles(V, dtype):
    """Rows of exactly 64 sampling tiles (2048 bf16 or 1024 fp32 ids each)
    take the pick's one-wave tile choice, rows of 65 the block-wide one; both
    in the sampling launch's last block (B=8) and in the pick launch (B=96),
    against the oracle, with rejections and bonus tokens in the mix."""
    import speculative_sampling_verification_vocab_amd as sv
    for B in (8, 96):
        fused = sv.spec_verify_launch_count(B, 3, V, torch.bfloat16 if dtype == "bf16" else torch.float32,
                                            "sample") == 2
        print(f"case V={V} dtype={dtype} B={B} fused pick={fused}", flush=True)
        assert fused == (B == 8)
        c = _case(B, 3, V, dtype, sigma=0.3, key=(26, V, B))
        rep, out, orc = check_case(c)
        assert np.any(out[0] == 3) and np.any(out[0] < 3)


@pytest.mark.parametrize("V,dtype", [(600000, "bf16"), (300000, "f32")])
def test_sample_long_rows(V, dtype):
    """147 statistics tiles and 293 sampling tiles per row: the combine over
    more than 64 tiles and the pick over more tiles than one block's threads."""
    print(f"case V={V} dtype={dtype}", flush=True)
    c = _case(2, 3, V, dtype, key=(24, V))
    check_case(c)


def test_greedy_max_k_and_long_rows():
    for B, K, V in ((3, 64, 3000), (2, 3, 600000)):
        print(f"case greedy B={B} K={K} V={V}", flush=True)
        g = torch.Generator().manual_seed(K + V)
        x = torch.randn(B, K + 1, V, generator=g).to(torch.bfloat16)
        tok = torch.argmax(x[:, :K].float(), dim=-1)
        tok[:, K // 2] = (tok[:, K // 2] + 1) % V    # a mismatch half way
        c = VerifyCase(x, None, tok.to(torch.int32), verify_uniforms(B, K, (2,)), 0.0, "bf16")
        rep, out, orc = check_case(c, mode="greedy")
        assert np.all(out[0] == K // 2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [50257, 4096, 7])
def test_greedy(dtype, V):
    g = torch.Generator().manual_seed(V)
    B, K = 16, 5
    # coarse values: ties are common and the lowest id must win
    x = torch.randint(-20, 20, (B, K + 1, V), generator=g).to(torch.float32) * 0.25
    x = x.to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    a = torch.argmax(x.float(), dim=-1)
    tok = a[:, :K].clone()
    flip = torch.rand(B, K, generator=g) < 0.2
    tok[flip] = torch.randint(0, V, (int(flip.sum()),), generator=g)
    c = VerifyCase(x, None, tok.to(torch.int32), verify_uniforms(B, K, (1,)), 0.0, dtype)
    check_case(c, mode="greedy")


def test_greedy_faulty():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(4, 3, 3000, generator=g).to(torch.bfloat16)
    tok = torch.argmax(x[:, :2].float(), -1).to(torch.int32)
    tok[1, 1] = 3000
    x[2, 2] = float("-inf")
    c = VerifyCase(x, None, tok, verify_uniforms(4, 2, (1,)), 0.0, "bf16")
    rep, out, orc = check_case(c, mode="greedy")
    assert out[0][1] == -1 and out[0][2] == -1


def test_repeat_calls_are_identical():
    """Bit-identical reruns (no float atomics; counters reset by the library)."""
    c = _case(32, 5, 50000, "bf16", key=(20,))
    a = run_gpu(c)
    b = run_gpu(c)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_shape_change_reuses_workspace():
    """A smaller call after a larger one on the same default workspace."""
    c1 = _case(16, 6, 40000, "bf16", key=(21,))
    c2 = _case(3, 2, 1000, "bf16", key=(22,))
    check_case(c1)
    check_case(c2)
    check_case(c1)


def test_chi_square_on_gpu():
    """Emitted tokens follow P_t on V = 8 over 10^6 sequences (GPU output)."""
    import scipy.special
    import scipy.stats
    import speculative_sampling_verification_vocab_amd as sv
    rng = np.random.default_rng(42)
    V, K, B = 8, 4, 1_000_000
    xt = (rng.standard_normal((K + 1, V)) * 2).astype(np.float32)
    xd = (xt[:K] + rng.standard_normal((K, V)) * 1.0).astype(np.float32)
    pt = scipy.special.softmax(xt.astype(np.float64), axis=-1)
    pd = scipy.special.softmax(xd.astype(np.float64), axis=-1)
    tok = np.stack([rng.choice(V, size=B, p=pd[i]) for i in range(K)], axis=1).astype(np.int32)
    uni = rng.random((B, K + 1, 2), dtype=np.float32)
    dev = torch.device("cuda", 0)
    tgt = torch.from_numpy(xt).to(dev).expand(B, K + 1, V).contiguous()
    dr = torch.from_numpy(xd).to(dev).expand(B, K, V).contiguous()
    n, out = sv.spec_verify(tgt, dr, torch.from_numpy(tok).to(dev), torch.from_numpy(uni).to(dev), 1.0)
    n, out = n.cpu().numpy(), out.cpu().numpy()
    for i in range(K + 1):
        sel = n >= i
        cnt = np.bincount(out[sel, i], minlength=V)
        p = scipy.stats.chisquare(cnt, pt[i] * cnt.sum()).pvalue
        assert p > 1e-3 / (K + 1), (i, p)
        assert 0.5 * np.abs(cnt / cnt.sum() - pt[i]).sum() < 0.01


@pytest.mark.parametrize("mode", ["sample", "greedy", "sample_early_exit"])
def test_empty_batch(mode):
    """B = 0 launches nothing and returns empty outputs; the next call on the
    same stream is unaffected."""
    import speculative_sampling_verification_vocab_amd as sv
    print(f"case empty batch mode={mode}", flush=True)
    dev = torch.device("cuda", 0)
    t = torch.empty((0, 4, 100), dtype=torch.bfloat16, device=dev)
    d = torch.empty((0, 3, 100), dtype=torch.bfloat16, device=dev)
    tok = torch.empty((0, 3), dtype=torch.int32, device=dev)
    uni = torch.empty((0, 4, 2), dtype=torch.float32, device=dev)
    assert sv.spec_verify_launch_count(0, 3, 100, torch.bfloat16, mode) == 0
    acc, out = sv.spec_verify(t, d, tok, uni, 1.0, mode)
    torch.cuda.synchronize()
    assert acc.shape == (0,) and out.shape == (0, 4)
    c = _case(3, 3, 5000, "bf16", key=(26,))
    check_case(c)


def test_offsets_past_4_gib():
    """A 4.25 GiB target tensor (B=17, K=1, V=2^26 bf16): the last sequence's
    rows start at byte 2^32 of the target and 2^31 of the draft, so addresses
    beyond 32 bits are exercised.  That sequence is checked against the oracle
    in SAMPLE and GREEDY; SAMPLE_EARLY_EXIT gives SAMPLE's outputs."""
    import speculative_sampling_verification_vocab_amd as sv
    from tests.parity_util import compare
    print("case offsets past 4 GiB: B=17 K=1 V=2^26 bf16", flush=True)
    dev = torch.device("cuda", 0)
    B, K, V = 17, 1, 1 << 26
    c = verify_case(B, K, V, "bf16", target_std=3.0, zipf_s=1.1, sigma=0.7, temperature=1.0, key=(27,),
                    device=dev)
    assert c.target.numel() * 2 > (1 << 32) and c.draft.numel() * 2 > (1 << 31)
    outs = {}
    for m in ("sample", "sample_early_exit", "greedy"):
        res = sv.spec_verify(c.target, c.draft, c.draft_tokens, c.uniforms,
                             c.temperature if m != "greedy" else 0.0, m, return_probs=True)
        torch.cuda.synchronize()
        outs[m] = [r.cpu().numpy() for r in res]
    np.testing.assert_array_equal(outs["sample_early_exit"][0], outs["sample"][0])
    np.testing.assert_array_equal(outs["sample_early_exit"][1], outs["sample"][1])
    s = slice(B - 1, B)
    last = VerifyCase(c.target[s].cpu(), c.draft[s].cpu(), c.draft_tokens[s].cpu(), c.uniforms[s].cpu(),
                      c.temperature, c.dtype)
    del c
    for m in ("sample", "greedy"):
        o = outs[m]
        greedy = m == "greedy"
        rep = compare(o[0][s], o[1][s], run_oracle(last, m, gpu=(o[0][s], o[1][s])), K, greedy=greedy,
                      gpu_pt=None if greedy else o[2][s], gpu_pd=None if greedy else o[3][s])
        assert not rep.failures, rep.failures
        assert rep.prob_max_rel < 1e-5


def test_largest_vocabulary():
    """V = 2^30, the largest vocabulary the library takes (B=1, K=2, bf16: 10
    GiB of logits).  Every logit is -inf except at a few ids spread over the
    row, including the last ones, so the rule's outcome depends only on those
    ids: the oracle runs on the rows compressed to them (same order, so the
    inverse CDF over token ids is the same) and its ids are mapped back.  The
    GPU reads the full rows in SAMPLE, SAMPLE_EARLY_EXIT and GREEDY."""
    import speculative_sampling_verification_vocab_amd as sv
    print("case largest vocabulary: B=1 K=2 V=2^30 bf16", flush=True)
    dev = torch.device("cuda", 0)
    B, K, V = 1, 2, 1 << 30
    ids = np.array([0, 5, 4095, 4096, (1 << 29) + 7, V - 4097, V - 9, V - 2, V - 1], np.int64)
    rng = np.random.default_rng(30)
    lt = rng.normal(0.0, 1.5, (K + 1, ids.size)).astype(np.float32)
    ld = (lt[:K] + rng.normal(0.0, 1.0, (K, ids.size))).astype(np.float32)
    ld[0, 1] = -np.inf   # a target token the draft never proposes
    lt[1, 6] = -np.inf   # a draft token the target rules out
    ld[0, 7] = lt[0, 7] + 3.0  # the draft overweights its first token
    lt_b = torch.from_numpy(lt).to(torch.bfloat16)
    ld_b = torch.from_numpy(ld).to(torch.bfloat16)
    tok_i = np.array([[7, 6]], np.int32)            # indices into ids: V - 2, then V - 9

    def prob(row, i):
        x = row.float().numpy().astype(np.float64)
        return float(np.exp(x[i] - x.max()) / np.exp(x - x.max()).sum())

    ratio = prob(lt_b[0], 7) / prob(ld_b[0], 7)
    assert ratio < 0.9
    for u_acc in (0.5 * ratio, 0.5 * (1.0 + ratio)):  # accept position 0, then reject it
        uni = np.full((B, K + 1, 2), 0.5, np.float32)
        uni[0, 0, 0] = u_acc
        uni[0, :, 1] = [0.61, 0.37, 0.83]
        target = torch.full((B, K + 1, V), float("-inf"), dtype=torch.bfloat16, device=dev)
        draft = torch.full((B, K, V), float("-inf"), dtype=torch.bfloat16, device=dev)
        idx = torch.from_numpy(ids).to(dev)
        target[0][:, idx] = lt_b.to(dev)
        draft[0][:, idx] = ld_b.to(dev)
        tok = torch.from_numpy(ids[tok_i].astype(np.int32)).to(dev)
        uni_d = torch.from_numpy(uni).to(dev)
        outs = {}
        for m in ("sample", "sample_early_exit", "greedy"):
            res = sv.spec_verify(target, draft, tok, uni_d, 1.0 if m != "greedy" else 0.0, m, return_probs=True)
            torch.cuda.synchronize()
            outs[m] = [r.cpu().numpy() for r in res]
        del target, draft
        torch.cuda.empty_cache()
        np.testing.assert_array_equal(outs["sample_early_exit"][0], outs["sample"][0])
        np.testing.assert_array_equal(outs["sample_early_exit"][1], outs["sample"][1])
        small = VerifyCase(lt_b[None], ld_b[None], torch.from_numpy(tok_i), torch.from_numpy(uni), 1.0, "bf16")
        for m in ("sample", "greedy"):
            o = outs[m]
            # GPU ids back to indices into `ids` (-1 stays -1)
            pos = {int(v): i for i, v in enumerate(ids)}
            o_idx = np.vectorize(lambda v: pos.get(int(v), -2) if v >= 0 else -1)(o[1]).astype(np.int32)
            assert np.all(o_idx >= -1), o[1]
            greedy = m == "greedy"
            rep = compare(o[0], o_idx, run_oracle(small, m, gpu=(o[0], o_idx)), K, greedy=greedy,
                          gpu_pt=None if greedy else o[2], gpu_pd=None if greedy else o[3])
            assert not rep.failures, (u_acc, m, rep.failures)
            assert rep.prob_max_rel < 1e-5
        assert (outs["sample"][0][0] == 0) == (u_acc > ratio)


def test_concurrent_streams_use_separate_default_workspaces():
    """Two calls on two streams at once, without explicit workspaces: each
    stream gets its own default scratch, so both match their single-stream
    results (and the oracle)."""
    import speculative_sampling_verification_vocab_amd as sv
    print("case concurrent streams: 2 x (B=64 K=4 V=40000 bf16)", flush=True)
    dev = torch.device("cuda", 0)
    cases = [verify_case(64, 4, 40000, "bf16", target_std=3.0, zipf_s=1.1, sigma=0.7, temperature=1.0,
                         key=(31, j), device=dev) for j in range(2)]
    ref = []
    for c in cases:
        res = sv.spec_verify(c.target, c.draft, c.draft_tokens, c.uniforms, c.temperature, "sample")
        ref.append([r.cpu().numpy() for r in res])
    streams = [torch.cuda.Stream(dev) for _ in cases]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream(dev))
    outs = []
    for rep in range(3):
        outs = []
        for c, s in zip(cases, streams):
            with torch.cuda.stream(s):
                outs.append(sv.spec_verify(c.target, c.draft, c.draft_tokens, c.uniforms, c.temperature, "sample"))
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            np.testing.assert_array_equal(o[0].cpu().numpy(), r[0])
            np.testing.assert_array_equal(o[1].cpu().numpy(), r[1])
    for c, r in zip(cases, ref):
        hc = VerifyCase(c.target.cpu(), c.draft.cpu(), c.draft_tokens.cpu(), c.uniforms.cpu(), c.temperature, c.dtype)
        rep = compare(r[0], r[1], run_oracle(hc, gpu=r), c.K)
        assert not rep.failures, rep.failures[:3]


@pytest.mark.parametrize("mode", ["sample", "greedy", "sample_early_exit"])
def test_verify_plan_matches_spec_verify(mode):
    """VerifyPlan (outputs and workspace allocated once, one C call per step)
    gives spec_verify's outputs on consecutive calls with different inputs."""
    import speculative_sampling_verification_vocab_amd as sv
    print(f"case verify plan {mode}: B=8 K=5 V=30000 bf16", flush=True)
    dev = torch.device("cuda", 0)
    plan = sv.VerifyPlan(8, 5, 30000, torch.bfloat16, mode, device=dev, return_probs=True)
    for j in range(3):
        c = verify_case(8, 5, 30000, "bf16", target_std=3.0, zipf_s=1.1, sigma=0.5, temperature=0.8,
                        key=(33, j), device=dev)
        greedy = mode == "greedy"
        got = [t.cpu().numpy() for t in plan(c.target, c.draft, c.draft_tokens, c.uniforms, c.temperature)]
        ref = sv.spec_verify(c.target, None if greedy else c.draft, c.draft_tokens, None if greedy else c.uniforms,
                             0.0 if greedy else c.temperature, mode, return_probs=True)
        for g, r in zip(got, ref):
            np.testing.assert_array_equal(g, r.cpu().numpy())
    with pytest.raises(ValueError):
        plan(c.target[:4], c.draft, c.draft_tokens, c.uniforms, c.temperature)
    with pytest.raises(ValueError):  # not on the plan's device
        plan(c.target.cpu(), c.draft, c.draft_tokens, c.uniforms, c.temperature)
