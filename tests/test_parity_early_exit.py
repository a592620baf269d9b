"""GPU early-exit verify schedule (mode "sample_early_exit").

Position i is processed only for sequences that accepted every earlier
position, so rows after a sequence's first rejection are never read (they
cannot change its output: Speculative Decoding lesson, nextadmin.net, "Core
algorithm" step 5).  Checked here:
  - accepted_len and out_tokens bit-identical to the full SAMPLE schedule, and
    the same comparison with the fp64 oracle as every other SAMPLE test;
  - P_t(d_i), P_d(d_i) bit-identical up to the first rejection, NaN after;
  - outputs do not change when every row after the first rejection (and the
    draft tokens there, within range) is replaced: the rows are not read;
  - faults: out-of-range draft tokens anywhere and non-finite rows up to the
    first rejection mark the sequence as in the full schedule; a non-finite row
    after it is never seen.
"""
import numpy as np
import pytest
import torch

from tests.parity_util import PROB_RTOL, compare, run_gpu, run_oracle
from workloads import verify_case, workload_case

pytestmark = pytest.mark.gpu

EE = "sample_early_exit"


def _case(B, K, V, dtype, T=1.0, std=3.0, zipf=1.1, sigma=0.7, key=(7,)):
    return verify_case(B, K, V, dtype, target_std=std, zipf_s=zipf, sigma=sigma, temperature=T, key=key)


def check_early_exit(case, vs_oracle=True):
    full = run_gpu(case, "sample")
    ee = run_gpu(case, EE)
    np.testing.assert_array_equal(ee[0], full[0])
    np.testing.assert_array_equal(ee[1], full[1])
    n, K = ee[0], case.K
    for k in (2, 3):
        # every reported probability is the full schedule's, bit for bit
        rep_mask = ~np.isnan(ee[k])
        np.testing.assert_array_equal(ee[k][rep_mask], full[k][rep_mask])
        for b in range(case.B):
            if n[b] < 0:
                continue      # a fault found at position i (or at the bonus row) stops the evaluation there
            upto = min(int(n[b]), K - 1) + 1
            assert not np.any(np.isnan(ee[k][b, :upto]))
            assert np.all(np.isnan(ee[k][b, upto:]))
    if vs_oracle:
        orc = dict(run_oracle(case, gpu=ee))
        for key, k in (("p_target", 2), ("p_draft", 3)):
            q = np.array(orc[key], dtype=np.float64, copy=True)
            q[np.isnan(ee[k])] = np.nan
            orc[key] = q
        rep = compare(ee[0], ee[1], orc, K, gpu_pt=ee[2], gpu_pd=ee[3])
        assert not rep.failures, rep.failures[:5]
        assert rep.prob_max_rel <= PROB_RTOL
    return ee


@pytest.mark.parametrize("B,K,V,dtype", [
    (6, 3, 4096, "bf16"),
    (6, 3, 10000, "f32"),      # ragged last tile, fp32 logits
    (6, 3, 5003, "bf16"),      # rows that are not 16-byte multiples
    (5, 0, 9000, "bf16"),      # no draft positions: bonus token only
    (4, 20, 3000, "bf16"),     # K > 16: the full schedule's generic combine path
    (3, 4, 300000, "bf16"),    # more than 64 statistics tiles per row
    (512, 2, 20000, "bf16"),   # enough phase blocks for two tiles per wave; 5 tiles per row (odd)
    (3, 64, 3000, "bf16"),     # K = SPEC_MAX_K: 66 launches
])
def test_early_exit_shapes(B, K, V, dtype):
    print(f"case B={B} K={K} V={V} {dtype}", flush=True)
    check_early_exit(_case(B, K, V, dtype, key=(31, V, K)))


@pytest.mark.parametrize("sigma,T", [(0.0, 1.0), (4.0, 1.0), (0.7, 0.37), (0.7, 2.5), (0.7, 0.02), (0.7, 50.0)])
def test_early_exit_acceptance_regimes(sigma, T):
    """Identical draft (all accepted), low acceptance, and two temperatures."""
    print(f"case sigma={sigma} T={T}", flush=True)
    c = _case(16, 6, 20000, "bf16", T=T, sigma=sigma, key=(32, int(sigma * 10), int(T * 100)))
    out = check_early_exit(c)
    if sigma == 0.0:
        assert np.all(out[0] == 6)


@pytest.mark.parametrize("T", [1e-7, 1e-20])
def test_early_exit_tiny_temperatures(T):
    """Wide exponent references (|m * s| >= 2^26) in the phase and sampling kernels."""
    print(f"case early exit T={T}", flush=True)
    out = check_early_exit(_case(8, 4, 12345 * 8, "bf16", T=T, key=(39, int(-np.log10(T)))))
    assert np.all(out[0] >= 0)


def test_early_exit_large_logit_magnitudes():
    """fp32 logits shifted by +3000: large exponent reference offsets in the
    per-position statistics and decisions."""
    from workloads import VerifyCase
    print("case early exit, logits shifted by 3000", flush=True)
    c = _case(8, 4, 20000, "f32", key=(37,))
    check_early_exit(VerifyCase(c.target + 3000.0, c.draft + 3000.0, c.draft_tokens, c.uniforms, c.temperature,
                                c.dtype))


def test_early_exit_shortlist_rows_and_boundary_uniforms():
    c = _case(8, 4, 16384, "bf16", key=(33,))
    mask = torch.ones(16384, dtype=torch.bool)
    mask[::3] = False
    c.draft[..., mask] = float("-inf")
    keep = torch.nonzero(~mask).flatten()
    g = torch.Generator().manual_seed(6)
    c.draft_tokens = keep[torch.randint(0, len(keep), (8, 4), generator=g)].to(torch.int32)
    c.uniforms[:2] = 0.0
    c.uniforms[2:4] = 1.0 - 2.0 ** -24
    check_early_exit(c)


def test_rows_after_first_rejection_are_not_read():
    c = _case(24, 6, 12000, "bf16", sigma=1.5, key=(34,))
    first = run_gpu(c, EE)
    n = first[0]
    assert np.any((n >= 0) & (n < 5))
    g = torch.Generator().manual_seed(35)
    c2 = _case(24, 6, 12000, "bf16", sigma=1.5, key=(34,))
    for b in range(c.B):
        if n[b] < 0 or n[b] >= c.K:
            continue
        j = int(n[b]) + 1                     # rows j.. of the target (incl. the bonus row) and draft
        c2.target[b, j:] = (torch.randn(c.K + 1 - j, c.V, generator=g) * 5).to(c2.target.dtype)
        c2.draft[b, j:] = (torch.randn(c.K - j, c.V, generator=g) * 5).to(c2.draft.dtype)
        c2.draft_tokens[b, j:] = torch.randint(0, c.V, (c.K - j,), generator=g, dtype=torch.int32)
        c2.uniforms[b, j:] = torch.rand(c.K + 1 - j, 2, generator=g)
    second = run_gpu(c2, EE)
    np.testing.assert_array_equal(first[0], second[0])
    np.testing.assert_array_equal(first[1], second[1])
    # the full schedule reads those rows but its outputs cannot depend on them either
    full2 = run_gpu(c2, "sample")
    np.testing.assert_array_equal(full2[0], second[0])
    np.testing.assert_array_equal(full2[1], second[1])


def test_early_exit_faults():
    c = _case(8, 4, 8192, "bf16", sigma=0.0, key=(36,))   # identical draft: every position accepted
    c.draft_tokens[1, 3] = 8192          # out of range at the last position
    c.draft_tokens[2, 0] = -5
    c.target[3, 0, :] = float("-inf")    # row 0 has no finite maximum
    c.draft[4, 2, :] = float("-inf")     # read: every earlier position is accepted
    c.target[5, 4, :] = float("-inf")    # bonus row, sampled because all drafts are accepted
    out = check_early_exit(c)
    for b in (1, 2, 3, 4, 5):
        assert out[0][b] == -1 and np.all(out[1][b] == -1)
    assert np.all(out[0][[0, 6, 7]] == 4)


def test_non_finite_row_after_rejection_is_not_seen():
    """The one documented difference from the full schedule."""
    c = _case(8, 5, 8192, "bf16", sigma=4.0, key=(37,))
    ee = run_gpu(c, EE)
    b = int(np.nonzero((ee[0] >= 0) & (ee[0] < 3))[0][0])
    n = int(ee[0][b])
    c.target[b, n + 1, :] = float("-inf")
    full = run_gpu(c, "sample")
    ee2 = run_gpu(c, EE)
    assert full[0][b] == -1                       # the full schedule reads the row
    assert ee2[0][b] == n                         # early exit never does
    np.testing.assert_array_equal(ee2[1][b], ee[1][b])


@pytest.mark.parametrize("trial", [0, 1, 2])
def test_early_exit_b256_k7_v262144(trial):
    """The benchmark batch: bit-identical to the full schedule, and against the oracle."""
    c = workload_case("b256_k7_v262144_bf16", trial=trial, device=torch.device("cuda", 0))
    c.target, c.draft = c.target.cpu(), c.draft.cpu()
    c.draft_tokens, c.uniforms = c.draft_tokens.cpu(), c.uniforms.cpu()
    out = check_early_exit(c)
    print(f"trial {trial}: mean tokens {np.mean(out[0] + 1):.3f}", flush=True)


def test_early_exit_workspace_reuse_after_full_acceptance():
    """A call where every sequence accepts every position leaves every
    continue flag set; a later call on the same workspace whose sequences
    reject early must not read those flags (regression test)."""
    import speculative_sampling_verification_vocab_amd as sv
    dev = torch.device("cuda", 0)
    ws = sv.Workspace(dev)
    accept_all = _case(12, 6, 9000, "bf16", sigma=0.0, key=(38,))
    reject_early = _case(12, 6, 9000, "bf16", sigma=4.0, key=(39,))
    for c in (accept_all, reject_early, accept_all, reject_early):
        full = run_gpu(c, "sample", workspace=ws)
        ee = run_gpu(c, EE, workspace=ws)
        np.testing.assert_array_equal(ee[0], full[0])
        np.testing.assert_array_equal(ee[1], full[1])
    assert np.all(run_gpu(accept_all, EE, workspace=ws)[0] == 6)
