"""CPU checks of the seeded input generators and of bench.py's host-side logic.

The generators feed both the oracle and the GPU path, so what they promise is
pinned here against definitions that do not depend on them: torch's own
bf16 conversion (round to nearest even), the softmax a Gumbel-max draw must
follow (a chi-square test), the 24-bit grid of the uniforms, and keyed
determinism.  bench.py is checked for its one-GPU refusal and for using a
committed profile figure only while the kernel source still matches it.
"""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch
from scipy import stats

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from workloads import generators as G  # noqa: E402


def test_cases_are_keyed_and_deterministic():
    a = G.workload_case("b1_k4_v32000_f32")
    b = G.workload_case("b1_k4_v32000_f32")
    c = G.workload_case("b1_k4_v32000_f32", trial=1)
    assert torch.equal(a.target, b.target) and torch.equal(a.draft, b.draft)
    assert torch.equal(a.draft_tokens, b.draft_tokens) and torch.equal(a.uniforms, b.uniforms)
    assert not torch.equal(a.target, c.target)
    assert not torch.equal(a.uniforms, c.uniforms)
    assert a.target.shape == (1, 5, 32000) and a.draft.shape == (1, 4, 32000)
    assert a.draft_tokens.dtype == torch.int32 and a.uniforms.shape == (1, 5, 2)


def test_uniforms_lie_on_the_24_bit_grid():
    u = G.verify_uniforms(64, 7, (123, 4))
    assert u.dtype == torch.float32 and u.shape == (64, 8, 2)
    assert float(u.min()) >= 0.0 and float(u.max()) < 1.0
    k = u.double() * (1 << 24)
    assert torch.equal(k, torch.round(k))
    # both columns are used and differ
    assert not torch.equal(u[..., 0], u[..., 1])


def test_bf16_rounding_is_nearest_even():
    x = torch.randn(100000, generator=torch.Generator().manual_seed(7)) * 5
    # exact halfway cases between neighbouring bf16 values (8 significant bits)
    ties = torch.tensor([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 2 + 2.0 ** -7, 3 * 2.0 ** -9 + 2.0 ** -18])
    for v in (x, ties):
        got = G.round_to(v, "bf16")
        assert got.dtype == torch.bfloat16
        assert torch.equal(got.view(torch.int16), v.to(torch.bfloat16).view(torch.int16))
    got = G.round_to(ties[:2], "bf16").float()
    assert got.tolist() == [1.0, 1 + 2.0 ** -6]  # ties go to the even mantissa


def test_gumbel_max_draws_follow_the_tempered_softmax():
    y = torch.tensor([1.5, 0.0, -1.0, 2.2, 0.7, -3.0], dtype=torch.float32)
    T = 0.7
    n = 40000
    tok = G.gumbel_max_tokens(y.expand(n, -1).contiguous(), T, (99, 1), chunk_rows=4096)
    assert tok.dtype == torch.int32 and tok.shape == (n,)
    counts = np.bincount(tok.numpy(), minlength=6)
    p = torch.softmax(y.double() / T, 0).numpy()
    chi2, pval = stats.chisquare(counts, p * n)
    assert pval > 1e-4, (counts, p * n)
    # a different temperature gives a visibly different distribution
    tok2 = G.gumbel_max_tokens(y.expand(n, -1).contiguous(), 3.0, (99, 1), chunk_rows=4096)
    assert abs(float((tok2 == 3).float().mean()) - p[3]) > 0.1


def test_gumbel_max_on_a_single_finite_logit():
    y = torch.full((3, 10), float("-inf"))
    y[0, 4] = 0.0
    y[1, 9] = -5.0
    y[2, 0] = 3.0
    assert G.gumbel_max_tokens(y, 1.0, (5,)).tolist() == [4, 9, 0]


def test_argmax_tokens_take_the_first_maximum():
    x = torch.tensor([[0.0, 2.0, 2.0, 1.0], [5.0, 5.0, 5.0, 5.0]])
    assert G.argmax_tokens(x).tolist() == [1, 0]


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_profile_figures_are_used_only_for_the_source_they_were_taken_on(tmp_path):
    import bench
    src = tmp_path / "kernel.hip"
    src.write_text("__global__ void k() {}\n")
    summary = tmp_path / "summary.md"
    summary.write_text(f"source_sha256: {bench.source_hash([str(src)])}\nhbm_bytes_per_launch: 1234.5\n")
    assert bench.profile_value(str(summary), "hbm_bytes_per_launch", [str(src)]) == 1234.5
    assert bench.profile_value(str(summary), "missing_key", [str(src)]) is None
    assert bench.profile_value(str(tmp_path / "absent.md"), "hbm_bytes_per_launch", [str(src)]) is None
    src.write_text("__global__ void k() { /* changed */ }\n")
    assert bench.profile_value(str(summary), "hbm_bytes_per_launch", [str(src)]) is None


def test_acceptance_report_counts_the_tests_taken():
    """alpha = accepted drafts / accept tests taken: a sequence that accepted n
    of K drafts took min(n + 1, K) tests; faulty sequences (-1) are left out."""
    import bench
    r = bench.acceptance_report(np.array([0, 4, 2, -1]), 4)
    assert r["accepted_drafts"] == 6 and r["accept_tests"] == 1 + 4 + 3
    assert r["alpha_observed"] == 6 / 8
    assert r["mean_tokens_per_verify"] == (1 + 5 + 3) / 3
    a = 0.75
    assert abs(r["closed_form_tokens_at_alpha_observed"] - (1 - a ** 5) / (1 - a)) < 1e-12
    assert bench.acceptance_report(np.array([3, 3]), 3)["closed_form_tokens_at_alpha_observed"] == 4.0
