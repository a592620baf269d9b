"""Verify against the fp64 oracle on seeded random shapes and input regimes.

The other parity tests pick their shapes by hand (tile edges, ragged rows,
the benchmarked workloads).  This sweep draws B, K, V, the logit dtype, the
temperature (a third of the cases anywhere from 1e-25 to 1e25), the
target's spread and prior and the draft's distance from the target at
random (a fixed seed, so every run checks the same cases), and runs each
case through SAMPLE (against the oracle, decision by decision), the
early-exit schedule (bit-identical to SAMPLE) and GREEDY (against the
oracle's argmax rule).  The case's parameters are printed before its GPU
calls.
"""
import numpy as np
import pytest

from tests.parity_util import check_case, compare, run_gpu, run_oracle
from workloads import verify_case

pytestmark = pytest.mark.gpu

N_CASES = 48


def _draw(i):
    r = np.random.default_rng([71, i])
    # a quarter of the cases are batches large enough for the separate
    # decision and pick launches; the rest pick inside the sampling launch
    big = i % 4 == 3
    B = int(r.integers(100, 301)) if big else int(r.integers(1, 41))
    K = int(r.choice([0, 1, 2, 3, 4, 5, 7, 8, 12, 16, 33]))
    V = int(r.choice([1, 2, 7, 64, 511, 2048, 4095, 4096, 4097, 8193, 20000, 32000, 65537]))
    if r.random() < 0.3:
        V = int(r.integers(1, 70000))
    if big:
        V = int(r.integers(20000, 40001))
    dtype = "bf16" if r.random() < 0.6 else "f32"
    T = float(np.exp(r.uniform(np.log(0.05), np.log(20.0))))
    if i % 3 == 2:  # a third of the cases anywhere from 1e-25 to 1e25
        T = float(np.float32(np.exp(r.uniform(np.log(1e-25), np.log(1e25)))))
    std = float(r.uniform(0.5, 5.0))
    zipf = float(r.choice([0.0, 1.1]))
    sigma = float(r.choice([0.0, 0.05, 0.3, 0.7, 1.5, 3.0]))
    return B, K, V, dtype, T, std, zipf, sigma


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    B, K, V, dtype, T, std, zipf, sigma = _draw(i)
    print(f"random case {i}: B={B} K={K} V={V} {dtype} T={T:.4g} std={std:.3g} zipf={zipf} sigma={sigma}",
          flush=True)
    c = verify_case(B, K, V, dtype, target_std=std, zipf_s=zipf, sigma=sigma, temperature=T, key=(72, i))
    rep, out, orc = check_case(c)

    # the early-exit schedule takes the same decisions and draws the same tokens
    ee = run_gpu(c, "sample_early_exit")
    np.testing.assert_array_equal(ee[0], out[0])
    np.testing.assert_array_equal(ee[1], out[1])

    # greedy on the same target rows, against the oracle's lowest-id argmax rule
    g = run_gpu(c, "greedy", return_probs=False)
    go = run_oracle(c, "greedy")
    grep_ = compare(g[0], g[1], go, K, greedy=True)
    assert not grep_.failures, grep_.failures[:3]


@pytest.mark.parametrize("i", range(16))
def test_random_sparse_draft_case(i):
    """The sparse-draft form (compact draft rows over per-position cluster
    shortlists) on seeded random shapes, against the oracle on the dense form."""
    from tests.test_parity_sparse_draft import check_sparse
    from workloads import sparse_draft_case
    r = np.random.default_rng([75, i])
    B = int(r.integers(100, 301)) if i % 4 == 3 else int(r.integers(1, 41))
    K = int(r.choice([0, 1, 2, 3, 4, 7]))
    cs = int(r.choice([1, 7, 50, 64, 501]))
    nc = int(r.integers(1, 80)) if cs > 1 else int(r.integers(64, 40000))
    V = nc * cs
    n_sel = [int(r.integers(1, nc + 1)) for _ in range(K)]
    dtype = "bf16" if r.random() < 0.6 else "f32"
    T = float(np.exp(r.uniform(np.log(0.1), np.log(10.0))))
    sigma = float(r.choice([0.05, 0.3, 0.7, 1.5]))
    print(f"random sparse case {i}: B={B} K={K} V={V} clusters={nc}x{cs} n_sel={n_sel} {dtype} T={T:.4g} "
          f"sigma={sigma}", flush=True)
    check_sparse(sparse_draft_case(B, K, V, cs, n_sel, dtype, temperature=T, sigma=sigma, key=(76, i)))
