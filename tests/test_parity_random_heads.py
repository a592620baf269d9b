"""The two drafter heads against the fp64 oracle head on seeded random shapes.

Shapes are drawn from a fixed seed: the number of contexts, positions and
hidden dims (multiples of 256, of 64, of 8 and none of these, so every load
path of both kernels is taken), the number and size of clusters and how many
each context keeps, and the output dtypes (the static head both with d split over blocks and
in one launch).  Tolerances are those of the
hand-picked head tests: 1e-5 of sum_j |h_j W_tj| per logit, plus the bf16
unit roundoff for bf16 outputs, and the dense output's -inf pattern exact.
"""
import numpy as np
import pytest
import torch

from tests.test_parity_head import _check as check_shortlist, _small
from tests.test_parity_static_head import DEV, HEAD_TOL, _check as check_static, _static_ids
from workloads import head_case

pytestmark = pytest.mark.gpu

N_CASES = 24
WORK = 1.5e9   # oracle multiply-adds per case (M * N * d), so each case checks in seconds


def _d(r):
    kind = int(r.integers(0, 4))
    if kind == 0:
        return 256 * int(r.integers(1, 5))
    if kind == 1:
        return 64 * int(r.integers(1, 12))
    if kind == 2:
        return 8 * int(r.integers(1, 100))
    return int(r.integers(1, 700))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shortlist_head(i):
    r = np.random.default_rng([73, i])
    B = int(r.integers(1, 41))
    K = int(r.integers(1, 9))
    d = _d(r)
    nc = int(r.integers(1, 65))
    cs = int(r.choice([1, 3, 16, 63, 64, 65, 130, 200]))
    n_sel = int(r.integers(1, nc + 1))
    while n_sel > 1 and B * K * n_sel * cs * d > WORK:
        n_sel //= 2
    dense = torch.float32 if r.random() < 0.5 else torch.bfloat16
    print(f"shortlist head case {i}: B={B} K={K} d={d} clusters={nc}x{cs} n_sel={n_sel} dense={dense}", flush=True)
    check_shortlist(_small(B, K, d, nc, cs, n_sel, seed=7300 + i), dense_dtype=dense)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_static_head(i):
    r = np.random.default_rng([74, i])
    B = int(r.integers(1, 41))
    K = int(r.integers(1, 9))
    d = _d(r)
    cs = int(r.choice([1, 7, 64, 101, 501]))
    nc = int(r.integers(1, 200)) if cs > 1 else int(r.integers(64, 40000))
    V = nc * cs
    n_sel = int(r.integers(1, nc + 1))
    while n_sel > 1 and B * K * n_sel * cs * d > WORK:
        n_sel //= 2
    dtype = torch.float32 if r.random() < 0.5 else torch.bfloat16
    print(f"static head case {i}: B={B} K={K} d={d} V={V} clusters={nc}x{cs} n_sel={n_sel} out={dtype}",
          flush=True)
    hc = head_case(B, K, d, V, nc, 1, trial=7400 + i)
    ids = _static_ids(V, cs, n_sel, seed=7400 + i)
    got, ref = check_static(hc.h, hc.W, ids, cs, dtype)
    # the single-launch form (no split of d over blocks) against the same oracle values
    import speculative_sampling_verification_vocab_amd as sv
    one = sv.spec_draft_head_static(hc.h.to(DEV), hc.W.to(DEV), ids.to(DEV), cs, dtype=dtype, split=False)
    torch.cuda.synchronize()
    one = one.float().cpu().numpy()
    tol = HEAD_TOL * ref["absdot"] + 1e-30
    if dtype == torch.bfloat16:
        tol = tol + np.abs(ref["compact"]) * 2.0 ** -8
    assert np.all(np.abs(one - ref["compact"]) <= tol)
