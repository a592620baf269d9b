"""GPU drafter head over one static shortlist shared by every context (bf16
MFMA GEMM, fp32 accumulation) against the fp64 oracle's shortlisted head with
the same cluster ids repeated for every context.

Tolerance: |gpu - oracle| <= 1e-5 * sum_j |h_j W_tj| per logit, as for the
per-context head; bf16 output adds the bf16 unit roundoff (2^-8) of the exact value.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import head_case

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
HEAD_TOL = 1e-5


def _static_ids(V, cs, n_sel, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.sort(torch.randperm(V // cs, generator=g)[:n_sel]).values.to(torch.int32)


def _oracle(h, W, ids, cs):
    B = h.shape[0]
    return oracle.head(h, W, ids.reshape(1, -1).repeat(B, 1).contiguous(), cs, threads=oracle.default_threads())


def _gpu(h, W, ids, cs, dtype=torch.float32):
    import speculative_sampling_verification_vocab_amd as sv
    out = sv.spec_draft_head_static(h.to(DEV), W.to(DEV), ids.to(DEV), cs, dtype=dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _check(h, W, ids, cs, dtype=torch.float32):
    got = _gpu(h, W, ids, cs, dtype)
    ref = _oracle(h, W, ids, cs)
    assert got.shape == ref["compact"].shape
    tol = HEAD_TOL * ref["absdot"] + 1e-30
    if dtype == torch.bfloat16:
        tol = tol + np.abs(ref["compact"]) * 2.0 ** -8   # bf16 unit roundoff (8-bit significand)
    err = np.abs(got - ref["compact"])
    assert np.all(err <= tol), float(np.max(err / tol))
    return got, ref


@pytest.mark.parametrize("B,K,d,V,n_clusters,n_sel", [
    (3, 5, 200, 1010, 101, 7),        # M = 15 < one row tile, N = 70: a ragged column tile
    (13, 10, 256, 6000, 100, 23),     # M = 130: two row tiles, the second of 2 rows
    (2, 4, 203, 999, 333, 50),        # d not a multiple of 8: the element-wise load path
    (1, 1, 64, 4096, 4096, 300),      # one context, token-level shortlist (cluster size 1)
])
def test_static_head_shapes(B, K, d, V, n_clusters, n_sel):
    hc = head_case(B, K, d, V, n_clusters, 1, trial=5)
    ids = _static_ids(V, V // n_clusters, n_sel, seed=B * 1000 + d)
    _check(hc.h, hc.W, ids, V // n_clusters)


@pytest.mark.parametrize("B,K,d,V", [
    (2, 4, 200, 32000),       # d % 64 != 0: register-staged kernel, 128 x 128 tiles
    (2, 4, 203, 32000),       # element loads, 128 x 128 tiles
    (13, 10, 256, 32000),     # LDS-DMA kernel, 128 x 128 tiles, two row tiles (M = 130)
])
def test_static_head_wide_tiles(B, K, d, V):
    """Shortlists wide enough for the 128 x 128-tile instances (N = 25000 token
    ids, at least 192 tiles), ragged in both directions."""
    hc = head_case(B, K, d, V, V, 1, trial=11)
    ids = _static_ids(V, 1, 25000, seed=d)
    _check(hc.h, hc.W, ids, 1)


@pytest.mark.parametrize("B,K,V,cs,n_sel", [
    (4, 6, 8192, 128, 9),      # N even: column pairs stored as dwords
    (3, 5, 4096, 1, 301),      # N odd: one bf16 per store; M = 15 ragged
    (13, 10, 6000, 60, 37),    # N even, M = 130: two row tiles
])
def test_static_head_bf16_out(B, K, V, cs, n_sel):
    hc = head_case(B, K, 512, V, V // cs, 1, trial=6)
    ids = _static_ids(V, cs, n_sel, seed=1)
    _check(hc.h, hc.W, ids, cs, torch.bfloat16)


def test_static_head_matches_per_context_head():
    """Same clusters for every context: the shared-shortlist head and the
    per-context head compute the same logits (both within tolerance of the
    oracle; their fp32 results may differ in summation order only)."""
    import speculative_sampling_verification_vocab_amd as sv
    hc = head_case(8, 4, 1024, 32000, 250, 1, trial=7)
    ids = _static_ids(32000, 128, 12, seed=2)
    got, ref = _check(hc.h, hc.W, ids, 128)
    comp, _ = sv.spec_draft_head_shortlist(hc.h.to(DEV), hc.W.to(DEV), ids.reshape(1, -1).repeat(8, 1).to(DEV),
                                           128, dense=False)
    tol = 2 * HEAD_TOL * ref["absdot"] + 1e-30
    assert np.all(np.abs(comp.cpu().numpy() - got) <= tol)


def test_static_head_full_size_sampled():
    """Llama-3-8B-like head, d = 4096, V = 128256 in 256 clusters of 501, a
    static shortlist of 64 clusters (N = 32064), all 128 rows on the GPU; the
    oracle checks 3 of the 32 contexts."""
    hc = head_case(trial=8)
    ids = _static_ids(128256, 501, 64, seed=3)
    got = _gpu(hc.h, hc.W, ids, 501)
    assert got.shape == (32, 4, 64 * 501)
    for b in (0, 17, 31):
        ref = _oracle(hc.h[b:b + 1], hc.W, ids, 501)
        tol = HEAD_TOL * ref["absdot"][0] + 1e-30
        assert np.all(np.abs(got[b] - ref["compact"][0]) <= tol), b


def test_static_head_frequency_shortlist_size():
    """FR-Spec's 32k-token static shortlist at token granularity (cluster size 1)
    on a d = 4096 head; two contexts checked against the oracle."""
    hc = head_case(2, 4, 4096, 128256, 128256, 1, trial=9)
    ids = _static_ids(128256, 1, 32768, seed=4)
    _check(hc.h, hc.W, ids, 1)


def test_static_head_out_of_range_ids_read_zero():
    hc = head_case(2, 3, 128, 1000, 10, 1, trial=10)
    ids = torch.tensor([1, 10, -1, 4], dtype=torch.int32)
    got = _gpu(hc.h, hc.W, ids, 100)
    assert np.all(got[..., 100:300] == 0.0)
    ref = _oracle(hc.h, hc.W, torch.tensor([1, 4], dtype=torch.int32), 100)["compact"]
    assert np.allclose(got[..., :100], ref[..., :100], rtol=0, atol=1e-4)
    assert np.allclose(got[..., 300:], ref[..., 100:], rtol=0, atol=1e-4)


def test_static_head_empty():
    import speculative_sampling_verification_vocab_amd as sv
    W = torch.zeros((100, 64), dtype=torch.bfloat16, device=DEV)
    out = sv.spec_draft_head_static(torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV), W,
                                    torch.tensor([0], dtype=torch.int32, device=DEV), 10)
    assert out.shape == (0, 10)
    out = sv.spec_draft_head_static(torch.zeros((3, 64), dtype=torch.bfloat16, device=DEV), W,
                                    torch.zeros((0,), dtype=torch.int32, device=DEV), 10)
    assert out.shape == (3, 0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_static_head_k_split_against_oracle_and_single_launch(dtype):
    """Narrow shortlists with d % 64 == 0 split d over blocks (fp32 partial tiles
    added in a fixed order by a second launch): M = 130 (two row tiles, the
    second of 2 rows), d = 1024 (four slices of 4 stages), N = 1000 in clusters
    of 8; against the oracle and against the unsplit kernel."""
    import speculative_sampling_verification_vocab_amd as sv
    hc = head_case(13, 10, 1024, 8000, 1000, 1, trial=11)
    ids = _static_ids(8000, 8, 125, seed=13)
    assert sv._native.load().spec_draft_head_static_workspace_bytes(130, 1024, 8000, 8, 125) == 4 * 130 * 1000 * 4
    got, ref = _check(hc.h, hc.W, ids, 8, dtype)
    one = sv.spec_draft_head_static(hc.h.to(DEV), hc.W.to(DEV), ids.to(DEV), 8, dtype=dtype, split=False)
    torch.cuda.synchronize()
    tol = 2 * HEAD_TOL * ref["absdot"] + 1e-30
    if dtype == torch.bfloat16:
        tol = tol + np.abs(ref["compact"]) * 2.0 ** -7
    assert np.all(np.abs(one.float().cpu().numpy() - got) <= tol)
    # repeated calls (the workspace is reused) give identical results
    again = _gpu(hc.h, hc.W, ids, 8, dtype)
    np.testing.assert_array_equal(again, got)


def test_static_head_k_split_out_of_range_ids_read_zero():
    hc = head_case(2, 3, 512, 1000, 10, 1, trial=12)
    ids = torch.tensor([1, 10, -1, 4], dtype=torch.int32)
    got = _gpu(hc.h, hc.W, ids, 100)
    assert np.all(got[..., 100:300] == 0.0)
    ref = _oracle(hc.h, hc.W, torch.tensor([1, 4], dtype=torch.int32), 100)
    tol = HEAD_TOL * ref["absdot"] + 1e-30
    assert np.all(np.abs(got[..., :100] - ref["compact"][..., :100]) <= tol[..., :100])
    assert np.all(np.abs(got[..., 300:] - ref["compact"][..., 100:]) <= tol[..., 100:])
