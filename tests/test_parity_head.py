"""GPU shortlisted head (bf16 MFMA, fp32 accumulation) against the fp64 oracle,
and verify of a shortlisted draft (P_d = 0 off the shortlist).

Tolerance: |gpu - oracle| <= 1e-5 * sum_j |h_j W_tj| per logit (relative to the
magnitude of the terms, so cancellation cannot fail it).  The -inf pattern of
the dense output must match exactly.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.parity_util import check_case
from workloads import VerifyCase, gumbel_max_tokens, head_case, normal_logits, verify_uniforms

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
HEAD_TOL = 1e-5


def _run_gpu(hc, dense_dtype=torch.float32):
    import speculative_sampling_verification_vocab_amd as sv
    comp, dense = sv.spec_draft_head_shortlist(hc.h.to(DEV), hc.W.to(DEV), hc.cluster_ids.to(DEV), hc.cluster_size,
                                               dense_dtype=dense_dtype)
    torch.cuda.synchronize()
    return comp.cpu().numpy(), dense.float().cpu().numpy()


def _check(hc, dense_dtype=torch.float32):
    comp, dense = _run_gpu(hc, dense_dtype)
    ref = oracle.head(hc.h.cpu(), hc.W.cpu(), hc.cluster_ids.cpu(), hc.cluster_size, dense=True,
                      threads=oracle.default_threads())
    tol = HEAD_TOL * ref["absdot"] + 1e-30
    err = np.abs(comp - ref["compact"])
    assert np.all(err <= tol), float(np.max(err / tol))
    ninf_ref = np.isneginf(ref["dense"])
    assert np.array_equal(np.isneginf(dense), ninf_ref)
    fin = ~ninf_ref
    if dense_dtype == torch.float32:
        np.testing.assert_array_equal(dense[fin].reshape(-1), _dense_from_compact(hc, comp)[fin].reshape(-1))
    else:
        # bf16 rounding of the fp32 result: within half a bf16 ulp plus the fp32 tolerance
        dref = ref["dense"][fin]
        ulp = np.abs(dref) * 2.0 ** -8
        assert np.all(np.abs(dense[fin] - dref) <= ulp + HEAD_TOL * np.abs(ref["dense"][fin]).max())
    return comp, dense, ref


def _dense_from_compact(hc, comp):
    B, K, L = comp.shape
    V = hc.W.shape[0]
    cs = hc.cluster_size
    out = np.full((B, K, V), -np.inf, np.float32)
    cid = hc.cluster_ids.cpu().numpy()
    for b in range(B):
        for s, c in enumerate(cid[b]):
            out[b, :, c * cs:(c + 1) * cs] = comp[b, :, s * cs:(s + 1) * cs]
    return out


def _small(B, K, d, n_clusters, cs, n_sel, seed):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn(B, K, d, generator=g).to(torch.bfloat16)
    W = (torch.randn(n_clusters * cs, d, generator=g) * 0.05).to(torch.bfloat16)
    scores = torch.randn(B, n_clusters, generator=g)
    from workloads import top_clusters
    from workloads.generators import HeadCase
    return HeadCase(h, W, top_clusters(scores, n_sel), cs)


@pytest.mark.parametrize("B,K,d,nc,cs,n_sel", [
    (3, 2, 96, 24, 10, 4),        # d below one LDS chunk
    (5, 4, 1000, 12, 70, 3),      # d not a multiple of 32; cs above one 64-token slab
    (2, 3, 100, 8, 16, 8),        # d % 8 != 0: element loads; every cluster selected
    (4, 40, 64, 6, 64, 2),        # K > 32: several row passes per context
    (40, 1, 128, 4, 32, 3),       # many contexts share a cluster
    (3, 2, 256, 10, 70, 3),       # whole-stage rows, one stage: no loads inside the stage loop
    (4, 4, 512, 12, 64, 4),       # whole-stage rows, two stages
])
def test_head_small(B, K, d, nc, cs, n_sel):
    print(f"head B={B} K={K} d={d} clusters={nc}x{cs} n_sel={n_sel}", flush=True)
    _check(_small(B, K, d, nc, cs, n_sel, seed=B * 1000 + K))


def test_head_max_contexts():
    """1024 contexts (the most one cluster's context list holds), each keeping
    every cluster: every block lists all 1024 and makes 128 passes of 32
    (context, position) rows over its slab."""
    _check(_small(1024, 4, 64, 4, 32, 4, seed=13), dense_dtype=torch.bfloat16)


def test_head_all_clusters_is_dense_gemm():
    hc = _small(3, 4, 256, 10, 24, 10, seed=5)
    comp, dense, ref = _check(hc)
    full = hc.h.double().numpy() @ hc.W.double().numpy().T
    assert np.all(np.abs(dense - full) <= HEAD_TOL * ref["absdot"].max())


def test_head_bf16_dense():
    _check(_small(4, 4, 512, 16, 40, 5, seed=9), dense_dtype=torch.bfloat16)


def test_head_deterministic_and_selection_independent():
    hc = _small(6, 4, 512, 16, 40, 5, seed=11)
    c1, d1 = _run_gpu(hc)
    c2, d2 = _run_gpu(hc)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(d1, d2)
    # move context 0's selection: shared clusters keep their logits (within tolerance)
    other = hc.cluster_ids.clone()
    other[0] = torch.tensor([0, 3, 7, 9, 15], dtype=torch.int32)
    from workloads.generators import HeadCase
    c3, d3 = _run_gpu(HeadCase(hc.h, hc.W, other, hc.cluster_size))
    common = set(hc.cluster_ids[0].tolist()) & set(other[0].tolist())
    for c in common:
        sl = slice(c * 40, (c + 1) * 40)
        np.testing.assert_allclose(d3[0][:, sl], d1[0][:, sl], rtol=0, atol=1e-5)


def test_head_full_shortlist_workload():
    """B=32 contexts, K=4, d=4096, V=128256 in 256 clusters of 501, top 16."""
    hc = head_case(device=DEV)
    comp, dense, ref = _check(hc)
    sizes = hc.cluster_ids.shape[1] * hc.cluster_size
    assert comp.shape == (32, 4, sizes) and sizes == 8016


def test_verify_on_shortlisted_draft():
    """Full-vocabulary verify of a shortlisted draft: draft logits are -inf off
    the shortlist (DynaSpec summary: verification keeps the full vocabulary)."""
    hc = head_case(B=8, K=4, d=1024, V=32064, n_clusters=64, n_sel=8, device="cpu")
    ref = oracle.head(hc.h, hc.W, hc.cluster_ids, hc.cluster_size, dense=True, threads=oracle.default_threads())
    draft = torch.from_numpy(ref["dense"]).to(torch.bfloat16)          # input from the oracle, not the GPU
    target = normal_logits((8, 5, 32064), 3.0, 1.1, (0, 5, 1, 0, 0)).to(torch.bfloat16)
    tok = gumbel_max_tokens(draft, 1.0, (0, 5, 1, 2, 0))
    uni = verify_uniforms(8, 4, (0, 5, 1, 3, 0))
    case = VerifyCase(target, draft, tok, uni, 1.0, "bf16")
    rep, out, orc = check_case(case)
    # drafts lie in the shortlist, so P_d(d) > 0 everywhere
    assert np.all(orc["p_draft"] > 0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_head_per_position_budget(dtype):
    """A shortlist per draft position (DynaSpec's position-aware budget, k_max = 8):
    each position's compact logits against the oracle head run on that position alone."""
    import speculative_sampling_verification_vocab_amd as sv
    from workloads import top_clusters
    g = torch.Generator().manual_seed(61)
    B, K, d, nc, cs = 6, 4, 320, 20, 48
    n_sel = [sv.position_budget(t, 8) for t in range(K)]          # [8, 8, 1, 1]
    S = max(n_sel)
    h = torch.randn(B, K, d, generator=g).to(torch.bfloat16)
    W = (torch.randn(nc * cs, d, generator=g) * 0.05).to(torch.bfloat16)
    cids = torch.full((B, K, S), -1, dtype=torch.int32)
    for k in range(K):
        cids[:, k, :n_sel[k]] = top_clusters(torch.randn(B, nc, generator=g), n_sel[k])
    L = S * cs + 5
    out = sv.spec_draft_head_positions(h.to(DEV), W.to(DEV), cids.to(DEV), n_sel, cs, L=L, dtype=dtype)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    for k in range(K):
        ref = oracle.head(h[:, k:k + 1].contiguous(), W, cids[:, k, :n_sel[k]].contiguous(), cs,
                          threads=oracle.default_threads())
        n = n_sel[k] * cs
        g_k = got[:, k:k + 1, :n]
        tol = HEAD_TOL * ref["absdot"] + (np.abs(ref["compact"]) * 2.0 ** -8 if dtype == torch.bfloat16 else 0)
        assert np.all(np.abs(g_k - ref["compact"]) <= tol + 1e-30), k
