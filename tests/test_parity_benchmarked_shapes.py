"""Parity at the shapes the benchmark times, in the configuration it times them.

- The shortlisted-drafter chain: the GPU head's dense bf16 draft logits
  (-inf off each context's shortlist) feed Gumbel-max draft tokens and a dense
  spec_verify at B=32, K=4, V=128256.  The head is checked against the oracle
  head; the oracle verify then runs on the GPU head's own draft bytes (DynaSpec
  summary, abstract: the drafter sees a shortlist, verification keeps the full
  vocabulary and the exact rule).
- The static shared shortlist of 16 clusters of 501 (N = 8016) on all 128 rows
  at d = 4096: the narrow-tile instance of the static head.
- Greedy verify on the whole B=256, K=7, V=262144 bf16 batch, every sequence
  against the oracle (LLMs-from-Scratch lesson 25, "Greedy case").
"""
import numpy as np
import pytest
import torch

import oracle
from tests.parity_util import PROB_RTOL, compare, probe_tokens
from workloads import gumbel_max_tokens, head_case, normal_logits, verify_uniforms, workload_case

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
HEAD_TOL = 1e-5


@pytest.mark.timeout(600)
def test_shortlist_head_then_dense_verify_chain():
    import speculative_sampling_verification_vocab_amd as sv
    print("case shortlist chain: head B=32 K=4 d=4096 V=128256 top-16 of 256, then dense verify", flush=True)
    hc = head_case(device=DEV)
    B, K, d = hc.h.shape
    V = hc.W.shape[0]
    cs = hc.cluster_size
    # the benchmark's inputs (same generator keys)
    target = normal_logits((B, K + 1, V), 3.0, 1.1, (0, 5, 0, 0, 0), DEV).to(torch.bfloat16)
    comp, dense = sv.spec_draft_head_shortlist(hc.h, hc.W, hc.cluster_ids, cs, compact=True,
                                               dense_dtype=torch.bfloat16)
    tok = gumbel_max_tokens(dense, 1.0, (0, 5, 0, 2, 0))
    uni = verify_uniforms(B, K, (0, 5, 0, 3, 0), DEV)
    acc, out, pt, pd = sv.spec_verify(target, dense, tok, uni, 1.0, "sample", return_probs=True)
    torch.cuda.synchronize()

    # the head against the oracle head
    ref = oracle.head(hc.h.cpu(), hc.W.cpu(), hc.cluster_ids.cpu(), cs, threads=oracle.default_threads())
    c32 = comp.cpu().numpy()
    err = np.abs(c32 - ref["compact"])
    assert np.all(err <= HEAD_TOL * ref["absdot"] + 1e-30), float(np.max(err / (HEAD_TOL * ref["absdot"])))
    # the dense bf16 draft holds the compact logits (rounded to bf16) at their ids, -inf elsewhere
    dn = dense.float().cpu().numpy()
    cid = hc.cluster_ids.cpu().numpy()
    want = np.full((B, K, V), -np.inf, np.float32)
    c16 = torch.from_numpy(c32).to(torch.bfloat16).float().numpy()
    for b in range(B):
        for s, c in enumerate(cid[b]):
            want[b, :, c * cs:(c + 1) * cs] = c16[b, :, s * cs:(s + 1) * cs]
    np.testing.assert_array_equal(dn, want)

    # drafts lie in each context's shortlist
    tk = tok.cpu().numpy()
    for b in range(B):
        assert np.all(np.isin(tk[b] // cs, cid[b]))

    # the oracle verify on the GPU head's own draft bytes
    o = [acc.cpu().numpy(), out.cpu().numpy(), pt.cpu().numpy(), pd.cpu().numpy()]
    orc = oracle.verify(target.cpu(), dense.cpu(), tok.cpu(), uni.cpu(), 1.0, threads=oracle.default_threads(),
                        probe_token=probe_tokens(o[0], o[1]))
    rep = compare(o[0], o[1], orc, K, gpu_pt=o[2], gpu_pd=o[3])
    print(f"chain: mean tokens per verify {np.mean(o[0] + 1):.3f}, excused {rep.excused} of {rep.decisions}",
          flush=True)
    assert not rep.failures, rep.failures[:3]
    assert rep.prob_max_rel <= PROB_RTOL
    assert rep.excused <= rep.allowed_excused()
    assert np.all(orc["p_draft"] > 0)


@pytest.mark.timeout(600)
def test_static_head_narrow_tiles_full_shape():
    """M = 128 rows, N = 8016 (16 clusters of 501), d = 4096: the shape bench.py
    times, which takes the narrow-tile instance; every row checked."""
    print("case static head narrow: M=128 N=8016 d=4096", flush=True)
    hc = head_case(trial=0)
    B, K, d = hc.h.shape
    V = hc.W.shape[0]
    g = torch.Generator().manual_seed(12)                 # the benchmark's shortlist of 16 clusters
    ids = torch.sort(torch.randperm(V // 501, generator=g)[:16]).values.to(torch.int32)
    import speculative_sampling_verification_vocab_amd as sv
    for dtype in (torch.float32, torch.bfloat16):
        got = sv.spec_draft_head_static(hc.h.reshape(B * K, d).to(DEV), hc.W.to(DEV), ids.to(DEV), 501,
                                        dtype=dtype).float().cpu().numpy().reshape(B, K, -1)
        if dtype == torch.float32:
            ref = oracle.head(hc.h, hc.W, ids.reshape(1, -1).repeat(B, 1).contiguous(), 501,
                              threads=oracle.default_threads())
        tol = HEAD_TOL * ref["absdot"] + 1e-30
        if dtype == torch.bfloat16:
            tol = tol + np.abs(ref["compact"]) * 2.0 ** -8
        err = np.abs(got - ref["compact"])
        assert got.shape == (B, K, 8016)
        assert np.all(err <= tol), (dtype, float(np.max(err / tol)))


@pytest.mark.timeout(600)
def test_greedy_full_benchmark_batch():
    """Greedy on the whole B=256, K=7, V=262144 bf16 batch (the benchmark's
    logits, argmax draft tokens), every sequence against the oracle."""
    import speculative_sampling_verification_vocab_amd as sv
    print("case greedy full batch: B=256 K=7 V=262144 bf16", flush=True)
    c = workload_case("b256_k7_v262144_bf16", device=DEV, greedy=True)
    acc, out = sv.spec_verify(c.target, None, c.draft_tokens, None, 0.0, "greedy")
    torch.cuda.synchronize()
    acc, out = acc.cpu().numpy(), out.cpu().numpy()
    orc = oracle.verify(c.target.cpu(), None, c.draft_tokens.cpu(), None, 1.0, mode=oracle.GREEDY,
                        threads=oracle.default_threads())
    rep = compare(acc, out, orc, c.K, greedy=True)
    assert not rep.failures, rep.failures[:3]
    print(f"greedy full batch: mean tokens per verify {np.mean(acc + 1):.3f}", flush=True)
