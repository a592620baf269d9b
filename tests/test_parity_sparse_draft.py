"""GPU verify with a sparse draft (spec_verify_sparse_draft) against the fp64 oracle.

The oracle runs on the dense form of the same draft (the compact logits at
their token ids, -inf elsewhere, so P_d = 0 off the shortlist); the
comparison is the SAMPLE comparison of every other verify test (exact
integers up to the 1e-6 tie band, probabilities within 1e-5 relative).
Shortlists follow DynaSpec's per-position budget where a test says so."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity_util import PROB_RTOL, compare, probe_tokens, run_gpu
from workloads import VerifyCase, sparse_draft_case

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def run_sparse(c):
    import speculative_sampling_verification_vocab_amd as sv
    res = sv.spec_verify_sparse_draft(c.target.to(DEV), c.compact.to(DEV), c.cluster_ids.to(DEV), c.n_sel,
                                      c.cluster_size, c.draft_tokens.to(DEV), c.uniforms.to(DEV), c.temperature,
                                      return_probs=True)
    torch.cuda.synchronize()
    return [r.cpu().numpy() for r in res]


def check_sparse(c):
    out = run_sparse(c)
    orc = oracle.verify(c.target.cpu(), c.dense_draft.cpu(), c.draft_tokens.cpu(), c.uniforms.cpu(),
                        c.temperature, threads=oracle.default_threads(), probe_token=probe_tokens(out[0], out[1]))
    rep = compare(out[0], out[1], orc, c.K, gpu_pt=out[2], gpu_pd=out[3])
    assert not rep.failures, rep.failures[:5]
    assert rep.prob_max_rel <= PROB_RTOL, rep.prob_max_rel
    return rep, out, orc


def _budget(K, k_max, nc):
    import speculative_sampling_verification_vocab_amd as sv
    return [min(nc, sv.position_budget(t, k_max)) for t in range(K)]


@pytest.mark.parametrize("B,K,V,cs,n_sel,dtype", [
    (6, 3, 8192, 64, [8, 4, 2], "bf16"),
    (6, 3, 10020, 501, [20, 4, 1], "bf16"),     # every cluster at position 0; ragged last tile
    (5, 2, 7000, 7, [100, 30], "f32"),           # 7-id clusters: a lane's 8 ids cross clusters
    (4, 1, 4096, 256, [3], "bf16"),
    (3, 0, 5010, 501, [], "bf16"),               # no drafts: bonus token only
    (512, 2, 20000, 50, [20, 10], "bf16"),       # large batch: decisions in a launch of their own
])
def test_sparse_shapes(B, K, V, cs, n_sel, dtype):
    print(f"case B={B} K={K} V={V} cs={cs} n_sel={n_sel} {dtype}", flush=True)
    check_sparse(sparse_draft_case(B, K, V, cs, n_sel, dtype, key=(51, V, cs)))


@pytest.mark.parametrize("sigma", [0.2, 0.7, 2.0])
def test_sparse_position_budget(sigma):
    """DynaSpec's position-aware budget with k_max = 16 over 40 clusters of 501."""
    c = sparse_draft_case(8, 4, 20040, 501, _budget(4, 16, 40), "bf16", sigma=sigma, key=(52, int(sigma * 10)))
    assert c.n_sel == [16, 16, 2, 2]
    check_sparse(c)


@pytest.mark.parametrize("T", [0.02, 50.0, 1e-7, 1e-20])
def test_sparse_extreme_temperatures(T):
    """Near-greedy and near-uniform temperatures on compact draft rows, whose
    exponent reference is the draft row maximum."""
    print(f"case sparse T={T}", flush=True)
    check_sparse(sparse_draft_case(6, 3, 8192, 64, [8, 4, 2], "bf16", temperature=T, key=(53, int(T * 100))))


def test_draft_token_off_the_shortlist_is_accepted():
    c = sparse_draft_case(4, 3, 8192, 64, [4, 4, 4], "bf16", key=(53,))
    # token 0 of sequence 0 moved off position 0's shortlist: P_d = 0 there
    off = [v for v in range(8192) if v // 64 not in c.cluster_ids[0, 0, :4].tolist()][17]
    c.draft_tokens[0, 0] = off
    rep, out, orc = check_sparse(c)
    assert out[0][0] >= 1 and out[3][0, 0] == 0.0


def test_full_shortlist_matches_dense_verify():
    """Every cluster selected: the sparse draft is the dense draft."""
    c = sparse_draft_case(8, 3, 6000, 500, [12, 12, 12], "bf16", key=(54,))
    assert torch.equal(c.compact.float().reshape(8, 3, -1), c.dense_draft.float())
    rep, out, orc = check_sparse(c)
    dense = run_gpu(VerifyCase(c.target, c.dense_draft, c.draft_tokens, c.uniforms, c.temperature, "bf16"))
    orc2 = oracle.verify(c.target, c.dense_draft, c.draft_tokens, c.uniforms, c.temperature,
                         probe_token=probe_tokens(dense[0], dense[1]))
    rep2 = compare(dense[0], dense[1], orc2, c.K)
    assert not rep2.failures
    np.testing.assert_array_equal(out[0], dense[0])


def test_sparse_faults():
    c = sparse_draft_case(5, 3, 8192, 64, [6, 3, 2], "bf16", sigma=0.0, key=(55,))
    c.draft_tokens[1, 1] = 8192                   # out of range
    c.target[2, 0, :] = float("-inf")             # no finite maximum
    rep, out, orc = check_sparse(c)
    assert out[0][1] == -1 and out[0][2] == -1


def test_shortlist_workload_b32_k4_v128256():
    """B=32, K=4, V=128256 in 256 clusters of 501, DynaSpec budget k_max = 16."""
    c = sparse_draft_case(32, 4, 128256, 501, _budget(4, 16, 256), "bf16", key=(56,), device=DEV)
    c.target, c.compact, c.dense_draft = c.target.cpu(), c.compact.cpu(), c.dense_draft.cpu()
    c.cluster_ids, c.draft_tokens, c.uniforms = c.cluster_ids.cpu(), c.draft_tokens.cpu(), c.uniforms.cpu()
    rep, out, orc = check_sparse(c)
    print(f"mean tokens per verify {np.mean(out[0] + 1):.3f}, excused {rep.excused}", flush=True)
