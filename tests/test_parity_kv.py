"""GPU KV-cache commit (spec_kv_commit) against the oracle, byte for byte.

Covers the lesson's rollback exercise, random shapes on the 16-byte vector
path and the element path (rows that are not 16-byte multiples), every
accepted_len class (faulty -1, 0..K, > K), caches too full to take the
commit, and a verify -> commit chain."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_commit_exercise.json")


def _bits(t):
    """Host numpy view with exact bit patterns (bf16 as uint16)."""
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def _run(cache, staging, acc, ln):
    import speculative_sampling_verification_vocab_amd as sv
    c, s = cache.to(DEV).contiguous(), staging.to(DEV).contiguous()
    a, l = torch.as_tensor(acc, dtype=torch.int32).to(DEV), torch.as_tensor(ln, dtype=torch.int32).to(DEV)
    st = sv.spec_kv_commit(c, s, a, l)
    torch.cuda.synchronize()
    return _bits(c), l.cpu().numpy(), st.cpu().numpy()


def _check(cache, staging, acc, ln):
    got_c, got_l, got_s = _run(cache, staging, acc, ln)
    exp_c, exp_l, exp_s = oracle.kv_commit(_bits(cache), _bits(staging), np.asarray(acc), np.asarray(ln))
    np.testing.assert_array_equal(got_s, exp_s)
    np.testing.assert_array_equal(got_l, exp_l)
    assert np.array_equal(got_c.view(np.uint8), exp_c.view(np.uint8))
    return got_c, got_l, got_s


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_exercise_on_gpu(dtype):
    g = json.load(open(GOLDEN))
    P, E, Lmax, L0, K, n = 4, 8, 32, g["prefix_len"], g["drafts"], g["accepted"]
    cache = torch.full((P, 1, Lmax, E), -1.0)
    for p in range(L0):
        cache[:, 0, p] = 1000 + p
    staging = torch.zeros(P, 1, K, E)
    for j in range(K):
        staging[:, 0, j] = 2000 + j
    c, ln, st = _check(cache.to(dtype), staging.to(dtype), [n], [L0])
    assert ln[0] == g["expected_len_after_commit"] and st[0] == 0


@pytest.mark.parametrize("P,B,K,Lmax,E,dtype", [
    (4, 16, 7, 40, 64, torch.bfloat16),       # 128-byte rows: vector path
    (6, 8, 5, 24, 1024, torch.bfloat16),      # 2 KiB rows (8 KV heads x 128)
    (3, 12, 4, 20, 33, torch.bfloat16),       # 66-byte rows: element path
    (2, 9, 6, 30, 17, torch.float32),         # 68-byte rows: element path, fp32
    (5, 7, 3, 16, 12, torch.float32),         # 48-byte rows: vector path, fp32
    (1, 300, 2, 8, 8, torch.bfloat16),        # more than one block of sequences in the finalize launch
])
def test_random_commits(P, B, K, Lmax, E, dtype):
    print(f"case P={P} B={B} K={K} Lmax={Lmax} E={E} {dtype}", flush=True)
    g = torch.Generator().manual_seed(P * 1000 + B * 10 + K)
    cache = torch.randn(P, B, Lmax, E, generator=g).to(dtype)
    staging = torch.randn(P, B, K, E, generator=g).to(dtype)
    acc = torch.randint(-1, K + 2, (B,), generator=g)                 # includes -1 and K + 1
    ln = torch.randint(0, Lmax + 1, (B,), generator=g)                 # some too full to take n
    _check(cache, staging, acc.numpy(), ln.numpy())


def test_zero_planes_and_zero_drafts_still_write_lengths():
    cache = torch.zeros(0, 4, 10, 8, dtype=torch.bfloat16)
    staging = torch.zeros(0, 4, 3, 8, dtype=torch.bfloat16)
    c, ln, st = _run(cache, staging, [0, 1, 3, 4], [2, 9, 5, 0])
    assert st.tolist() == [0, 0, 0, 2] and ln.tolist() == [2, 10, 8, 0]
    cache = torch.zeros(2, 3, 10, 8, dtype=torch.bfloat16)
    staging = torch.zeros(2, 3, 0, 8, dtype=torch.bfloat16)
    c, ln, st = _run(cache, staging, [0, 0, 1], [3, 10, 4])
    assert st.tolist() == [0, 0, 2] and ln.tolist() == [3, 10, 4]


def test_verify_then_commit():
    """accepted_len straight from spec_verify drives the commit on the GPU."""
    import speculative_sampling_verification_vocab_amd as sv
    from workloads import verify_case
    c = verify_case(16, 5, 20000, "bf16", target_std=3.0, zipf_s=1.1, sigma=0.7, temperature=1.0, key=(41,))
    n, _ = sv.spec_verify(c.target.to(DEV), c.draft.to(DEV), c.draft_tokens.to(DEV), c.uniforms.to(DEV), 1.0)
    g = torch.Generator().manual_seed(42)
    P, Lmax, E = 8, 64, 256
    cache = torch.randn(P, 16, Lmax, E, generator=g).to(torch.bfloat16).to(DEV)
    staging = torch.randn(P, 16, 5, E, generator=g).to(torch.bfloat16).to(DEV)
    ln = torch.randint(0, 40, (16,), generator=g).to(torch.int32).to(DEV)
    exp = oracle.kv_commit(_bits(cache), _bits(staging), n.cpu().numpy(), ln.cpu().numpy())
    st = sv.spec_kv_commit(cache, staging, n, ln)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(cache), exp[0])
    np.testing.assert_array_equal(ln.cpu().numpy(), exp[1])
    np.testing.assert_array_equal(st.cpu().numpy(), exp[2])
    assert np.all(exp[2] == 0)


def test_caller_status_tensor_is_checked():
    """A caller-supplied status tensor must be int32 [B] on the cache's device
    (the kernel writes B entries into it)."""
    import speculative_sampling_verification_vocab_amd as sv
    dev = torch.device("cuda", 0)
    cache = torch.zeros(2, 3, 10, 8, dtype=torch.bfloat16, device=dev)
    staging = torch.zeros(2, 3, 2, 8, dtype=torch.bfloat16, device=dev)
    n = torch.tensor([0, 1, 2], dtype=torch.int32, device=dev)
    ln = torch.tensor([1, 2, 3], dtype=torch.int32, device=dev)
    for bad in (torch.zeros(2, dtype=torch.int32, device=dev), torch.zeros(3, dtype=torch.int64, device=dev),
                torch.zeros(3, dtype=torch.int32)):
        with pytest.raises(ValueError):
            sv.spec_kv_commit(cache, staging, n, ln, bad)
    good = torch.full((3,), 7, dtype=torch.int32, device=dev)
    assert sv.spec_kv_commit(cache, staging, n, ln, good) is good
    assert good.tolist() == [0, 0, 0] and ln.tolist() == [1, 3, 5]
