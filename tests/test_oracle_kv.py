"""Pins of the oracle's KV-cache commit (CPU).

The page's exercise (tests/golden/kv_commit_exercise.json), a multi-step
simulation in which the cache must always hold exactly the entries of the
committed token stream, and the status cases."""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_commit_exercise.json")


def test_exercise_prefix_plus_accepted_drafts():
    g = json.load(open(GOLDEN))
    P, E, Lmax = 4, 6, 32                      # two layers x {K, V}, 6 values per entry
    L0, K, n = g["prefix_len"], g["drafts"], g["accepted"]
    assert n == g["rejected_position_one_based"] - 1
    cache = np.full((P, 1, Lmax, E), -1.0, np.float32)
    for p in range(L0):
        cache[:, 0, p, :] = 1000 + p
    staging = np.zeros((P, 1, K, E), np.float32)
    for j in range(K):
        staging[:, 0, j, :] = 2000 + j
    new, ln, st = oracle.kv_commit(cache, staging, [n], [L0])
    assert st[0] == 0 and ln[0] == g["expected_len_after_commit"]
    read = new[:, 0, :ln[0], 0]                # what the next iteration reads
    expect = [1000 + p for p in range(L0)] + [2000 + j for j in range(n)]
    assert np.array_equal(read, np.tile(np.array(expect, np.float32), (P, 1)))
    assert np.all(new[:, 0, ln[0]:] == -1.0)   # nothing written past the accepted prefix


def _entry(pos, tok, P, E):
    """A token's KV entry as a deterministic function of its position and id."""
    base = np.float32(pos * 100003 + tok * 7 + 1)
    return np.stack([np.arange(E, dtype=np.float32) + base + 0.5 * p for p in range(P)])


def test_multi_step_cache_holds_the_committed_stream():
    rng = np.random.default_rng(5)
    P, B, K, E, Lmax = 3, 4, 6, 5, 64
    cache = np.zeros((P, B, Lmax, E), np.float32)
    ln = np.zeros(B, np.int32)
    streams = [[] for _ in range(B)]           # committed (position, token) per sequence
    for step in range(8):
        drafts = rng.integers(0, 1000, (B, K))
        staging = np.zeros((P, B, K, E), np.float32)
        for b in range(B):
            for j in range(K):
                staging[:, b, j] = _entry(int(ln[b]) + j, int(drafts[b, j]), P, E)
        n = rng.integers(0, K + 1, B).astype(np.int32)
        cache, new_ln, st = oracle.kv_commit(cache, staging, n, ln)
        for b in range(B):
            if st[b] == 0:
                streams[b] += [(int(ln[b]) + j, int(drafts[b, j])) for j in range(n[b])]
            else:
                assert st[b] == 1 and new_ln[b] == ln[b]   # only "no room" can happen here
        ln = new_ln
        for b in range(B):
            assert len(streams[b]) == ln[b]
            for pos, tok in streams[b]:
                assert np.array_equal(cache[:, b, pos], _entry(pos, tok, P, E))


def test_status_cases_commit_nothing():
    P, B, K, E, Lmax = 2, 5, 4, 3, 10
    cache = np.arange(P * B * Lmax * E, dtype=np.float32).reshape(P, B, Lmax, E)
    staging = -np.ones((P, B, K, E), np.float32)
    n = np.array([-1, 5, 3, 0, 4], np.int32)       # faulty, > K, no room (8 + 3 > 10), zero, fits exactly
    ln = np.array([2, 2, 8, 4, 6], np.int32)
    new, new_ln, st = oracle.kv_commit(cache, staging, n, ln)
    assert st.tolist() == [2, 2, 1, 0, 0]
    assert new_ln.tolist() == [2, 2, 8, 4, 10]
    for b in range(4):
        assert np.array_equal(new[:, b], cache[:, b])
    assert np.all(new[:, 4, 6:10] == -1.0) and np.array_equal(new[:, 4, :6], cache[:, 4, :6])


def test_bytes_are_copied_exactly():
    """bf16 bit patterns (as uint16) and NaN payloads survive the copy."""
    P, B, K, E, Lmax = 1, 2, 3, 8, 6
    cache = np.zeros((P, B, Lmax, E), np.uint16)
    staging = np.random.default_rng(1).integers(0, 65536, (P, B, K, E)).astype(np.uint16)
    staging[0, 0, 0, 0] = 0x7fc1                  # a NaN payload as bf16
    new, ln, st = oracle.kv_commit(cache, staging, [3, 1], [0, 5])
    assert np.array_equal(new[0, 0, :3], staging[0, 0]) and np.array_equal(new[0, 1, 5:6], staging[0, 1, :1])
