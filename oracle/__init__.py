"""fp64 CPU oracle for the speculative-sampling verify step and the shortlisted head.

TEST INFRASTRUCTURE ONLY.  The library path never imports this package; only
the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg do.
It shares no code with the GPU implementation.  The arithmetic lives in
``oracle.c`` (plain C, IEEE double, scalar loops in token-id order); this module
only builds it with gcc, marshals numpy arrays and splits batches over threads.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

F32, BF16 = 0, 1
SAMPLE, GREEDY = 0, 1


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math: IEEE double semantics)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
                               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            i32 = ctypes.c_int32
            lib.oracle_verify.argtypes = [P, P, ctypes.c_int, P, P, i32, i32, i32, ctypes.c_float,
                                          ctypes.c_int, P, P, P, P, P, P, P, P, P, P]
            lib.oracle_verify.restype = ctypes.c_int
            lib.oracle_row_stats.argtypes = [P, ctypes.c_int, i32, i32, ctypes.c_float, P, P]
            lib.oracle_row_stats.restype = ctypes.c_int
            lib.oracle_overlap.argtypes = [P, P, ctypes.c_int, i32, i32, ctypes.c_float, P]
            lib.oracle_overlap.restype = ctypes.c_int
            lib.oracle_head.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, P, P, P]
            lib.oracle_head.restype = ctypes.c_int
            lib.oracle_kv_commit.argtypes = [P, P, P, P, P, i32, i32, i32, i32, ctypes.c_int64]
            lib.oracle_kv_commit.restype = ctypes.c_int
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _as_logits(x):
    """numpy view of logits: uint16 bit patterns for bf16, float32 otherwise."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            t = x.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16), BF16
            return t.to(torch.float32).numpy(), F32
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, BF16
    return x.astype(np.float32, copy=False), F32


def _np(x, dtype):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(x, dtype=dtype)


def verify(target, draft, draft_tokens, uniforms, temperature, mode=SAMPLE, threads=1, probe_token=None):
    """Run the oracle over a batch.

    target [B,K+1,V] and draft [B,K,V]: bf16 torch tensors, uint16 bit arrays or
    float32 arrays.  draft may be None in GREEDY mode.  Returns a dict of numpy
    arrays: accepted_len, out_tokens, p_target, p_draft, accept_margin,
    sample_margin, residual_mass, fallbacks, and probe_gap when probe_token
    (int32 [B], a token per sequence) is given: the normalised mass between
    u*S and that token's cumulative interval at the oracle's sampled position.
    """
    lib = _load()
    tgt, dt = _as_logits(target)
    B, K1, V = tgt.shape
    K = K1 - 1
    if draft is None:
        dr = np.zeros((B, K, V), dtype=tgt.dtype) if mode == GREEDY else None
        ddt = dt
    else:
        dr, ddt = _as_logits(draft)
    assert ddt == dt and dr.shape == (B, K, V)
    tok = _np(draft_tokens, np.int32).reshape(B, K)
    uni = _np(uniforms, np.float32).reshape(B, K + 1, 2) if uniforms is not None else \
        np.zeros((B, K + 1, 2), np.float32)
    out = dict(
        accepted_len=np.empty(B, np.int32), out_tokens=np.empty((B, K + 1), np.int32),
        p_target=np.empty((B, K), np.float64), p_draft=np.empty((B, K), np.float64),
        accept_margin=np.empty((B, K), np.float64), sample_margin=np.empty(B, np.float64),
        residual_mass=np.empty(B, np.float64), fallbacks=np.empty(B, np.int32))
    probe = None
    if probe_token is not None:
        probe = _np(probe_token, np.int32).reshape(B)
        out["probe_gap"] = np.empty(B, np.float64)

    def run(b0, b1):
        n = b1 - b0
        if n <= 0:
            return
        sl = slice(b0, b1)
        lib.oracle_verify(_ptr(tgt[sl]), _ptr(dr[sl]), dt, _ptr(tok[sl]), _ptr(uni[sl]),
                          n, K, V, float(np.float32(temperature)), mode,
                          _ptr(out["accepted_len"][sl]), _ptr(out["out_tokens"][sl]),
                          _ptr(out["p_target"][sl]), _ptr(out["p_draft"][sl]),
                          _ptr(out["accept_margin"][sl]), _ptr(out["sample_margin"][sl]),
                          _ptr(out["residual_mass"][sl]), _ptr(out["fallbacks"][sl]),
                          _ptr(probe[sl]) if probe is not None else None,
                          _ptr(out["probe_gap"][sl]) if probe is not None else None)

    if threads <= 1 or B <= 1:
        run(0, B)
    else:
        step = (B + threads - 1) // threads
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda b0: run(b0, min(B, b0 + step)), range(0, B, step)))
    return out


def row_stats(x, temperature):
    """(m, Z) per row of x[..., V] in fp64: m = max, Z = sum exp((x - m)/T)."""
    lib = _load()
    arr, dt = _as_logits(x)
    V = arr.shape[-1]
    R = int(np.prod(arr.shape[:-1]))
    m = np.empty(R, np.float64)
    Z = np.empty(R, np.float64)
    lib.oracle_row_stats(_ptr(arr), dt, R, V, float(np.float32(temperature)), _ptr(m), _ptr(Z))
    return m.reshape(arr.shape[:-1]), Z.reshape(arr.shape[:-1])


def overlap(target, draft, temperature, threads=1):
    """beta = sum_v min(P_t(v), P_d(v)) in fp64 per pair of rows: target and
    draft of the same shape [..., V] (for verify inputs pass target[:, :K])."""
    lib = _load()
    ta, dt1 = _as_logits(target)
    da, dt2 = _as_logits(draft)
    assert dt1 == dt2 and ta.shape == da.shape
    V = ta.shape[-1]
    R = int(np.prod(ta.shape[:-1]))
    ta = ta.reshape(R, V)
    da = da.reshape(R, V)
    beta = np.empty(R, np.float64)
    T = float(np.float32(temperature))

    def run(r0, r1):
        if r1 > r0:
            lib.oracle_overlap(_ptr(ta[r0:r1]), _ptr(da[r0:r1]), dt1, r1 - r0, V, T, _ptr(beta[r0:r1]))

    if threads <= 1 or R <= 1:
        run(0, R)
    else:
        step = (R + threads - 1) // threads
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda r0: run(r0, min(R, r0 + step)), range(0, R, step)))
    return beta.reshape(target.shape[:-1])


def head(h, W, cluster_ids, cluster_size, dense=False, threads=1):
    """Shortlisted head in fp64.  h bf16 [B,K,d], W bf16 [V,d], cluster_ids int32 [B,n_sel].

    Returns dict(compact [B,K,n_sel*cs], absdot [same], dense [B,K,V] or None).
    """
    lib = _load()
    hb, dt1 = _as_logits(h)
    Wb, dt2 = _as_logits(W)
    assert dt1 == BF16 and dt2 == BF16
    cid = _np(cluster_ids, np.int32)
    B, K, d = hb.shape
    V = Wb.shape[0]
    n_sel = cid.shape[1]
    L = n_sel * cluster_size
    compact = np.empty((B, K, L), np.float64)
    absdot = np.empty((B, K, L), np.float64)
    dn = np.empty((B, K, V), np.float64) if dense else None
    rc = [0]

    def run(b0, b1):
        if b1 <= b0:
            return
        r = lib.oracle_head(_ptr(hb[b0:b1]), _ptr(Wb), _ptr(cid[b0:b1]), b1 - b0, K, d, V,
                            cluster_size, n_sel, _ptr(compact[b0:b1]), _ptr(absdot[b0:b1]),
                            _ptr(dn[b0:b1]) if dn is not None else None)
        if r:
            rc[0] = r

    if threads <= 1 or B <= 1:
        run(0, B)
    else:
        step = (B + threads - 1) // threads
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda b0: run(b0, min(B, b0 + step)), range(0, B, step)))
    if rc[0]:
        raise ValueError("cluster ids out of range or not strictly ascending")
    return dict(compact=compact, absdot=absdot, dense=dn)


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def kv_commit(cache, staging, accepted_len, cache_len):
    """KV-cache commit (see oracle_kv_commit in oracle.c).

    cache [P, B, Lmax, E] and staging [P, B, K, E] numpy arrays of any
    fixed-size dtype (copied byte for byte); accepted_len, cache_len int32 [B].
    Returns (new cache, new cache_len, status) without modifying the inputs."""
    cache = np.array(cache, copy=True, order="C")
    staging = np.ascontiguousarray(staging)
    if staging.dtype != cache.dtype:
        raise ValueError("cache and staging must share a dtype")
    P, B, Lmax = cache.shape[:3]
    K = staging.shape[2]
    if staging.shape[:2] != (P, B) or staging.shape[3:] != cache.shape[3:]:
        raise ValueError("staging must be [P, B, K, ...] matching the cache")
    row_bytes = int(np.prod(cache.shape[3:], dtype=np.int64)) * cache.dtype.itemsize
    acc = np.ascontiguousarray(accepted_len, dtype=np.int32)
    ln = np.array(cache_len, dtype=np.int32, copy=True)
    status = np.zeros(B, dtype=np.int32)
    _load().oracle_kv_commit(_ptr(cache), _ptr(staging), _ptr(acc), _ptr(ln), _ptr(status),
                             P, B, K, Lmax, row_bytes)
    return cache, ln, status
