"""MI355X (gfx950) speculative-sampling verify over large vocabularies.

Python face of libspecverify.so.  Functions take torch tensors on a ROCm GPU
and call the C ABI on torch's current stream; results are new tensors on the
same device.  See include/specverify.h for the full contract.

    accepted_len, out_tokens = spec_verify(target, draft, draft_tokens, uniforms,
                                           temperature=1.0, mode="sample")
    compact, dense = spec_draft_head_shortlist(h, W, cluster_ids, cluster_size)
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _native
from ._native import SpecVerifyError  # noqa: F401

__all__ = ["spec_verify", "VerifyPlan", "spec_verify_noalloc", "spec_verify_workspace_bytes", "spec_verify_launch_count", "spec_draft_head_shortlist",
           "spec_kv_commit", "spec_verify_sparse_draft", "position_budget", "spec_draft_head_positions",
           "spec_draft_head_static",
           "Workspace", "SpecVerifyError", "abi_version"]

_DTYPES = {torch.bfloat16: _native.SPEC_BF16, torch.float32: _native.SPEC_F32}
_MODES = {"sample": _native.SPEC_MODE_SAMPLE, "greedy": _native.SPEC_MODE_GREEDY,
          "sample_early_exit": _native.SPEC_MODE_SAMPLE_EARLY_EXIT}
_SAMPLING = ("sample", "sample_early_exit")


def abi_version() -> int:
    return _native.load().spec_abi_version()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_gpu(t: torch.Tensor, name: str, device: Optional[torch.device] = None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (there is no CPU path)")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, the device of the call's first tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_of(device: torch.device, stream=None):
    return stream if stream is not None else torch.cuda.current_stream(device)


def _stream_handle(device: torch.device, stream=None):
    return ctypes.c_void_p(_stream_of(device, stream).cuda_stream)


def spec_verify_workspace_bytes(B: int, K: int, V: int, dtype: torch.dtype, mode: str = "sample") -> int:
    return int(_native.load().spec_verify_workspace_bytes(B, K, V, _DTYPES[dtype], _MODES[mode]))


def spec_verify_launch_count(B: int, K: int, V: int, dtype: torch.dtype, mode: str = "sample") -> int:
    """Kernel launches of one spec_verify call (timing events needed: this + 1)."""
    return int(_native.load().spec_verify_launch_count(B, K, V, _DTYPES[dtype], _MODES[mode]))


class Workspace:
    """A device scratch buffer reused across calls; it grows to the largest size asked for.

    Calls that share one Workspace must be ordered on the GPU (same stream, or
    synchronised).  The buffer is allocated on the stream of the call that
    grows it, and every use on another stream is recorded with the caching
    allocator (``record_stream``), so a buffer that is replaced is not handed
    out again while kernels on any stream that used it may still run."""

    def __init__(self, device):
        self.device = torch.device(device)
        self.buf = torch.empty(0, dtype=torch.uint8, device=self.device)
        self._stream = None

    def get(self, nbytes: int, stream=None, device=None) -> torch.Tensor:
        if device is not None and torch.device(device) != self.device:
            raise ValueError(f"this workspace is on {self.device}, the call on {device}")
        s = _stream_of(self.device, stream)
        if self.buf.numel() < nbytes:
            with torch.cuda.stream(s):
                self.buf = torch.empty(max(nbytes, 2 * self.buf.numel()), dtype=torch.uint8, device=self.device)
            self._stream = s
        elif s != self._stream:
            self.buf.record_stream(s)
        return self.buf


_default_ws = {}


def _workspace_for(device, stream=None) -> Workspace:
    """The default workspace of (device, stream): calls on different streams never share scratch."""
    dev = torch.device(device)
    key = (dev, _stream_of(dev, stream).cuda_stream)
    ws = _default_ws.get(key)
    if ws is None:
        ws = _default_ws[key] = Workspace(dev)
    return ws


def spec_verify(target: torch.Tensor, draft: Optional[torch.Tensor], draft_tokens: Optional[torch.Tensor],
                uniforms: Optional[torch.Tensor], temperature: float = 1.0, mode: str = "sample", *,
                return_probs: bool = False, workspace: Optional[Workspace] = None, stream=None,
                events: Optional[Sequence] = None):
    """Speculative-sampling verify step on the GPU.

    target [B, K+1, V] and draft [B, K, V] (bf16 or float32), draft_tokens int32
    [B, K], uniforms float32 [B, K+1, 2].  Returns (accepted_len int32 [B],
    out_tokens int32 [B, K+1]) and, with return_probs, also (P_t(d), P_d(d))
    float32 [B, K].  `events`: recorded torch.cuda.Event objects, re-recorded
    before each kernel launch and after the last (see spec_verify_timed).

    mode: "sample" (every row read once), "sample_early_exit" (the same
    accepted_len and out_tokens, reading only the rows up to each sequence's
    first rejection; probabilities after it are NaN) or "greedy".
    """
    B, K, V, dt, sampling = _check_verify_inputs(target, draft, draft_tokens, uniforms, mode)
    dev = target.device
    lib = _native.load()
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    pt = torch.empty((B, K), dtype=torch.float32, device=dev) if return_probs else None
    pd = torch.empty((B, K), dtype=torch.float32, device=dev) if return_probs else None
    need = lib.spec_verify_workspace_bytes(B, K, V, dt, _MODES[mode])
    ws = (workspace or _workspace_for(dev, stream)).get(need, stream, dev)
    args = [_ptr(target), _ptr(draft) if sampling else None,
            _ptr(draft_tokens) if K > 0 else None, _ptr(uniforms) if sampling else None,
            B, K, V, dt, ctypes.c_float(temperature if sampling else 0.0), _MODES[mode],
            _ptr(acc), _ptr(out), _ptr(pt), _ptr(pd), _ptr(ws), ws.numel(), _stream_handle(dev, stream)]
    if events is not None:
        evs = list(events)
        arr = (ctypes.c_void_p * max(1, len(evs)))(*[e.cuda_event if e is not None else None for e in evs])
        st = lib.spec_verify_timed(*args, arr, len(evs))
    else:
        st = lib.spec_verify(*args)
    _native.check(st, "spec_verify")
    if return_probs:
        return acc, out, pt, pd
    return acc, out


class VerifyPlan:
    """spec_verify prepared once for a fixed shape, for serving loops.

    The output tensors and the workspace are allocated when the plan is made
    and reused by every call, which is then only argument packing and one C
    call (no allocation).  Each call returns the same output tensors,
    overwritten in place: copy them before the next call if they must be kept.
    Inputs must have the shapes and dtype the plan was made for (checked) and
    be contiguous tensors on the plan's device.  Calls run on the stream the
    plan was made for (`stream`, else the current stream at that time), and
    calls that overlap in time on one plan race on its workspace and outputs."""

    def __init__(self, B: int, K: int, V: int, dtype: torch.dtype = torch.bfloat16, mode: str = "sample", *,
                 device="cuda", stream=None, return_probs: bool = False):
        if mode not in _MODES:
            raise ValueError(f"mode must be one of {list(_MODES)}")
        if dtype not in _DTYPES:
            raise ValueError("logits must be bfloat16 or float32")
        dev = torch.device(device)
        if dev.index is None:
            dev = torch.device(dev.type, torch.cuda.current_device())
        self.B, self.K, self.V, self.dtype, self.mode = int(B), int(K), int(V), dtype, mode
        self.device = dev
        self._sampling = mode in _SAMPLING
        lib = _native.load()
        self._lib = lib
        self._dt, self._m = _DTYPES[dtype], _MODES[mode]
        self.accepted_len = torch.empty(B, dtype=torch.int32, device=dev)
        self.out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        self.p_target = torch.empty((B, K), dtype=torch.float32, device=dev) if return_probs else None
        self.p_draft = torch.empty((B, K), dtype=torch.float32, device=dev) if return_probs else None
        s = _stream_of(dev, stream)
        need = lib.spec_verify_workspace_bytes(B, K, V, self._dt, self._m)
        with torch.cuda.stream(s):
            self._ws = torch.empty(max(1, need), dtype=torch.uint8, device=dev)
        self._stream = s.cuda_stream
        self._tail = [self.accepted_len.data_ptr(), self.out_tokens.data_ptr(),
                      self.p_target.data_ptr() if return_probs else None,
                      self.p_draft.data_ptr() if return_probs else None,
                      self._ws.data_ptr(), self._ws.numel(), self._stream]
        self._shapes = ((B, K + 1, V), (B, K, V), (B, K), (B, K + 1, 2))
        self._out = (self.accepted_len, self.out_tokens) + ((self.p_target, self.p_draft) if return_probs else ())

    def _arg(self, t, shape, dtype, name):
        if t.shape != shape or t.dtype != dtype or t.device != self.device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dtype} {list(shape)} tensor on {self.device}")
        return t.data_ptr()

    def __call__(self, target, draft, draft_tokens, uniforms, temperature: float = 1.0, events=None):
        sh = self._shapes
        tp = self._arg(target, sh[0], self.dtype, "target")
        dp = up = kp = None
        if self.K > 0:
            kp = self._arg(draft_tokens, sh[2], torch.int32, "draft_tokens")
        if self._sampling:
            if self.K > 0:
                dp = self._arg(draft, sh[1], self.dtype, "draft")
            up = self._arg(uniforms, sh[3], torch.float32, "uniforms")
        args = [tp, dp, kp, up, self.B, self.K, self.V, self._dt,
                ctypes.c_float(temperature if self._sampling else 0.0), self._m, *self._tail]
        if events is None:
            st = self._lib.spec_verify(*args)
        else:
            evs = list(events)
            arr = (ctypes.c_void_p * max(1, len(evs)))(*[e.cuda_event if e is not None else None for e in evs])
            st = self._lib.spec_verify_timed(*args, arr, len(evs))
        if st:
            _native.check(st, "spec_verify")
        return self._out


def _check_verify_inputs(target, draft, draft_tokens, uniforms, mode):
    """Shape and dtype checks shared by spec_verify and spec_verify_noalloc."""
    if mode not in _MODES:
        raise ValueError(f"mode must be one of {list(_MODES)}")
    _need_gpu(target, "target")
    if target.dim() != 3:
        raise ValueError("target must be [B, K+1, V]")
    B, K1, V = target.shape
    K = K1 - 1
    dt = _DTYPES.get(target.dtype)
    if dt is None:
        raise ValueError("logits must be bfloat16 or float32")
    sampling = mode in _SAMPLING
    if sampling and K > 0:
        if draft is None:
            raise ValueError("draft logits are required in sample mode")
        _need_gpu(draft, "draft", target.device)
        if draft.dtype != target.dtype or tuple(draft.shape) != (B, K, V):
            raise ValueError("draft must match target dtype and be [B, K, V]")
    if K > 0:
        if draft_tokens is None:
            raise ValueError("draft_tokens are required when K > 0")
        _need_gpu(draft_tokens, "draft_tokens", target.device)
        if draft_tokens.dtype != torch.int32 or tuple(draft_tokens.shape) != (B, K):
            raise ValueError("draft_tokens must be int32 [B, K]")
    if sampling:
        if uniforms is None:
            raise ValueError("uniforms are required in sample mode")
        _need_gpu(uniforms, "uniforms", target.device)
        if uniforms.dtype != torch.float32 or tuple(uniforms.shape) != (B, K + 1, 2):
            raise ValueError("uniforms must be float32 [B, K+1, 2]")
    return B, K, V, dt, sampling


def spec_verify_noalloc(target: torch.Tensor, draft: Optional[torch.Tensor], draft_tokens: Optional[torch.Tensor],
                        uniforms: Optional[torch.Tensor], temperature: float = 1.0, mode: str = "sample", *,
                        out: Sequence[torch.Tensor], stream=None):
    """spec_verify into caller-owned outputs with the library's static scratch
    (spec_verify_noalloc of the C ABI): neither this call nor the library
    allocates device memory.  out = (accepted_len int32 [B], out_tokens int32
    [B, K+1]) or those plus (p_target, p_draft) float32 [B, K].  Calls that
    overlap on one GPU race on the shared scratch."""
    B, K, V, dt, sampling = _check_verify_inputs(target, draft, draft_tokens, uniforms, mode)
    if len(out) not in (2, 4):
        raise ValueError("out must hold 2 or 4 tensors")
    want = [((B,), torch.int32), ((B, K + 1), torch.int32), ((B, K), torch.float32), ((B, K), torch.float32)]
    for t, (shape, dtype) in zip(out, want):
        _need_gpu(t, "out", target.device)
        if tuple(t.shape) != shape or t.dtype != dtype:
            raise ValueError(f"out tensor must be {dtype} {list(shape)}")
    pt, pd = (out[2], out[3]) if len(out) == 4 else (None, None)
    st = _native.load().spec_verify_noalloc(
        _ptr(target), _ptr(draft) if sampling else None, _ptr(draft_tokens) if K > 0 else None,
        _ptr(uniforms) if sampling else None, B, K, V, dt, ctypes.c_float(temperature if sampling else 0.0),
        _MODES[mode], _ptr(out[0]), _ptr(out[1]), _ptr(pt), _ptr(pd), _stream_handle(target.device, stream))
    _native.check(st, "spec_verify_noalloc")
    return tuple(out)


def spec_draft_head_shortlist(h: torch.Tensor, W: torch.Tensor, cluster_ids: torch.Tensor, cluster_size: int, *,
                              compact: bool = True, dense: bool = True, dense_dtype: torch.dtype = torch.float32,
                              stream=None):
    """Shortlisted drafter head.  h bf16 [B, K, d], W bf16 [V, d], cluster_ids int32 [B, n_sel]
    (ascending).  Returns (compact float32 [B, K, n_sel*cluster_size] or None,
    dense [B, K, V] of dense_dtype with -inf off the shortlist, or None)."""
    for t, name in ((h, "h"), (W, "W"), (cluster_ids, "cluster_ids")):
        _need_gpu(t, name, h.device)
    if h.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
        raise ValueError("h and W must be bfloat16")
    if cluster_ids.dtype != torch.int32:
        raise ValueError("cluster_ids must be int32")
    B, K, d = h.shape
    V = W.shape[0]
    if W.shape[1] != d:
        raise ValueError("W must be [V, d]")
    n_sel = cluster_ids.shape[1]
    dev = h.device
    comp = torch.empty((B, K, n_sel * cluster_size), dtype=torch.float32, device=dev) if compact else None
    dn = torch.empty((B, K, V), dtype=dense_dtype, device=dev) if dense else None
    lib = _native.load()
    st = lib.spec_draft_head_shortlist(_ptr(h), _ptr(W), _ptr(cluster_ids), B, K, d, V, cluster_size, n_sel,
                                       _ptr(comp), _ptr(dn), _DTYPES[dense_dtype] if dense else 0, None, 0,
                                       _stream_handle(dev, stream))
    _native.check(st, "spec_draft_head_shortlist")
    return comp, dn


def spec_kv_commit(cache: torch.Tensor, staging: torch.Tensor, accepted_len: torch.Tensor,
                   cache_len: torch.Tensor, status: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Commit the accepted drafts' KV entries (see spec_kv_commit in specverify.h).

    cache [P, B, L_max, ...] and staging [P, B, K, ...] (same trailing shape,
    bf16 or float32, contiguous, on the GPU); accepted_len int32 [B] from
    spec_verify; cache_len int32 [B], advanced in place.  Returns the status
    tensor (int32 [B]: 0 committed, 1 no room, 2 accepted_len outside [0, K])."""
    for t, name in ((cache, "cache"), (staging, "staging"), (accepted_len, "accepted_len"), (cache_len, "cache_len")):
        _need_gpu(t, name, cache.device)
    dt = _DTYPES.get(cache.dtype)
    if dt is None or staging.dtype != cache.dtype:
        raise ValueError("cache and staging must both be bfloat16 or both float32")
    if cache.dim() < 3 or staging.dim() != cache.dim() or staging.shape[:2] != cache.shape[:2] \
            or staging.shape[3:] != cache.shape[3:]:
        raise ValueError("cache must be [P, B, L_max, ...] and staging [P, B, K, ...] with the same trailing shape")
    if not (cache.is_contiguous() and staging.is_contiguous()):
        raise ValueError("cache and staging must be contiguous")
    P, B, Lmax = cache.shape[:3]
    K = staging.shape[2]
    E = 1
    for x in cache.shape[3:]:
        E *= int(x)
    for t, name in ((accepted_len, "accepted_len"), (cache_len, "cache_len")):
        if t.dtype != torch.int32 or tuple(t.shape) != (B,) or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous int32 [B]")
    if status is None:
        status = torch.empty(B, dtype=torch.int32, device=cache.device)
    else:
        _need_gpu(status, "status", cache.device)
        if status.dtype != torch.int32 or tuple(status.shape) != (B,):
            raise ValueError("status must be contiguous int32 [B]")
    st = _native.load().spec_kv_commit(_ptr(cache), _ptr(staging), _ptr(accepted_len), _ptr(cache_len),
                                       _ptr(status), P, B, K, Lmax, E, dt, _stream_handle(cache.device, stream))
    _native.check(st, "spec_kv_commit")
    return status


def position_budget(t: int, k_max: int) -> int:
    """Clusters selected at draft position t (spec_position_budget of the C ABI)."""
    r = int(_native.load().spec_position_budget(int(t), int(k_max)))
    if r < 0:
        raise ValueError("t >= 0 and k_max >= 1")
    return r


def spec_verify_sparse_draft(target: torch.Tensor, draft_compact: torch.Tensor, cluster_ids: torch.Tensor,
                             n_sel, cluster_size: int, draft_tokens: torch.Tensor, uniforms: torch.Tensor,
                             temperature: float = 1.0, *, return_probs: bool = False,
                             workspace: Optional[Workspace] = None, stream=None):
    """Speculative-sampling verify with a sparse draft (see spec_verify_sparse_draft in specverify.h).

    target [B, K+1, V]; draft_compact [B, K, L] (same dtype) holding position
    i's logits on its shortlist in ascending token id; cluster_ids int32
    [B, K, S] (ascending, first n_sel[i] used); n_sel: K ints.  Returns what
    spec_verify returns in sample mode."""
    _need_gpu(target, "target")
    if target.dim() != 3:
        raise ValueError("target must be [B, K+1, V]")
    B, K1, V = target.shape
    K = K1 - 1
    dt = _DTYPES.get(target.dtype)
    if dt is None:
        raise ValueError("logits must be bfloat16 or float32")
    if len(n_sel) != K:
        raise ValueError("n_sel must have K entries")
    ns = (ctypes.c_int32 * max(1, K))(*[int(x) for x in n_sel])
    L = S = 1
    if K > 0:
        for t, name in ((draft_compact, "draft_compact"), (cluster_ids, "cluster_ids"),
                        (draft_tokens, "draft_tokens")):
            _need_gpu(t, name, target.device)
        if draft_compact.dtype != target.dtype or draft_compact.dim() != 3 or draft_compact.shape[:2] != (B, K):
            raise ValueError("draft_compact must be [B, K, L] with the target's dtype")
        if cluster_ids.dtype != torch.int32 or cluster_ids.dim() != 3 or cluster_ids.shape[:2] != (B, K):
            raise ValueError("cluster_ids must be int32 [B, K, S]")
        if draft_tokens.dtype != torch.int32 or tuple(draft_tokens.shape) != (B, K):
            raise ValueError("draft_tokens must be int32 [B, K]")
        L, S = draft_compact.shape[2], cluster_ids.shape[2]
        draft_compact, cluster_ids = draft_compact.contiguous(), cluster_ids.contiguous()
    _need_gpu(uniforms, "uniforms", target.device)
    if uniforms.dtype != torch.float32 or tuple(uniforms.shape) != (B, K + 1, 2):
        raise ValueError("uniforms must be float32 [B, K+1, 2]")
    lib = _native.load()
    dev = target.device
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    pt = torch.empty((B, K), dtype=torch.float32, device=dev) if return_probs else None
    pd = torch.empty((B, K), dtype=torch.float32, device=dev) if return_probs else None
    need = lib.spec_verify_workspace_bytes(B, K, V, dt, _MODES["sample"])
    ws = (workspace or _workspace_for(dev, stream)).get(need, stream, dev)
    st = lib.spec_verify_sparse_draft(_ptr(target), _ptr(draft_compact) if K > 0 else None,
                                      _ptr(cluster_ids) if K > 0 else None, ns, L, S, int(cluster_size),
                                      _ptr(draft_tokens) if K > 0 else None, _ptr(uniforms), B, K, V, dt,
                                      ctypes.c_float(temperature), _ptr(acc), _ptr(out), _ptr(pt), _ptr(pd),
                                      _ptr(ws), ws.numel(), _stream_handle(dev, stream))
    _native.check(st, "spec_verify_sparse_draft")
    return (acc, out, pt, pd) if return_probs else (acc, out)


def spec_draft_head_positions(h: torch.Tensor, W: torch.Tensor, cluster_ids: torch.Tensor, n_sel,
                              cluster_size: int, L: Optional[int] = None, dtype: torch.dtype = torch.bfloat16,
                              out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Drafter head with a shortlist per draft position (see spec_draft_head_positions in specverify.h).

    h bf16 [B, K, d]; W bf16 [V, d]; cluster_ids int32 [B, K, S] (first n_sel[k]
    ascending for position k); n_sel: K ints.  Returns compact logits
    [B, K, L] of `dtype` (L defaults to S * cluster_size), the input that
    spec_verify_sparse_draft takes."""
    for t, name in ((h, "h"), (W, "W"), (cluster_ids, "cluster_ids")):
        _need_gpu(t, name, h.device)
    if h.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
        raise ValueError("h and W must be bfloat16")
    B, K, d = h.shape
    V = W.shape[0]
    if cluster_ids.dtype != torch.int32 or cluster_ids.dim() != 3 or cluster_ids.shape[:2] != (B, K):
        raise ValueError("cluster_ids must be int32 [B, K, S]")
    if len(n_sel) != K:
        raise ValueError("n_sel must have K entries")
    S = cluster_ids.shape[2]
    L = S * cluster_size if L is None else int(L)
    dt = _DTYPES.get(dtype)
    if dt is None:
        raise ValueError("dtype must be bfloat16 or float32")
    if out is None:
        out = torch.empty((B, K, L), dtype=dtype, device=h.device)
    elif out.dtype != dtype or tuple(out.shape) != (B, K, L) or not out.is_contiguous() \
            or out.device != h.device:
        raise ValueError("out must be on h's device, a contiguous [B, K, L] tensor of dtype")
    ns = (ctypes.c_int32 * max(1, K))(*[int(x) for x in n_sel])
    st = _native.load().spec_draft_head_positions(_ptr(h.contiguous()), _ptr(W.contiguous()),
                                                  _ptr(cluster_ids.contiguous()), ns, B, K, d, V,
                                                  int(cluster_size), S, L, _ptr(out), dt,
                                                  _stream_handle(h.device, stream))
    _native.check(st, "spec_draft_head_positions")
    return out


def spec_draft_head_static(h: torch.Tensor, W: torch.Tensor, cluster_ids: torch.Tensor, cluster_size: int,
                           dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None,
                           stream=None, workspace: Optional[Workspace] = None, split: bool = True) -> torch.Tensor:
    """Drafter head over one shortlist shared by every context (see
    spec_draft_head_static in specverify.h).  h bf16 [..., d] (all leading
    dims are rows), W bf16 [V, d], cluster_ids int32 [n_sel].  Returns logits
    [..., n_sel * cluster_size] of dtype.  With split (default) narrow
    shortlists split d over blocks through a workspace (the stream's default
    one unless given); split=False runs the single-launch kernel."""
    for t, name in ((h, "h"), (W, "W"), (cluster_ids, "cluster_ids")):
        _need_gpu(t, name, h.device)
    if h.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
        raise ValueError("h and W must be bfloat16")
    if cluster_ids.dtype != torch.int32 or cluster_ids.dim() != 1:
        raise ValueError("cluster_ids must be int32 [n_sel]")
    d = h.shape[-1]
    M = h.numel() // d
    V = W.shape[0]
    N = cluster_ids.numel() * cluster_size
    dt = _DTYPES.get(dtype)
    if dt is None:
        raise ValueError("dtype must be bfloat16 or float32")
    shape = tuple(h.shape[:-1]) + (N,)
    if out is None:
        out = torch.empty(shape, dtype=dtype, device=h.device)
    elif out.dtype != dtype or tuple(out.shape) != shape or not out.is_contiguous() \
            or out.device != h.device:
        raise ValueError("out must be on h's device, contiguous with shape h.shape[:-1] + (N,) and dtype")
    lib = _native.load()
    ws, wsb = None, 0
    need = lib.spec_draft_head_static_workspace_bytes(M, d, V, int(cluster_size), cluster_ids.numel()) \
        if split and M > 0 and cluster_ids.numel() > 0 else 0
    if need:
        buf = (workspace or _workspace_for(h.device, stream)).get(need, stream, h.device)
        ws, wsb = _ptr(buf), buf.numel()
    st = lib.spec_draft_head_static(_ptr(h.contiguous()), _ptr(W.contiguous()),
                                    _ptr(cluster_ids.contiguous()), M, d, V, int(cluster_size),
                                    cluster_ids.numel(), _ptr(out), dt, ws, wsb,
                                    _stream_handle(h.device, stream))
    _native.check(st, "spec_draft_head_static")
    return out
