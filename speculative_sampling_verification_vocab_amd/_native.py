"""ctypes binding of libspecverify.so (the C ABI declared in include/specverify.h).

This module only marshals arguments: torch tensors provide device memory and
the current HIP stream; every step of the verify path runs in the library's
HIP kernels.  There is no CPU fallback: a missing library or a non-GPU tensor
raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SPEC_F32, SPEC_BF16 = 0, 1
SPEC_MODE_SAMPLE, SPEC_MODE_GREEDY, SPEC_MODE_SAMPLE_EARLY_EXIT = 0, 1, 2
SPEC_OK = 0

_lib = None
_lock = threading.Lock()


class SpecVerifyError(RuntimeError):
    """A non-zero spec_status_t returned by the library."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


def load() -> ctypes.CDLL:
    """Load libspecverify.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(LIB_PATH)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        lib.spec_abi_version.argtypes = []
        lib.spec_abi_version.restype = ctypes.c_int
        lib.spec_status_string.argtypes = [ctypes.c_int]
        lib.spec_status_string.restype = ctypes.c_char_p
        lib.spec_verify_workspace_bytes.argtypes = [i32, i32, i32, ctypes.c_int, ctypes.c_int]
        lib.spec_verify_workspace_bytes.restype = sz
        verify_args = [P, P, P, P, i32, i32, i32, ctypes.c_int, ctypes.c_float, ctypes.c_int,
                       P, P, P, P, P, sz, P]
        lib.spec_verify.argtypes = verify_args
        lib.spec_verify.restype = ctypes.c_int
        lib.spec_verify_noalloc.argtypes = verify_args[:-3] + [P]
        lib.spec_verify_noalloc.restype = ctypes.c_int
        lib.spec_verify_timed.argtypes = verify_args + [P, i32]
        lib.spec_verify_timed.restype = ctypes.c_int
        lib.spec_verify_launch_count.argtypes = [i32, i32, i32, ctypes.c_int, ctypes.c_int]
        lib.spec_verify_launch_count.restype = i32
        lib.spec_draft_head_shortlist.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, P, P,
                                                  ctypes.c_int, P, sz, P]
        lib.spec_draft_head_shortlist.restype = ctypes.c_int
        lib.spec_verify_sparse_draft.argtypes = [P, P, P, P, i32, i32, i32, P, P, i32, i32, i32, ctypes.c_int,
                                                 ctypes.c_float, P, P, P, P, P, sz, P]
        lib.spec_verify_sparse_draft.restype = ctypes.c_int
        lib.spec_draft_head_positions.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i32, i32, P, ctypes.c_int, P]
        lib.spec_draft_head_positions.restype = ctypes.c_int
        lib.spec_draft_head_static.argtypes = [P, P, P, i32, i32, i32, i32, i32, P, ctypes.c_int, P, sz, P]
        lib.spec_draft_head_static_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        lib.spec_draft_head_static_workspace_bytes.restype = sz
        lib.spec_draft_head_static.restype = ctypes.c_int
        lib.spec_read_stream_probe.argtypes = [P, sz, P, P]
        lib.spec_read_stream_probe.restype = ctypes.c_int
        lib.spec_position_budget.argtypes = [i32, i32]
        lib.spec_position_budget.restype = i32
        lib.spec_kv_commit.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, ctypes.c_int, P]
        lib.spec_kv_commit.restype = ctypes.c_int
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load().spec_status_string(int(status)).decode()


def check(status: int, what: str) -> None:
    if status != SPEC_OK:
        raise SpecVerifyError(status, what)
