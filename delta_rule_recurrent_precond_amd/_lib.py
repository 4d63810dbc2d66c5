"""ctypes binding of libosdn.so (argument marshalling only).

Every step of the forward runs in the HIP kernels behind the C ABI declared in
include/osdn.h; this module only checks tensors, allocates outputs with torch
and passes raw device pointers plus the current HIP stream.  There is no CPU
fallback: if the library or a GPU is missing, calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libosdn.so")

OSDN_OK = 0
OSDN_ERR_NULL = -1
OSDN_ERR_SHAPE = -2
OSDN_ERR_UNSUPPORTED = -3
OSDN_ERR_WORKSPACE = -4
OSDN_ERR_HIP = -5
OSDN_ERR_TOO_LARGE = -6
OSDN_NOALLOC_MAX_BYTES = 64 << 20
OSDN_BF16 = 0
OSDN_F32 = 1
OSDN_PRECOND_OFF = 1
OSDN_NORM_QK = 2
OSDN_GATE_LOGITS = 4
OSDN_GATE_PER_CHANNEL = 8

_lib = None
_lock = threading.Lock()

P = ctypes.c_void_p
I = ctypes.c_int
F = ctypes.c_float
SIGNATURES = {
    "osdn_precond_scan": (I, [P, P, P, P, F, I, I, I, I, I, P, P, P, P, P, ctypes.c_size_t, P]),
    "osdn_precond_scan_workspace_bytes": (ctypes.c_size_t, [I, I, I, I, I]),
    "osdn_chunk_fwd": (I, [P, P, P, P, P, P, P, I, I, I, I, I, I, I, ctypes.c_uint, P, P, P,
                           ctypes.c_size_t, P]),
    "osdn_chunk_fwd_workspace_bytes": (ctypes.c_size_t, [I, I, I, I, I, I, I, ctypes.c_uint]),
    "osdn_step": (I, [P, P, P, P, P, P, F, I, I, I, I, I, ctypes.c_uint, P, P, P, P, P]),
    "osdn_forward": (I, [P, P, P, P, P, P, P, P, F, I, I, I, I, I, I, I, ctypes.c_uint,
                         P, P, P, P, P, ctypes.c_size_t, P]),
    "osdn_forward_workspace_bytes": (ctypes.c_size_t, [I, I, I, I, I, I, I, ctypes.c_uint]),
    "osdn_forward_noalloc": (I, [P, P, P, P, P, P, P, P, F, I, I, I, I, I, I, I, ctypes.c_uint,
                                 P, P, P, P, P]),
    "osdn_status_str": (ctypes.c_char_p, [I]),
    "osdn_forward_path": (ctypes.c_char_p, [I, I, I, I, I, I, I, ctypes.c_uint,
                                            ctypes.c_size_t]),
}


class OsdnError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s failed: %d (%s)" % (fn, status, status_str(status)))


def load(path: str = LIB_PATH):
    """Load libosdn.so (built in-tree by build.py); raises if it is missing."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError(
                    "libosdn.so is not built (%s); run `python -m "
                    "delta_rule_recurrent_precond_amd.build`" % path)
            lib = ctypes.CDLL(path)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def status_str(status: int) -> str:
    return load().osdn_status_str(int(status)).decode()


def check(fn: str, status: int):
    if status != OSDN_OK:
        raise OsdnError(fn, status)
