"""The C ABI without a GPU: the library loads, exports exactly what
include/osdn.h declares, and rejects bad arguments with the documented codes
before touching the HIP runtime."""
import ctypes
import os
import re
import subprocess

import pytest

from delta_rule_recurrent_precond_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "osdn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(osdn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libosdn.so not built")
    return _lib.load()


def test_header_declares_the_entry_points():
    names = _declared()
    for want in ("osdn_precond_scan", "osdn_chunk_fwd", "osdn_forward",
                 "osdn_forward_workspace_bytes", "osdn_status_str", "osdn_forward_path"):
        assert want in names
    assert set(names) == set(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(set(re.findall(r"\bT (osdn_\w+)$", out, flags=re.M)))
    assert exported == _declared()


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        s = lib.osdn_status_str(code).decode()
        assert s and s != "unknown status"
    assert lib.osdn_status_str(12345).decode() == "unknown status"


NULL = None


def _fwd(lib, B=1, H=1, T=4, dk=16, dv=16, chunk=16, dtype=0, flags=0, ptr=1):
    p = ptr  # non-NULL dummy address: never dereferenced on these paths
    return lib.osdn_forward(p, p, p, p, None, None, None, None, 0.1, B, H, T, dk, dv, chunk, dtype,
                            flags, p, None, None, None, None, 0, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), _lib.OSDN_ERR_SHAPE),
    (dict(T=-3), _lib.OSDN_ERR_SHAPE),
    (dict(dk=48), _lib.OSDN_ERR_UNSUPPORTED),
    (dict(dv=256), _lib.OSDN_ERR_UNSUPPORTED),
    (dict(chunk=128), _lib.OSDN_ERR_UNSUPPORTED),
    (dict(chunk=0), _lib.OSDN_ERR_UNSUPPORTED),
    (dict(dtype=7), _lib.OSDN_ERR_UNSUPPORTED),
    (dict(flags=16), _lib.OSDN_ERR_UNSUPPORTED),
    (dict(flags=8), _lib.OSDN_ERR_NULL),   # the per-channel gate needs alpha
    (dict(ptr=None), _lib.OSDN_ERR_NULL),
    (dict(B=1 << 30, H=1 << 10), _lib.OSDN_ERR_SHAPE),
])
def test_forward_rejects(lib, kw, code):
    assert _fwd(lib, **kw) == code


def test_forward_needs_workspace_on_two_phase_path(lib):
    # fp32 data always takes the two-launch path, which stages k~ in the workspace
    assert lib.osdn_forward_path(1, 1, 4, 16, 16, 16, 1, 0, 0).decode() == "two-phase"
    assert _fwd(lib, dtype=1) == _lib.OSDN_ERR_WORKSPACE


def test_empty_batch_is_a_no_op(lib):
    assert _fwd(lib, B=0, ptr=None) == _lib.OSDN_OK
    assert lib.osdn_forward_path(0, 4, 8, 16, 16, 16, 0, 0, 0).decode() == "none"
    assert lib.osdn_precond_scan(None, None, None, None, 0.1, 3, 0, 5, 16, 0, None, None, None,
                                 None, None, 0, None) == _lib.OSDN_OK
    assert lib.osdn_chunk_fwd(None, None, None, None, None, None, None, 0, 2, 5, 16, 16, 16, 0, 0,
                              None, None, None, 0, None) == _lib.OSDN_OK


def test_scan_and_chunk_reject(lib):
    p = 1
    assert lib.osdn_precond_scan(p, p, None, None, 0.1, 1, 1, 4, 24, 0, p, None, None, None, None, 0,
                                 None) == _lib.OSDN_ERR_UNSUPPORTED
    assert lib.osdn_precond_scan(None, p, None, None, 0.1, 1, 1, 4, 16, 0, p, None, None, None, None, 0,
                                 None) == _lib.OSDN_ERR_NULL
    assert lib.osdn_precond_scan(p, p, None, None, 0.1, 1, 1, 4, 16, 0, None, None, None, None, None, 0,
                                 None) == _lib.OSDN_ERR_NULL
    assert lib.osdn_chunk_fwd(p, p, None, p, p, None, None, 1, 1, 4, 16, 16, 16, 0, 0, p, None,
                              None, 0, None) == _lib.OSDN_ERR_NULL
    assert lib.osdn_chunk_fwd(p, p, p, p, p, None, None, 1, 1, 4, 16, 16, 8, 0, 0, p, None,
                              None, 0, None) == _lib.OSDN_ERR_UNSUPPORTED
    assert lib.osdn_chunk_fwd(p, p, p, p, p, None, None, 1, -1, 4, 16, 16, 16, 0, 0, p, None,
                              None, 0, None) == _lib.OSDN_ERR_SHAPE
    # flags: only the per-channel gate, and it needs alpha
    assert lib.osdn_chunk_fwd(p, p, p, p, p, None, None, 1, 1, 4, 16, 16, 16, 0, 2, p, None,
                              None, 0, None) == _lib.OSDN_ERR_UNSUPPORTED
    assert lib.osdn_chunk_fwd(p, p, p, p, p, None, None, 1, 1, 4, 16, 16, 16, 0,
                              _lib.OSDN_GATE_PER_CHANNEL, p, None, None, 0,
                              None) == _lib.OSDN_ERR_NULL


def test_step_rejects(lib):
    p = 1
    assert lib.osdn_step(None, None, None, None, None, None, 0.1, 0, 4, 16, 16, 0, 0, None, None, None,
                         None, None) == _lib.OSDN_OK
    assert lib.osdn_step(p, p, p, p, None, None, 0.1, 1, 1, 16, 16, 0, 0, None, p, p, None,
                         None) == _lib.OSDN_ERR_NULL
    assert lib.osdn_step(p, p, p, p, None, None, 0.1, 1, 1, 24, 16, 0, 0, p, p, p, None,
                         None) == _lib.OSDN_ERR_UNSUPPORTED
    assert lib.osdn_step(p, p, p, p, None, None, 0.1, 1, -2, 16, 16, 0, 0, p, p, p, None,
                         None) == _lib.OSDN_ERR_SHAPE


def test_chunk_workspace_bytes(lib):
    # one 32 KB record per (b, h, chunk of 64) on the bf16 dk = dv = 128 shapes
    assert lib.osdn_chunk_fwd_workspace_bytes(2, 3, 130, 128, 128, 64, 0, 0) == 2 * 3 * 3 * 32768
    assert lib.osdn_chunk_fwd_workspace_bytes(2, 3, 130, 128, 128, 64, 0,
                                              _lib.OSDN_GATE_PER_CHANNEL) == 2 * 3 * 3 * 66048
    assert lib.osdn_chunk_fwd_workspace_bytes(2, 3, 0, 128, 128, 64, 0, 0) == 0
    assert lib.osdn_chunk_fwd_workspace_bytes(2, 3, 130, 64, 128, 64, 0, 0) == 0
    assert lib.osdn_chunk_fwd_workspace_bytes(2, 3, 130, 128, 128, 64, 1, 0) == 0
    assert lib.osdn_chunk_fwd_workspace_bytes(2, 3, 130, 128, 128, 24, 0, 0) == (1 << 64) - 1
    assert lib.osdn_chunk_fwd_workspace_bytes(2, 3, 130, 128, 128, 64, 0, 2) == (1 << 64) - 1


def test_split_workspace_bytes(lib):
    # matrix-core shapes: chunk records (32 KB; the walk records of 17.25 KB use the same
    # space first) and walk results (768 B) per (b, h, chunk of 64); with at most 32
    # heads the walk records get their own space and three 8-byte flags per chunk
    # follow (the one-launch forward); the walk alone: its records (17 KB) plus
    # results plus two 8-byte flags
    few = 17664 + 24
    assert lib.osdn_forward_workspace_bytes(2, 3, 130, 128, 128, 64, 0, 0) == 2 * 3 * 3 * (32768 + 768 + few)
    assert lib.osdn_forward_workspace_bytes(2, 3, 130, 128, 128, 64, 0, 1) == 2 * 3 * 3 * (32768 + 768 + few)
    assert lib.osdn_forward_workspace_bytes(4, 9, 130, 128, 128, 64, 0, 0) == 4 * 9 * 3 * (32768 + 768)
    assert lib.osdn_precond_scan_workspace_bytes(2, 3, 130, 128, 0) == 2 * 3 * 3 * (17664 + 768 + 16)
    assert lib.osdn_precond_scan_workspace_bytes(2, 3, 130, 64, 0) == 0
    assert lib.osdn_precond_scan_workspace_bytes(2, 3, 130, 128, 1) == 0
    assert lib.osdn_precond_scan_workspace_bytes(2, 3, 130, 48, 0) == (1 << 64) - 1
    n = lib.osdn_forward_workspace_bytes(2, 3, 130, 128, 128, 64, 0, 0)
    assert lib.osdn_forward_path(2, 3, 130, 128, 128, 64, 0, 0, n).decode() == "split"
    assert lib.osdn_forward_path(2, 3, 130, 128, 128, 64, 0, 0, n - 1).decode() == "fused"
    assert lib.osdn_forward_path(2, 3, 130, 128, 128, 64, 0, 1, n).decode() == "split"


def test_workspace_bytes(lib):
    n = lib.osdn_forward_workspace_bytes(2, 3, 100, 64, 32, 32, 1, 0)
    path = lib.osdn_forward_path(2, 3, 100, 64, 32, 32, 1, 0, 0).decode()
    if path == "two-phase":
        assert n >= 2 * 3 * 100 * 64 * 4 and n % 256 == 0
    else:
        assert n == 0
    assert lib.osdn_forward_workspace_bytes(2, 3, 100, 64, 32, 32, 1, 1) == 0
    assert lib.osdn_forward_workspace_bytes(2, 3, 100, 48, 32, 32, 1, 0) == ctypes.c_size_t(-1).value
    assert lib.osdn_forward_path(2, 3, 100, 48, 32, 32, 1, 0, 0).decode() == "invalid"


def test_python_binding_refuses_cpu_tensors():
    import torch
    import delta_rule_recurrent_precond_amd as osdn
    q = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ValueError, match="no CPU path"):
        osdn.forward(q, q, q, torch.zeros(1, 1, 4))


def test_transform_flags(lib):
    """Input transforms: accepted where the multi-launch or two-phase path runs,
    refused where only the single fused kernel could (validated before any launch;
    the dummy pointers are never dereferenced on these paths)."""
    assert lib.osdn_forward_path(1, 1, 64, 128, 128, 64, 0, 2, 0).decode() == "unsupported"
    assert lib.osdn_forward_path(1, 1, 64, 128, 128, 64, 0, 6, 1 << 40).decode() == "split"
    assert lib.osdn_forward_path(1, 1, 64, 64, 64, 64, 1, 7, 0).decode() == "two-phase"
    assert _fwd(lib, B=1, H=1, T=64, dk=128, dv=128, chunk=64, flags=2) == _lib.OSDN_ERR_UNSUPPORTED
    assert lib.osdn_forward_workspace_bytes(1, 1, 64, 128, 128, 64, 0, 7) > 0
    assert lib.osdn_step(1, 1, 1, 1, None, None, 0.1, 1, 1, 16, 16, 0, 16, 1, 1, 1, None,
                         None) == _lib.OSDN_ERR_UNSUPPORTED


def test_per_channel_gate_flag(lib):
    """OSDN_GATE_PER_CHANNEL: the multi-launch pipeline on its shapes given its
    (larger) workspace, else the two-phase path (never the single fused kernel);
    alpha is required (validated before any launch)."""
    PC = _lib.OSDN_GATE_PER_CHANNEL
    n = lib.osdn_forward_workspace_bytes(2, 3, 100, 128, 128, 64, 0, PC)
    assert n == 2 * 3 * 2 * (66048 + 768)   # chunk records with K (.) G, Q (.) G and g_L
    assert lib.osdn_forward_workspace_bytes(2, 3, 100, 128, 128, 64, 0, PC | 1) == n
    assert lib.osdn_forward_path(2, 3, 100, 128, 128, 64, 0, PC, n).decode() == "split"
    assert lib.osdn_forward_path(2, 3, 100, 128, 128, 64, 0, PC, n - 1).decode() == "two-phase"
    assert lib.osdn_forward_path(1, 1, 64, 128, 128, 64, 0, PC | 1, 0).decode() == "two-phase"
    assert lib.osdn_forward_path(1, 1, 64, 32, 16, 16, 1, PC | 6, 0).decode() == "two-phase"
    assert lib.osdn_forward_workspace_bytes(2, 3, 100, 64, 64, 64, 1, PC) == 2 * 3 * 100 * 64 * 4
    assert _fwd(lib, B=1, H=1, T=64, dk=128, dv=128, chunk=64, flags=PC) == _lib.OSDN_ERR_NULL
    assert lib.osdn_step(1, 1, 1, 1, None, None, 0.1, 1, 1, 16, 16, 0, PC, 1, 1, 1, None,
                         None) == _lib.OSDN_ERR_NULL


def test_noalloc_rejects_calls_beyond_its_fixed_scratch(lib):
    """osdn_forward_noalloc refuses, before touching the HIP runtime, a call whose
    scratch would exceed OSDN_NOALLOC_MAX_BYTES (dummy pointers: never dereferenced)."""
    p = 1
    need = lib.osdn_forward_workspace_bytes(4, 16, 4096, 128, 128, 64, 0, 0)
    assert need > _lib.OSDN_NOALLOC_MAX_BYTES
    st = lib.osdn_forward_noalloc(p, p, p, p, None, None, None, None, 0.05, 4, 16, 4096, 128, 128,
                                  64, 0, 0, p, None, None, None, None)
    assert st == _lib.OSDN_ERR_TOO_LARGE
    # argument checks come first, as on every entry point
    assert lib.osdn_forward_noalloc(p, p, p, p, None, None, None, None, 0.05, 1, 1, 64, 48, 128,
                                    64, 0, 0, p, None, None, None, None) == _lib.OSDN_ERR_UNSUPPORTED
