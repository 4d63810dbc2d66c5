"""OSDN (Online Scaled DeltaNet) forward hot path for AMD MI355X (gfx950).

Python face of libosdn.so.  The functions mirror the C ABI of include/osdn.h:

  precond_scan(k, beta, r, d0, eta)            phase 1: the preconditioner walk
  chunk_fwd(q, k, k_tilde, v, beta, S0, chunk)  phase 2: chunkwise pass with k~
  forward(q, k, v, beta, r, d0, S0, eta, chunk) both phases

Tensors are torch tensors on a ROCm device, contiguous, in the [B,H,T,D]
layout; q/k/v/k~/o are bfloat16 or float32, gates and states float32.  Outputs
are allocated with torch on the inputs' device and the work is enqueued on the
current stream.  Source of the method: gist.science technical summary of
"OSDN: Improving Delta Rule with Provable Online Preconditioning in Linear
Attention" (arXiv 2605.13473).
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib
from ._lib import OsdnError, load  # noqa: F401

__all__ = ["precond_scan", "chunk_fwd", "forward", "forward_noalloc", "step",
           "forward_workspace_bytes", "forward_path",
           "precond_scan_workspace_bytes", "chunk_fwd_workspace_bytes",
           "OsdnError", "load"]


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.OSDN_BF16
    if t.dtype == torch.float32:
        return _lib.OSDN_F32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % t.dtype)


def _dev(t: Optional[torch.Tensor], name: str, shape=None, dtype=None, device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a ROCm device (got %s); there is no CPU path" %
                         (name, t.device))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    return t


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def precond_scan_workspace_bytes(B, H, T, dk, dtype_code) -> int:
    n = _lib.load().osdn_precond_scan_workspace_bytes(B, H, T, dk, dtype_code)
    if n == (1 << 64) - 1:
        raise ValueError("invalid arguments for osdn_precond_scan")
    return int(n)


def precond_scan(k, beta, r=None, d0=None, eta=0.05, *, want_d_all=False, want_log_ratio=False,
                 workspace=True):
    """Phase 1.  Returns dict(k_tilde, d_final[, d_all][, log_ratio]).

    ``workspace``: True allocates the scratch that selects the three-launch
    walk (when it exists for these shapes), a uint8 device tensor passes one,
    None runs the single-kernel walk."""
    _dev(k, "k")
    B, H, T, dk = k.shape
    dev = k.device
    _dev(beta, "beta", (B, H, T), torch.float32, dev)
    _dev(r, "r", (B, H, T), torch.float32, dev)
    _dev(d0, "d0", (B, H, dk), torch.float32, dev)
    out = {
        "k_tilde": torch.empty_like(k),
        "d_final": torch.empty((B, H, dk), dtype=torch.float32, device=dev),
    }
    if want_d_all:
        out["d_all"] = torch.empty((B, H, T, dk), dtype=torch.float32, device=dev)
    if want_log_ratio:
        out["log_ratio"] = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    if workspace is True:
        n = precond_scan_workspace_bytes(B, H, T, dk, _dtype_code(k))
        workspace = torch.empty(n, dtype=torch.uint8, device=dev) if n else None
    ws_bytes = 0 if workspace is None else workspace.numel()
    st = _lib.load().osdn_precond_scan(
        _ptr(k), _ptr(beta), _ptr(r), _ptr(d0), float(eta), B, H, T, dk, _dtype_code(k),
        _ptr(out["k_tilde"]), _ptr(out["d_final"]), _ptr(out.get("d_all")),
        _ptr(out.get("log_ratio")), _ptr(workspace), ws_bytes, _stream(dev))
    _lib.check("osdn_precond_scan", st)
    return out


def chunk_fwd_workspace_bytes(B, H, T, dk, dv, chunk, dtype_code, per_channel=False) -> int:
    n = _lib.load().osdn_chunk_fwd_workspace_bytes(
        B, H, T, dk, dv, chunk, dtype_code, _lib.OSDN_GATE_PER_CHANNEL if per_channel else 0)
    if n == (1 << 64) - 1:
        raise ValueError("invalid arguments for osdn_chunk_fwd")
    return int(n)


def chunk_fwd(q, k, k_tilde, v, beta, S0=None, chunk=64, *, alpha=None, workspace=True):
    """Phase 2 with a given write key k~.  Returns (o, S_final).

    ``alpha`` [B,H,T] fp32 is the optional state gate ([B,H,T,dk]: one gate per
    key dimension).  ``workspace``: True
    allocates the scratch that selects the chunk-parallel path (when one exists
    for these shapes), a uint8 device tensor passes one, None runs the
    single-kernel pass."""
    _dev(q, "q")
    B, H, T, dk = q.shape
    dev = q.device
    _dev(k, "k", q.shape, q.dtype, dev)
    _dev(k_tilde, "k_tilde", q.shape, q.dtype, dev)
    _dev(v, "v", None, q.dtype, dev)
    if v.shape[:3] != (B, H, T):
        raise ValueError("v has shape %s, expected [%d,%d,%d,dv]" % (tuple(v.shape), B, H, T))
    dv = v.shape[3]
    _dev(beta, "beta", (B, H, T), torch.float32, dev)
    chan = alpha is not None and alpha.dim() == 4
    _dev(alpha, "alpha", (B, H, T, dk) if chan else (B, H, T), torch.float32, dev)
    _dev(S0, "S0", (B, H, dv, dk), torch.float32, dev)
    o = torch.empty_like(v)
    S_final = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    if workspace is True:
        n = chunk_fwd_workspace_bytes(B, H, T, dk, dv, int(chunk), _dtype_code(q), chan)
        workspace = torch.empty(n, dtype=torch.uint8, device=dev) if n else None
    ws_bytes = 0 if workspace is None else workspace.numel()
    st = _lib.load().osdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(k_tilde), _ptr(v), _ptr(beta),
                                    _ptr(alpha), _ptr(S0), B, H, T, dk, dv, int(chunk), _dtype_code(q),
                                    _lib.OSDN_GATE_PER_CHANNEL if chan else 0,
                                    _ptr(o), _ptr(S_final), _ptr(workspace), ws_bytes,
                                    _stream(dev))
    _lib.check("osdn_chunk_fwd", st)
    return o, S_final


def _transform_flags(norm_qk, gate_logits):
    return (_lib.OSDN_NORM_QK if norm_qk else 0) | (_lib.OSDN_GATE_LOGITS if gate_logits else 0)


def step(q, k, v, beta, S, d, r=None, eta=0.05, *, alpha=None, o=None, want_log_ratio=False,
         norm_qk=False, gate_logits=False):
    """One decoding step.  q, k [B,H,dk], v [B,H,dv] (bf16 or fp32), beta, r and
    the optional state gate alpha [B,H] fp32 (or [B,H,dk]: one gate per key
    dimension); S [B,H,dv,dk] and d [B,H,dk] fp32 are updated in place.  ``norm_qk``: q, k are unnormalised (the kernel
    divides them by their norms); ``gate_logits``: beta, r are logits.
    Returns dict(o[, log_ratio])."""
    _dev(q, "q")
    B, H, dk = q.shape
    dev = q.device
    _dev(k, "k", q.shape, q.dtype, dev)
    _dev(v, "v", None, q.dtype, dev)
    if v.dim() != 3 or v.shape[:2] != (B, H):
        raise ValueError("v has shape %s, expected [%d,%d,dv]" % (tuple(v.shape), B, H))
    dv = v.shape[2]
    _dev(beta, "beta", (B, H), torch.float32, dev)
    _dev(r, "r", (B, H), torch.float32, dev)
    chan = alpha is not None and alpha.dim() == 3
    _dev(alpha, "alpha", (B, H, dk) if chan else (B, H), torch.float32, dev)
    _dev(S, "S", (B, H, dv, dk), torch.float32, dev)
    _dev(d, "d", (B, H, dk), torch.float32, dev)
    o = torch.empty_like(v) if o is None else o
    lr = torch.empty((B, H), dtype=torch.float32, device=dev) if want_log_ratio else None
    st = _lib.load().osdn_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(r), _ptr(alpha),
                               float(eta), B, H, dk, dv, _dtype_code(q),
                               _transform_flags(norm_qk, gate_logits)
                               | (_lib.OSDN_GATE_PER_CHANNEL if chan else 0),
                               _ptr(S), _ptr(d), _ptr(o),
                               _ptr(lr), _stream(dev))
    _lib.check("osdn_step", st)
    out = {"o": o}
    if want_log_ratio:
        out["log_ratio"] = lr
    return out


def forward_workspace_bytes(B, H, T, dk, dv, chunk, dtype_code, precond=True,
                            per_channel=False) -> int:
    flags = ((0 if precond else _lib.OSDN_PRECOND_OFF)
             | (_lib.OSDN_GATE_PER_CHANNEL if per_channel else 0))
    n = _lib.load().osdn_forward_workspace_bytes(B, H, T, dk, dv, chunk, dtype_code, flags)
    if n == (1 << 64) - 1:
        raise ValueError("invalid arguments for osdn_forward")
    return int(n)


def forward_path(B, H, T, dk, dv, chunk, dtype_code, precond=True, workspace_bytes=0,
                 per_channel=False) -> str:
    flags = ((0 if precond else _lib.OSDN_PRECOND_OFF)
             | (_lib.OSDN_GATE_PER_CHANNEL if per_channel else 0))
    return _lib.load().osdn_forward_path(B, H, T, dk, dv, chunk, dtype_code, flags,
                                         int(workspace_bytes)).decode()


def forward(q, k, v, beta, r=None, d0=None, S0=None, eta=0.05, chunk=64, precond=True,
            *, alpha=None, out=None, workspace=True, norm_qk=False, gate_logits=False):
    """Both phases.  Returns dict(o, S_final, d_final, log_ratio_sum).

    ``norm_qk``: q and k are unnormalised and the kernels divide each by its L2
    norm; ``gate_logits``: beta and r are logits and the kernels take their
    sigmoid (multi-launch and two-phase paths; the single fused kernel refuses
    them).

    ``alpha`` [B,H,T] fp32 is the optional state gate (Gated DeltaNet backbone;
    with precond=False, Gated DeltaNet itself); [B,H,T,dk] is the per-channel
    gate, one per key dimension (Kimi Delta Attention backbone), which runs on
    the two-phase path.

    ``out`` may pass preallocated outputs (same keys) to keep the call free of
    allocations.  ``workspace``: True allocates the scratch of the fastest path
    (forward_workspace_bytes), a uint8 device tensor passes one, None passes
    only what the path requires (none on the shapes of the single fused
    kernel, which then runs).
    """
    _dev(q, "q")
    B, H, T, dk = q.shape
    dev = q.device
    _dev(k, "k", q.shape, q.dtype, dev)
    _dev(v, "v", None, q.dtype, dev)
    if v.shape[:3] != (B, H, T):
        raise ValueError("v has shape %s, expected [%d,%d,%d,dv]" % (tuple(v.shape), B, H, T))
    dv = v.shape[3]
    _dev(beta, "beta", (B, H, T), torch.float32, dev)
    _dev(r, "r", (B, H, T), torch.float32, dev)
    chan = alpha is not None and alpha.dim() == 4
    _dev(alpha, "alpha", (B, H, T, dk) if chan else (B, H, T), torch.float32, dev)
    _dev(d0, "d0", (B, H, dk), torch.float32, dev)
    _dev(S0, "S0", (B, H, dv, dk), torch.float32, dev)
    code = _dtype_code(q)
    flags = ((0 if precond else _lib.OSDN_PRECOND_OFF) | _transform_flags(norm_qk, gate_logits)
             | (_lib.OSDN_GATE_PER_CHANNEL if chan else 0))
    if out is None:
        out = {
            "o": torch.empty_like(v),
            "S_final": torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev),
            "d_final": (torch.empty((B, H, dk), dtype=torch.float32, device=dev)
                        if precond else None),
            "log_ratio_sum": torch.empty((B, H), dtype=torch.float32, device=dev),
        }
    single = forward_path(B, H, T, dk, dv, chunk, code, precond, per_channel=chan) == "fused"
    if workspace is True or (workspace is None and not single):
        need = forward_workspace_bytes(B, H, T, dk, dv, chunk, code, precond, per_channel=chan)
        workspace = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.load().osdn_forward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(r), _ptr(alpha), _ptr(d0), _ptr(S0),
        float(eta),
        B, H, T, dk, dv, int(chunk), code, flags, _ptr(out["o"]), _ptr(out.get("S_final")),
        _ptr(out.get("d_final")), _ptr(out.get("log_ratio_sum")), _ptr(workspace), ws_bytes,
        _stream(dev))
    _lib.check("osdn_forward", st)
    return out


def forward_noalloc(q, k, v, beta, r=None, d0=None, S0=None, eta=0.05, chunk=64, precond=True,
                    *, alpha=None, out=None, norm_qk=False, gate_logits=False):
    """osdn_forward_noalloc: the forward with its scratch in the library's fixed
    device array (OSDN_NOALLOC_MAX_BYTES per GPU) instead of a workspace.  Same
    arguments and results as forward(); with ``out`` given the call allocates
    nothing.  Calls that overlap on one GPU race on that array."""
    _dev(q, "q")
    B, H, T, dk = q.shape
    dev = q.device
    _dev(k, "k", q.shape, q.dtype, dev)
    _dev(v, "v", None, q.dtype, dev)
    if v.shape[:3] != (B, H, T):
        raise ValueError("v has shape %s, expected [%d,%d,%d,dv]" % (tuple(v.shape), B, H, T))
    dv = v.shape[3]
    _dev(beta, "beta", (B, H, T), torch.float32, dev)
    _dev(r, "r", (B, H, T), torch.float32, dev)
    chan = alpha is not None and alpha.dim() == 4
    _dev(alpha, "alpha", (B, H, T, dk) if chan else (B, H, T), torch.float32, dev)
    _dev(d0, "d0", (B, H, dk), torch.float32, dev)
    _dev(S0, "S0", (B, H, dv, dk), torch.float32, dev)
    flags = ((0 if precond else _lib.OSDN_PRECOND_OFF) | _transform_flags(norm_qk, gate_logits)
             | (_lib.OSDN_GATE_PER_CHANNEL if chan else 0))
    if out is None:
        out = {
            "o": torch.empty_like(v),
            "S_final": torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev),
            "d_final": (torch.empty((B, H, dk), dtype=torch.float32, device=dev)
                        if precond else None),
            "log_ratio_sum": torch.empty((B, H), dtype=torch.float32, device=dev),
        }
    st = _lib.load().osdn_forward_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(r), _ptr(alpha), _ptr(d0), _ptr(S0),
        float(eta), B, H, T, dk, dv, int(chunk), _dtype_code(q), flags, _ptr(out["o"]),
        _ptr(out.get("S_final")), _ptr(out.get("d_final")), _ptr(out.get("log_ratio_sum")),
        _stream(dev))
    _lib.check("osdn_forward_noalloc", st)
    return out
