"""Seeded synthetic workloads for the OSDN forward path.

This module only draws inputs; it holds none of the method's arithmetic, so
both the GPU path's tests/benchmark and the fp64 oracle can take their inputs
from it.  Generation is in fp64 with numpy's PCG64, keys and queries are
L2-normalised per token in fp64, the gates go through a logistic sigmoid, and
q/k/v are cast once (round-to-nearest-even) to the stored dtype.  Those stored
bits are the inputs of every implementation.

Draw order per seed: q, k, v, beta-logits, r-logits, alpha-logits (state
gate, gated workloads only; one per key dimension for the per-channel gate).  Raw workloads skip the normalisation and the
sigmoids (the same draws, so their transforms give the plain workload's values
before rounding).  The recall workload draws its key pool, value
pool and index sequence first.

The pages measure on recall/perplexity datasets that are not available here;
the repeated-key workload below stands in for the structure of their
repeated-context ("JRT twice") recall setting: keys come from a fixed pool and
the same index sequence is emitted twice.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int
    dtype: str          # "f32" or "bf16" for q, k, v (and k~, o)
    eta: float
    apf: bool           # retention gate r present
    beta_mu: float = 0.0
    beta_sigma: float = 1.0
    r_mu: float = 3.0
    r_sigma: float = 1.0
    recall_pool: int = 0  # >0: repeated-key recall structure with this pool size
    seed: int = 0
    gated: bool = False   # state gate alpha present (Gated DeltaNet backbone)
    alpha_mu: float = 3.0
    alpha_sigma: float = 1.0
    gate_channels: bool = False  # with gated: one gate per key dimension (KDA backbone)
    raw: bool = False     # q, k not normalised and beta, r as logits (the kernels transform them)

    @property
    def tokens(self) -> int:
        return self.B * self.T

    @property
    def token_heads(self) -> int:
        return self.B * self.H * self.T


# The five measured configurations (sizes, distributions and step sizes as
# specified for this path).
TINY_F32 = Workload("tiny-f32 B1 H1 T256 d16 C16", 1, 1, 256, 16, 16, 16, "f32", 0.1, False,
                    seed=1001)
L340M_VANILLA = Workload("340M-layer vanilla B8 H8 T2048 d128 C64 bf16", 8, 8, 2048, 128, 128, 64,
                         "bf16", 0.05, False, seed=1002)
L340M_APF = Workload("340M-layer APF B8 H8 T2048 d128 C64 bf16", 8, 8, 2048, 128, 128, 64,
                     "bf16", 0.05, True, seed=1003)
L13B_APF = Workload("1.3B-layer APF B4 H16 T4096 d128 C64 bf16", 4, 16, 4096, 128, 128, 64,
                    "bf16", 0.05, True, seed=1004)
RECALL_VANILLA = Workload("recall x2 vanilla B2 H16 T16384 d128 C64 bf16", 2, 16, 16384, 128, 128,
                          64, "bf16", 0.05, False, beta_mu=1.0, beta_sigma=0.5, recall_pool=512,
                          seed=1005)
RECALL_APF = replace(RECALL_VANILLA, name="recall x2 APF B2 H16 T16384 d128 C64 bf16", apf=True)

# The 1.3B-style layer on the Gated DeltaNet backbone: the same draws plus a
# per-token state gate alpha = sigmoid(3 + N(0,1)) (mostly 0.88..0.98).
L13B_APF_GATED = replace(L13B_APF, name="1.3B-layer APF gated B4 H16 T4096 d128 C64 bf16",
                         gated=True)

# The same layer on the Kimi Delta Attention backbone: one gate per key
# dimension, alpha[..., i] = sigmoid(3 + N(0,1)) drawn independently.
L13B_APF_KDA = replace(L13B_APF, name="1.3B-layer APF per-channel gate B4 H16 T4096 d128 C64 bf16",
                       gated=True, gate_channels=True)

CONFIGS = {
    "tiny": TINY_F32,
    "340m": L340M_VANILLA,
    "340m-apf": L340M_APF,
    "1.3b-apf": L13B_APF,
    "recall": RECALL_VANILLA,
    "recall-apf": RECALL_APF,
    "1.3b-apf-gated": L13B_APF_GATED,
    "1.3b-apf-kda": L13B_APF_KDA,
}

# The throughput metric is quoted on the 1.3B-style layer (H=16, dk=dv=128, T=4096).
METRIC_WORKLOAD = L13B_APF

# One decoding step of a batch of 64 sequences on the same layer shape (the
# persistent-state update): q, k, v of one token per (b, h), APF gates.
DECODE = Workload("decode step B64 H16 d128 bf16 APF", 64, 16, 1, 128, 128, 64, "bf16", 0.05,
                  True, seed=1006)


def custom(B, H, T, dk, dv, chunk, dtype="bf16", eta=0.05, apf=False, seed=7, **kw) -> Workload:
    name = "custom B%d H%d T%d dk%d dv%d C%d %s%s" % (B, H, T, dk, dv, chunk, dtype,
                                                       " APF" if apf else "")
    return Workload(name, B, H, T, dk, dv, chunk, dtype, eta, apf, seed=seed, **kw)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _l2n(x):
    n = np.sqrt(np.einsum("...i,...i->...", x, x))[..., None]
    x /= np.where(n > 0, n, 1.0)
    return x


def _store(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.float32) if dtype == "f32" else t.to(torch.bfloat16)


@dataclass
class Inputs:
    q: torch.Tensor        # [B,H,T,dk] stored dtype
    k: torch.Tensor        # [B,H,T,dk]
    v: torch.Tensor        # [B,H,T,dv]
    beta: torch.Tensor     # [B,H,T] fp32
    r: Optional[torch.Tensor]  # [B,H,T] fp32 or None (no APF)
    eta: float
    workload: Workload
    alpha: Optional[torch.Tensor] = None  # [B,H,T] (or [B,H,T,dk]) fp32 state gate or None

    def to(self, device):
        mv = lambda t: None if t is None else t.to(device)
        return Inputs(mv(self.q), mv(self.k), mv(self.v), mv(self.beta), mv(self.r), self.eta,
                      self.workload, mv(self.alpha))


def generate(w: Workload, seed: Optional[int] = None) -> Inputs:
    """Draw the workload's inputs on the CPU (fp64 -> stored dtype)."""
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    if w.recall_pool > 0:
        P = w.recall_pool
        keys = _l2n(rng.standard_normal((H, P, dk)))          # per-head key pool
        vals = rng.standard_normal((H, P, dv))                 # paired values
        half = T // 2
        idx = rng.integers(0, P, size=(B, half))               # per-batch index sequence
        idx = np.concatenate([idx, idx, idx[:, : T - 2 * half]], axis=1)
        k = np.empty((B, H, T, dk))
        v = np.empty((B, H, T, dv))
        for b in range(B):
            k[b] = keys[:, idx[b], :]
            v[b] = vals[:, idx[b], :]
        q = k.copy()                                           # queries are the keys
    else:
        q = rng.standard_normal((B, H, T, dk))
        k = rng.standard_normal((B, H, T, dk))
        if not w.raw:
            q, k = _l2n(q), _l2n(k)
        v = rng.standard_normal((B, H, T, dv))
    gate = (lambda x: x) if w.raw else _sigmoid
    beta = gate(w.beta_mu + w.beta_sigma * rng.standard_normal((B, H, T)))
    r = gate(w.r_mu + w.r_sigma * rng.standard_normal((B, H, T))) if w.apf else None
    gshape = (B, H, T, dk) if w.gate_channels else (B, H, T)
    alpha = (_sigmoid(w.alpha_mu + w.alpha_sigma * rng.standard_normal(gshape))
             if w.gated else None)
    f32 = lambda x: None if x is None else torch.from_numpy(x).to(torch.float32)
    return Inputs(_store(q, w.dtype), _store(k, w.dtype), _store(v, w.dtype), f32(beta), f32(r),
                  float(w.eta), w, f32(alpha))
