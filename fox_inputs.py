"""Seeded synthetic inputs for causal FoX attention (shared by tests, bench, oracle checks).

This module only draws numbers; it holds none of the attention arithmetic.
The one transformation it applies is the gate recipe of the workloads
(``log f = logsigmoid(logit)``, the sigmoid forget gate of the FoX module page,
``ForgettingAttention.forward``, taken in log space without the module's 1e-6
epsilon), which produces the kernel *input* ``log f``.

Recipe (all CPU, one ``torch.Generator`` per slab, fixed draw order):

* forward workloads: per batch index b, a generator seeded with
  ``_slab_seed(tag, seed, b)`` draws Q[b], K[b], V[b] (each [H,N,d], N(0,1) in
  fp32, then rounded to bf16 with round-to-nearest-even when the dtype is bf16)
  and then the gate logits [H,N] ~ N(mu, sigma) in fp32;
* decode workload: per sequence s, a generator seeded with
  ``_slab_seed(tag, seed, s)`` draws q[s] [H,d], K[s] [H,L,d], V[s] [H,L,d] and
  the gate logits [H,L]; ``logf_all[..., :L-1]`` is the history whose prefix
  sums form the cache and ``logf_all[..., L-1]`` is the new token's gate.

Because every slab has its own seed, any slab can be regenerated alone (the
oracle's sampled checks at full size do exactly that).
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass, replace

import torch

__all__ = ["FwdConfig", "DecodeConfig", "FWD", "DECODE", "fwd_inputs", "decode_inputs", "digest"]


@dataclass(frozen=True)
class FwdConfig:
    tag: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32" or "bf16" (Q, K, V and O); log f is always fp32
    mu: float = 0.0
    sigma: float = 1.0
    gate: str = "logsigmoid"  # "logsigmoid" | "ones" (log f = 0) | "const" (log f = -m)
    m: float = 0.0

    @property
    def desc(self) -> str:
        g = {"logsigmoid": f"gate logits N({self.mu:g},{self.sigma:g})", "ones": "f=1",
             "const": f"f=exp(-{self.m:g})"}[self.gate]
        return f"fox_attn_fwd {self.dtype} B={self.B} H={self.H} N={self.N} d={self.d}, {g}"


@dataclass(frozen=True)
class DecodeConfig:
    tag: str
    S: int
    H: int
    L: int
    d: int
    dtype: str
    mu: float
    sigma: float

    @property
    def desc(self) -> str:
        return (f"fox_attn_decode {self.dtype} S={self.S} H={self.H} L={self.L} d={self.d}, "
                f"gate logits N({self.mu:g},{self.sigma:g})")


# The five workloads: shapes, dtypes and gate distributions.
FWD = {
    "c1": FwdConfig("c1", 1, 2, 128, 32, "f32", 2.0, 1.0),
    "c2": FwdConfig("c2", 4, 12, 1024, 64, "bf16", 3.0, 1.5),
    "c2_f1": FwdConfig("c2_f1", 4, 12, 1024, 64, "bf16", 3.0, 1.5, gate="ones"),
    "c2_alibi": FwdConfig("c2_alibi", 4, 12, 1024, 64, "bf16", 3.0, 1.5, gate="const", m=0.05),
    "c3": FwdConfig("c3", 2, 16, 4096, 128, "bf16", 4.0, 2.0),
    "c4": FwdConfig("c4", 1, 32, 16384, 128, "bf16", 6.0, 1.0),
}
DECODE = {
    "c5": DecodeConfig("c5", 64, 32, 8192, 128, "bf16", 4.0, 2.0),
}

_TAG_ID = {"c1": 1, "c2": 2, "c2_f1": 2, "c2_alibi": 2, "c3": 3, "c4": 4, "c5": 5}


def _slab_seed(tag: str, seed: int, slab: int) -> int:
    base = _TAG_ID.get(tag)
    if base is None:  # ad-hoc shapes: stable id from the tag text
        base = 100 + int(hashlib.sha256(tag.encode()).hexdigest()[:6], 16)
    return (base * 1_000_003 + seed * 65_537 + slab) & 0x7FFF_FFFF_FFFF


def _torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _gate_logf(logits: torch.Tensor, cfg) -> torch.Tensor:
    """Kernel input log f from the drawn logits, per the workload's gate recipe."""
    gate = getattr(cfg, "gate", "logsigmoid")
    if gate == "ones":
        return torch.zeros_like(logits, dtype=torch.float32)
    if gate == "const":
        return torch.full_like(logits, -cfg.m, dtype=torch.float32)
    return torch.nn.functional.logsigmoid(logits.double()).float()


def fwd_inputs(cfg: FwdConfig, seed: int = 0, **override) -> dict:
    """Q, K, V [B,H,N,d] (cfg.dtype) and log f [B,H,N] (fp32), CPU tensors.

    ``override`` replaces fields of ``cfg`` (e.g. ``N=77`` for a ragged case).
    """
    if override:
        cfg = replace(cfg, **override)
    dt = _torch_dtype(cfg.dtype)
    q = torch.empty(cfg.B, cfg.H, cfg.N, cfg.d, dtype=dt)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    logf = torch.empty(cfg.B, cfg.H, cfg.N, dtype=torch.float32)
    for b in range(cfg.B):
        g = torch.Generator().manual_seed(_slab_seed(cfg.tag, seed, b))
        for t in (q, k, v):
            t[b] = torch.randn(cfg.H, cfg.N, cfg.d, generator=g).to(dt)
        logits = torch.randn(cfg.H, cfg.N, generator=g) * cfg.sigma + cfg.mu
        logf[b] = _gate_logf(logits, cfg)
    return {"q": q, "k": k, "v": v, "logf": logf, "scale": float(torch.tensor(cfg.d ** -0.5, dtype=torch.float32)),
            "cfg": cfg}


def decode_slab(cfg: DecodeConfig, seed: int, s: int, out=None):
    """One sequence's draws: q [H,d], K [H,L,d], V [H,L,d] (cfg.dtype), log f [H,L] fp32.

    ``out`` = (q, k, v, logf) destination views to fill in place (same values; avoids
    re-faulting fresh host pages for every slab of a large cache).
    """
    dt = _torch_dtype(cfg.dtype)
    g = torch.Generator().manual_seed(_slab_seed(cfg.tag, seed, s))
    if out is None:
        out = (torch.empty(cfg.H, cfg.d, dtype=dt), torch.empty(cfg.H, cfg.L, cfg.d, dtype=dt),
               torch.empty(cfg.H, cfg.L, cfg.d, dtype=dt), torch.empty(cfg.H, cfg.L, dtype=torch.float32))
    oq, ok, ov, ol = out
    oq.copy_(torch.randn(cfg.H, cfg.d, generator=g))
    buf = torch.empty(cfg.H, cfg.L, cfg.d)
    for dst in (ok, ov):
        buf.normal_(generator=g)  # same stream as torch.randn(..., generator=g)
        dst.copy_(buf)
    logits = torch.randn(cfg.H, cfg.L, generator=g) * cfg.sigma + cfg.mu
    ol.copy_(_gate_logf(logits, cfg))
    return out


def decode_inputs(cfg: DecodeConfig, seed: int = 0, seqs=None, **override) -> dict:
    """q [S,H,d], K, V caches [S,H,L,d] (new token at slot L-1), log f history [S,H,L] fp32.

    ``logf_all[..., :L-1]`` are the gates whose prefix sums fill the cache;
    ``logf_all[..., L-1]`` is the new token's gate.  ``seqs`` selects a subset
    of sequence indices (each regenerated from its own seed).
    """
    if override:
        cfg = replace(cfg, **override)
    seqs = list(range(cfg.S)) if seqs is None else list(seqs)
    dt = _torch_dtype(cfg.dtype)
    S = len(seqs)
    q = torch.empty(S, cfg.H, cfg.d, dtype=dt)
    k = torch.empty(S, cfg.H, cfg.L, cfg.d, dtype=dt)
    v = torch.empty_like(k)
    logf = torch.empty(S, cfg.H, cfg.L, dtype=torch.float32)
    for i, s in enumerate(seqs):
        decode_slab(cfg, seed, s, out=(q[i], k[i], v[i], logf[i]))
    return {"q": q, "k": k, "v": v, "logf_all": logf,
            "scale": float(torch.tensor(cfg.d ** -0.5, dtype=torch.float32)), "cfg": cfg, "seqs": seqs}


def digest(*tensors: torch.Tensor) -> str:
    """SHA-256 over the raw bytes of the given CPU tensors (logged so both sides provably saw the same inputs)."""
    h = hashlib.sha256()
    for t in tensors:
        h.update(t.contiguous().reshape(-1).view(torch.uint8).numpy())
    return h.hexdigest()[:16]
