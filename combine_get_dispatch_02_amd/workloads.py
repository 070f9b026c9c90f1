"""Seeded synthetic MoE routing workloads (CPU, numpy).

This module only *draws* inputs: token activations ``x`` (bf16 bits),
routing ``topk_idx`` and softmax ``topk_weights``.  It contains none of the
dispatch/combine arithmetic, so that the CPU oracle and the HIP path can both
consume its output without sharing any code of the method.

Shapes follow the expert-parallel problem statement of the page
"[Not ready] MSCCLPP EP implementation #852" (torch-tensor ABI of
``get_dispatch_layout`` / dispatch / combine: x[T,H] bf16, topk_idx[T,k]
int64, topk_weights[T,k] fp32).  The five named workloads are synthetic; two
of them take the shapes that the same page aligns its benchmark knobs to: the
high-throughput default (256 experts, top-8) and the low-latency default (128
tokens, hidden 7168, top-8).

Every draw uses ``numpy.random.default_rng([2026, cfg_id])`` in the fixed
order routing -> logits -> x, so both sides of a parity test see identical
bytes.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Workload", "CONFIGS", "make_workload", "make_routing", "bf16_bits",
           "random_bf16", "expert_outputs", "pooled_expert_outputs", "mask_slots"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """A named problem size plus the routing distribution used to draw it."""
    name: str
    cfg_id: int
    T: int            # tokens
    H: int            # hidden size (bf16 channels)
    k: int            # top-k
    E: int            # experts
    R: int            # destination partitions ("ranks")
    P: int            # partitions per group (two-level grouping)
    routing: str      # "uniform" | "zipf" | "two_level"
    sigma: float = 1.0
    zipf_s: float = 1.2
    confined_frac: float = 0.5
    fp8: bool = False

    @property
    def G(self) -> int:
        return self.R // self.P

    @property
    def N(self) -> int:
        return self.T * self.k

    def describe(self) -> str:
        return (f"{self.name}: T={self.T} H={self.H} k={self.k} E={self.E} "
                f"R={self.R} G={self.G} routing={self.routing}")

    def scaled(self, T: int, H: Optional[int] = None, name: Optional[str] = None) -> "Workload":
        """Same routing law, fewer tokens / channels (for oracle-sized parity runs)."""
        return dataclasses.replace(self, T=T, H=self.H if H is None else H,
                                   name=name or f"{self.name}@T{T}")


# Partitions per group defaults to min(8, R): the pages' two-level layout
# groups 8 GPUs per node.
CONFIGS = {
    "tiny":   Workload("tiny",   1, T=128,   H=256,  k=2, E=16,  R=4,  P=4, routing="uniform"),
    "dsv3":   Workload("dsv3",   2, T=4096,  H=7168, k=8, E=256, R=8,  P=8, routing="uniform"),
    "skewed": Workload("skewed", 3, T=8192,  H=4096, k=6, E=64,  R=8,  P=8, routing="zipf"),
    "ll_fp8": Workload("ll_fp8", 4, T=128,   H=7168, k=8, E=256, R=16, P=8, routing="uniform",
                       sigma=2.0, fp8=True),
    "large":  Workload("large",  5, T=32768, H=7168, k=8, E=256, R=32, P=8, routing="two_level"),
}


def _distinct_uniform(rng: np.random.Generator, T: int, E: int, k: int) -> np.ndarray:
    # A random permutation of the experts per token (argsort of iid uniforms),
    # truncated to k: k distinct experts, uniformly, kept in draw order.
    return np.argsort(rng.random((T, E)), axis=1, kind="stable")[:, :k]


def make_routing(rng: np.random.Generator, wl: Workload) -> np.ndarray:
    """Draw topk_idx [T,k] int64 for the workload's routing law."""
    T, E, k = wl.T, wl.E, wl.k
    if wl.routing == "uniform":
        idx = _distinct_uniform(rng, T, E, k)
    elif wl.routing == "zipf":
        # Without-replacement sampling with p_e proportional to (e+1)^-s via
        # Gumbel-top-k; expert 0 is the most popular, so partition 0 is hot.
        logp = -wl.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
        keys = logp[None, :] + rng.gumbel(size=(T, E))
        idx = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    elif wl.routing == "two_level":
        # Half of the tokens keep all k experts inside one uniformly chosen
        # group of E/G experts; the rest draw from all E.
        G = wl.G
        epg = E // G
        confined = rng.random(T) < wl.confined_frac
        grp = rng.integers(0, G, size=T)
        local = _distinct_uniform(rng, T, epg, k) + epg * grp[:, None]
        glob = _distinct_uniform(rng, T, E, k)
        idx = np.where(confined[:, None], local, glob)
    else:
        raise ValueError(f"unknown routing {wl.routing!r}")
    return np.ascontiguousarray(idx, dtype=np.int64)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def random_bf16(rng: np.random.Generator, rows: int, cols: int, sigma: float = 1.0,
                chunk_rows: int = 2048) -> np.ndarray:
    """N(0, sigma^2) activations as bf16 bits [rows, cols]; drawn in row chunks
    (the generator's stream is consumed in C order, so chunking does not change
    the values)."""
    out = np.empty((rows, cols), dtype=np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        blk = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if sigma != 1.0:
            blk *= np.float32(sigma)
        out[r0:r1] = bf16_bits(blk)
    return out


def _softmax_fp32(logits: np.ndarray) -> np.ndarray:
    l = logits.astype(np.float32)
    m = l.max(axis=1, keepdims=True)
    e = np.exp(l - m, dtype=np.float32)
    return (e / e.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)


def make_workload(wl: Workload, seed_extra: int = 0, with_x: bool = True):
    """Return (x_bits[T,H] uint16 or None, topk_idx[T,k] int64, topk_weights[T,k] fp32)."""
    rng = np.random.default_rng([2026, wl.cfg_id, seed_extra] if seed_extra else [2026, wl.cfg_id])
    idx = make_routing(rng, wl)
    w = _softmax_fp32(rng.standard_normal((wl.T, wl.k), dtype=np.float32))
    x = random_bf16(rng, wl.T, wl.H, wl.sigma) if with_x else None
    return x, idx, np.ascontiguousarray(w, dtype=np.float32)


def expert_outputs(wl: Workload, rows: int, seed_extra: int = 0) -> np.ndarray:
    """Seeded stand-in expert outputs y[rows, H] (bf16 bits), N(0,1)."""
    rng = np.random.default_rng([2026, wl.cfg_id, 7, seed_extra])
    return random_bf16(rng, rows, wl.H, 1.0)


def pooled_expert_outputs(wl: Workload, rows: int, pool_rows: int = 4096, seed_extra: int = 0):
    """Seeded stand-in expert outputs for full-size batches, where drawing
    rows x H normals would dominate a test: y[r] = pool[sel[r]] with pool
    N(0,1) bf16 bits [pool_rows, H] and sel uniform over the pool.  Returns
    (pool, sel), so each side can form y (or index the pool) without the host
    holding rows x H values."""
    rng = np.random.default_rng([2026, wl.cfg_id, 8, seed_extra])
    pool = random_bf16(rng, pool_rows, wl.H, 1.0)
    sel = rng.integers(0, pool_rows, size=rows).astype(np.int32)
    return pool, sel


def mask_slots(idx: np.ndarray, frac: float, seed: int = 0) -> np.ndarray:
    """Copy of idx with a seeded fraction of slots set to -1 (empty slots)."""
    rng = np.random.default_rng([2026, 99, seed])
    out = idx.copy()
    out[rng.random(idx.shape) < frac] = -1
    return out
