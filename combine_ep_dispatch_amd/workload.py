"""Seeded synthetic workloads for MoE expert-parallel dispatch and combine.

This module only draws inputs: token activations, top-k expert ids and
routing probabilities.  It holds none of the dispatch/combine arithmetic, so
that the CPU oracle (under ``oracle/``) and the HIP path can both be fed from
it without sharing any of the method.

Recipe (one ``numpy.random.default_rng(seed)`` PCG64 stream, draws in this
order):

1. ``x      = rng.standard_normal((T, H), float32)``
2. ``U      = rng.random((T, E))``
3. ``logits = rng.standard_normal((T, K)) * sigma``
4. outlier rows (only when ``outlier_frac > 0``):
   ``rng.choice(T, round(outlier_frac * T), replace=False)``; those rows of
   ``x`` are multiplied by ``outlier_scale``.

``x`` is then rounded to bfloat16 (round-to-nearest-even, through torch).
Expert ids are ``K`` distinct experts per token:

* uniform: the first ``K`` columns of a stable argsort of ``U``;
* Zipf(s): Gumbel-top-k sampling without replacement with weights
  ``w_e = (e + 1) ** -s``, i.e. the ``K`` largest ``log w_e - log(-log U)``.

Routing probabilities are the softmax of ``logits`` over the K chosen slots,
taken in float64 and stored as float32 (the router's fp32 output, as the
NeMo AutoModel ``token_dispatcher`` page's ``TokenDispatcherConfig.
moe_router_dtype`` describes).
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Workload", "CONFIGS", "make_workload", "make_tensor_like_rows", "bf16_bits"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Sizes and routing recipe of one synthetic workload."""

    name: str
    T: int                 # tokens of this GPU's share
    H: int                 # hidden size (bf16 elements per token)
    E: int                 # routed experts
    S: int                 # destination segments (modelled EP ranks)
    K: int                 # top-k
    align: int = 1         # per-expert row padding multiple
    capacity: int = 0      # rows per segment (0 = packed, unbounded)
    shared_expert: int = 0 # 1: every token also goes to the shared group
    src_segment: int = 0   # segment that owns the shared expert
    routing: str = "uniform"  # "uniform" | "zipf"
    zipf_s: float = 0.0
    sigma: float = 1.0     # std-dev of the router logits
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    seed: int = 0

    capacity_factor: float = 0.0  # > 0: capacity = factor x mean segment load (recomputed per T)

    @property
    def Kp(self) -> int:
        return self.K + self.shared_expert

    def at_tokens(self, T: int) -> "Workload":
        """The same recipe with T tokens (capacity recomputed from its factor)."""
        cap = self.capacity
        if self.capacity_factor > 0:
            cap = _capacity_rows(T, self.K, self.S, self.capacity_factor, 4)
        return dataclasses.replace(self, T=T, capacity=cap)


def _capacity_rows(T: int, K: int, S: int, factor: float, multiple: int) -> int:
    # Capacity = mean per-segment load times a factor, rounded up to the
    # 4-token slack alignment (NeMo AutoModel token_dispatcher page,
    # _HybridEPManager._calibrate_hybridep_capacity and
    # _HYBRIDEP_TOKEN_ALIGNMENT).  Integer arithmetic only.
    mean_num = T * K  # mean load is T*K / S
    # ceil(factor * T*K / S) with factor = 11/10 exactly
    num = int(round(factor * 10)) * mean_num
    den = 10 * S
    c = -(-num // den)
    return -(-c // multiple) * multiple


CONFIGS = {
    "tiny": Workload("tiny", T=128, H=256, E=8, S=2, K=2, align=16),
    "dsv3": Workload("dsv3", T=4096, H=7168, E=256, S=8, K=8, align=128),
    "skewed": Workload("skewed", T=8192, H=4096, E=128, S=8, K=8, align=128,
                       routing="zipf", zipf_s=1.2, sigma=2.0),
    "nvfp4": Workload("nvfp4", T=4096, H=7168, E=256, S=8, K=8, align=128,
                      shared_expert=1, src_segment=0,
                      outlier_frac=0.01, outlier_scale=50.0),
    "capacity": Workload("capacity", T=16384, H=2048, E=64, S=4, K=6, align=1,
                         capacity=_capacity_rows(16384, 6, 4, 1.1, 4), capacity_factor=1.1,
                         routing="zipf", zipf_s=1.5),
}


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (RNE) through torch and return the uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _route(U: np.ndarray, K: int, routing: str, zipf_s: float) -> np.ndarray:
    if routing == "uniform":
        return np.argsort(U, axis=1, kind="stable")[:, :K].astype(np.int32)
    if routing == "zipf":
        E = U.shape[1]
        logw = -zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
        keys = logw[None, :] - np.log(-np.log(U))
        return np.argsort(-keys, axis=1, kind="stable")[:, :K].astype(np.int32)
    raise ValueError(f"unknown routing {routing!r}")


def make_workload(w: Workload, T: Optional[int] = None, seed: Optional[int] = None,
                  with_x: bool = True) -> dict:
    """Draw the inputs of workload ``w``.

    Returns a dict with ``x`` (uint16 bf16 bits [T, H]), ``topk_ids``
    (int32 [T, K]), ``probs`` (float32 [T, K]) and ``outliers`` (int64 row
    indices).  ``T`` overrides the token count (same recipe, fewer rows).
    """
    T = w.T if T is None else T
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, w.H), dtype=np.float32)
    U = rng.random((T, w.E))
    logits = rng.standard_normal((T, w.K)) * w.sigma
    outliers = np.zeros(0, dtype=np.int64)
    if w.outlier_frac > 0 and T > 0:
        outliers = rng.choice(T, int(round(w.outlier_frac * T)), replace=False)
        x[outliers] *= np.float32(w.outlier_scale)
    ids = _route(U, w.K, w.routing, w.zipf_s) if T > 0 else np.zeros((0, w.K), np.int32)
    z = logits - logits.max(axis=1, keepdims=True) if T > 0 else logits
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True) if T > 0 else 1.0
    out = {
        "topk_ids": np.ascontiguousarray(ids, dtype=np.int32),
        "probs": np.ascontiguousarray(p, dtype=np.float32),
        "outliers": outliers,
    }
    if with_x:
        out["x"] = bf16_bits(x)
    return out


def make_tensor_like_rows(rows: int, H: int, seed: int) -> np.ndarray:
    """Standard-normal bf16 rows (bits), e.g. stand-in expert outputs or gradients."""
    rng = np.random.default_rng(seed)
    return bf16_bits(rng.standard_normal((rows, H), dtype=np.float32))


def min_recv_rows(w: Workload) -> int:
    """Receive rows a caller must allocate for ``w`` without reading counts."""
    if w.capacity > 0:
        return w.S * w.capacity
    routed = w.T * w.Kp
    groups = w.E + w.shared_expert
    return routed + min(routed, groups) * (w.align - 1)


def describe(w: Workload) -> str:
    s = f"{w.name}: T={w.T} H={w.H} E={w.E}/S={w.S} K={w.K}"
    if w.shared_expert:
        s += "+shared"
    s += f" A={w.align}"
    if w.capacity:
        s += f" C={w.capacity}"
    if w.routing == "zipf":
        s += f" zipf({w.zipf_s})"
    return s

