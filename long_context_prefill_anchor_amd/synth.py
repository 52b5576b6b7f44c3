"""Seeded synthetic inputs shared by the GPU path, the oracle tests and the bench.

This module holds no routing arithmetic: it only draws drifting chunk
representations and encodes them in the dtype the routing kernels read.

Recipe (one ``numpy.random.default_rng(seed)`` stream, PCG64, draws in this order):
  1. if the workload's drift is a range (lo, hi): sigma_l ~ U[lo, hi) for l = 0..L-1
     (sigma_0 is drawn and unused: layer 0 has no predecessor);
  2. Q^0 then K^0, each [H, n, d] float32 standard normal, scaled by 1/sqrt(d);
  3. for l = 1..L-1: dQ then dK, each [H, n, d] float32 standard normal, and
     Q^l = Q^{l-1} + step_l * dQ, K^l = K^{l-1} + step_l * dK in float32, with
     step_l = sigma_l ("absolute") or sigma_l / sqrt(d) ("relative").
The walk stays in float32; bf16 workloads hand out round-to-nearest-even bf16
copies of each layer (the walk itself is never re-rounded).

Workloads with ``drift_model == "local"`` (the persistent-preferred-chunk setting,
RouteRelay Section 5.1) use instead, from the same kind of stream:
  1. sigma_l as above;
  2. base Q then base K, [H, nq, d] and [H, nk, d], N(0,1)/sqrt(d);
  3. per head, each query row's preferred chunks: the first ``preferred`` entries of
     ``rng.permutation(nk)`` drawn row by row; the row's base query gains
     pref_gain * (sum of the base keys of its preferred chunks) / sqrt(preferred);
  4. for l = 0..L-1: dQ then dK as above and Q^l = base Q + step_l * dQ,
     K^l = base K + step_l * dK (the drift is local to each layer; it does not accumulate).
Where the pages leave that generator open (preference strength, how preferences enter the
vectors) these are this module's choices.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Iterator

import numpy as np

from .workloads import Workload


def fp32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) and return the raw uint16 bits.

    Inputs are finite by construction (Gaussian draws), so no NaN handling.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = u + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_fp32(b: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bits to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class LayerInput:
    layer: int
    sigma: float
    q: np.ndarray   # float32 [H, n, d] or uint16 bf16 bits [H, n, d]
    k: np.ndarray


def layer_sigmas(w: Workload, rng: np.random.Generator) -> np.ndarray:
    lo, hi = w.drift
    if lo == hi:
        return np.full(w.layers, lo, dtype=np.float64)
    return rng.uniform(lo, hi, size=w.layers)


def generate(w: Workload, heads: slice | None = None) -> Iterator[LayerInput]:
    """Yield the workload's layers one at a time (only one layer is held in memory).

    ``heads`` optionally restricts the *returned* arrays to a head slice; the
    random stream is always drawn for all heads so a slice sees the same values
    as the full run.
    """
    if w.drift_model == "local":
        yield from _generate_local(w, heads)
        return
    rng = np.random.default_rng(w.seed)
    sig = layer_sigmas(w, rng)
    shape = (w.heads, w.n, w.d)
    inv = np.float32(1.0 / np.sqrt(w.d))
    q = rng.standard_normal(shape, dtype=np.float32) * inv
    k = rng.standard_normal(shape, dtype=np.float32) * inv
    sel = heads if heads is not None else slice(None)

    def emit(layer: int) -> LayerInput:
        qs, ks = q[sel], k[sel]
        if w.dtype == "bf16":
            return LayerInput(layer, float(sig[layer]), fp32_to_bf16_bits(qs), fp32_to_bf16_bits(ks))
        return LayerInput(layer, float(sig[layer]), np.ascontiguousarray(qs), np.ascontiguousarray(ks))

    yield emit(0)
    for layer in range(1, w.layers):
        step = sig[layer] if w.drift_scale == "absolute" else sig[layer] / np.sqrt(w.d)
        step32 = np.float32(step)
        q = q + step32 * rng.standard_normal(shape, dtype=np.float32)
        k = k + step32 * rng.standard_normal(shape, dtype=np.float32)
        yield emit(layer)


def _generate_local(w: Workload, heads: slice | None) -> Iterator[LayerInput]:
    """Persistent preferred chunks plus layer-local drift (recipe in the module docstring)."""
    rng = np.random.default_rng(w.seed)
    sig = layer_sigmas(w, rng)
    inv = np.float32(1.0 / np.sqrt(w.d))
    qb = rng.standard_normal((w.heads, w.nq, w.d), dtype=np.float32) * inv
    kb = rng.standard_normal((w.heads, w.nk, w.d), dtype=np.float32) * inv
    if w.preferred > 0:
        gain = np.float32(w.pref_gain / np.sqrt(w.preferred))
        for h in range(w.heads):
            for i in range(w.nq):
                pref = rng.permutation(w.nk)[: w.preferred]
                qb[h, i] += gain * kb[h, pref].sum(axis=0, dtype=np.float32)
    sel = heads if heads is not None else slice(None)
    for layer in range(w.layers):
        step = sig[layer] if w.drift_scale == "absolute" else sig[layer] / np.sqrt(w.d)
        step32 = np.float32(step)
        q = qb + step32 * rng.standard_normal(qb.shape, dtype=np.float32)
        k = kb + step32 * rng.standard_normal(kb.shape, dtype=np.float32)
        qs, ks = q[sel], k[sel]
        if w.dtype == "bf16":
            yield LayerInput(layer, float(sig[layer]), fp32_to_bf16_bits(qs), fp32_to_bf16_bits(ks))
        else:
            yield LayerInput(layer, float(sig[layer]), np.ascontiguousarray(qs), np.ascontiguousarray(ks))


def integer_inputs(heads: int, n: int, d: int, seed: int, lo: int = -2, hi: int = 2,
                   dtype: str = "f32") -> tuple[np.ndarray, np.ndarray]:
    """Q, K with integer entries in [lo, hi]: every score is an exact small integer
    in fp32 and in bf16, so ties are frequent and decided only by chunk index."""
    rng = np.random.default_rng(seed)
    q = rng.integers(lo, hi + 1, size=(heads, n, d)).astype(np.float32)
    k = rng.integers(lo, hi + 1, size=(heads, n, d)).astype(np.float32)
    if dtype == "bf16":
        return fp32_to_bf16_bits(q), fp32_to_bf16_bits(k)
    return q, k


def gaussian_inputs(heads: int, nq: int, nk: int, d: int, seed: int,
                    dtype: str = "f32") -> tuple[np.ndarray, np.ndarray]:
    """One layer of N(0,1)/sqrt(d) chunk vectors (nq may differ from nk)."""
    rng = np.random.default_rng(seed)
    inv = np.float32(1.0 / np.sqrt(d))
    q = rng.standard_normal((heads, nq, d), dtype=np.float32) * inv
    k = rng.standard_normal((heads, nk, d), dtype=np.float32) * inv
    if dtype == "bf16":
        return fp32_to_bf16_bits(q), fp32_to_bf16_bits(k)
    return q, k


def perturb(x: np.ndarray, sigma: float, seed: int, dtype: str = "f32") -> np.ndarray:
    """x + sigma * N(0,1) in float32 (x given in the workload dtype); used to build
    a relay layer close to a given anchor layer."""
    rng = np.random.default_rng(seed)
    base = bf16_bits_to_fp32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)
    y = base + np.float32(sigma) * rng.standard_normal(base.shape, dtype=np.float32)
    return fp32_to_bf16_bits(y) if dtype == "bf16" else y.astype(np.float32)
