"""Named routing workloads: shapes, drift, anchor schedule and sentinel widths.

Each workload describes a stack of layers whose chunk representations
Q^l (nq x d) and K^l (nk x d) drift from layer to layer, as in the synthetic
setting of "RouteRelay: Event-Triggered Cross-Layer Route Reuse for Efficient
Dynamic Sparse Attention" (Section 5, Table 1; Sections 5.1-5.3).  Only shapes
and schedules live here; the seeded generator is in ``synth.py``.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    heads: int
    layers: int
    n: int                      # query chunk rows per head (and key chunks unless nk_ is set)
    d: int                      # routing representation width
    dtype: str                  # "f32" or "bf16": what the routing kernels read
    drift: Tuple[float, float]  # (lo, hi): lo == hi -> fixed sigma, else sigma_l ~ U[lo, hi)
    drift_scale: str            # "absolute": step = sigma*N(0,1); "relative": step = (sigma/sqrt(d))*N(0,1)
    anchors: Tuple[int, ...]    # forced anchor layers (Section 3.2, "Forced anchors")
    k: int = 12                 # route width (Eq. 2)
    m: int = 12                 # near-miss sentinels (Section 3.1, item 1)
    r: int = 8                  # random sentinels (Section 3.1, item 2)
    causal: bool = False        # key chunk j allowed for query chunk i only if j <= i
    gamma: float = 0.0          # guard margin of Eq. 8
    seed: int = 0
    sink: int = 0               # mandatory sink sentinels (Section 3.1, item 3)
    recent: int = 0             # mandatory recent sentinels (Section 3.1, item 3)
    min_reuse: int = 0          # hysteresis (Section 3.2): untested reuse after a refresh
    gamma_extra: float = 0.0    # hysteresis: extra guard after a refresh until a test passes
    nk_: int = 0                # key chunks per head when it differs from n (0: nk = n)
    drift_model: str = "walk"   # "walk": Q^l = Q^{l-1} + step*N; "local": Q^l = base + step*N
    preferred: int = 0          # "local": preferred key chunks per query row
    pref_gain: float = 0.0      # "local": weight of the preferred chunks in the row's base query

    @property
    def nq(self) -> int:
        return self.n

    @property
    def nk(self) -> int:
        return self.nk_ or self.n

    @property
    def c(self) -> int:
        return self.k + self.m + self.sink + self.recent + self.r

    def is_anchor(self, layer: int) -> bool:
        return layer == 0 or layer in self.anchors

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def stride_anchors(layers: int, stride: int) -> Tuple[int, ...]:
    """Layers 0, stride, 2*stride, ... below ``layers``."""
    return tuple(range(0, layers, stride))


def tiny_chain() -> Workload:
    """1 head, 128 chunks, 8 fp32 layers, literal random-walk drift 0.03, anchors {0, 4}."""
    return Workload("tiny_chain", heads=1, layers=8, n=128, d=64, dtype="f32",
                    drift=(0.03, 0.03), drift_scale="absolute", anchors=(0, 4))


def drift_sweep(sigma: float, seed: int = 0) -> Workload:
    """1 head, 256 chunks, 16 fp32 layers, anchor stride 8; sigma in {0.01, 0.03, 0.06}, seeds 0-9."""
    return Workload(f"drift_sweep_s{sigma:g}_seed{seed}", heads=1, layers=16, n=256, d=64,
                    dtype="f32", drift=(sigma, sigma), drift_scale="relative",
                    anchors=stride_anchors(16, 8), seed=seed)


def scale_sweep(n: int, seed: int = 0) -> Workload:
    """1 head, n in {128, 256, 512, 1024} chunks, 32 bf16 layers, drift 0.03, anchor stride 8."""
    return Workload(f"scale_sweep_n{n}_seed{seed}", heads=1, layers=32, n=n, d=64, dtype="bf16",
                    drift=(0.03, 0.03), drift_scale="relative",
                    anchors=stride_anchors(32, 8), seed=seed)


def batched_heads() -> Workload:
    """32 heads x 32 layers, 1024 chunks (128K tokens / 128-token chunks), bf16,
    per-layer drift sigma_l ~ U[0.01, 0.06), anchor stride 8, non-causal."""
    return Workload("batched_heads", heads=32, layers=32, n=1024, d=64, dtype="bf16",
                    drift=(0.01, 0.06), drift_scale="relative",
                    anchors=stride_anchors(32, 8))


def causal_large() -> Workload:
    """64 heads x 32 layers, 4096 chunks (512K tokens / 128-token chunks), bf16,
    drift 0.03, causal chunk mask, anchor stride 8."""
    return Workload("causal_large", heads=64, layers=32, n=4096, d=64, dtype="bf16",
                    drift=(0.03, 0.03), drift_scale="relative",
                    anchors=stride_anchors(32, 8), causal=True)


def preferred_chunks(sigma: float, seed: int = 0) -> Workload:
    """The cross-layer stability setting (Section 5.1): 1 head, 384 query rows, 192 key chunks,
    32 fp32 layers; each query row leans towards 12 preferred chunks of its own that persist
    through depth, and every layer adds its own Gaussian drift around those persistent
    representations (not a random walk).  The page gives neither the preference strength nor
    the anchor schedule: gain 1.0 (a preferred chunk's score is raised by about two standard
    deviations of the scores) and anchors every 8 layers are this module's choices.  Sentinels
    as on the page: 24 near-miss and 12 random."""
    return Workload(f"preferred_s{sigma:g}_seed{seed}", heads=1, layers=32, n=384, d=64,
                    dtype="f32", drift=(sigma, sigma), drift_scale="relative",
                    anchors=stride_anchors(32, 8), k=12, m=24, r=12, seed=seed, nk_=192,
                    drift_model="local", preferred=12, pref_gain=1.0)


def all_named():
    out = [tiny_chain()]
    out += [drift_sweep(s, seed) for s in (0.01, 0.03, 0.06) for seed in range(10)]
    out += [scale_sweep(n) for n in (128, 256, 512, 1024)]
    out += [batched_heads(), causal_large()]
    out += [preferred_chunks(s, seed) for s in (0.01, 0.03, 0.06, 0.1) for seed in range(10)]
    return out
