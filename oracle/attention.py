"""Sparse attention over routed chunks: the oracle of the downstream consumer.

TEST INFRASTRUCTURE ONLY (part of the oracle): see ``oracle/__init__.py``.

Source: "RouteRelay: Event-Triggered Cross-Layer Route Reuse for Efficient Dynamic Sparse
Attention", Section 2.1 (the selected chunks are expanded into token indices for a sparse
online-softmax kernel) and Section 2.2, Eq. 3: o_i = softmax(q_i K_R^T / sqrt(d)) V_R, with
R the route of the query's chunk.  Plain float64 NumPy, one query token at a time.

Readings (the page names no token layout):
  * chunk j covers tokens j*T .. j*T+T-1 of the key sequence; query chunk i covers query
    tokens i*T .. i*T+T-1, and every query token of chunk i uses chunk i's route;
  * route entries of -1 are padding; a query token with no routed key gets output 0;
  * causal mode (query and key sequences are the same tokens): query token t sees key token
    s of a routed chunk only if s <= t;
  * inputs are the bf16 values handed to the GPU (decoded exactly); the softmax is exact
    (float64, max-subtracted), the scale is 1/sqrt(d).
"""
from __future__ import annotations

import numpy as np

from .routing import decode


def sparse_attention(q_tok: np.ndarray, k_tok: np.ndarray, v_tok: np.ndarray,
                     routes: np.ndarray, T: int, causal: bool, dtype: str = "bf16") -> np.ndarray:
    """q_tok [H, nq*T, d], k_tok / v_tok [H, nk*T, d] (raw bf16 bits or fp32), routes
    [H, nq, k] int32; returns float64 [H, nq*T, d]."""
    Q, K, V = decode(q_tok, dtype), decode(k_tok, dtype), decode(v_tok, dtype)
    H, nqT, d = Q.shape
    nq = routes.shape[1]
    assert nqT == nq * T
    scale = 1.0 / np.sqrt(d)
    out = np.zeros((H, nqT, d))
    for h in range(H):
        for i in range(nq):
            chunks = [int(j) for j in routes[h, i] if j >= 0]
            if not chunks:
                continue
            toks = np.concatenate([np.arange(j * T, (j + 1) * T) for j in chunks])
            for t in range(i * T, (i + 1) * T):
                keep = toks[toks <= t] if causal else toks
                if keep.size == 0:
                    continue
                s = (K[h, keep] @ Q[h, t]) * scale
                w = np.exp(s - s.max())
                out[h, t] = (w / w.sum()) @ V[h, keep]
    return out
