"""Pins for the sparse-attention oracle (Section 2.2, Eq. 3; token expansion of Section 2.1).

Each test states what the page and the mathematics fix, independently of the oracle's loop."""
import numpy as np
import pytest

import oracle as O
from long_context_prefill_anchor_amd import synth


def _tok(H, n, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((H, n, d)) / 8).astype(np.float32)


def test_uniform_scores_average_the_routed_values():
    """q = 0: every routed token gets the same weight, so o = mean of V over the routed tokens."""
    T, d = 4, 8
    q = np.zeros((1, 2 * T, d), np.float32)
    k, v = _tok(1, 3 * T, d, 1), _tok(1, 3 * T, d, 2)
    routes = np.array([[[2, 0], [1, -1]]], np.int32)
    out = O.sparse_attention(q, k, v, routes, T, causal=False, dtype="f32")
    want0 = np.concatenate([v[0, 8:12], v[0, 0:4]]).astype(np.float64).mean(axis=0)
    want1 = v[0, 4:8].astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(out[0, :T], np.broadcast_to(want0, (T, d)), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(out[0, T:], np.broadcast_to(want1, (T, d)), rtol=1e-12, atol=1e-15)


def test_dominant_key_selects_its_value():
    """One key aligned with the query and far above the rest: o is that key's value."""
    T, d = 4, 8
    q = np.zeros((1, T, d), np.float32)
    q[0, :, 0] = 1.0
    k = np.zeros((1, 2 * T, d), np.float32)
    k[0, 5, 0] = 400.0                      # s = 400 / sqrt(8) for token 5, 0 for the others
    v = _tok(1, 2 * T, d, 3)
    out = O.sparse_attention(q, k, v, np.array([[[1, 0]]], np.int32), T, False, "f32")
    np.testing.assert_allclose(out[0], np.broadcast_to(v[0, 5].astype(np.float64), (T, d)), atol=1e-12)


def test_full_route_equals_dense_attention():
    """A route holding every chunk is plain softmax attention; compared with a dense
    formulation written with scipy's softmax over the whole score matrix."""
    from scipy.special import softmax
    T, d, n = 4, 16, 5
    q, k, v = _tok(2, n * T, d, 4), _tok(2, n * T, d, 5), _tok(2, n * T, d, 6)
    routes = np.tile(np.arange(n, dtype=np.int32)[::-1], (2, n, 1))     # order does not matter
    out = O.sparse_attention(q, k, v, routes, T, False, "f32")
    for h in range(2):
        S = q[h].astype(np.float64) @ k[h].astype(np.float64).T / np.sqrt(d)
        np.testing.assert_allclose(out[h], softmax(S, axis=1) @ v[h].astype(np.float64), rtol=1e-10, atol=1e-13)
    # causal: the dense form with the upper triangle masked
    out_c = O.sparse_attention(q, k, v, routes, T, True, "f32")
    for h in range(2):
        S = q[h].astype(np.float64) @ k[h].astype(np.float64).T / np.sqrt(d)
        S[np.triu_indices(n * T, 1)] = -np.inf
        np.testing.assert_allclose(out_c[h], softmax(S, axis=1) @ v[h].astype(np.float64), rtol=1e-10, atol=1e-13)


def test_padding_and_empty_rows():
    """-1 entries are ignored; a chunk with no routed key gets zeros; in causal mode the first
    token of a chunk routed only to itself attends to itself alone."""
    T, d = 4, 8
    q, k, v = _tok(1, 2 * T, d, 7), _tok(1, 2 * T, d, 8), _tok(1, 2 * T, d, 9)
    routes = np.array([[[-1, -1], [1, -1]]], np.int32)
    out = O.sparse_attention(q, k, v, routes, T, causal=True, dtype="f32")
    assert np.all(out[0, :T] == 0)
    np.testing.assert_allclose(out[0, T], v[0, T].astype(np.float64), atol=1e-15)


def test_bf16_inputs_are_decoded_exactly():
    """bf16 bits in, the same values as their fp32 widening."""
    T, d = 4, 8
    q, k, v = _tok(1, T, d, 10), _tok(1, T, d, 11), _tok(1, T, d, 12)
    qb, kb, vb = (synth.fp32_to_bf16_bits(x) for x in (q, k, v))
    routes = np.array([[[0]]], np.int32)
    a = O.sparse_attention(qb, kb, vb, routes, T, False, "bf16")
    b = O.sparse_attention(*(synth.bf16_bits_to_fp32(x) for x in (qb, kb, vb)), routes, T, False, "f32")
    np.testing.assert_array_equal(a, b)
