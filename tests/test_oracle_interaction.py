"""Pins of the oracle's dot interaction ("Deep Learning Recommendation Model
for Personalization and Recommendation Systems", review page, "Proposed
method": second-order interactions are the dot products between the
embedding vectors and the processed dense features, concatenated with the
dense features).

Each check ties the oracle to something other than its own loops: a
hand-worked example (tests/golden/dot_interaction_tiny.json), the lower
triangle of numpy's float64 Gram matrix, closed forms (orthogonal rows,
equal rows, d = 1), exact scaling by powers of two, and the output width.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dot_interaction_tiny.json")


def _gram_lower(dense, pooled):
    Z = np.concatenate([dense[:, None, :], pooled], axis=1).astype(np.float64)
    G = np.matmul(Z, np.transpose(Z, (0, 2, 1)))
    i, j = np.tril_indices(Z.shape[1], -1)
    return G[:, i, j], np.matmul(np.abs(Z), np.transpose(np.abs(Z), (0, 2, 1)))[:, i, j]


def test_hand_worked_example():
    g = json.load(open(GOLDEN))
    out, absd = oracle.dot_interaction(np.array(g["dense"], np.float32), np.array(g["pooled"], np.float32))
    assert np.array_equal(out, np.array(g["out"]))
    assert np.array_equal(absd[:, 2:], out[:, 2:])  # all products positive


@pytest.mark.parametrize("T,dim", [(0, 5), (1, 1), (2, 3), (15, 16), (26, 64), (64, 128), (7, 1000)])
def test_width_and_numpy_gram(T, dim):
    g = np.random.default_rng(100 + T * 7 + dim)
    B = 9
    dense = g.standard_normal((B, dim)).astype(np.float32)
    pooled = (g.standard_normal((B, T, dim)) * g.uniform(0.01, 10, size=(B, T, 1))).astype(np.float32)
    out, absd = oracle.dot_interaction(dense, pooled)
    assert out.shape == (B, dim + T * (T + 1) // 2) == (B, oracle.interaction_width(T, dim))
    assert np.array_equal(out[:, :dim], dense.astype(np.float64))
    assert np.all(absd[:, :dim] == 0)
    ref, ref_abs = _gram_lower(dense, pooled)
    assert np.all(np.abs(out[:, dim:] - ref) <= 1e-12 * ref_abs + 1e-300)
    assert np.allclose(absd[:, dim:], ref_abs, rtol=1e-12, atol=0)


def test_orthogonal_rows_give_zero():
    B, T, dim = 3, 6, 8
    eye = np.eye(dim, dtype=np.float32)
    dense = np.tile(eye[0] * 3.0, (B, 1)).astype(np.float32)
    pooled = np.tile((eye[1:T + 1] * np.arange(1, T + 1, dtype=np.float32)[:, None])[None], (B, 1, 1))
    out, _ = oracle.dot_interaction(dense, pooled)
    assert np.all(out[:, dim:] == 0)


def test_equal_rows_give_the_squared_norm():
    v = np.array([0.5, -1.25, 2.0, 0.125], np.float32)
    T = 5
    out, _ = oracle.dot_interaction(v[None], np.tile(v, (1, T, 1)))
    assert np.all(out[0, 4:] == float(np.sum(v.astype(np.float64) ** 2)))


def test_one_dimension_is_products():
    g = np.random.default_rng(3)
    T = 10
    z = g.standard_normal(T + 1).astype(np.float32)
    out, _ = oracle.dot_interaction(z[None, :1], z[None, 1:, None])
    i, j = np.tril_indices(T + 1, -1)
    assert np.array_equal(out[0, 1:], z[i].astype(np.float64) * z[j].astype(np.float64))


def test_scaling_dense_by_two_scales_exactly_its_pairs():
    g = np.random.default_rng(4)
    B, T, dim = 4, 9, 33
    dense = g.standard_normal((B, dim)).astype(np.float32)
    pooled = g.standard_normal((B, T, dim)).astype(np.float32)
    a, _ = oracle.dot_interaction(dense, pooled)
    b, _ = oracle.dot_interaction(dense * np.float32(2), pooled)
    i, j = np.tril_indices(T + 1, -1)
    with_dense = j == 0
    assert np.array_equal(b[:, dim:][:, with_dense], 2 * a[:, dim:][:, with_dense])
    assert np.array_equal(b[:, dim:][:, ~with_dense], a[:, dim:][:, ~with_dense])
    assert np.array_equal(b[:, :dim], 2 * a[:, :dim])


def test_empty_batch():
    out, _ = oracle.dot_interaction(np.zeros((0, 4), np.float32), np.zeros((0, 3, 4), np.float32))
    assert out.shape == (0, 10)
