"""Pins of the oracle's Hadamard matrix: scipy's Sylvester construction, orthonormality,
symmetry, norm preservation, and an explicit radix-2 butterfly."""

import numpy as np
import scipy.linalg

from oracle import hadamard


def test_equals_scipy_sylvester():
    assert np.array_equal(hadamard.H128 * np.sqrt(128.0), scipy.linalg.hadamard(128).astype(float))


def test_orthonormal_and_symmetric():
    h = hadamard.H128
    assert np.allclose(h @ h.T, np.eye(128), atol=1e-14, rtol=0)
    assert np.array_equal(h, h.T)
    assert np.allclose(h @ h, np.eye(128), atol=1e-14, rtol=0)


def test_norm_preserved():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 128)) * np.exp(rng.standard_normal(128))
    y = hadamard.rotate(x)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_matches_radix2_butterflies():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(128)
    y = x.copy()
    half = 1
    while half < 128:                       # 7 butterfly stages
        for start in range(0, 128, 2 * half):
            for i in range(start, start + half):
                a, b = y[i], y[i + half]
                y[i], y[i + half] = a + b, a - b
        half *= 2
    assert np.allclose(y / np.sqrt(128.0), hadamard.rotate(x), atol=1e-13, rtol=0)


def test_small_orders():
    assert np.array_equal(hadamard.hadamard(2) * np.sqrt(2), np.array([[1, 1], [1, -1]], float))
    for n in (4, 8, 16):
        assert np.array_equal(hadamard.hadamard(n) * np.sqrt(n), scipy.linalg.hadamard(n))
