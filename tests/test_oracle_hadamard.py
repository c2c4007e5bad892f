"""Pins of the oracle's Hadamard matrix: scipy's routine, an independent
Kronecker construction, orthogonality, and rotation invariants."""
import numpy as np
import scipy.linalg

from oracle.hadamard import hadamard
from oracle.quantize import rotate_keys


def test_matches_scipy():
    for n in (1, 2, 4, 16, 128):
        np.testing.assert_array_equal(hadamard(n), scipy.linalg.hadamard(n) / np.sqrt(n))


def test_matches_kronecker_recursion():
    H = np.array([[1.0]])
    while H.shape[0] < 128:
        H = np.block([[H, H], [H, -H]])
    np.testing.assert_array_equal(hadamard(128) * np.sqrt(128), H)


def test_order_two_literal():
    r = 1 / np.sqrt(2)
    np.testing.assert_array_equal(hadamard(2), np.array([[r, r], [r, -r]]))


def test_orthogonal_and_involutive():
    Hs = hadamard(128) * np.sqrt(128)   # exact +-1 integers
    assert np.all(np.abs(Hs) == 1)
    np.testing.assert_array_equal(Hs @ Hs.T, 128 * np.eye(128))
    np.testing.assert_array_equal(Hs, Hs.T)
    H = hadamard(128)
    np.testing.assert_allclose(H @ H, np.eye(128), atol=1e-14)


def test_unit_vectors_map_to_columns():
    H = hadamard(128)
    for j in (0, 1, 5, 64, 127):
        e = np.zeros((1, 128)); e[0, j] = 1.0
        np.testing.assert_allclose(rotate_keys(e)[0], H[:, j], atol=0)


def test_rotation_preserves_norms_and_dots():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((64, 128)) * rng.lognormal(0, 1, (64, 1))
    q = rng.standard_normal((64, 128))
    yk, yq = rotate_keys(k), rotate_keys(q)
    np.testing.assert_allclose(np.linalg.norm(yk, axis=1), np.linalg.norm(k, axis=1), rtol=1e-12)
    np.testing.assert_allclose(np.sum(yk * yq, 1), np.sum(k * q, 1), rtol=1e-10, atol=1e-10)


def test_rotation_spreads_channel_outliers():
    """Method sanity (Canalized Rotation spreads channel-outlier energy over
    all channels): the max |component| / norm drops sharply after rotation."""
    from synthetic import workload, keys_slice, bf16_bits_to_f64
    k = bf16_bits_to_f64(keys_slice(workload(0), 0, 0))
    y = rotate_keys(k)
    before = np.median(np.abs(k).max(1) / np.linalg.norm(k, axis=1))
    after = np.median(np.abs(y).max(1) / np.linalg.norm(y, axis=1))
    assert after < 0.6 * before
