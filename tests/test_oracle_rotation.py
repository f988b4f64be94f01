"""Pins for oracle.splitmix and oracle.rotation (CPU).

  * SplitMix64 reproduces the published seed-0 output sequence of the
    reference generator (Steele, Lea, Flood 2014; Vigna's splitmix64.c).
  * H is orthogonal and equals scipy.linalg.hadamard(d) / sqrt(d).
  * R = H D_s is orthogonal, R^-1 = R^T = D_s H, and preserves dot products
    (OCTOPUS paper, App. B, Proposition 1).
"""
import numpy as np
import pytest
import scipy.linalg

from oracle import rotation, splitmix


def test_splitmix64_published_sequence():
    # First three outputs of SplitMix64 started from state 0.
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert [splitmix.splitmix64_output(0, j) for j in range(3)] == want


def test_signs_are_bit63_and_streams_disjoint():
    s = splitmix.sign_vector(7, 0, 256)
    for j in range(256):
        assert s[j] == (-1 if splitmix.splitmix64_output(7, j) >> 63 else 1)
    assert np.array_equal(rotation.qjl_signs(128, 7), np.array(s[128:256], dtype=float))
    assert 40 < sum(1 for v in s[:128] if v < 0) < 88


@pytest.mark.parametrize("d", [1, 2, 4, 8, 64, 128, 256])
def test_hadamard_orthogonal_and_matches_scipy(d):
    h = rotation.hadamard(d)
    assert np.allclose(h.T @ h, np.eye(d), atol=1e-13)
    assert np.allclose(h, scipy.linalg.hadamard(d) / np.sqrt(d), atol=0)
    assert np.allclose(h, h.T)


def test_rotation_inverse_and_dot_product_invariance():
    d = 128
    r = rotation.rotation_matrix(d, 3)
    s = rotation.signs(d, 3)
    assert np.allclose(r.T @ r, np.eye(d), atol=1e-13)
    assert np.allclose(r.T, np.diag(s) @ rotation.hadamard(d), atol=1e-15)
    rng = np.random.default_rng(0)
    q, k = rng.standard_normal((2, 50, d))
    lhs = ((q @ r.T) * (k @ r.T)).sum(1)
    assert np.allclose(lhs, (q * k).sum(1), rtol=1e-12, atol=1e-12)
    assert np.allclose(rotation.unrotate(rotation.rotate(q, 3), 3), q, atol=1e-13)


def test_rotation_depends_on_seed():
    assert not np.array_equal(rotation.signs(128, 0), rotation.signs(128, 1))
    assert not np.array_equal(rotation.signs(128, 0), rotation.qjl_signs(128, 0))
