"""Pins for oracle.octahedral (CPU).

  * encode -> decode is the identity on unit vectors (Eq. 5 / Eq. 6 are
    inverse on the octahedron, OCTOPUS paper App. C.6-C.7).
  * the map is continuous across the equator and sends the poles and axes to
    the expected corners; a zero triplet gets the (0, 0) placeholder.
  * uniform directions produce the density g of Eq. 7 on the square, whose
    xi-marginal is the f_xi printed in Sec. 3.2 (both formulas from the paper;
    the test checks them against each other and against samples).
"""
import numpy as np
from scipy import integrate, stats

from oracle.octahedral import oct_decode, oct_encode, oct_unfold


def unit_vectors(n, seed=0):
    v = np.random.default_rng(seed).standard_normal((n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def f_xi(xi):
    """Sec. 3.2 printed marginal of one octahedral coordinate."""
    a = np.abs(xi)
    return (1.0 / (np.pi * np.sqrt(a * a + (1 - a) ** 2))) * (
        (1 - a) / (1 - 2 * a + 3 * a * a) + a / (2 - 4 * a + 3 * a * a))


def g_density(xi, eta):
    """Eq. 7: g = (1/4pi) ||q(xi, eta)||^-3 with q the octahedron point."""
    q = oct_unfold(np.asarray(xi, float), np.asarray(eta, float))
    return (1.0 / (4 * np.pi)) * np.linalg.norm(q, axis=-1) ** -3


def test_round_trip_unit_vectors():
    n = unit_vectors(200000)
    xi, eta, _ = oct_encode(n)
    assert np.all(np.abs(xi) <= 1) and np.all(np.abs(eta) <= 1)
    assert np.abs(oct_decode(xi, eta) - n).max() < 1e-12


def test_scale_invariance_of_encode():
    n = unit_vectors(1000, 1)
    xi1, eta1, _ = oct_encode(n)
    xi2, eta2, _ = oct_encode(0.0137 * n)
    assert np.allclose(xi1, xi2, atol=1e-15) and np.allclose(eta1, eta2, atol=1e-15)


def test_special_points_and_placeholder():
    pts = np.array([[0, 0, 1], [0, 0, -1], [1, 0, 0], [0, -1, 0], [0, 0, 0]], float)
    xi, eta, _ = oct_encode(pts)
    assert np.allclose(np.stack([xi, eta], 1), [[0, 0], [1, 1], [1, 0], [0, -1], [0, 0]])
    dec = oct_decode(xi, eta)
    assert np.allclose(dec[:4], pts[:4], atol=1e-15)
    assert np.allclose(dec[4], [0, 0, 1])          # zero triplet -> pole placeholder


def test_equator_continuity():
    rng = np.random.default_rng(2)
    phi = rng.uniform(0, 2 * np.pi, 1000)
    for eps in (1e-9, -1e-9):
        v = np.stack([np.cos(phi), np.sin(phi), np.full_like(phi, eps)], 1)
        xi, eta, _ = oct_encode(v)
        w = np.stack([np.cos(phi), np.sin(phi), np.zeros_like(phi)], 1)
        xi0, eta0, _ = oct_encode(w)
        assert np.abs(xi - xi0).max() < 1e-8 and np.abs(eta - eta0).max() < 1e-8


def test_eq7_density_normalized_and_marginal_is_f_xi():
    tot, _ = integrate.dblquad(lambda e, x: g_density(x, e), -1, 1, -1, 1, epsabs=1e-10)
    assert abs(tot - 1.0) < 1e-6
    for x in (0.0, 0.1, 0.3, 0.5, 0.77, 0.95):
        m, _ = integrate.quad(lambda e: g_density(x, e), -1, 1, points=[-(1 - x), 1 - x], epsabs=1e-12)
        assert abs(m - f_xi(x)) < 1e-8, (x, m, f_xi(x))
    tot_f, _ = integrate.quad(f_xi, -1, 1, points=[0], epsabs=1e-12)
    assert abs(tot_f - 1.0) < 1e-9


def test_samples_follow_f_xi():
    n = unit_vectors(400000, 3)
    xi, eta, _ = oct_encode(n)

    def cdf(x):
        x = np.atleast_1d(x)
        return np.array([integrate.quad(f_xi, -1, v, points=[0] if v > 0 else None)[0] for v in x])

    grid = np.linspace(-1, 1, 401)
    table = cdf(grid)
    for sample in (xi, eta):
        res = stats.kstest(sample, lambda v: np.interp(v, grid, table))
        assert res.pvalue > 1e-3, res


def test_samples_follow_eq7_on_cells():
    n = unit_vectors(400000, 4)
    xi, eta, _ = oct_encode(n)
    edges = np.linspace(-1, 1, 9)
    counts, _, _ = np.histogram2d(xi, eta, bins=[edges, edges])
    expect = np.zeros_like(counts)
    for i in range(8):
        for j in range(8):
            expect[i, j] = integrate.dblquad(lambda e, x: g_density(x, e), edges[i], edges[i + 1],
                                             edges[j], edges[j + 1], epsabs=1e-9)[0] * n.shape[0]
    chi2 = ((counts - expect) ** 2 / expect).sum()
    assert stats.chi2.sf(chi2, 63) > 1e-3, chi2
