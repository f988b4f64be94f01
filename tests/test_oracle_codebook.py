"""Pins for oracle.codebook and the codebook artifact (CPU).

  * Lloyd-Max centroid condition on the training sample: every centroid of the
    artifact is the mean of its nearest-neighbour cell (OCTOPUS paper Sec. 3.4).
  * C_xi is exactly antisymmetric; sizes are 2^b; at b = 4 the (5, 3) split has
    32 + 8 centroids (Sec. 3.4).
  * Agreement with Lloyd-Max computed independently by quadrature on the
    analytic densities printed in the paper: f_xi (Sec. 3.2) and the
    triplet-norm law f_rho (Eq. 4).
  * One level: the centroid is E[rho] = B(2,(d-3)/2) / B(3/2,(d-3)/2).
  * E[rho^2] = 3/d (App. C.10, Eq. 9) on the sample.
  * lloyd_max_1d equals a brute-force Lloyd (explicit argmin) on a small set.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import beta as B

from oracle.codebook import lloyd_max_1d, monte_carlo_samples

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ART = os.path.join(ROOT, "quantized_decode_attention_octo_amd", "codebooks", "octopus_d128.json")
CLAIMS = json.load(open(os.path.join(ROOT, "tests", "golden", "paper_claims.json")))


@pytest.fixture(scope="module")
def art():
    return json.load(open(ART))


@pytest.fixture(scope="module")
def samples(art):
    p = art["provenance"]
    return monte_carlo_samples(art["d"], p["n_keys"], p["mc_seed"], p["rotation_seed"])


def f_xi(xi):
    a = np.abs(xi)
    return (1.0 / (np.pi * np.sqrt(a * a + (1 - a) ** 2))) * (
        (1 - a) / (1 - 2 * a + 3 * a * a) + a / (2 - 4 * a + 3 * a * a))


def f_rho(r, d):
    return 2 * r * r * (1 - r * r) ** ((d - 5) / 2) / B(1.5, (d - 3) / 2)


def quadrature_lloyd(lo, hi, dens, K, n=400001, iters=20000):
    x = np.linspace(lo, hi, n)
    w = dens(x)
    w /= w.sum()
    cw = np.concatenate([[0], np.cumsum(w)])
    cxw = np.concatenate([[0], np.cumsum(w * x)])
    c = np.interp((np.arange(K) + 0.5) / K, np.cumsum(w), x)
    for _ in range(iters):
        cut = np.searchsorted(x, 0.5 * (c[:-1] + c[1:]), side="right")
        a = np.concatenate([[0], cut])
        b = np.concatenate([cut, [n]])
        new = (cxw[b] - cxw[a]) / np.maximum(cw[b] - cw[a], 1e-300)
        if np.abs(new - c).max() < 1e-13:
            c = new
            break
        c = new
    return c


def test_sizes_symmetry_budget(art):
    for b, c in art["c_xi"].items():
        c = np.array(c, dtype=np.float32)
        assert c.size == 2 ** int(b)
        assert np.all(np.diff(c) > 0)
        assert np.array_equal(c, -c[::-1])
    for b, c in art["c_rho"].items():
        c = np.array(c)
        assert c.size == 2 ** int(b) and np.all(np.diff(c) > 0) and c[0] > 0 and c[-1] < 1
    assert len(art["c_xi"]["5"]) + len(art["c_rho"]["3"]) == CLAIMS["codebook_size"]["max_centroids"]


def test_centroid_condition_on_training_sample(art, samples):
    s_xi, s_rho = samples
    pooled = np.concatenate([s_xi, -s_xi])
    for table, data in (("c_xi", pooled), ("c_rho", s_rho)):
        for b, c in art[table].items():
            c = np.array(c, dtype=np.float64)
            idx = np.argmin(np.abs(data[:, None] - c[None, :]), axis=1) if c.size <= 8 else \
                np.searchsorted(0.5 * (c[:-1] + c[1:]), data, side="left")
            means = np.array([data[idx == k].mean() for k in range(c.size)])
            assert np.abs(means - c).max() < 2e-6, (table, b, np.abs(means - c).max())


@pytest.mark.parametrize("b_dir", [1, 2, 3, 4, 5])
def test_c_xi_matches_quadrature_on_f_xi(art, b_dir):
    q = quadrature_lloyd(-1, 1, f_xi, 2 ** b_dir)
    assert np.abs(q - np.array(art["c_xi"][str(b_dir)])).max() < 1e-3


@pytest.mark.parametrize("b_nrm", [1, 2, 3, 4])
def test_c_rho_matches_quadrature_on_eq4(art, b_nrm):
    q = quadrature_lloyd(0, 1, lambda r: f_rho(r, 128), 2 ** b_nrm)
    assert np.abs(q - np.array(art["c_rho"][str(b_nrm)])).max() < 1e-3


def test_single_level_is_mean_norm(art):
    d = 128
    e_rho = B(2, (d - 3) / 2) / B(1.5, (d - 3) / 2)
    assert abs(e_rho - 0.1413231) < 1e-6
    assert abs(art["c_rho"]["0"][0] - e_rho) < 5e-4


def test_second_moment_of_triplet_norm(samples):
    _, s_rho = samples
    want = CLAIMS["triplet_norm_second_moment"]["value"]
    assert want == 3 / 128
    assert abs((s_rho ** 2).mean() - want) < 1e-4


def test_lloyd_equals_bruteforce_lloyd():
    x = np.random.default_rng(5).beta(2, 5, 3000)
    for K in (2, 4, 8):
        c, info = lloyd_max_1d(x, K)
        ref = np.sort(x)[np.minimum(((np.arange(K) + 0.5) / K * x.size).astype(int), x.size - 1)]
        for _ in range(100000):
            idx = np.argmin(np.abs(x[:, None] - ref[None, :]), axis=1)
            new = np.array([x[idx == k].mean() if np.any(idx == k) else ref[k] for k in range(K)])
            if np.array_equal(new, ref):
                break
            ref = new
        assert info["converged"]
        assert np.abs(c - ref).max() < 1e-12
