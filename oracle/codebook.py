"""Lloyd-Max codebooks C_xi(b_dir) and C_rho(d, b_nrm).

OCTOPUS paper, Sec. 3.4: two Lloyd-Max codebooks suffice, C_rho(d, b_nrm) on
[0, 1] matched to the triplet-norm marginal (Eq. 4) and C_xi(b_dir) on [-1, 1]
matched to the empirical xi marginal; both are trained offline with the
standard alternating assignment / update Lloyd-Max iteration "to distortion
1e-10", serialized, and depend only on (d, b_dir, b_nrm).

Readings (the paper leaves these open):
  * samples are drawn by seeded Monte Carlo through the implementation itself:
    Gaussian keys in R^d -> unit norm -> R = H D_s -> triplets -> Eq. 5.  Only
    the full triplets (the first floor(d/3)) are pooled, since the zero-padded
    last triplet has a different law.
  * xi and eta are pooled into one sample set, and the set is symmetrized
    (every value also enters negated): the xi marginal printed in Sec. 3.2
    depends on |xi| only.  The finished codebook is made exactly antisymmetric
    (c_k = -c_{K-1-k}) by averaging each pair; the size of that correction is
    recorded.
  * initial centroids are the sample quantiles at (k + 1/2) / K.
  * "to distortion 1e-10" is read as: stop when the relative decrease of the
    mean squared distortion falls below 1e-10 and no centroid moves by more
    than 1e-10, or after max_iter iterations.

The Lloyd step is the textbook one.  Assignment sends each sample to its
nearest centroid; in one dimension with sorted centroids the cell of c_k is
the interval between the midpoints to its neighbours (a sample exactly on a
midpoint goes to the lower index).  Update moves each centroid to the mean of
its cell.  Cell sums are read off prefix sums of the sorted samples.

Parity: pinned by the Lloyd centroid/midpoint conditions, exact symmetry,
agreement with quadrature Lloyd-Max on the analytic densities of Sec. 3.2 and
Eq. 4, the closed form E[rho] for one level, and a brute-force Lloyd on a
small sample (tests/test_oracle_codebook.py).
"""
import numpy as np

from .octahedral import oct_encode
from .rotation import rotation_matrix


def lloyd_max_1d(samples, levels, rel_tol=1e-10, move_tol=1e-10, max_iter=100000):
    """Lloyd-Max quantizer of a 1-D sample set.  Returns (centroids, info)."""
    x = np.sort(np.asarray(samples, dtype=np.float64).ravel())
    n = x.size
    if levels == 1:
        c = np.array([x.mean()])
        dist = float(((x - c[0]) ** 2).mean())
        return c, {"iterations": 0, "distortion": dist, "converged": True}
    csum = np.concatenate([[0.0], np.cumsum(x)])
    csum2 = np.concatenate([[0.0], np.cumsum(x * x)])
    pos = np.minimum(((np.arange(levels) + 0.5) / levels * n).astype(np.int64), n - 1)
    c = x[pos].copy()
    prev = np.inf
    converged = False
    it = 0
    dist = np.inf
    for it in range(1, max_iter + 1):
        # assignment: nearest-centroid cells are the intervals between midpoints
        mid = 0.5 * (c[:-1] + c[1:])
        cut = np.searchsorted(x, mid, side="right")
        lo = np.concatenate([[0], cut])
        hi = np.concatenate([cut, [n]])
        cnt = hi - lo
        s1 = csum[hi] - csum[lo]
        s2 = csum2[hi] - csum2[lo]
        dist = float((s2 - 2.0 * c * s1 + c * c * cnt).sum() / n)
        # update: each centroid moves to the mean of its cell
        new_c = np.where(cnt > 0, s1 / np.maximum(cnt, 1), c)
        move = float(np.abs(new_c - c).max())
        c = new_c
        if prev - dist <= rel_tol * dist and move <= move_tol:
            converged = True
            break
        prev = dist
    return c, {"iterations": it, "distortion": dist, "converged": converged}


def monte_carlo_samples(d, n_keys, mc_seed, rot_seed=0):
    """(xi_eta pooled samples, rho samples) from seeded Gaussian keys."""
    rng = np.random.default_rng(mc_seed)
    k = rng.standard_normal((n_keys, d))
    u_tilde = k / np.linalg.norm(k, axis=1, keepdims=True)
    u = u_tilde @ rotation_matrix(d, rot_seed).T
    n_full = d // 3
    t = u[:, : 3 * n_full].reshape(n_keys, n_full, 3)
    rho = np.sqrt((t * t).sum(axis=-1))
    xi, eta, _ = oct_encode(t)
    return np.concatenate([xi.ravel(), eta.ravel()]), rho.ravel()


def train_xi(samples_xi, b_dir, **kw):
    """C_xi(b_dir): Lloyd-Max on the symmetrized pooled oct-coordinate sample."""
    sym = np.concatenate([samples_xi, -samples_xi])
    c, info = lloyd_max_1d(sym, 2 ** b_dir, **kw)
    anti = 0.5 * (c - c[::-1])
    info["symmetrization_correction"] = float(np.abs(anti - c).max())
    return anti, info


def train_rho(samples_rho, b_nrm, **kw):
    """C_rho(d, b_nrm): Lloyd-Max on the triplet-norm sample."""
    return lloyd_max_1d(samples_rho, 2 ** b_nrm, **kw)
