"""The OCTOPUS encoder, one step at a time, in float64.

Follows the OCTOPUS paper in its own order:
  Sec. 3.1 / App. C.1   gamma = ||k||_2, u~ = k / gamma (eps-safe divisor)
  Sec. 3.1 / App. C.2   u = R u~, R = H D_s
  Sec. 3.2 / App. C.4   zero-pad u to 3*ceil(d/3), triplets t_i, rho_i = ||t_i||
  Sec. 3.2 Eq. 5        octahedral coordinates (xi_i, eta_i) of the direction
  Sec. 3.5              scalar Lloyd seeds (i_xi, i_eta) = nearest centroids;
                        local 3x3 joint rounding: among the nine clamped
                        neighbours of the seed take the direction maximizing
                        s = t^T n(xi^, eta^), then rho^ = the C_rho centroid
                        nearest s (App. C.13 summary)
  App. A/E summaries    Delta = {(0,0)} gives the legacy scalar rounding
                        (direction = seed, rho^ nearest rho); the full grid
                        search over all 2^(2 b_dir) codes is the reference
                        upper bound
  Sec. 3.6 / App. C.15  optional QJL residual: r = u - u^, sigma = sign(R' r),
                        gamma_r = ||r|| stored as fp16

Readings where the paper is silent:
  * eps = 1e-20; gamma is stored as fp32 (round to nearest even).
  * nearest centroid = brute-force argmin |x - c_k|, ties -> lowest index.
  * 3x3 tie rule: start from the seed (0, 0), visit the other eight in
    row-major order (dx outer, dy inner, -1 -> +1), replace only on a strictly
    larger s.
  * full-grid tie rule: lowest (i_xi, i_eta) in row-major order.
  * sign(0) = +1 for sigma; the zero pad coordinate is not part of r.

Every decision also yields a margin: the distance (in the units of the quantity
decided on) to the nearest point where the decision would change.  Per triplet
the margin is the minimum over: |p_z| (hemisphere), |p_x| and |p_y| on the
lower hemisphere (fold signs), the seed distances to their cell boundaries, the
gap between the best and the best different candidate s, and the distance of
s* (or rho) to the C_rho cell boundaries.  For sigma_j it is |(R' r)_j|.

Parity: pinned by tests/test_oracle_encode.py (tiny-d exhaustive joint search,
l_full <= l_3x3 <= l_scalar, equality of argmax-s/nearest-rho with the literal
minimum of Eq. 12, the paper's statistical claims for the bit split and the
rounding ablation, QJL unbiasedness).
"""
import numpy as np

from .octahedral import oct_decode, oct_encode, sign0
from .rotation import qjl_rotation_matrix, rotation_matrix

EPS = 1e-20
ROUND_LOCAL3X3 = "local3x3"
ROUND_SCALAR = "scalar"
ROUND_FULL = "full"


def n_triplets(d):
    return -(-d // 3)


def nearest_centroid(x, c):
    """Brute-force nearest centroid (ties -> lowest index) and its margin."""
    dist = np.abs(x[..., None] - c)
    idx = np.argmin(dist, axis=-1)
    if c.size == 1:
        return idx, np.full(x.shape, np.inf)
    best = np.take_along_axis(dist, idx[..., None], axis=-1)
    other = np.where(np.arange(c.size) == idx[..., None], np.inf, dist)
    margin = 0.5 * (other.min(axis=-1) - best[..., 0])
    return idx, margin


def magnitude_split(x):
    gamma = np.sqrt((x * x).sum(axis=-1))
    return gamma, x / np.maximum(gamma, EPS)[..., None]


def split_triplets(u):
    d = u.shape[-1]
    nt = n_triplets(d)
    pad = np.zeros(u.shape[:-1] + (3 * nt - d,), dtype=u.dtype)
    return np.concatenate([u, pad], axis=-1).reshape(u.shape[:-1] + (nt, 3))


def candidate_directions(c_xi):
    """n^(i, j) for every code pair: [K, K, 3]."""
    xi = c_xi[:, None] * np.ones((1, c_xi.size))
    eta = np.ones((c_xi.size, 1)) * c_xi[None, :]
    return oct_decode(xi, eta)


def encode(x, c_xi, c_rho, seed, rounding=ROUND_LOCAL3X3, qjl=False):
    """Encode vectors x[N, d] (float64 copies of fp32/bf16 data).

    c_xi, c_rho: the fp32 codebook values (ascending), promoted to float64.
    Returns a dict of float64 / int64 arrays:
      gamma[N], gamma_f32[N], i_xi, i_eta, i_rho [N, n_tri], margin [N, n_tri],
      u_hat [N, 3*n_tri] (the rotated-frame reconstruction), and with qjl:
      sigma_neg [N, d] (True where sigma = -1), sigma_margin [N, d],
      gamma_r_f16 [N] (float16), r_norm [N].
    """
    x = np.asarray(x, dtype=np.float64)
    c_xi = np.asarray(c_xi, dtype=np.float64)
    c_rho = np.asarray(c_rho, dtype=np.float64)
    n, d = x.shape
    K = c_xi.size

    gamma, u_tilde = magnitude_split(x)
    u = u_tilde @ rotation_matrix(d, seed).T
    t = split_triplets(u)                                   # [N, nt, 3]
    rho = np.sqrt((t * t).sum(axis=-1))
    xi, eta, p = oct_encode(t)

    lower = p[..., 2] < 0
    margin = np.abs(p[..., 2])
    margin = np.minimum(margin, np.where(lower, np.abs(p[..., 0]), np.inf))
    margin = np.minimum(margin, np.where(lower, np.abs(p[..., 1]), np.inf))

    seed_xi, m_xi = nearest_centroid(xi, c_xi)
    seed_eta, m_eta = nearest_centroid(eta, c_xi)
    dirs = candidate_directions(c_xi)                       # [K, K, 3]

    if rounding == ROUND_SCALAR:
        i_xi, i_eta = seed_xi, seed_eta
        margin = np.minimum(margin, np.minimum(m_xi, m_eta))
        i_rho, m_rho = nearest_centroid(rho, c_rho)
        margin = np.minimum(margin, m_rho)
        n_hat = dirs[i_xi, i_eta]
    elif rounding == ROUND_LOCAL3X3:
        margin = np.minimum(margin, np.minimum(m_xi, m_eta))
        order = [(0, 0)] + [(a, b) for a in (-1, 0, 1) for b in (-1, 0, 1) if (a, b) != (0, 0)]
        cx = np.stack([np.clip(seed_xi + a, 0, K - 1) for a, _ in order], axis=-1)
        cy = np.stack([np.clip(seed_eta + b, 0, K - 1) for _, b in order], axis=-1)
        s = (t[..., None, :] * dirs[cx, cy]).sum(axis=-1)   # [N, nt, 9]
        best = np.zeros(s.shape[:-1], dtype=np.int64)
        best_s = s[..., 0].copy()
        for k in range(1, 9):
            take = s[..., k] > best_s
            best = np.where(take, k, best)
            best_s = np.where(take, s[..., k], best_s)
        i_xi = np.take_along_axis(cx, best[..., None], axis=-1)[..., 0]
        i_eta = np.take_along_axis(cy, best[..., None], axis=-1)[..., 0]
        code = cx * K + cy
        best_code = i_xi * K + i_eta
        rival = np.where(code == best_code[..., None], -np.inf, s).max(axis=-1)
        margin = np.minimum(margin, best_s - rival)
        i_rho, m_rho = nearest_centroid(best_s, c_rho)
        margin = np.minimum(margin, m_rho)
        n_hat = dirs[i_xi, i_eta]
    elif rounding == ROUND_FULL:
        s = np.einsum("ntc,abc->ntab", t, dirs).reshape(n, -1, K * K)
        flat = np.argmax(s, axis=-1)                        # first max = lowest code
        best_s = np.take_along_axis(s, flat[..., None], axis=-1)[..., 0]
        rival = np.where(np.arange(K * K) == flat[..., None], -np.inf, s).max(axis=-1)
        margin = np.minimum(margin, best_s - rival)
        i_xi, i_eta = flat // K, flat % K
        i_rho, m_rho = nearest_centroid(best_s, c_rho)
        margin = np.minimum(margin, m_rho)
        n_hat = dirs[i_xi, i_eta]
    else:
        raise ValueError(rounding)

    u_hat = (c_rho[i_rho][..., None] * n_hat).reshape(n, -1)
    out = {
        "gamma": gamma,
        "gamma_f32": gamma.astype(np.float32),
        "i_xi": i_xi.astype(np.int64),
        "i_eta": i_eta.astype(np.int64),
        "i_rho": i_rho.astype(np.int64),
        "margin": margin,
        "u": u,
        "u_hat": u_hat,
    }
    if qjl:
        r = u - u_hat[:, :d]
        proj = r @ qjl_rotation_matrix(d, seed).T
        r_norm = np.sqrt((r * r).sum(axis=-1))
        out["sigma_neg"] = sign0(proj) < 0
        out["sigma_margin"] = np.abs(proj)
        out["r_norm"] = r_norm
        out["gamma_r_f16"] = r_norm.astype(np.float16)
    return out
