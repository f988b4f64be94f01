"""Octahedral map of a triplet direction to the square [-1, 1]^2.

OCTOPUS paper, Sec. 3.2 Eq. 5 (encode) and App. C.6 / C.7 (encode, decode);
the App. C summary adds that the encoder folds the L1-normalized direction,
uses sign(0) = +1 and clamps denominators, and that decode inverts the fold
and renormalizes onto S^2.

Encode: p = t / max(||t||_1, eps);  if p_z >= 0: (xi, eta) = (p_x, p_y),
        else (sign(p_x)(1 - |p_y|), sign(p_y)(1 - |p_x|)).
Decode: z = 1 - |xi| - |eta|; if z < 0 the x, y pair is unfolded as
        (sign(xi)(1 - |eta|), sign(eta)(1 - |xi|)); n = (x, y, z) / ||(x, y, z)||.

A zero triplet (rho = 0) gives p = 0, hence (xi, eta) = (0, 0), whose decode is
the pole (0, 0, 1): that is the placeholder direction the paper asks for.

Parity: pinned by the encode->decode round trip on unit vectors, continuity on
the equator, and the Eq. 7 density (tests/test_oracle_octahedral.py).
"""
import numpy as np

EPS = 1e-20


def sign0(x):
    """sign with sign(0) = +1 (paper, App. C summary)."""
    return np.where(x >= 0, 1.0, -1.0)


def oct_encode(t: np.ndarray):
    """Eq. 5 on triplets t[..., 3] (any scale).  Returns (xi, eta, p)."""
    l1 = np.abs(t).sum(axis=-1)
    p = t / np.maximum(l1, EPS)[..., None]
    px, py, pz = p[..., 0], p[..., 1], p[..., 2]
    upper = pz >= 0
    xi = np.where(upper, px, sign0(px) * (1.0 - np.abs(py)))
    eta = np.where(upper, py, sign0(py) * (1.0 - np.abs(px)))
    return xi, eta, p


def oct_unfold(xi: np.ndarray, eta: np.ndarray) -> np.ndarray:
    """The un-normalized point q(xi, eta) on the octahedron |x|+|y|+|z| = 1."""
    z = 1.0 - np.abs(xi) - np.abs(eta)
    lower = z < 0
    x = np.where(lower, sign0(xi) * (1.0 - np.abs(eta)), xi)
    y = np.where(lower, sign0(eta) * (1.0 - np.abs(xi)), eta)
    return np.stack([x, y, z], axis=-1)


def oct_decode(xi: np.ndarray, eta: np.ndarray) -> np.ndarray:
    """Eq. 6 followed by normalization onto S^2: n[..., 3]."""
    q = oct_unfold(xi, eta)
    nrm = np.sqrt((q * q).sum(axis=-1))
    return q / np.maximum(nrm, EPS)[..., None]
