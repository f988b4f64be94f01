"""Sign-flipped Walsh-Hadamard rotation (OCTOPUS paper, Sec. 3.1; App. C.2).

R = H D_s with H the normalized Walsh-Hadamard matrix in natural (Sylvester)
order and D_s = diag(s).  H is symmetric and orthogonal, so
R^{-1} = R^T = D_s H (paper, App. C.2 summary).  The QJL residual uses a second
rotation R' = H D_{s'} with an independent sign vector (Sec. 3.6).

Here H is built explicitly from the Sylvester recursion
H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]] and scaled by 1/sqrt(d); the
rotation is a plain float64 matrix product (no fast transform).

Parity: pinned by H^T H = I, agreement with scipy.linalg.hadamard, and
(Rq).(Rk) = q.k (paper, App. B, Proposition 1) in tests/test_oracle_rotation.py.
"""
import numpy as np

from .splitmix import sign_vector


def hadamard(d: int) -> np.ndarray:
    """Normalized Sylvester-order Hadamard matrix, float64 [d, d]."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two (paper, Sec. 3)")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(d)


def signs(d: int, seed: int) -> np.ndarray:
    """s in {+-1}^d for R."""
    return np.array(sign_vector(seed, 0, d), dtype=np.float64)


def qjl_signs(d: int, seed: int) -> np.ndarray:
    """s' in {+-1}^d for R' (the next d draws of the same stream)."""
    return np.array(sign_vector(seed, d, d), dtype=np.float64)


def rotation_matrix(d: int, seed: int) -> np.ndarray:
    """R = H diag(s)."""
    return hadamard(d) * signs(d, seed)[None, :]


def qjl_rotation_matrix(d: int, seed: int) -> np.ndarray:
    """R' = H diag(s')."""
    return hadamard(d) * qjl_signs(d, seed)[None, :]


def rotate(x: np.ndarray, seed: int) -> np.ndarray:
    """u = R x for every row of x ([..., d] float64)."""
    d = x.shape[-1]
    return x @ rotation_matrix(d, seed).T


def unrotate(u: np.ndarray, seed: int) -> np.ndarray:
    """x = R^T u for every row of u."""
    d = u.shape[-1]
    return u @ rotation_matrix(d, seed)
