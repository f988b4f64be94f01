"""Pins for oracle.attention (CPU).

  * score factorization (OCTOPUS paper Sec. 3.6 Eq. 13 / App. C.14):
    q . k^ computed from the explicit reconstruction equals gamma q_rot . u^.
  * decode attention equals torch's scaled_dot_product_attention (float64, CPU)
    run on the explicitly reconstructed K^, V^, per GQA group.
  * the QJL-corrected score equals the estimator of Sec. 3.6 computed through
    the explicit matrices (R' R q) . sigma.
  * chunk attention equals SDPA over the concatenation of the reconstructed
    cached window and the full-precision current chunk.
  * attention on the quantized cache approaches exact attention as b grows;
    an empty context gives zeros.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import cache as C
from oracle.rotation import qjl_rotation_matrix, rotation_matrix
from tests.oracle_codecs import codec


def build(bits, B=2, H=2, T=100, cap=128, qjl=False, seed=0):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((B, H, T, 128)).astype(np.float32)
    V = rng.standard_normal((B, H, T, 128)).astype(np.float32)
    kc, vc = codec(bits, qjl=qjl, seed=5), codec(bits, seed=5)
    kk, vv = C.empty_cache(kc, B, H, cap), C.empty_cache(vc, B, H, cap)
    C.encode_into(kk, kc, K)
    C.encode_into(vv, vc, V)
    return K, V, kc, vc, kk, vv


def test_score_factorization_eq13():
    K, V, kc, vc, kk, vv = build(3)
    q = np.random.default_rng(9).standard_normal((7, 128))
    k_hat, rec = A.reconstruct(kk, kc, 1, 0, 0, 100)
    from oracle.cache import u_hat_from_indices
    u_hat = u_hat_from_indices(kc, rec["i_xi"], rec["i_eta"], rec["i_rho"])
    q_rot = np.concatenate([q @ rotation_matrix(128, 5).T, np.zeros((7, 1))], 1)
    lhs = q @ k_hat.T
    rhs = rec["gamma"][None, :] * (q_rot @ u_hat.T)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-11)


@pytest.mark.parametrize("qjl", [False, True])
def test_decode_matches_sdpa_on_explicit_reconstruction(qjl):
    K, V, kc, vc, kk, vv = build(2, qjl=qjl)
    B, Hkv, G = 2, 2, 3
    q = np.random.default_rng(4).standard_normal((B, Hkv * G, 128))
    seq = np.array([100, 37])
    out = A.decode_attention(q, kk, vv, kc, vc, seq)
    for b in range(B):
        for g in range(Hkv):
            L = seq[b]
            k_hat, rec = A.reconstruct(kk, kc, b, g, 0, L)
            v_hat, _ = A.reconstruct(vv, vc, b, g, 0, L)
            qg = torch.tensor(q[b, g * G:(g + 1) * G])
            mask = None
            if qjl:
                # the estimator as an additive score term, through explicit matrices
                sigma = np.where(rec["sigma_neg"], -1.0, 1.0)
                M = qjl_rotation_matrix(128, 5) @ rotation_matrix(128, 5)
                corr = np.sqrt(np.pi / 256) * rec["gamma"][None, :] * rec["gamma_r"][None, :] * ((q[b, g * G:(g + 1) * G] @ M.T) @ sigma.T)
                mask = torch.tensor(corr / np.sqrt(128))
            ref = torch.nn.functional.scaled_dot_product_attention(
                qg[None], torch.tensor(k_hat)[None], torch.tensor(v_hat)[None], attn_mask=mask)[0]
            assert np.allclose(out[b, g * G:(g + 1) * G], ref.numpy(), atol=1e-12)


def test_chunk_matches_sdpa_on_concatenation():
    K, V, kc, vc, kk, vv = build(2, B=1, H=2, T=70, cap=128)
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 2, 9, 128))
    kcur = rng.standard_normal((1, 2, 5, 128))
    vcur = rng.standard_normal((1, 2, 5, 128))
    out = A.chunk_attention(q, kk, vv, kc, vc, 70, kcur, vcur)
    for h in range(2):
        kh, _ = A.reconstruct(kk, kc, 0, h, 0, 70)
        vh, _ = A.reconstruct(vv, vc, 0, h, 0, 70)
        keys = torch.tensor(np.concatenate([kh, kcur[0, h]]))
        vals = torch.tensor(np.concatenate([vh, vcur[0, h]]))
        ref = torch.nn.functional.scaled_dot_product_attention(torch.tensor(q[0, h])[None], keys[None], vals[None])[0]
        assert np.allclose(out[0, h], ref.numpy(), atol=1e-12)
    part = A.chunk_attention(q, kk, vv, kc, vc, 70, kcur, vcur, q_rows=[0, 4])
    assert np.allclose(part[0, :, [0, 4]], out[0, :, [0, 4]], atol=1e-13)
    assert np.all(part[0, :, [1, 2, 3]] == 0)


def test_approaches_exact_attention_and_empty_context():
    errs = []
    for bits in (2, 3, 4):
        K, V, kc, vc, kk, vv = build(bits, B=1, H=1, T=100, seed=3)
        q = np.random.default_rng(8).standard_normal((1, 1, 128)) * 0.3
        out = A.decode_attention(q, kk, vv, kc, vc, [100])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q, dtype=torch.float64)[:, :, None], torch.tensor(K, dtype=torch.float64),
            torch.tensor(V, dtype=torch.float64))[:, :, 0].numpy()
        errs.append(np.abs(out - ref).max())
    assert errs[0] > errs[1] > errs[2] and errs[2] < 0.05
    out = A.decode_attention(q, kk, vv, kc, vc, [0])
    assert np.all(out == 0)


def test_chunk_edge_windows():
    """No cached tokens: plain attention over the current chunk (SDPA); no
    current tokens: attention over the reconstructed window; neither: zeros."""
    K, V, kc, vc, kk, vv = build(2, B=1, H=1, T=40, cap=64)
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 1, 3, 128))
    kcur = rng.standard_normal((1, 1, 6, 128))
    vcur = rng.standard_normal((1, 1, 6, 128))
    out = A.chunk_attention(q, kk, vv, kc, vc, 0, kcur, vcur)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q[0]), torch.tensor(kcur[0]), torch.tensor(vcur[0]))
    assert np.allclose(out[0], ref.numpy(), atol=1e-12)
    empty = np.zeros((1, 1, 0, 128))
    out = A.chunk_attention(q, kk, vv, kc, vc, 40, empty, empty)
    kh, _ = A.reconstruct(kk, kc, 0, 0, 0, 40)
    vh, _ = A.reconstruct(vv, vc, 0, 0, 0, 40)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q[0]), torch.tensor(kh)[None], torch.tensor(vh)[None])
    assert np.allclose(out[0], ref.numpy(), atol=1e-12)
    out = A.chunk_attention(q, kk, vv, kc, vc, 0, empty, empty)
    assert np.all(out == 0)
