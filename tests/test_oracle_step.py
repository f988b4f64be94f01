"""Pins for oracle.step, the decode step with a native residual window (CPU).

  * while nothing has left the window, a step is plain softmax attention over
    the native rows: torch's scaled_dot_product_attention (float64);
  * eviction: after S steps with window W, the packed tokens [0, S - W + 1)
    are bit for bit the cache that encoding those tokens at once gives, and
    the ring holds the last W - 1 tokens at their slots;
  * with tokens packed, a step equals SDPA over the explicitly reconstructed
    packed keys and values followed by the native rows (one softmax);
  * W = 1 compresses every token right after the step that adds it;
  * with QJL keys, the step output is the two-part softmax mixture (packed
    part from the decode attention of the packed cache alone, native part),
    weighted by the parts' softmax masses.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import cache as C
from oracle import step as S
from tests.oracle_codecs import codec

D = 128


def bf16(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def stream(B, Hkv, Hq, steps, seed):
    rng = np.random.default_rng(seed)
    K = bf16(rng.standard_normal((B, Hkv, steps, D)))
    V = bf16(rng.standard_normal((B, Hkv, steps, D)))
    Q = bf16(rng.standard_normal((steps, B, Hq, D)))
    return K, V, Q


def sdpa(q, keys, vals):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None], torch.tensor(keys)[None], torch.tensor(vals)[None])[0].numpy()


def test_window_only_is_plain_attention():
    B, Hkv, Hq, W = 2, 2, 4, 8
    kc, vc = codec(3, seed=1), codec(3, seed=1)
    st = S.new_state(kc, vc, B, Hkv, 64, W)
    K, V, Q = stream(B, Hkv, Hq, W, 0)
    for t in range(W):
        out = S.decode_step(st, Q[t], K[:, :, t], V[:, :, t], kc, vc)
        for b in range(B):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                ref = sdpa(Q[t, b, h][None], K[b, g, :t + 1], V[b, g, :t + 1])[0]
                assert np.abs(out[b, h] - ref).max() < 1e-12
    assert list(st["P"]) == [1, 1] and list(st["n"]) == [W - 1, W - 1]


@pytest.mark.parametrize("qjl", [False, True])
def test_eviction_equals_encoding_at_once(qjl):
    B, Hkv, Hq, W, steps = 2, 2, 2, 4, 11
    kc, vc = codec(2, qjl=qjl, seed=3), codec(2, seed=3)
    st = S.new_state(kc, vc, B, Hkv, 64, W)
    K, V, Q = stream(B, Hkv, Hq, steps, 1)
    for t in range(steps):
        S.decode_step(st, Q[t], K[:, :, t], V[:, :, t], kc, vc)
    P = steps - W + 1
    assert list(st["P"]) == [P] * B and list(st["n"]) == [W - 1] * B
    kk, vv = C.empty_cache(kc, B, Hkv, 64), C.empty_cache(vc, B, Hkv, 64)
    C.encode_into(kk, kc, K[:, :, :P])
    C.encode_into(vv, vc, V[:, :, :P])
    for name in kk:
        if isinstance(kk[name], np.ndarray):
            assert np.array_equal(st["k"][name], kk[name]), name
    for name in vv:
        if isinstance(vv[name], np.ndarray):
            assert np.array_equal(st["v"][name], vv[name]), name
    for j in range(P, steps):
        assert np.array_equal(st["k_ring"][:, :, j % W], K[:, :, j])
        assert np.array_equal(st["v_ring"][:, :, j % W], V[:, :, j])


@pytest.mark.parametrize("W", [1, 5])
def test_step_is_attention_over_reconstruction_and_window(W):
    B, Hkv, Hq, steps = 1, 2, 4, 9
    kc, vc = codec(3, seed=2), codec(3, seed=2)
    st = S.new_state(kc, vc, B, Hkv, 64, W)
    K, V, Q = stream(B, Hkv, Hq, steps, 2)
    for t in range(steps):
        P = int(st["P"][0])
        out = S.decode_step(st, Q[t], K[:, :, t], V[:, :, t], kc, vc)
        # every token below t + 1 - W is packed, the rest native
        assert P == max(0, t + 1 - W)
        for h in range(Hq):
            g = h // (Hq // Hkv)
            if P:
                k_hat, _ = A.reconstruct(st["k"], kc, 0, g, 0, P)
                v_hat, _ = A.reconstruct(st["v"], vc, 0, g, 0, P)
            else:
                k_hat = v_hat = np.zeros((0, D))
            keys = np.concatenate([k_hat, K[0, g, P:t + 1]])
            vals = np.concatenate([v_hat, V[0, g, P:t + 1]])
            ref = sdpa(Q[t, 0, h][None], keys, vals)[0]
            assert np.abs(out[0, h] - ref).max() < 1e-12
    if W == 1:
        assert st["P"][0] == steps and st["n"][0] == 0


def test_qjl_step_is_two_part_mixture():
    B, Hkv, Hq, W, steps = 1, 1, 3, 3, 8
    kc, vc = codec(2, qjl=True, seed=4), codec(2, seed=4)
    st = S.new_state(kc, vc, B, Hkv, 64, W)
    K, V, Q = stream(B, Hkv, Hq, steps, 3)
    for t in range(steps - 1):
        S.decode_step(st, Q[t], K[:, :, t], V[:, :, t], kc, vc)
    P = int(st["P"][0])
    packed_out = A.decode_attention(Q[-1], st["k"], st["v"], kc, vc, [P])
    out = S.decode_step(st, Q[-1], K[:, :, -1], V[:, :, -1], kc, vc)
    scale = 1 / np.sqrt(D)
    for h in range(Hq):
        # log-masses of the two parts: the packed part's from its scores
        k_hat, krec = A.reconstruct(st["k"], kc, 0, 0, 0, P)
        sp = scale * (Q[-1, 0, h] @ k_hat.T + A.qjl_correction(Q[-1, 0, h][None], krec, kc)[0])
        sw = scale * (K[0, 0, P:] @ Q[-1, 0, h])
        m = max(sp.max(), sw.max())
        mp, mw = np.exp(sp - m).sum(), np.exp(sw - m).sum()
        win = np.exp(sw - m) @ V[0, 0, P:] / mw
        ref = (mp * packed_out[0, h] + mw * win) / (mp + mw)
        assert np.abs(out[0, h] - ref).max() < 1e-12
