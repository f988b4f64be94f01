"""Pins of the Jensen-bias correction of the oracle (oracle/group.py,
oracle/attention.chunk_attention(correction=True)).

"Quantized Keys Steal Attention" (Sec. 4.1-4.2, appendix "Taylor
approximation"): uniform round-to-nearest noise on a cached key inflates its
expected exponentiated score by prod_c sinh(a_c)/a_c, a_c = tau q_c Delta_c/2;
Eq. 15 is the Taylor form tau^2/24 sum_j Delta_j^2 ||q_j||^2.  Pinned by the
series of log(sinh a / a), a Monte-Carlo estimate of the expectation itself,
the over-estimation the page states, invariances of the softmax, and the
page's attention-mass claim measured with the real quantizer.
"""
import numpy as np

from oracle import group as G
from oracle.attention import chunk_attention
from oracle.cache import empty_cache, encode_into
from tests.oracle_codecs import group_codec


def test_taylor_form_is_the_series_of_the_exact_correction():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((6, 128))
    s8 = rng.integers(40, 60, (9, 4)).astype(np.uint8)              # steps ~0.2 .. 0.9
    tau = 1 / np.sqrt(128)
    t = G.jensen_bias(q, s8, 32, tau)
    e = G.jensen_bias_exact(q, s8, 32, tau)
    dh = np.repeat(G.from_e4m3(s8), 32, axis=1)
    a = np.abs(tau * q[:, None, :] * dh[None] / 2)
    assert a.max() < 0.5
    # log(sinh a / a) = a^2/6 - a^4/180 + a^6/2835 - ...
    fourth = (a ** 4).sum(axis=-1) / 180
    assert np.all(t >= e)                                            # the Taylor term over-estimates
    assert np.allclose(t - e, fourth, rtol=0.05, atol=1e-12)


def test_exact_correction_is_the_expected_noise_factor():
    # Monte Carlo of E[exp(tau q . eps)], eps_c ~ U(-Delta_c/2, Delta_c/2)
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 128)) * 3.0
    s8 = np.array([[0x40, 0x44, 0x48, 0x3C]], dtype=np.uint8)       # 2, 3, 4, 1.5
    tau = 1 / np.sqrt(128)
    dh = np.repeat(G.from_e4m3(s8), 32, axis=1)[0]
    n = 200000
    eps = (rng.random((n, 128)) - 0.5) * dh
    mc = np.log(np.mean(np.exp(tau * eps @ q[0])))
    exact = G.jensen_bias_exact(q, s8, 32, tau)[0, 0]
    assert exact > 0.1
    assert abs(mc - exact) < 0.02 * exact


def test_eq15_at_tau_one_over_sqrt_d():
    # with tau = 1/sqrt(d) the correction is 1/(24 d) sum_j Delta_j^2 ||q_j||^2
    rng = np.random.default_rng(2)
    q = rng.standard_normal((3, 128))
    s8 = rng.integers(30, 70, (5, 8)).astype(np.uint8)
    per_coord = np.array([[sum(q[a, c] ** 2 * G.from_e4m3(s8[i, c // 16]) ** 2 for c in range(128))
                           for i in range(5)] for a in range(3)]) / (24 * 128)
    assert np.allclose(G.jensen_bias(q, s8, 16, 1 / np.sqrt(128)), per_coord, rtol=1e-12)


def _setup(seed, cached=256, cur=32, Tq=16, bits=2, group=32, const=False):
    rng = np.random.default_rng(seed)
    kc, vc = group_codec(bits, group, seed=seed), group_codec(bits, group, seed=seed + 1)
    k = rng.standard_normal((1, 1, cached, 128))
    if const:
        k[:] = k[:, :, :1]                                           # one key repeated
    v = rng.standard_normal((1, 1, cached, 128))
    kcache, vcache = empty_cache(kc, 1, 1, cached), empty_cache(vc, 1, 1, cached)
    encode_into(kcache, kc, k)
    encode_into(vcache, vc, v)
    q = rng.standard_normal((1, 1, Tq, 128)) * 2.0
    kcur = rng.standard_normal((1, 1, cur, 128))
    vcur = rng.standard_normal((1, 1, cur, 128))
    return q, kcache, vcache, kc, vc, kcur, vcur, k, v


def test_constant_bias_without_current_tokens_changes_nothing():
    # one key repeated: every cached token has the same steps, so the bias is
    # the same for all of them and cancels in the softmax
    q, kcache, vcache, kc, vc, kcur, vcur, *_ = _setup(3, const=True)
    none = np.zeros((1, 1, 0, 128))
    a = chunk_attention(q, kcache, vcache, kc, vc, 256, none, none)
    b = chunk_attention(q, kcache, vcache, kc, vc, 256, none, none, correction=True)
    assert np.allclose(a, b, atol=1e-12)
    c = chunk_attention(q, kcache, vcache, kc, vc, 256, kcur, vcur, correction=True)
    assert not np.allclose(a, c)


def test_keys_on_a_flat_grid_need_no_correction():
    # keys constant within every group in the rotated frame: their steps are
    # (near) zero, so the correction is (near) zero and nothing changes
    from oracle.rotation import rotation_matrix
    rng = np.random.default_rng(4)
    kc, vc = group_codec(2, 32, seed=4), group_codec(2, 32, seed=5)
    u = np.repeat(rng.standard_normal((1, 1, 64, 4)), 32, axis=-1)
    k = u @ rotation_matrix(128, 4)                                    # R^T u
    v = rng.standard_normal((1, 1, 64, 128))
    kcache, vcache = empty_cache(kc, 1, 1, 64), empty_cache(vc, 1, 1, 64)
    encode_into(kcache, kc, k)
    encode_into(vcache, vc, v)
    q = rng.standard_normal((1, 1, 8, 128))
    kcur, vcur = rng.standard_normal((1, 1, 16, 128)), rng.standard_normal((1, 1, 16, 128))
    a = chunk_attention(q, kcache, vcache, kc, vc, 64, kcur, vcur)
    b = chunk_attention(q, kcache, vcache, kc, vc, 64, kcur, vcur, correction=True)
    assert np.allclose(a, b, atol=1e-9)


def test_attention_mass_claim_with_the_real_quantizer():
    # QKSA Sec. 5 / Fig. 4: under INT2 the cached tokens gain attention mass
    # (Delta P_S > 0); the correction moves it back toward zero (and may
    # over-correct slightly).  Exact mass from the unquantized keys; the same
    # queries and current tokens; averaged over seeds.
    def masses(seed):
        rng = np.random.default_rng(seed)
        cached, cur, Tq, d = 512, 64, 32, 128
        kc = group_codec(2, 32, seed=seed)
        k = rng.standard_normal((1, 1, cached, d))
        q = rng.standard_normal((Tq, d)) * 1.5
        kcur = rng.standard_normal((cur, d))
        kcache = empty_cache(kc, 1, 1, cached)
        encode_into(kcache, kc, k)
        from oracle.attention import reconstruct
        from oracle.rotation import rotation_matrix
        k_hat, rec = reconstruct(kcache, kc, 0, 0, 0, cached)
        tau = 1 / np.sqrt(d)

        def mass(keys_cached, bias=0.0):
            lc = tau * q @ keys_cached.T - bias
            lr = tau * q @ kcur.T
            m = np.maximum(lc.max(1, keepdims=True), lr.max(1, keepdims=True))
            zc, zr = np.exp(lc - m).sum(1), np.exp(lr - m).sum(1)
            return np.mean(zc / (zc + zr))
        b = G.jensen_bias(q @ rotation_matrix(d, seed).T, rec["scale8"], 32, tau)
        return mass(k[0, 0]), mass(k_hat), mass(k_hat, b)
    m = np.array([masses(s) for s in range(12)])
    d_plain = np.mean(m[:, 1] - m[:, 0])
    d_corr = np.mean(m[:, 2] - m[:, 0])
    assert d_plain > 0.0
    assert abs(d_corr) < 0.5 * d_plain
