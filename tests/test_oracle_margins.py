"""Pins for the oracle's decision margins (CPU).

The GPU parity tests forgive a disagreement in an index only where the
oracle's margin says the decision's input lies within 1e-6 of a decision
threshold.  These tests pin every margin to the distance at which its
decision actually changes: each decision input is nudged (through the
oracle's own nudge arguments) by 0.999 of its reported margin in every
direction of the max-norm ball, which must leave the decision as it is, and
by 1.001 of it in the worst direction, which must change it.  A margin off by
any factor, measured to the wrong cell edge or with a wrong sign fails one of
the two.  Covered: the hemisphere test, the fold signs, the Lloyd seeds, the
3x3 and full-grid argmax and the norm index of the OCTOPUS encoder (every
default and uniform split, all rounding modes), the QJL signs, and the E4M3
scale, BF16 zero-point and code decisions of the group-wise value codec.  A
joint nudge of every input by less than the triplet's smallest margin leaves
all indices unchanged.
"""
import itertools

import numpy as np
import pytest

from oracle import encode as E
from oracle import group as Gc
from oracle.rotation import rotation_matrix
from tests.oracle_codecs import codec

IN, OUT = 0.999, 1.001


def triplets(bits_seed, n_vec=60):
    """Rotated-frame triplets of unit Gaussian keys at d = 128 (the encoder's
    inputs), plus triplets with tiny components that sit near the hemisphere
    and fold thresholds."""
    rng = np.random.default_rng(bits_seed)
    x = rng.standard_normal((n_vec, 128))
    u = (x / np.linalg.norm(x, axis=1, keepdims=True)) @ rotation_matrix(128, 0).T
    t = E.split_triplets(u).reshape(-1, 3)
    near = rng.standard_normal((200, 3)) * 0.1
    near[:100, 2] *= 1e-4                      # near the equator
    near[100:, 0] *= 1e-4                      # near a fold sign
    return np.concatenate([t, near])


SPLITS = [(3, 1), (4, 2), (5, 3), (2, 2), (3, 3), (4, 4)]


def _cands(e, K, rounding):
    """Codes of the argmax candidates in the encoder's order."""
    if rounding == E.ROUND_FULL:
        return np.broadcast_to(np.arange(K * K), e["code"].shape + (K * K,))
    cx = np.stack([np.clip(e["seed_xi"] + a, 0, K - 1) for a, _ in E.ORDER], axis=-1)
    cy = np.stack([np.clip(e["seed_eta"] + b, 0, K - 1) for _, b in E.ORDER], axis=-1)
    return cx * K + cy


def _check_component(t, c, rounding, comp):
    cx, cr = c["c_xi"], c["c_rho"]
    K = cx.size
    base = E.encode_triplets(t, cx, cr, rounding)
    m = base["m_" + comp]
    sel = np.isfinite(m) & (m > 1e-12)
    assert sel.sum() > 20, (comp, int(sel.sum()))
    t, m = t[sel], m[sel]
    base = {k: v[sel] for k, v in base.items()}
    dec = {
        "hemi": lambda e: [e["upper"]],
        "fold": lambda e: [e["neg_x"], e["neg_y"]],
        "seed": lambda e: [e["seed_xi"], e["seed_eta"]],
        "gap": lambda e: [e["code"]],
        "rho": lambda e: [e["i_rho"]],
    }[comp]
    same = lambda e: np.logical_and.reduce([a == b for a, b in zip(dec(e), dec(base))])  # noqa: E731
    run = lambda nudge: E.encode_triplets(t, cx, cr, rounding, nudge)                    # noqa: E731
    if comp == "gap":
        cand = _cands(base, K, rounding)
        own = cand == base["code"][:, None]
        sgn = np.where(own, -1.0, 1.0)                 # the worst corner: best down, rivals up
        assert same(run({"s": IN * m[:, None] * sgn})).all()
        assert not same(run({"s": OUT * m[:, None] * sgn})).any()
        return
    keys = {"hemi": ["pz"], "fold": ["px", "py"], "seed": ["xi", "eta"], "rho": ["s_star"]}[comp]
    # inside: every corner of the max-norm ball of radius 0.999 m
    for signs in itertools.product((-1.0, 1.0), repeat=len(keys)):
        nudge = {k: IN * sg * m for k, sg in zip(keys, signs)}
        assert same(run(nudge)).all(), (comp, signs)
    # outside: some single input moved by 1.001 m changes the decision
    changed = np.zeros(len(m), dtype=bool)
    for k in keys:
        for sg in (-1.0, 1.0):
            changed |= ~same(run({k: OUT * sg * m}))
    assert changed.all(), (comp, int((~changed).sum()))


@pytest.mark.parametrize("split", SPLITS)
@pytest.mark.parametrize("rounding", [E.ROUND_LOCAL3X3, E.ROUND_SCALAR])
def test_encoder_margins_are_distances_to_decision_points(split, rounding):
    c = codec(b_dir=split[0], b_nrm=split[1])
    t = triplets(10 * split[0] + split[1])
    comps = ["hemi", "fold", "seed", "rho"] + (["gap"] if rounding == E.ROUND_LOCAL3X3 else [])
    for comp in comps:
        _check_component(t, c, rounding, comp)


@pytest.mark.parametrize("split", [(3, 1), (2, 2)])
def test_full_grid_gap_margin(split):
    c = codec(b_dir=split[0], b_nrm=split[1])
    t = triplets(7, n_vec=20)
    for comp in ("gap", "rho"):
        _check_component(t, c, E.ROUND_FULL, comp)


@pytest.mark.parametrize("split", SPLITS)
def test_joint_nudge_below_the_margin_keeps_every_index(split):
    """All inputs moved at once, each by less than the triplet's smallest
    margin (random directions): the indices (i_xi, i_eta, i_rho) stay."""
    c = codec(b_dir=split[0], b_nrm=split[1])
    t = triplets(3 + split[0])
    base = E.encode_triplets(t, c["c_xi"], c["c_rho"])
    sel = np.isfinite(base["margin"]) & (base["margin"] > 1e-12)
    t = t[sel]
    m = base["margin"][sel]
    rng = np.random.default_rng(1)
    for _ in range(5):
        r = lambda *sh: IN * m.reshape((-1,) + (1,) * len(sh)) * rng.uniform(-1, 1, (len(m),) + sh)  # noqa: E731
        nudge = {"pz": r(), "px": r(), "py": r(), "xi": r(), "eta": r(), "s": r(9)}
        e = E.encode_triplets(t, c["c_xi"], c["c_rho"], nudge=nudge)
        for k in ("i_xi", "i_eta", "i_rho"):
            assert np.array_equal(e[k], base[k][sel]), k


def test_margin_is_smallest_component_and_zero_on_ties():
    c = codec(3)
    t = triplets(5)
    e = E.encode_triplets(t, c["c_xi"], c["c_rho"])
    comp = np.minimum.reduce([e["m_hemi"], e["m_fold"], e["m_seed"], e["m_gap"], e["m_rho"]])
    assert np.array_equal(e["margin"], comp)
    # a triplet on the equator and one exactly between two C_xi centroids
    cx = c["c_xi"].astype(np.float64)
    mid = 0.5 * (cx[3] + cx[4])
    tie = np.array([[0.3, 0.2, 0.0], [mid * 0.5, 0.1, 0.5 - abs(mid * 0.5) - 0.1 + 0.5]])
    e2 = E.encode_triplets(tie, c["c_xi"], c["c_rho"])
    assert e2["m_hemi"][0] == 0.0 and e2["margin"][0] == 0.0


def test_qjl_sign_margins():
    rng = np.random.default_rng(2)
    r = rng.standard_normal((40, 128)) * 0.05
    neg, m = E.qjl_signs(r, 0)
    for sg in (-1.0, 1.0):
        assert np.array_equal(E.qjl_signs(r, 0, IN * sg * m)[0], neg)
    flipped = (E.qjl_signs(r, 0, OUT * m)[0] != neg) | (E.qjl_signs(r, 0, -OUT * m)[0] != neg)
    assert flipped.all()


def _fp32_ok(x, m):
    """Margins large enough that a 0.001 m step is resolved in fp32."""
    ulp = np.spacing(np.abs(np.asarray(x, dtype=np.float32))).astype(np.float64)
    return np.isfinite(m) & (m > 4e3 * ulp)


def test_e4m3_margins():
    rng = np.random.default_rng(3)
    vals = Gc.e4m3_values()
    x = np.concatenate([rng.uniform(0, 470, 3000), rng.uniform(0, 0.05, 1000),
                        vals[8:] * (1 + rng.uniform(-0.03, 0.03, vals[8:].size)),   # binade edges
                        vals[1:] * (1 + 1e-3)])
    x = np.abs(x).astype(np.float32).astype(np.float64)
    code, m = Gc.to_e4m3(x)
    ok = _fp32_ok(x, m) & (x - m > 0)
    x, m, code = x[ok], m[ok], code[ok]
    assert len(x) > 3000
    for sg in (-1.0, 1.0):
        assert np.array_equal(Gc.to_e4m3(x + IN * sg * m)[0], code)
    ch = (Gc.to_e4m3(x + OUT * m)[0] != code) | (Gc.to_e4m3(np.maximum(x - OUT * m, 0))[0] != code)
    assert ch.all()
    # the saturated cell reaches down to the midpoint of 416 and 448
    assert Gc.to_e4m3(np.array([500.0]))[1][0] == pytest.approx(500.0 - 432.0)


def test_bf16_margins():
    rng = np.random.default_rng(4)
    p2 = 2.0 ** rng.integers(-20, 20, 2000)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-6, 6, 3000),
                        p2 * (1 + rng.uniform(-2e-3, 2e-3, 2000)) * rng.choice([-1, 1], 2000)])
    x = x.astype(np.float32).astype(np.float64)
    h, m = Gc.to_bf16(x)
    ok = _fp32_ok(x, m)
    x, m, h = x[ok], m[ok], h[ok]
    assert len(x) > 3000
    for sg in (-1.0, 1.0):
        assert np.array_equal(Gc.to_bf16(x + IN * sg * m)[0], h)
    ch = (Gc.to_bf16(x + OUT * m)[0] != h) | (Gc.to_bf16(x - OUT * m)[0] != h)
    assert ch.all()


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_group_code_margins(bits):
    rng = np.random.default_rng(5 + bits)
    u = rng.standard_normal((400, 32)).astype(np.float32) * 0.1
    dh = np.float32(0.2 / ((1 << bits) - 1))
    zh = np.float32(-0.1)
    q, m = Gc.group_codes(u, dh, zh, bits)
    # the decision is taken on (u - z^) / Delta^ in fp32: resolve a 0.001 m
    # step in that quotient, not only in u
    qf = (u - zh) / dh
    ok = _fp32_ok(u, m) & _fp32_ok(u - zh, m) & _fp32_ok(qf, m / dh)
    u, m, q = u[ok], m[ok], q[ok]
    assert len(u) > 5000
    for sg in (-1.0, 1.0):
        assert np.array_equal(Gc.group_codes(u, dh, zh, bits, IN * sg * m)[0], q)
    ch = (Gc.group_codes(u, dh, zh, bits, OUT * m)[0] != q) | \
         (Gc.group_codes(u, dh, zh, bits, -OUT * m)[0] != q)
    assert ch.all()
