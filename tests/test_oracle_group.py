"""Pins of the group-wise value codec oracle (oracle/group.py).

The codec follows "Quantized Keys Steal Attention" (Sec. 3, quantization
granularity and Hadamard rotation; Sec. 4.3, B_eff = B + 24/g with FP8 E4M3
scales and BF16 zero-points; Sec. 5, asymmetric round-to-nearest) as the value
codec that the OCTOPUS page's experiments share (Sec. 4).  Each pin checks the
oracle against something other than itself: the E4M3 format definition,
torch's float8_e4m3fn / bfloat16 conversions, exact rational search, closed
error bounds or a statement of the pages.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import group as G
from oracle import pack
from oracle.attention import decode_attention, reconstruct
from oracle.cache import empty_cache, encode_into
from oracle.rotation import rotation_matrix
from tests.oracle_codecs import codec, group_codec


def test_e4m3_format_points():
    v = G.e4m3_values()
    assert v.size == 127 and np.all(np.diff(v) > 0)
    assert v[0x38] == 1.0 and v[0x7E] == 448.0
    assert v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x30] == 0.5 and v[0x3C] == 1.5


def test_e4m3_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (np.abs(rng.standard_normal(50000)) * 2.0 ** rng.integers(-12, 9, 50000)).astype(np.float32)
    v = G.e4m3_values()
    mids = (0.5 * (v[1:] + v[:-1])).astype(np.float32)          # every tie, exact in fp32
    x = np.concatenate([x[x < 448], mids, v.astype(np.float32), np.float32([0.0, 2.0 ** -11])])
    code, _ = G.to_e4m3(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(code, ref)
    # ties go to the even code: 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39)
    assert G.to_e4m3(np.float32([1.0625, 1.1875]))[0].tolist() == [0x38, 0x3A]


def test_e4m3_saturates():
    code, _ = G.to_e4m3(np.float32([448.0, 449.0, 463.9, 500.0, 1e30]))
    assert code.tolist() == [0x7E] * 5


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(50000) * 2.0 ** rng.integers(-20, 20, 50000)).astype(np.float32)
    ties = ((rng.integers(0, 2 ** 15, 1000, dtype=np.int64) << 16) | 0x8000).astype(np.uint32).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)], -ties[np.isfinite(ties)]])
    code, _ = G.to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(code, ref)


def test_record_size_is_b_eff():
    # Sec. 4.3 of the QKSA page: B_eff = B + 24/g bits per coordinate
    for bits in (2, 3, 4):
        for g in (16, 32):
            assert G.record_words(128, bits, g) * 32 == 128 * (bits + 24 / g)


def test_pack_layout_positions():
    rng = np.random.default_rng(2)
    for bits in (2, 3, 4):
        for g in (16, 32):
            n = 128 // g
            codes = rng.integers(0, 1 << bits, (5, 128))
            s8 = rng.integers(0, 127, (5, n)).astype(np.uint8)
            z16 = rng.integers(0, 1 << 16, (5, n)).astype(np.uint16)
            w = G.pack_record(codes, s8, z16, bits)
            assert w.shape == (5, G.record_words(128, bits, g))
            big = [sum(int(x) << (32 * i) for i, x in enumerate(row)) for row in w]
            for t in range(5):
                for c in (0, 1, 77, 127):
                    assert (big[t] >> (c * bits)) & ((1 << bits) - 1) == codes[t, c]
                for j in range(n):
                    assert (big[t] >> (128 * bits + 8 * j)) & 0xFF == s8[t, j]
                    assert (big[t] >> (128 * bits + 8 * n + 16 * j)) & 0xFFFF == z16[t, j]
            c2, s2, z2 = G.unpack_record(w, 128, bits, g)
            assert np.array_equal(c2, codes) and np.array_equal(s2, s8) and np.array_equal(z2, z16)


def test_codes_are_nearest_grid_points_exactly():
    # brute force in exact rational arithmetic over the stored (Delta^, z^):
    # the code is the nearest of the 2^b grid points wherever the fp32
    # quotient is not within 1e-6 (relative) of a tie
    rng = np.random.default_rng(3)
    u = (rng.standard_normal((40, 128)) * rng.uniform(0.01, 20, (40, 1))).astype(np.float32)
    for bits in (2, 3, 4):
        for g in (16, 32):
            r = G.quantize_rotated(u, bits, g)
            n = 128 // g
            for t in range(0, 40, 3):
                for c in range(0, 128, 5):
                    j = c // g
                    dh = Fraction(float(G.from_e4m3(r["scale8"][t, j])))
                    zh = Fraction(float(G.from_bf16(r["zero16"][t, j])))
                    x = Fraction(float(u[t, c]))
                    dist = [abs(x - (zh + k * dh)) for k in range(1 << bits)]
                    best = min(dist)
                    cands = [k for k in range(1 << bits) if dist[k] == best]
                    if r["code_margin"][t, c] < 1e-6 * float(np.abs(u[t]).max()):
                        continue
                    assert r["codes"][t, c] in cands
            assert r["scale8"].shape == (40, n)


def test_half_step_bound_and_norm_bound():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 128))
    x[:, [3, 50, 90, 111]] *= 10.0            # outlier channels
    for bits in (2, 3, 4):
        for g in (16, 32):
            r = G.encode(x, bits, g, seed=7)
            u_hat = G.dequantize_rotated(r["codes"], r["scale8"], r["zero16"], g)
            dh = np.repeat(G.from_e4m3(r["scale8"]), g, axis=1)
            zh = np.repeat(G.from_bf16(r["zero16"]), g, axis=1)
            top = zh + ((1 << bits) - 1) * dh
            inside = (r["u32"] >= zh - dh / 2) & (r["u32"] <= top + dh / 2)
            err = np.abs(r["u32"] - u_hat)
            assert np.all(err[inside] <= dh[inside] / 2 * (1 + 1e-6) + 1e-30)
            # outside the grid the code is the nearer end point
            lo = r["u32"] < zh - dh / 2
            assert np.all(r["codes"][lo] == 0)
            hi = r["u32"] > top + dh / 2
            assert np.all(r["codes"][hi] == (1 << bits) - 1)
            # R is orthogonal: the reconstruction error of v is that of u
            x_hat = G.reconstruct(r["codes"], r["scale8"], r["zero16"], g, seed=7)
            assert np.allclose(np.linalg.norm(x - x_hat, axis=1),
                               np.linalg.norm(r["u"] - u_hat, axis=1), rtol=1e-9, atol=1e-9)


def test_grid_values_round_trip():
    # values that sit on the grid of their group decode exactly
    rng = np.random.default_rng(5)
    for bits in (2, 3, 4):
        levels = (1 << bits) - 1
        dh = np.float32(0.25)
        zh = np.float32(-1.5)
        codes = rng.integers(0, levels + 1, (8, 128))
        codes[:, ::16] = 0
        codes[:, 1::16] = levels              # every group spans the full range
        u = (zh + dh * codes).astype(np.float32)
        r = G.quantize_rotated(u, bits, 16)
        assert np.all(G.from_e4m3(r["scale8"]) == 0.25) and np.all(G.from_bf16(r["zero16"]) == -1.5)
        assert np.array_equal(r["codes"], codes)


def test_constant_group_and_zero_vector():
    u = np.zeros((2, 128), dtype=np.float32)
    u[1] = 3.0
    r = G.quantize_rotated(u, 2, 32)
    assert np.all(r["scale8"] == 0) and np.all(r["codes"] == 0)
    assert np.array_equal(G.dequantize_rotated(r["codes"], r["scale8"], r["zero16"], 32), u.astype(np.float64))


def test_uniform_noise_mse_is_delta_squared_over_12():
    # textbook: rounding error of a uniform quantizer on smooth data ~ U(-D/2, D/2)
    rng = np.random.default_rng(6)
    u = rng.uniform(-1, 1, (4000, 128)).astype(np.float32)
    r = G.quantize_rotated(u, 4, 32)
    u_hat = G.dequantize_rotated(r["codes"], r["scale8"], r["zero16"], 32)
    dh = np.repeat(G.from_e4m3(r["scale8"]), 32, axis=1)
    ratio = np.mean((u - u_hat) ** 2) / np.mean(dh ** 2 / 12)
    assert 0.95 < ratio < 1.05


def test_smaller_groups_give_smaller_error():
    # QKSA Sec. 3: the smaller the group sharing (Delta, z), the smaller the error
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2000, 128))
    for bits in (2, 3, 4):
        mse = {}
        for g in (16, 32):
            r = G.encode(x, bits, g, seed=0)
            x_hat = G.reconstruct(r["codes"], r["scale8"], r["zero16"], g, seed=0)
            mse[g] = np.mean((x - x_hat) ** 2)
        assert mse[16] < mse[32]


def test_rotation_spreads_outliers():
    # QKSA Sec. 3: outlier channels inflate the step size; the rotation spreads
    # their energy and lowers the error of the same quantizer
    rng = np.random.default_rng(8)
    x = rng.standard_normal((2000, 128))
    x[:, [5, 40, 77, 120]] *= 10.0
    for bits in (2, 3):
        r = G.encode(x, bits, 32, seed=0)
        rot = np.mean((x - G.reconstruct(r["codes"], r["scale8"], r["zero16"], 32, seed=0)) ** 2)
        p = G.quantize_rotated(x.astype(np.float32), bits, 32)
        plain = np.mean((x - G.dequantize_rotated(p["codes"], p["scale8"], p["zero16"], 32)) ** 2)
        assert rot < plain


def test_cache_round_trip_and_attention_on_explicit_values():
    rng = np.random.default_rng(9)
    B, H, T, d = 2, 2, 70, 128
    kc, vc = codec(bits=3), group_codec(bits=2, group=32, seed=0)
    k = rng.standard_normal((B, H, T, d))
    v = rng.standard_normal((B, H, T, d))
    kcache, vcache = empty_cache(kc, B, H, 128), empty_cache(vc, B, H, 128)
    encode_into(kcache, kc, k)
    enc = encode_into(vcache, vc, v)
    assert "gamma" not in vcache
    for b in range(B):
        for h in range(H):
            v_hat, rec = reconstruct(vcache, vc, b, h, 0, T)
            assert np.array_equal(rec["codes"], enc["codes"][b, h])
            direct = G.reconstruct(enc["codes"][b, h], enc["scale8"][b, h], enc["zero16"][b, h], 32, 0)
            assert np.array_equal(v_hat, direct)
    q = rng.standard_normal((B, 2 * H, d))
    lens = np.array([T, 33])
    out = decode_attention(q, kcache, vcache, kc, vc, lens)
    for b in range(B):
        for h in range(2 * H):
            g = h // 2
            k_hat, _ = reconstruct(kcache, kc, b, g, 0, lens[b])
            v_hat, _ = reconstruct(vcache, vc, b, g, 0, lens[b])
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b, h][None, None, None]), torch.from_numpy(k_hat[None, None]),
                torch.from_numpy(v_hat[None, None]))[0, 0, 0].numpy()
            assert np.allclose(out[b, h], ref, atol=1e-12)


def test_group_codec_converges_to_exact_attention():
    rng = np.random.default_rng(10)
    T, d = 200, 128
    kc = codec(bits=4)
    k = rng.standard_normal((1, 1, T, d))
    v = rng.standard_normal((1, 1, T, d))
    q = rng.standard_normal((1, 1, d))
    exact = torch.softmax(torch.from_numpy(q[0] @ k[0, 0].T / np.sqrt(d)), -1).numpy() @ v[0, 0]
    kcache = empty_cache(kc, 1, 1, 256)
    encode_into(kcache, kc, k)
    errs = []
    for bits in (2, 3, 4):
        vc = group_codec(bits=bits, group=16)
        vcache = empty_cache(vc, 1, 1, 256)
        encode_into(vcache, vc, v)
        out = decode_attention(q, kcache, vcache, kc, vc, np.array([T]))
        errs.append(np.abs(out[0] - exact).max())
    assert errs[0] > errs[1] > errs[2]
