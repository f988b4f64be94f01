"""GPU parity of octo_encode against the oracle encoder (bit-exact indices).

Covers the five workload shapes at sizes the oracle finishes in seconds (with
ragged tails), the full-size encodes on sampled tokens, appends at unaligned
token offsets, zero vectors, the scalar rounding mode and the uniform (b, b)
splits; large launches of the b_dir >= 5 splits (the encoder takes four
16-token tiles a wavefront there) in scalar rounding, fp32 input and two
sweep splits.
"""
import numpy as np
import pytest
import torch

from gpu_parity import (assert_encode_ok, codecs, compare_encode, encode_gpu, make_inputs, say,
                        workload)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("key,T", [("tiny", None), ("gqa32k", 333), ("batch16", 130),
                                   ("long128k", 200), ("chunk", 150)])
def test_encode_small(key, T):
    w = workload(key)
    say(f"encode {key} T={T}")
    inp = make_inputs(w, scale_T=T)
    kc, hk = codecs(w.bits, qjl=w.qjl)
    vc, hv = codecs(w.bits)
    for name, x, gc, hc in (("K", inp["K"], kc, hk), ("V", inp["V"], vc, hv)):
        cache = encode_gpu(x, gc)
        assert_encode_ok(compare_encode(cache.to_host(), hc, x), f"{key} {name}")


@pytest.mark.parametrize("key", ["gqa32k", "batch16", "long128k", "chunk"])
def test_encode_full_size_sampled(key):
    """Full-size encode (the configuration the benchmark times); the oracle
    re-encodes a seeded sample of tokens in two planes."""
    w = workload(key)
    say(f"encode full {key}")
    inp = make_inputs(w)
    for name, qjl in (("K", w.qjl), ("V", False)):
        gc, hc = codecs(w.bits, qjl=qjl)
        x = inp[name]
        cache = encode_gpu(x, gc, capacity=w.capacity)
        B, H, T, _ = x.shape
        rng = np.random.default_rng(1)
        tokens = np.sort(rng.choice(T, size=min(T, 384), replace=False))
        tokens[-1] = T - 1
        planes = [(0, 0), (B - 1, H - 1)]
        assert_encode_ok(compare_encode(cache.to_host(), hc, x, planes=planes, tokens=tokens),
                         f"{key} full {name}")
        del cache


def test_encode_append_unaligned_offsets():
    """Appends at token offsets that are not tile aligned land in the right words."""
    w = workload("gqa32k")
    inp = make_inputs(w, scale_T=200)
    gc, hc = codecs(4)
    x = inp["K"]
    cache = encode_gpu(x[:, :, :37], gc, capacity=256)
    for lo, hi in ((37, 100), (100, 101), (101, 200)):
        encode_gpu(x[:, :, lo:hi], gc, token_offset=lo, cache=cache)
    assert_encode_ok(compare_encode(cache.to_host(), hc, x), "append")


def test_encode_strided_input():
    """A non-contiguous [B, H, T, d] view (heads and tokens transposed)."""
    w = workload("gqa32k")
    inp = make_inputs(w, scale_T=96)
    x = inp["K"].transpose(1, 2).contiguous().transpose(1, 2)     # strides (T*H*d, d, H*d, 1)
    assert not x.is_contiguous()
    gc, hc = codecs(4)
    cache = encode_gpu(x.cuda(), gc)
    assert_encode_ok(compare_encode(cache.to_host(), hc, x), "strided")


def test_encode_zero_and_degenerate_vectors():
    """Zero vectors (gamma = 0, placeholder direction), one-hot vectors and a
    vector whose rotation hits triplet boundaries exactly."""
    x = torch.zeros(1, 1, 70, 128)
    x[0, 0, 1, 5] = 1.0
    x[0, 0, 2, :] = 1.0
    x[0, 0, 3, ::2] = -3.0
    x[0, 0, 4:] = torch.randn(66, 128, generator=torch.Generator().manual_seed(3))
    for bits in (2, 3, 4):
        gc, hc = codecs(bits)
        cache = encode_gpu(x, gc)
        h = cache.to_host()
        assert h["gamma"][0, 0, 0] == 0.0
        assert_encode_ok(compare_encode(h, hc, x), f"degenerate b={bits}")


# the (b + delta, b - delta) sweep splits of Sec. 3.3 besides delta = 0, +1
SWEEP = [(b, b + dl, b - dl) for b in (2, 3, 4) for dl in (-2, -1, 2)]


@pytest.mark.parametrize("bits,b_dir,b_nrm,rounding", [
    (3, None, None, "scalar"), (2, 2, 2, "local3x3"), (3, 3, 3, "local3x3"), (4, 4, 4, "scalar")]
    + [(b, bd, bn, "local3x3") for b, bd, bn in SWEEP])
def test_encode_modes(bits, b_dir, b_nrm, rounding):
    w = workload("tiny")
    inp = make_inputs(w)
    gc, hc = codecs(bits, b_dir=b_dir, b_nrm=b_nrm, rounding=rounding)
    cache = encode_gpu(inp["K"], gc)
    assert_encode_ok(compare_encode(cache.to_host(), hc, inp["K"]), f"mode {bits} {b_dir} {b_nrm} {rounding}")


def test_encode_qjl_small_all_splits():
    w = workload("tiny")
    inp = make_inputs(w)
    for bits in (2, 3, 4):
        gc, hc = codecs(bits, qjl=True, seed=5)
        cache = encode_gpu(inp["K"], gc)
        assert_encode_ok(compare_encode(cache.to_host(), hc, inp["K"]), f"qjl b={bits}")


def test_encode_deterministic():
    w = workload("gqa32k")
    inp = make_inputs(w, scale_T=300)
    gc, _ = codecs(4)
    a = encode_gpu(inp["K"], gc).to_host()
    b = encode_gpu(inp["K"], gc).to_host()
    for k in ("idx", "gamma"):
        assert np.array_equal(a[k], b[k])


@pytest.mark.parametrize("bits,b_dir,b_nrm,rounding,dtype", [
    (4, None, None, "scalar", torch.bfloat16), (4, None, None, "local3x3", torch.float32),
    (4, 6, 2, "local3x3", torch.bfloat16), (3, 5, 1, "local3x3", torch.bfloat16)])
def test_encode_large_launch_modes(bits, b_dir, b_nrm, rounding, dtype):
    """Launches of 4 x 25600 tokens with b_dir >= 5 (four tiles a wavefront):
    scalar rounding, fp32 input and two sweep splits, on sampled tokens of
    two planes."""
    g = torch.Generator().manual_seed(11)
    x = torch.randn(1, 4, 25600, 128, generator=g).to(dtype)
    gc, hc = codecs(bits, b_dir=b_dir, b_nrm=b_nrm, rounding=rounding, seed=7)
    say(f"large encode bits={bits} split=({b_dir},{b_nrm}) {rounding} {dtype}")
    cache = encode_gpu(x, gc)
    rng = np.random.default_rng(2)
    tokens = np.sort(rng.choice(25600, size=256, replace=False))
    tokens[-1] = 25599
    assert_encode_ok(compare_encode(cache.to_host(), hc, x, planes=[(0, 0), (0, 3)], tokens=tokens),
                     f"large {bits} {b_dir} {b_nrm} {rounding} {dtype}")
