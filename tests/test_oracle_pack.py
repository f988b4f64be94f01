"""Pins for oracle.pack and oracle.cache (CPU).

  * pack/unpack are inverse for every field width used (1..6 bits);
  * explicit bit positions of hand-made fields (LSB-first, little-endian);
  * padding bits are zero; words per token match the record-size table
    (I_dir 86 fields, I_nrm 43 fields, QJL 128 one-bit fields at d = 128);
  * the tile-64 word index formula, scatter/gather round trip, and an
    encode -> cache -> read round trip of the indices.
"""
import numpy as np
import pytest

from oracle import cache as C
from oracle import pack as P
from tests.oracle_codecs import codec


@pytest.mark.parametrize("width", [1, 2, 3, 4, 5, 6])
def test_round_trip(width):
    rng = np.random.default_rng(width)
    f = rng.integers(0, 2 ** width, size=(37, 86))
    words = P.pack_fields(f, width)
    assert words.shape == (37, -(-86 * width // 32))
    assert np.array_equal(P.unpack_fields(words, 86, width), f)


def test_explicit_bits_and_padding():
    w = P.pack_fields(np.array([[1, 0, 3]]), 2)
    assert w.shape == (1, 1) and int(w[0, 0]) == 1 | (0 << 2) | (3 << 4)
    # a 5-bit field straddling a word boundary: field 6 occupies bits 30..34
    f = np.zeros((1, 7), dtype=np.int64)
    f[0, 6] = 0b10111
    w = P.pack_fields(f, 5)
    assert int(w[0, 0]) == (0b11 << 30) and int(w[0, 1]) == 0b101
    # all-ones fields leave the padding bits zero
    f = np.full((1, 86), 31)
    w = P.pack_fields(f, 5)
    assert int(w[0, -1]) >> (430 - 13 * 32) == 0


def test_record_sizes():
    table = {4: (14, 5), 3: (11, 3), 2: (9, 2)}
    for b, (wd, wn) in table.items():
        s = C.stream_sizes(codec(b))
        assert (s["dir"], s["nrm"]) == (wd, wn)
    assert C.stream_sizes(codec(2, qjl=True))["qjl"] == 4
    # bytes per token: K and V records incl. fp32 gamma
    assert 4 * (14 + 5 + 1) == 80 and 4 * (11 + 3 + 1) == 60 and 4 * (9 + 2 + 1) == 48


def test_tile_index_and_scatter_gather():
    H, cap, W = 3, 192, 5
    assert P.tile_index(0, 0, 0, 0, H, cap, W) == 0
    assert P.tile_index(0, 0, 1, 0, H, cap, W) == 1
    assert P.tile_index(0, 0, 0, 1, H, cap, W) == 64
    assert P.tile_index(0, 0, 64, 0, H, cap, W) == 64 * W
    assert P.tile_index(0, 1, 0, 0, H, cap, W) == cap * W
    assert P.tile_index(1, 0, 0, 0, H, cap, W) == H * cap * W
    buf = np.zeros(2 * H * cap * W, dtype=np.uint32)
    words = np.random.default_rng(0).integers(0, 2 ** 32, size=(70, W), dtype=np.uint64).astype(np.uint32)
    P.scatter_tokens(buf, words, 1, 2, 100, H, cap)
    assert np.array_equal(P.gather_tokens(buf, 1, 2, 100, 70, H, cap, W), words)
    assert np.count_nonzero(buf) == np.count_nonzero(words)


@pytest.mark.parametrize("qjl", [False, True])
def test_encode_into_cache_round_trip(qjl):
    c = codec(2, qjl=qjl)
    x = np.random.default_rng(1).standard_normal((2, 2, 70, 128)).astype(np.float32)
    cache = C.empty_cache(c, 2, 2, 128)
    enc = C.encode_into(cache, c, x, token_offset=5)
    for b in range(2):
        for h in range(2):
            rec = C.read_tokens(cache, c, b, h, 5, 70)
            assert np.array_equal(rec["i_xi"], enc["i_xi"][b, h])
            assert np.array_equal(rec["i_eta"], enc["i_eta"][b, h])
            assert np.array_equal(rec["i_rho"], enc["i_rho"][b, h])
            assert np.array_equal(rec["gamma"], enc["gamma_f32"][b, h].astype(float))
            if qjl:
                assert np.array_equal(rec["sigma_neg"], enc["sigma_neg"][b, h])
    assert np.all(cache["gamma"][:, :, :5] == 0) and np.all(cache["gamma"][:, :, 75:] == 0)
