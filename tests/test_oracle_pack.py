"""Pins for oracle.pack and oracle.cache (CPU).

  * pack/unpack are inverse for every field width used (1..6 bits);
  * explicit bit positions of hand-made fields (LSB-first, little-endian);
  * padding bits are zero; words per token match the record-size table
    (43 triplet fields of 2 b_dir + b_nrm bits, QJL 128 one-bit fields at
    d = 128); a triplet field splits back into (xi, eta, rho) and holds the
    same bits as the I_dir pair followed by the I_nrm entry;
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
    # words per token: ceil(43 * (2 b_dir + b_nrm) / 32) for the splits 4 -> (5,3), 3 -> (4,2), 2 -> (3,1)
    table = {4: 18, 3: 14, 2: 10}
    for b, w in table.items():
        assert C.stream_sizes(codec(b))["idx"] == w
        bd, bn = codec(b)["b_dir"], codec(b)["b_nrm"]
        assert w == -(-43 * (2 * bd + bn) // 32)
    assert C.stream_sizes(codec(2, qjl=True))["qjl"] == 4
    # bytes per token: K and V records incl. fp32 gamma
    assert 4 * (18 + 1) == 76 and 4 * (14 + 1) == 60 and 4 * (10 + 1) == 44


def test_triplet_fields():
    rng = np.random.default_rng(3)
    for bd, bn in [(5, 3), (4, 2), (3, 1), (4, 4), (2, 2), (6, 0)]:
        xi = rng.integers(0, 2 ** bd, size=(5, 43))
        eta = rng.integers(0, 2 ** bd, size=(5, 43))
        rho = rng.integers(0, 2 ** bn, size=(5, 43)) if bn else np.zeros((5, 43), dtype=np.int64)
        f = P.triplet_fields(xi, eta, rho, bd)
        assert f.max() < 2 ** (2 * bd + bn)
        a, b, c = P.split_triplet_fields(f, bd, bn)
        assert np.array_equal(a, xi) and np.array_equal(b, eta) and np.array_equal(c, rho)
        # the packed field stream carries, triplet by triplet, the xi, eta (b_dir bits each)
        # and rho (b_nrm bits) fields in that order: bit p of the stream is the same bit
        # of the interleaved b_dir/b_dir/b_nrm sequence
        words = P.pack_fields(f, 2 * bd + bn)
        bits = []
        for i in range(43):
            for v, w in ((xi[0, i], bd), (eta[0, i], bd), (rho[0, i], bn)):
                bits += [(int(v) >> k) & 1 for k in range(w)]
        stream = [(int(words[0, p // 32]) >> (p % 32)) & 1 for p in range(len(bits))]
        assert stream == bits
    # explicit: xi = 1, eta = 2, rho = 3 at (b_dir, b_nrm) = (3, 2) -> 1 | 2 << 3 | 3 << 6
    assert int(P.triplet_fields([[1]], [[2]], [[3]], 3)[0, 0]) == 1 | (2 << 3) | (3 << 6)


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
