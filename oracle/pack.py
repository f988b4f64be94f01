"""Bit packing of the compressed state and the cache layout.

The OCTOPUS paper (Sec. 3) stores S(k) = (gamma, I_dir, I_nrm): the norm, a
packed stream of octahedral-coordinate indices and a packed stream of
triplet-norm indices; with QJL also sigma in {+-1}^d and gamma_r in fp16
(Sec. 3.6).  The paper fixes no bit layout.  The layout below is this
project's own and is written here independently of the HIP code from its
description:

  * A stream is a little-endian, LSB-first bit string: field j of width w
    occupies bits [j*w, (j+1)*w), bit p is bit (p % 8) of byte p // 8.
  * The index stream I holds one field per triplet, n_tri fields of
    B_tri = 2 b_dir + b_nrm bits (the per-triplet budget of Sec. 3.3): field i
    is xi_i | eta_i << b_dir | rho_i << 2 b_dir, i.e. the triplet's I_dir
    pair followed by its I_nrm entry.  (I_dir and I_nrm are the same bits,
    interleaved per triplet rather than kept as two streams.)
    The sigma stream holds d one-bit fields, 1 where sigma_j = -1.
  * Every stream is zero-padded to whole 32-bit words; W = words per token.
  * gamma is fp32 and gamma_r the fp16 bit pattern, each one value per token
    in a plain [B, H, capacity] array.
  * Cache layout ("tile-64"): for each (batch b, kv head h) a plane of
    `capacity` tokens (a multiple of 64); word w of token t of a stream with W
    words lives at word index
        ((b * H + h) * capacity / 64 + t // 64) * W * 64 + w * 64 + t % 64.
    So one 64-token tile stores its W words as W rows of 64 consecutive words.

Parity: pinned by pack/unpack round trips, explicit bit positions for
hand-made fields, zero padding and the record sizes per (b_dir, b_nrm, QJL)
(tests/test_oracle_pack.py).
"""
import numpy as np


def stream_words(n_fields, width):
    return -(-(n_fields * width) // 32)


def pack_fields(fields, width):
    """fields[N, F] (ints < 2^width) -> uint32 words [N, W] (LSB-first)."""
    fields = np.asarray(fields, dtype=np.uint64)
    n, f = fields.shape
    w = stream_words(f, width)
    if w == 0:
        return np.zeros((n, 0), dtype=np.uint32)
    bits = np.zeros((n, w * 32), dtype=np.uint8)
    for b in range(width):
        bits[:, b: f * width: width] = ((fields >> np.uint64(b)) & np.uint64(1)).astype(np.uint8)
    by = np.packbits(bits, axis=1, bitorder="little")
    return by.view("<u4").reshape(n, w)


def unpack_fields(words, n_fields, width):
    """uint32 words [N, W] -> fields [N, F] (int64)."""
    words = np.ascontiguousarray(np.asarray(words, dtype="<u4"))
    n = words.shape[0]
    if width == 0:
        return np.zeros((n, n_fields), dtype=np.int64)
    bits = np.unpackbits(words.view(np.uint8).reshape(n, -1), axis=1, bitorder="little")
    out = np.zeros((n, n_fields), dtype=np.int64)
    for b in range(width):
        out |= bits[:, b: n_fields * width: width].astype(np.int64) << b
    return out


def triplet_fields(i_xi, i_eta, i_rho, b_dir):
    """One B_tri-bit field per triplet: xi | eta << b_dir | rho << 2 b_dir."""
    i_xi, i_eta, i_rho = (np.asarray(a, dtype=np.int64) for a in (i_xi, i_eta, i_rho))
    return i_xi | (i_eta << b_dir) | (i_rho << (2 * b_dir))


def split_triplet_fields(f, b_dir, b_nrm):
    """Inverse of triplet_fields: (i_xi, i_eta, i_rho)."""
    f = np.asarray(f, dtype=np.int64)
    m = (1 << b_dir) - 1
    return f & m, (f >> b_dir) & m, (f >> (2 * b_dir)) & ((1 << b_nrm) - 1)


def tile_index(b, h, t, w, H, capacity, W):
    """Word index of word w of token t in the (b, h) plane (tile-64 layout)."""
    tiles = capacity // 64
    return ((b * H + h) * tiles + t // 64) * W * 64 + w * 64 + t % 64


def scatter_tokens(buf, words, b, h, t0, H, capacity):
    """Write words[T, W] of tokens t0..t0+T-1 into the flat uint32 buffer."""
    T, W = words.shape
    t = t0 + np.arange(T)
    for w in range(W):
        buf[tile_index(b, h, t, w, H, capacity, W)] = words[:, w]


def gather_tokens(buf, b, h, t0, T, H, capacity, W):
    """Read words[T, W] of tokens t0..t0+T-1 from the flat uint32 buffer."""
    t = t0 + np.arange(T)
    out = np.zeros((T, W), dtype=np.uint32)
    for w in range(W):
        out[:, w] = buf[tile_index(b, h, t, w, H, capacity, W)]
    return out
