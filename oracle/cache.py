"""Encode into, and decode out of, the packed cache layout (oracle side).

A cache for one tensor (K or V) of shape [B, H, capacity, d] is a dict of
flat host arrays in the layout documented in oracle.pack:
  "idx"    uint32, B*H*capacity*W_idx words (tile-64): the index stream
  "gamma"  float32, [B, H, capacity]
  "qjl"    uint32, B*H*capacity*W_sig words (tile-64)   (only with QJL)
  "gamma_r" uint16, [B, H, capacity] fp16 bit patterns  (only with QJL)

The codec is described by a plain dict:
  d, b_dir, b_nrm, seed, qjl (bool), c_xi, c_rho (float32 arrays), rounding;
or, for the group-wise value codec of oracle.group, kind="group", d, bits,
group, seed.  A group cache has only the "idx" stream (codes, scales and
zero-points in one record) and no "gamma".
"""
import numpy as np

from . import group as grp
from . import pack
from .encode import encode, n_triplets
from .octahedral import oct_decode


def is_group(codec):
    return codec.get("kind") == "group"


def stream_sizes(codec):
    if is_group(codec):
        return {"idx": grp.record_words(codec["d"], codec["bits"], codec["group"]), "qjl": 0}
    nt = n_triplets(codec["d"])
    return {
        "idx": pack.stream_words(nt, 2 * codec["b_dir"] + codec["b_nrm"]),
        "qjl": pack.stream_words(codec["d"], 1) if codec.get("qjl") else 0,
    }


def empty_cache(codec, B, H, capacity):
    if capacity % 64:
        raise ValueError("capacity must be a multiple of 64")
    w = stream_sizes(codec)
    c = {
        "idx": np.zeros(B * H * capacity * w["idx"], dtype=np.uint32),
        "B": B, "H": H, "capacity": capacity,
    }
    if not is_group(codec):
        c["gamma"] = np.zeros((B, H, capacity), dtype=np.float32)
    if codec.get("qjl"):
        c["qjl"] = np.zeros(B * H * capacity * w["qjl"], dtype=np.uint32)
        c["gamma_r"] = np.zeros((B, H, capacity), dtype=np.uint16)
    return c


def encode_into(cache, codec, x, token_offset=0):
    """Encode x[B, H, T, d] into tokens [token_offset, token_offset+T).

    Returns the per-vector encoder outputs (indices, margins, ...) reshaped to
    [B, H, T, ...] so that tests can compare decisions and margins."""
    B, H, T, d = x.shape
    flat = np.asarray(x, dtype=np.float64).reshape(B * H * T, d)
    if is_group(codec):
        enc = grp.encode(flat, codec["bits"], codec["group"], codec["seed"])
        words = grp.pack_record(enc["codes"], enc["scale8"], enc["zero16"], codec["bits"])
        for b in range(B):
            for h in range(H):
                sl = slice((b * H + h) * T, (b * H + h + 1) * T)
                pack.scatter_tokens(cache["idx"], words[sl], b, h, token_offset, H, cache["capacity"])
        return {k: v.reshape((B, H, T) + v.shape[1:]) for k, v in enc.items()}
    enc = encode(flat, codec["c_xi"], codec["c_rho"], codec["seed"],
                 rounding=codec.get("rounding", "local3x3"), qjl=codec.get("qjl", False))
    w = stream_sizes(codec)
    cap = cache["capacity"]
    idxw = pack.pack_fields(pack.triplet_fields(enc["i_xi"], enc["i_eta"], enc["i_rho"], codec["b_dir"]),
                            2 * codec["b_dir"] + codec["b_nrm"])
    if codec.get("qjl"):
        sigw = pack.pack_fields(enc["sigma_neg"].astype(np.int64), 1)
    for b in range(B):
        for h in range(H):
            sl = slice((b * H + h) * T, (b * H + h + 1) * T)
            pack.scatter_tokens(cache["idx"], idxw[sl].reshape(T, w["idx"]), b, h, token_offset, H, cap)
            cache["gamma"][b, h, token_offset:token_offset + T] = enc["gamma_f32"][sl]
            if codec.get("qjl"):
                pack.scatter_tokens(cache["qjl"], sigw[sl], b, h, token_offset, H, cap)
                cache["gamma_r"][b, h, token_offset:token_offset + T] = enc["gamma_r_f16"][sl].view(np.uint16)
    return {k: (v.reshape((B, H, T) + v.shape[1:]) if isinstance(v, np.ndarray) else v)
            for k, v in enc.items()}


def encode_at(cache, codec, x, b, h, token_offset):
    """Encode x[T, d] into tokens [token_offset, token_offset+T) of plane (b, h)
    alone (the other planes are untouched).  Returns the encoder outputs."""
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    if is_group(codec):
        enc = grp.encode(x, codec["bits"], codec["group"], codec["seed"])
        words = grp.pack_record(enc["codes"], enc["scale8"], enc["zero16"], codec["bits"])
        pack.scatter_tokens(cache["idx"], words, b, h, token_offset, cache["H"], cache["capacity"])
        return enc
    enc = encode(x, codec["c_xi"], codec["c_rho"], codec["seed"],
                 rounding=codec.get("rounding", "local3x3"), qjl=codec.get("qjl", False))
    w = stream_sizes(codec)
    H, cap = cache["H"], cache["capacity"]
    idxw = pack.pack_fields(pack.triplet_fields(enc["i_xi"], enc["i_eta"], enc["i_rho"], codec["b_dir"]),
                            2 * codec["b_dir"] + codec["b_nrm"])
    pack.scatter_tokens(cache["idx"], idxw.reshape(T, w["idx"]), b, h, token_offset, H, cap)
    cache["gamma"][b, h, token_offset:token_offset + T] = enc["gamma_f32"]
    if codec.get("qjl"):
        sigw = pack.pack_fields(enc["sigma_neg"].astype(np.int64), 1)
        pack.scatter_tokens(cache["qjl"], sigw, b, h, token_offset, H, cap)
        cache["gamma_r"][b, h, token_offset:token_offset + T] = enc["gamma_r_f16"].view(np.uint16)
    return enc


def read_tokens(cache, codec, b, h, t0, T):
    """Indices and side data of tokens [t0, t0+T) of plane (b, h)."""
    w = stream_sizes(codec)
    H, cap = cache["H"], cache["capacity"]
    idxw = pack.gather_tokens(cache["idx"], b, h, t0, T, H, cap, w["idx"])
    if is_group(codec):
        codes, s8, z16 = grp.unpack_record(idxw, codec["d"], codec["bits"], codec["group"])
        return {"codes": codes, "scale8": s8, "zero16": z16, "idx_words": idxw}
    nt = n_triplets(codec["d"])
    f = pack.unpack_fields(idxw, nt, 2 * codec["b_dir"] + codec["b_nrm"])
    i_xi, i_eta, i_rho = pack.split_triplet_fields(f, codec["b_dir"], codec["b_nrm"])
    out = {
        "i_xi": i_xi, "i_eta": i_eta, "i_rho": i_rho,
        "gamma": cache["gamma"][b, h, t0:t0 + T].astype(np.float64),
        "idx_words": idxw,
    }
    if codec.get("qjl"):
        sigw = pack.gather_tokens(cache["qjl"], b, h, t0, T, H, cap, w["qjl"])
        out["sigma_neg"] = pack.unpack_fields(sigw, codec["d"], 1).astype(bool)
        out["gamma_r"] = cache["gamma_r"][b, h, t0:t0 + T].view(np.float16).astype(np.float64)
    return out


def u_hat_from_indices(codec, i_xi, i_eta, i_rho):
    """Rotated-frame reconstruction u^ = rho^ n^(xi^, eta^) per triplet."""
    c_xi = np.asarray(codec["c_xi"], dtype=np.float64)
    c_rho = np.asarray(codec["c_rho"], dtype=np.float64)
    n_hat = oct_decode(c_xi[i_xi], c_xi[i_eta])
    u_hat = c_rho[i_rho][..., None] * n_hat
    return u_hat.reshape(u_hat.shape[:-2] + (-1,))
