"""Attention over the packed cache, as the plain definition, in float64.

Decode attention (one query per sequence, grouped-query heads):
  for query head h on KV head g = h // (H_q / H_kv) and cached tokens j < len_b
    k^_j = gamma_j R^T u^_j[:d]                      (OCTOPUS paper, Sec. 3.6,
    v^_j = gamma_v,j R^T u^_v,j[:d]                   Eq. 13 / App. C.14)
    score_j = q_h . k^_j  (+ gamma_j * sqrt(pi/(2d)) * gamma_r,j * (R' q_rot)^T sigma_j
                           with OCTOPUS-QJL, Sec. 3.6)
    o_h = sum_j softmax(scale * score)_j v^_j
The keys and values are reconstructed explicitly here; the HIP path never does
that (Sec. 3: the decoder never materializes K^).  V uses the same OCTOPUS
codec as K without QJL (reading; the paper's value-side group codec is never
defined).  An empty context (len_b = 0) gives an all-zero output (reading).

Chunk attention (the cached / current decomposition of the second page,
"Quantized Keys Steal Attention", Sec. 3 "Token Structure and Attention
Decomposition"): every query of the current chunk attends, in one softmax and
without a mask, to all cached (packed) tokens and to all current-chunk tokens,
the latter at full precision.  An empty window (no cached and no current
tokens) gives zero output rows, as an empty decode context does (reading).

Parity: pinned by the score factorization of Eq. 13 against the explicit
reconstruction, by torch's scaled_dot_product_attention on the explicit K^, V^,
and by exact attention as the bit width grows (tests/test_oracle_attention.py).
"""
import numpy as np

from . import group as grp
from .cache import is_group, read_tokens, u_hat_from_indices
from .rotation import qjl_rotation_matrix, rotation_matrix


def reconstruct(cache, codec, b, h, t0, T):
    """Explicit float64 vectors gamma R^T u^[:d] (OCTOPUS) or R^T u^ (group
    codec) for tokens [t0, t0+T)."""
    d = codec["d"]
    rec = read_tokens(cache, codec, b, h, t0, T)
    if is_group(codec):
        return grp.reconstruct(rec["codes"], rec["scale8"], rec["zero16"], codec["group"], codec["seed"]), rec
    u_hat = u_hat_from_indices(codec, rec["i_xi"], rec["i_eta"], rec["i_rho"])
    x_hat = rec["gamma"][:, None] * (u_hat[:, :d] @ rotation_matrix(d, codec["seed"]))
    return x_hat, rec


def qjl_correction(q, rec, codec):
    """gamma * sqrt(pi/(2d)) * gamma_r * (R' q_rot)^T sigma for q[G, d]."""
    d = codec["d"]
    q_rot = q @ rotation_matrix(d, codec["seed"]).T
    q_prime = q_rot @ qjl_rotation_matrix(d, codec["seed"]).T      # [G, d]
    sigma = np.where(rec["sigma_neg"], -1.0, 1.0)                   # [T, d]
    est = np.sqrt(np.pi / (2 * d)) * rec["gamma_r"][None, :] * (q_prime @ sigma.T)
    return rec["gamma"][None, :] * est                              # [G, T]


def softmax_rows(s):
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def decode_attention(q, k_cache, v_cache, k_codec, v_codec, seq_lens, scale=None):
    """q[B, H_q, d] -> out[B, H_q, d] (float64)."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = k_cache["H"]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None or scale <= 0 else scale
    out = np.zeros((B, Hq, d))
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        for g in range(Hkv):
            qg = q[b, g * G:(g + 1) * G]
            k_hat, krec = reconstruct(k_cache, k_codec, b, g, 0, L)
            v_hat, _ = reconstruct(v_cache, v_codec, b, g, 0, L)
            score = qg @ k_hat.T
            if k_codec.get("qjl"):
                score = score + qjl_correction(qg, krec, k_codec)
            out[b, g * G:(g + 1) * G] = softmax_rows(scale * score) @ v_hat
    return out


def chunk_attention(q, k_cache, v_cache, k_codec, v_codec, cached_tokens,
                    k_cur, v_cur, scale=None, q_rows=None, correction=False):
    """q[B, H_q, Tq, d], k_cur/v_cur[B, H_kv, Tc, d] -> out[B, H_q, Tq, d].

    q_rows: optional index array of query rows to evaluate (others are left 0),
    so that large chunks can be checked on a sample.
    correction: subtract the Jensen bias of oracle.group.jensen_bias (the
    Taylor form of "Quantized Keys Steal Attention", Eq. 15) from the logits
    of the cached tokens; the keys must use the group-wise codec, whose
    round-to-nearest noise the correction models."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, Tq, d = q.shape
    Hkv = k_cache["H"]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None or scale <= 0 else scale
    rows = np.arange(Tq) if q_rows is None else np.asarray(q_rows)
    out = np.zeros((B, Hq, Tq, d))
    for b in range(B):
        for g in range(Hkv):
            if cached_tokens:
                k_hat, krec = reconstruct(k_cache, k_codec, b, g, 0, cached_tokens)
                v_hat, _ = reconstruct(v_cache, v_codec, b, g, 0, cached_tokens)
            else:
                k_hat = v_hat = np.zeros((0, d))
            kc = np.asarray(k_cur[b, g], dtype=np.float64).reshape(-1, d)
            vc = np.asarray(v_cur[b, g], dtype=np.float64).reshape(-1, d)
            keys = np.concatenate([k_hat, kc], axis=0)
            vals = np.concatenate([v_hat, vc], axis=0)
            if keys.shape[0] == 0:
                continue            # nothing to attend to: zero rows (reading)
            for hh in range(G):
                h = g * G + hh
                qh = q[b, h][rows]
                score = qh @ keys.T
                if k_codec.get("qjl") and cached_tokens:
                    score[:, :cached_tokens] += qjl_correction(qh, krec, k_codec)
                logit = scale * score
                if correction and cached_tokens:
                    if not is_group(k_codec):
                        raise ValueError("the correction models round-to-nearest keys (group codec)")
                    q_rot = qh @ rotation_matrix(d, k_codec["seed"]).T
                    logit[:, :cached_tokens] -= grp.jensen_bias(q_rot, krec["scale8"],
                                                                k_codec["group"], scale)
                out[b, h][rows] = softmax_rows(logit) @ vals
    return out
