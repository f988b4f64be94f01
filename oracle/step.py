"""One decode step with a native-precision residual window, in float64.

Test infrastructure only: nothing outside tests/, the smoke check and the
CPU baseline of the benchmark may import this module.

The OCTOPUS paper's experiments keep a short window of the most recent tokens
at native precision beside the compressed cache (Sec. 4, "default recipe";
Sec. 4.2 uses a window of 32 tokens).  The paper gives no mechanism; this is
the reading implemented here and in the HIP path:

  State of a sequence: a packed cache holding tokens [0, P) and a ring of W
  native K/V rows holding tokens [P, P + n), n < W, token j in slot j mod W.

  A step with query q and the new token's k, v:
    1. the new token t = P + n is written to ring slot t mod W;
    2. attention: one softmax over the packed tokens [0, P) (decoded, with
       the QJL term when the key codec has it) and the native tokens
       [P, t] (n + 1 rows);
    3. if n + 1 == W, token P is encoded into packed slot P and leaves the
       window (P += 1, n stays W - 1); otherwise n += 1.

  So at every step the attention sees exactly the last min(W, t + 1) tokens
  at native precision, and a token is compressed when it leaves the window.
"""
import numpy as np

from .attention import qjl_correction, reconstruct, softmax_rows
from .cache import empty_cache, encode_at


def new_state(k_codec, v_codec, B, Hkv, capacity, W, d=128):
    """An empty state: no packed token, an empty ring of W rows."""
    return {
        "k": empty_cache(k_codec, B, Hkv, capacity),
        "v": empty_cache(v_codec, B, Hkv, capacity),
        "k_ring": np.zeros((B, Hkv, W, d)),
        "v_ring": np.zeros((B, Hkv, W, d)),
        "P": np.zeros(B, dtype=np.int64),
        "n": np.zeros(B, dtype=np.int64),
        "W": W,
    }


def decode_step(state, q, k_new, v_new, k_codec, v_codec, scale=None):
    """q[B, H_q, d], k_new/v_new[B, H_kv, d] -> out[B, H_q, d] (float64).

    Updates `state` in place (ring, packed caches, P and n)."""
    q = np.asarray(q, dtype=np.float64)
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = k_new.shape[1]
    G = Hq // Hkv
    W = state["W"]
    scale = 1.0 / np.sqrt(d) if scale is None or scale <= 0 else scale
    out = np.zeros((B, Hq, d))
    for b in range(B):
        P, n = int(state["P"][b]), int(state["n"][b])
        t = P + n
        state["k_ring"][b, :, t % W] = k_new[b]
        state["v_ring"][b, :, t % W] = v_new[b]
        slots = [(P + j) % W for j in range(n + 1)]
        for g in range(Hkv):
            qg = q[b, g * G:(g + 1) * G]
            kw = state["k_ring"][b, g, slots]                 # [n+1, d]
            vw = state["v_ring"][b, g, slots]
            score_w = qg @ kw.T
            if P > 0:
                k_hat, krec = reconstruct(state["k"], k_codec, b, g, 0, P)
                v_hat, _ = reconstruct(state["v"], v_codec, b, g, 0, P)
                score_p = qg @ k_hat.T
                if k_codec.get("qjl"):
                    score_p = score_p + qjl_correction(qg, krec, k_codec)
                score = np.concatenate([score_p, score_w], axis=1)
                vals = np.concatenate([v_hat, vw], axis=0)
            else:
                score, vals = score_w, vw
            out[b, g * G:(g + 1) * G] = softmax_rows(scale * score) @ vals
        if n + 1 == W:
            s = P % W
            for g in range(Hkv):
                encode_at(state["k"], k_codec, state["k_ring"][b, g, s][None], b, g, P)
                encode_at(state["v"], v_codec, state["v_ring"][b, g, s][None], b, g, P)
            state["P"][b] = P + 1
        else:
            state["n"][b] = n + 1
    return out
