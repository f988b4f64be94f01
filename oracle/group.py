"""Group-wise asymmetric integer codec for the values (test infrastructure).

Only tests/, the smoke check and the CPU baseline of the benchmark use this
module; the product path never does.

What the pages say.
  * OCTOPUS ("OCTOPUS: Optimized KV Cache for Transformers via Octahedral
    Parametrization ...", Sec. 4, default recipe; Sec. 4.2): every compared
    K codec shares one value codec with a value-side group size g in
    {16, 32} (32 for the language-model and video rows, 16 for audio).  The
    page does not define that codec.
  * "Quantized Keys Steal Attention" (Sec. 3, "Quantization granularity"):
    group-wise per-token quantization splits each token's d channels into
    groups of g, each with its own step size Delta and zero-point z.
    Sec. 3, "Hadamard rotation": a randomized orthogonal Hadamard rotation is
    applied before quantizing (QuaRot).  Sec. 4.3: B_eff = B + 24/g, the
    scale stored as FP8 E4M3 and the zero-point as BF16.  Sec. 5,
    "Quantization configuration": group-wise per-token asymmetric INT-B,
    round-to-nearest.

Reading (the "Integer quantization" paragraph of that Sec. 3 is lost in the
text; this is the plainest asymmetric round-to-nearest quantizer consistent
with the rest):
    u        = R v with the keys' rotation R = H diag(s) (same seed rule)
    per group j of g consecutive coordinates of u:
      Delta  = (max_j - min_j) / (2^b - 1)                     (fp32)
      Delta^ = E4M3(Delta), round to nearest even, saturating at 448
      z^     = BF16(min_j), round to nearest even (a zero minimum as +0)
      q_c    = clamp(rint((u_c - z^) / Delta^), 0, 2^b - 1)    (fp32), 0 if Delta^ = 0
      u^_c   = Delta^ q_c + z^
    v^ = R^T u^.
Every decision (E4M3, BF16, rint) is taken on fp32 values in fp32 arithmetic,
the precision of the kernels (the pages give none).

Record layout (this project's; the pages fix none): one LSB-first stream of
d fields of b bits (code of coordinate c at bits [c b, (c+1) b)), then G = d/g
fields of 8 bits (the E4M3 scale codes), then G fields of 16 bits (the BF16
zero-points), in 32-bit words: W = (b d + 24 G) / 32 words per token, which
is exactly B_eff = b + 24/g bits per coordinate.

Jensen-bias correction ("Quantized Keys Steal Attention", Sec. 4.1-4.2 and
the appendix "Taylor approximation"): round-to-nearest noise on a cached key,
uniform on [-Delta/2, Delta/2] per coordinate, raises the expected
exponentiated score by the factor prod_c sinh(a_c)/a_c, a_c = tau q_c Delta_c
/ 2 (tau the softmax scale, 1/sqrt(d) on the page), so log(sinh(a)/a) summed
over the coordinates is subtracted from the cached token's logit; its Taylor
form a^2/6 gives Eq. 15, b_i = tau^2/24 sum_j Delta_ij^2 ||q_j||^2 over the
groups j.  Under the rotation (that appendix, "Taylor approximation under
rotation") the noise lives in the rotated frame, so q_j are the groups of
R q.  jensen_bias is that Taylor form, jensen_bias_exact the log-sinh one.

Parity: pinned in tests/test_oracle_group.py by the E4M3 format table, torch's
float8_e4m3fn and bfloat16 conversions (library routines), brute-force
nearest-grid-point search in exact rational arithmetic, the half-step error
bound and the norm bound it implies through the orthogonal rotation, the
record size against B_eff and the claim that smaller groups give smaller
error.
"""
import numpy as np

from . import pack
from .rotation import rotation_matrix

E4M3_MAX_CODE = 0x7E        # 448; 0x7F is NaN in E4M3 (no infinities)


def e4m3_values():
    """Value of every non-negative finite E4M3 code 0..0x7E (float64).

    Format: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
    subnormal (m/8 * 2^-6), exponent 15 with mantissa 7 is NaN."""
    v = np.zeros(E4M3_MAX_CODE + 1)
    for c in range(E4M3_MAX_CODE + 1):
        e, m = c >> 3, c & 7
        v[c] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return v


_E4M3 = e4m3_values()


def to_e4m3(x):
    """Non-negative fp32 values -> E4M3 codes (uint8): nearest value, ties to
    the even code, values beyond the largest finite value saturate to 448.
    Also returns the decision margin: the distance of x to the nearer edge of
    the chosen code's rounding cell (the midpoints with the adjacent codes;
    the cell of 448 has no upper edge)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    if np.any(x < 0) or np.any(~np.isfinite(x)):
        raise ValueError("scales are finite and non-negative")
    hi = np.clip(np.searchsorted(_E4M3, x), 1, E4M3_MAX_CODE)     # _E4M3[hi-1] <= x <= _E4M3[hi]
    lo = hi - 1
    dl, dh = x - _E4M3[lo], _E4M3[hi] - x
    code = np.where((dh < dl) | ((dh == dl) & (hi % 2 == 0)), hi, lo)
    code = np.where(x >= _E4M3[-1], E4M3_MAX_CODE, code)
    below = np.where(code > 0, 0.5 * (_E4M3[np.maximum(code - 1, 0)] + _E4M3[code]), -np.inf)
    above = np.where(code < E4M3_MAX_CODE,
                     0.5 * (_E4M3[code] + _E4M3[np.minimum(code + 1, E4M3_MAX_CODE)]), np.inf)
    margin = np.minimum(x - below, above - x)
    return code.astype(np.uint8), margin


def from_e4m3(code):
    return _E4M3[np.asarray(code, dtype=np.int64)]


def to_bf16(x):
    """fp32 values -> BF16 bit patterns (uint16), round to nearest even.
    Also returns the decision margin: the distance of x to the nearer edge of
    the chosen value's rounding cell (the midpoints with the adjacent BF16
    values of the same sign; a zero's cell reaches down to zero)."""
    x32 = np.asarray(x, dtype=np.float32)
    bits = x32.view(np.uint32).astype(np.int64)
    low = bits & ~0xFFFF                       # truncation toward zero
    high = low + 0x10000                       # next value away from zero
    xv = x32.astype(np.float64)
    vlow = (low.astype(np.uint32)).view(np.float32).astype(np.float64)
    vhigh = (high.astype(np.uint32)).view(np.float32).astype(np.float64)
    dl, dh = np.abs(xv - vlow), np.abs(vhigh - xv)
    pick_high = (dh < dl) | ((dh == dl) & (((low >> 16) & 1) == 1))
    out = np.where(pick_high, high, low) >> 16
    # magnitudes of the chosen value and of its neighbours toward and away
    # from zero
    mag = out & 0x7FFF
    val = lambda m: np.abs(((m << 16).astype(np.uint32)).view(np.float32).astype(np.float64))  # noqa: E731
    v = val(mag)
    toward = np.where(mag > 0, 0.5 * (v + val(np.maximum(mag - 1, 0))), 0.0)
    away = 0.5 * (v + val(mag + 1))
    ax = np.abs(xv)
    margin = np.minimum(ax - toward, away - ax)
    return out.astype(np.uint16), margin


def from_bf16(h):
    return (np.asarray(h, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def n_groups(d, g):
    if g not in (16, 32) or d % g:
        raise ValueError("group size 16 or 32 dividing d")
    return d // g


def record_words(d, bits, g):
    return (bits * d + 24 * n_groups(d, g)) // 32


def quantize_rotated(u32, bits, g):
    """Quantize rotated fp32 vectors u32[N, d] group by group.

    Returns codes [N, d], scale codes [N, G] (E4M3), zero codes [N, G] (BF16)
    and the decision margins (u units) of each scale, zero-point and code."""
    u32 = np.asarray(u32, dtype=np.float32)
    N, d = u32.shape
    G = n_groups(d, g)
    levels = (1 << bits) - 1
    ug = u32.reshape(N, G, g)
    mn = ug.min(axis=-1) + np.float32(0.0)                # a zero minimum is +0 (reading)
    mx = ug.max(axis=-1)
    delta = (mx - mn) / np.float32(levels)                # fp32 subtract, fp32 divide
    s8, s_margin = to_e4m3(delta)
    z16, z_margin = to_bf16(mn)
    dh = from_e4m3(s8).astype(np.float32)[..., None]
    zh = from_bf16(z16).astype(np.float32)[..., None]
    q, q_margin = group_codes(ug, dh, zh, bits)
    return {
        "codes": q.reshape(N, d), "scale8": s8, "zero16": z16,
        "scale_margin": s_margin, "zero_margin": z_margin, "code_margin": q_margin.reshape(N, d),
        "u32": u32,
    }


def group_codes(u32, dh, zh, bits, nudge=None):
    """Codes q = clamp(rint((u - z^) / Delta^), 0, 2^b - 1) in fp32 (0 where
    Delta^ = 0) of fp32 coordinates u32 against fp32 steps dh and zero-points
    zh (broadcast), and their margins in u units: the distance of u to the
    nearer edge of its code's cell (the code changes where (u - z^) / Delta^
    crosses k + 1/2).  nudge: an additive perturbation of u (float64, taken
    to fp32 with u)."""
    levels = (1 << bits) - 1
    u32 = np.asarray(u32, dtype=np.float32)
    if nudge is not None:
        u32 = (u32.astype(np.float64) + nudge).astype(np.float32)
    dh = np.asarray(dh, dtype=np.float32)
    zh = np.asarray(zh, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = (u32 - zh) / dh                              # fp32
    qf = np.where(dh > 0, qf, np.float32(0))
    q = np.clip(np.rint(qf), 0, levels).astype(np.int64)
    q = np.where(dh > 0, q, 0)
    # code decisions turn at k + 1/2, k = 0 .. levels - 1
    bnd = np.arange(levels, dtype=np.float64) + 0.5
    dist = np.abs(qf.astype(np.float64)[..., None] - bnd).min(axis=-1) * dh.astype(np.float64)
    return q, np.where(dh > 0, dist, np.inf)


def dequantize_rotated(codes, scale8, zero16, g):
    """u^ = Delta^ q + z^ per coordinate (float64, rotated frame)."""
    codes = np.asarray(codes, dtype=np.float64)
    N, d = codes.shape
    G = n_groups(d, g)
    dh = from_e4m3(scale8).reshape(N, G, 1)
    zh = from_bf16(zero16).reshape(N, G, 1)
    return (dh * codes.reshape(N, G, g) + zh).reshape(N, d)


def encode(x, bits, g, seed):
    """x[N, d] -> the quantizer outputs for u = R x, u rounded to fp32."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    u = x @ rotation_matrix(d, seed).T
    out = quantize_rotated(u.astype(np.float32), bits, g)
    out["u"] = u
    return out


def reconstruct(codes, scale8, zero16, g, seed):
    """v^ = R^T u^ (float64)."""
    u_hat = dequantize_rotated(codes, scale8, zero16, g)
    return u_hat @ rotation_matrix(u_hat.shape[-1], seed)


def pack_record(codes, scale8, zero16, bits):
    """Token records as uint32 words [N, W] (layout in the module header)."""
    codes = np.asarray(codes, dtype=np.int64)
    parts = [pack.pack_fields(codes, bits),
             pack.pack_fields(np.asarray(scale8, dtype=np.int64), 8),
             pack.pack_fields(np.asarray(zero16, dtype=np.int64), 16)]
    return np.concatenate(parts, axis=1)


def unpack_record(words, d, bits, g):
    words = np.asarray(words, dtype=np.uint32)
    G = n_groups(d, g)
    wc, ws = bits * d // 32, G // 4
    codes = pack.unpack_fields(words[:, :wc], d, bits)
    s8 = pack.unpack_fields(words[:, wc:wc + ws], G, 8).astype(np.uint8)
    z16 = pack.unpack_fields(words[:, wc + ws:], G, 16).astype(np.uint16)
    return codes, s8, z16


def jensen_bias(q_rot, scale8, g, tau):
    """Eq. 15 of the QKSA page, generalized to softmax scale tau:
    b[q, i] = tau^2 / 24 * sum_j Delta^_ij^2 ||q_rot_j||^2 for query rows
    q_rot[Q, d] (rotated) and tokens' E4M3 scale codes scale8[T, G]."""
    q_rot = np.asarray(q_rot, dtype=np.float64)
    Q, d = q_rot.shape
    G = n_groups(d, g)
    qn2 = (q_rot.reshape(Q, G, g) ** 2).sum(axis=-1)                  # [Q, G]
    d2 = from_e4m3(scale8).reshape(-1, G) ** 2                        # [T, G]
    return tau * tau / 24.0 * (qn2 @ d2.T)


def jensen_bias_exact(q_rot, scale8, g, tau):
    """sum_c log(sinh(a_c) / a_c), a_c = tau q_c Delta^_ic / 2 (the exact
    log of the expected noise factor under uniform noise)."""
    q_rot = np.asarray(q_rot, dtype=np.float64)
    Q, d = q_rot.shape
    G = n_groups(d, g)
    dh = np.repeat(from_e4m3(scale8).reshape(-1, G), g, axis=1)       # [T, d]
    a = np.abs(tau * q_rot[:, None, :] * dh[None, :, :] / 2.0)       # [Q, T, d]
    small = a < 1e-4
    with np.errstate(divide="ignore", invalid="ignore"):
        f = np.where(small, a * a / 6.0, np.log(np.sinh(np.where(small, 1.0, a)) / np.where(small, 1.0, a)))
    return f.sum(axis=-1)
