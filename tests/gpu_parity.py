"""Helpers of the GPU parity tests: run the HIP path through the C ABI, read
the packed cache back to the host and compare it with the oracle.

Parity rules (the oracle is float64, the kernels fp32):
  * indices (xi, eta, rho) must be bit-exact; a triplet may differ only when
    the oracle's smallest decision margin for it is below 1e-6, and such
    mismatches are counted and reported;
  * QJL sign bits likewise, with margin |(R' r)_j| < 1e-6, or on tokens that
    already carry an allowed index mismatch (their residual differs);
  * gamma within 4 fp32 ulps; gamma_r within 1 fp16 ulp;
  * attention outputs within max-abs 2e-3 of the oracle evaluated on the
    GPU-written cache;
  * group-wise value codec: E4M3 scales, BF16 zero-points and codes bit-exact;
    a field may differ only where the oracle's decision margin is below 1e-6
    of the token's largest |u| (the codes of a group whose scale or
    zero-point differs that way are then not compared).
"""
import dataclasses
import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

import quantized_decode_attention_octo_amd as octo  # noqa: E402
from oracle import attention as oatt  # noqa: E402
from oracle import cache as ocache  # noqa: E402
from oracle import encode as oenc  # noqa: E402
from oracle import group as ogroup  # noqa: E402
from oracle_codecs import codec as oracle_codec  # noqa: E402
from oracle_codecs import group_codec as oracle_group_codec  # noqa: E402
from quantized_decode_attention_octo_amd.workloads import WORKLOADS, make_inputs  # noqa: E402

MARGIN = 1e-6
ATOL = 2e-3
# Every index comparison adds its counts here (case name -> counts): the
# GPU run's record of the mismatches the near-threshold rule forgave.
COUNTS_PATH = os.environ.get("OCTO_PARITY_COUNTS",
                             os.path.join(ROOT, "gpurun_out", "parity_counts.json"))


def record_counts(what, st):
    """Adds the counts of one comparison to the run's record (best effort:
    a read-only tree skips it)."""
    import json
    try:
        os.makedirs(os.path.dirname(COUNTS_PATH), exist_ok=True)
        try:
            with open(COUNTS_PATH) as f:
                rec = json.load(f)
        except (OSError, ValueError):
            rec = {"rule": "an index may differ from the oracle only where the oracle's smallest "
                           "decision margin is below 1e-6 (forgiven); bad = other mismatches",
                   "cases": {}}
        # a case name seen again in the run (a loop over steps) adds up
        old = rec["cases"].get(what, {})
        rec["cases"][what] = {k: (max(float(v), old.get(k, 0.0)) if isinstance(v, float)
                                  else int(v) + old.get(k, 0)) for k, v in st.items()}
        with open(COUNTS_PATH, "w") as f:
            json.dump(rec, f, indent=1, sort_keys=True)
    except OSError:
        pass


def say(*a):
    print(*a, flush=True)


def ceil64(n):
    return -(-n // 64) * 64


def codecs(bits, qjl=False, seed=0, b_dir=None, b_nrm=None, rounding="local3x3"):
    """(GPU codec, oracle codec dict) built from the same codebook artifact."""
    r = octo.binding.ROUND_SCALAR if rounding == "scalar" else octo.binding.ROUND_LOCAL3X3
    g = octo.Codec(bits=bits, seed=seed, qjl=qjl, b_dir=b_dir, b_nrm=b_nrm, rounding=r)
    h = oracle_codec(bits=bits, seed=seed, qjl=qjl, b_dir=b_dir, b_nrm=b_nrm, rounding=rounding)
    return g, h


def group_codecs(bits, group, seed=0):
    """(GPU codec, oracle codec dict) of the group-wise value codec."""
    return octo.Codec(bits=bits, seed=seed, group=group), oracle_group_codec(bits, group, seed)


def plane_of(h, b, g):
    """The host cache of plane (b, g) alone (same layout with B = H = 1)."""
    n = h["B"] * h["H"]
    p = b * h["H"] + g
    out = {"B": 1, "H": 1, "capacity": h["capacity"], "idx": h["idx"].reshape(n, -1)[p]}
    if "gamma" in h:
        out["gamma"] = h["gamma"][b:b + 1, g:g + 1]
    if "qjl" in h:
        out["qjl"] = h["qjl"].reshape(n, -1)[p]
        out["gamma_r"] = h["gamma_r"][b:b + 1, g:g + 1]
    return out


def compare_group_encode(host_cache, hcodec, x, token_offset=0, planes=None, tokens=None):
    """Compares GPU-written group records with the oracle's encoding of x."""
    B, H, T, d = x.shape
    planes = planes or [(b, h) for b in range(B) for h in range(H)]
    st = dict(codes=0, mismatch=0, bad=0, groups=0, meta_mismatch=0, meta_bad=0)
    g = hcodec["group"]
    for b, h in planes:
        ts = np.arange(T) if tokens is None else np.asarray(tokens)
        e = ogroup.encode(x[b, h].double().numpy()[ts], hcodec["bits"], g, hcodec["seed"])
        rec = ocache.read_tokens(host_cache, hcodec, b, h, token_offset, T)
        codes, s8, z16 = rec["codes"][ts], rec["scale8"][ts], rec["zero16"][ts]
        tol = MARGIN * np.abs(e["u"]).max(axis=1, keepdims=True)           # per token
        sm, zm = s8 != e["scale8"], z16 != e["zero16"]
        meta_bad = (sm & (e["scale_margin"] >= tol)) | (zm & (e["zero_margin"] >= tol))
        st["groups"] += sm.size
        st["meta_mismatch"] += int((sm | zm).sum())
        st["meta_bad"] += int(meta_bad.sum())
        skip = np.repeat(sm | zm, g, axis=1)                  # codes of a moved grid
        cm = (codes != e["codes"]) & ~skip
        bad = cm & (e["code_margin"] >= tol)
        st["codes"] += cm.size
        st["mismatch"] += int(cm.sum())
        st["bad"] += int(bad.sum())
        if bad.any() or meta_bad.any():
            i = np.argwhere(bad)[0] if bad.any() else np.argwhere(meta_bad)[0]
            say("first bad mismatch", (b, h, int(ts[i[0]]), int(i[1])), "gpu codes",
                codes[i[0]].tolist()[:16], "oracle", e["codes"][i[0]].tolist()[:16],
                "scales", s8[i[0]].tolist(), e["scale8"][i[0]].tolist(),
                "zeros", z16[i[0]].tolist(), e["zero16"][i[0]].tolist())
    return st


def assert_group_encode_ok(st, what):
    st = dict(st, forgiven=st["mismatch"] - st["bad"],
              meta_forgiven=st["meta_mismatch"] - st["meta_bad"])
    say(f"[{what}] codes {st['codes']} mismatches {st['mismatch']} (bad {st['bad']}); groups"
        f" {st['groups']} scale/zero mismatches {st['meta_mismatch']} (bad {st['meta_bad']})")
    record_counts("group " + what, st)
    assert st["bad"] == 0 and st["meta_bad"] == 0


def encode_gpu(x, gcodec, capacity=None, token_offset=0, cache=None):
    B, H, T, _ = x.shape
    if cache is None:
        cache = octo.PackedCache(gcodec, B, H, capacity or ceil64(token_offset + T))
    octo.octo_encode(gcodec, x.cuda(), cache, token_offset)
    torch.cuda.synchronize()
    return cache


def compare_encode(host_cache, hcodec, x, token_offset=0, planes=None, tokens=None):
    """Compares the GPU-written tokens [token_offset, token_offset + T) of the
    given planes (default all) at the given token positions (default all)
    with the oracle's encoding of x[b, h, t]."""
    B, H, T, d = x.shape
    planes = planes or [(b, h) for b in range(B) for h in range(H)]
    st = dict(triplets=0, mismatch=0, bad=0, gamma_err=0.0, sig_mismatch=0, sig_bad=0,
              gr_bad=0)
    for b, h in planes:
        ts = np.arange(T) if tokens is None else np.asarray(tokens)
        xv = x[b, h].double().numpy()[ts]
        e = oenc.encode(xv, hcodec["c_xi"], hcodec["c_rho"], hcodec["seed"],
                        rounding=hcodec["rounding"], qjl=hcodec["qjl"])
        rec = ocache.read_tokens(host_cache, hcodec, b, h, token_offset, T)
        gx, gy, gr = rec["i_xi"][ts], rec["i_eta"][ts], rec["i_rho"][ts]
        mism = (gx != e["i_xi"]) | (gy != e["i_eta"]) | (gr != e["i_rho"])
        bad = mism & (e["margin"] >= MARGIN)
        st["triplets"] += mism.size
        st["mismatch"] += int(mism.sum())
        st["bad"] += int(bad.sum())
        g = rec["gamma"][ts]
        rel = np.abs(g - e["gamma"]) / np.maximum(e["gamma"], 1e-30)
        st["gamma_err"] = max(st["gamma_err"], float(rel.max()) if rel.size else 0.0)
        if hcodec["qjl"]:
            tok_mism = mism.any(axis=1)
            sm = rec["sigma_neg"][ts] != e["sigma_neg"]
            sbad = sm & (e["sigma_margin"] >= MARGIN) & ~tok_mism[:, None]
            st["sig_mismatch"] += int(sm.sum())
            st["sig_bad"] += int(sbad.sum())
            gr16 = rec["gamma_r"][ts]
            ref16 = e["gamma_r_f16"].astype(np.float64)
            ulp = np.spacing(np.abs(ref16).astype(np.float16)).astype(np.float64)
            st["gr_bad"] += int(((np.abs(gr16 - ref16) > ulp * 1.01) & ~tok_mism).sum())
        if bad.any():
            i = np.argwhere(bad)[0]
            say("first bad mismatch", (b, h, int(ts[i[0]]), int(i[1])),
                "gpu", (gx[tuple(i)], gy[tuple(i)], gr[tuple(i)]),
                "oracle", (e["i_xi"][tuple(i)], e["i_eta"][tuple(i)], e["i_rho"][tuple(i)]),
                "margin", e["margin"][tuple(i)])
    return st


def assert_encode_ok(st, what):
    st = dict(st, forgiven=st["mismatch"] - st["bad"], sig_forgiven=st["sig_mismatch"] - st["sig_bad"])
    record_counts(what, st)
    say(f"[{what}] triplets {st['triplets']} mismatches {st['mismatch']} (all with margin < 1e-6"
        f" unless bad={st['bad']}); gamma rel err {st['gamma_err']:.2e}; sigma mismatches"
        f" {st['sig_mismatch']} bad {st['sig_bad']}; gamma_r bad {st['gr_bad']}")
    assert st["bad"] == 0
    assert st["gamma_err"] <= 4 * 2.0 ** -23
    assert st["sig_bad"] == 0
    assert st["gr_bad"] == 0


def workload(key, **changes):
    w = WORKLOADS[key]
    return dataclasses.replace(w, **changes) if changes else w
