"""Test helper: oracle codec dicts built from the codebook artifact."""
import json
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ART = os.path.join(ROOT, "quantized_decode_attention_octo_amd", "codebooks", "octopus_d128.json")
_art = None


def artifact():
    global _art
    if _art is None:
        with open(ART) as f:
            _art = json.load(f)
    return _art


def split_for(bits, b_dir=None, b_nrm=None):
    if b_dir is None:
        return bits + 1, bits - 1
    return b_dir, b_nrm


def codec(bits=3, seed=0, qjl=False, b_dir=None, b_nrm=None, rounding="local3x3", d=128):
    bd, bn = split_for(bits, b_dir, b_nrm)
    a = artifact()
    return {
        "d": d, "b_dir": bd, "b_nrm": bn, "seed": seed, "qjl": qjl, "rounding": rounding,
        "c_xi": np.array(a["c_xi"][str(bd)], dtype=np.float32),
        "c_rho": np.array(a["c_rho"][str(bn)], dtype=np.float32),
    }


def group_codec(bits=2, group=32, seed=0, d=128):
    """Oracle dict of the group-wise value codec (oracle.group)."""
    return {"kind": "group", "d": d, "bits": bits, "group": group, "seed": seed}
