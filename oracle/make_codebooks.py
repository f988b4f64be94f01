"""Train the Lloyd-Max codebooks and write the codebook artifact.

Usage:  python -m oracle.make_codebooks [--d 128] [--out PATH]

The OCTOPUS paper (Sec. 3.4) trains C_xi(b_dir) and C_rho(d, b_nrm) offline and
serializes them; they are tiny fp32 tables that depend only on
(d, b_dir, b_nrm).  This script is the offline step: it calls only
oracle.codebook and writes a JSON file of fp32 centroid values with their
provenance (seed, sample counts, iterations, final distortion).  The codec
takes the tables as inputs on both sides; the HIP library never trains them.

b_dir runs over 0..6 and b_nrm over 0..6 so that every split of the paper's
diagonal sweep (b +- delta, b in {2,3,4}, delta in -2..2, Sec. 3.3) exists.
"""
import argparse
import json
import os
import time

import numpy as np

from .codebook import monte_carlo_samples, train_rho, train_xi

DEFAULT_OUT = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "quantized_decode_attention_octo_amd", "codebooks", "octopus_d{d}.json")


def fp32_list(c):
    return [float(np.float32(v)) for v in c]


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--d", type=int, default=128)
    ap.add_argument("--n-keys", type=int, default=100_000)
    ap.add_argument("--mc-seed", type=int, default=0)
    ap.add_argument("--max-iter", type=int, default=100_000)
    ap.add_argument("--out", default=None)
    a = ap.parse_args(argv)
    t0 = time.time()
    s_xi, s_rho = monte_carlo_samples(a.d, a.n_keys, a.mc_seed)
    art = {
        "format": "octopus-codebooks-v1",
        "d": a.d,
        "provenance": {
            "mc_seed": a.mc_seed, "n_keys": a.n_keys, "rotation_seed": 0,
            "xi_samples": int(2 * s_xi.size), "rho_samples": int(s_rho.size),
            "stopping": "relative distortion decrease < 1e-10 and max move < 1e-10",
            "max_iter": a.max_iter,
        },
        "c_xi": {}, "c_rho": {}, "info_xi": {}, "info_rho": {},
    }
    for b in range(0, 7):
        c, info = train_xi(s_xi, b, max_iter=a.max_iter)
        art["c_xi"][str(b)] = fp32_list(c)
        art["info_xi"][str(b)] = info
        print(f"C_xi b_dir={b}: {info}", flush=True)
    for b in range(0, 7):
        c, info = train_rho(s_rho, b, max_iter=a.max_iter)
        art["c_rho"][str(b)] = fp32_list(c)
        art["info_rho"][str(b)] = info
        print(f"C_rho b_nrm={b}: {info}", flush=True)
    art["provenance"]["seconds"] = round(time.time() - t0, 1)
    out = a.out or DEFAULT_OUT.format(d=a.d)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with open(out, "w") as f:
        json.dump(art, f, indent=1)
    print("wrote", out)


if __name__ == "__main__":
    main()
