"""SplitMix64 counter generator and the rotation sign vectors it yields.

The OCTOPUS paper (Sec. 1 and the abstract) calls the codec "deterministic
given a seed" and builds R = H diag(s) with a random sign vector s (Sec. 3.1,
App. C.2) and, for the QJL residual, a second rotation R' = H diag(s') "with
independent seed" (Sec. 3.6).  It never names the generator.  Reading used
here: the j-th sign is drawn from the j-th output of a
SplitMix64 generator started at `seed`, i.e. the counter form

    z_j = mix64(seed + (j + 1) * 0x9E3779B97F4A7C15 mod 2^64)

with mix64 the SplitMix64 finalizer of Steele, Lea and Flood, "Fast Splittable
Pseudorandom Number Generators" (OOPSLA 2014), as published in Vigna's
reference splitmix64.c.  s_j = -1 when bit 63 of z_j is set, else +1.
s uses j = 0..d-1 and s' uses j = d..2d-1, so the two are independent draws of
one stream.

Parity: pinned by the published seed-0 output sequence of SplitMix64
(tests/test_oracle_rotation.py).
"""

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15


def mix64(z: int) -> int:
    """SplitMix64 output finalizer (shift-xor-multiply, 30/27/31)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def splitmix64_output(seed: int, j: int) -> int:
    """The j-th (0-based) 64-bit output of SplitMix64 seeded with `seed`."""
    return mix64((seed + (j + 1) * GOLDEN_GAMMA) & MASK64)


def sign_vector(seed: int, start: int, count: int):
    """Signs s_j in {+1, -1} for j = start .. start+count-1 (Python ints)."""
    out = []
    for j in range(start, start + count):
        out.append(-1 if (splitmix64_output(seed, j) >> 63) & 1 else 1)
    return out
