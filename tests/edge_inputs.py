"""Seeded pseudo-gradients at the edges of the quantizer's fixed-point histogram:
tensors whose mean dwarfs their spread, so that lo and hi round to fp32 steps
coarser than the bucket width and (hi - lo) / wd leaves its usual ~256 (down to
lo == hi), with elements above hi.  Inputs only: none of the method's arithmetic.
"""
import numpy as np


def mean_dominated(seed, n, mean, ulps_sd, above, up_ulps):
    """fp32 pseudo-gradients fl32(mean + N(0, (ulps_sd ulp)^2)), ulp the fp32 step at
    the mean, with `above` elements placed up_ulps steps above the mean."""
    rs = np.random.default_rng(seed)
    m = np.float32(mean)
    x = (np.float64(m) + float(np.spacing(m)) * ulps_sd * rs.standard_normal(n)).astype(np.float32)
    idx = rs.choice(n, above, replace=False)
    up = m
    for _ in range(up_ulps):
        up = np.nextafter(up, np.float32(np.inf))
    x[idx] = up
    return x


def ordinary(seed, n):
    """N(0, 1e-3^2) with a few elements at 10 sigma (above hi)."""
    rs = np.random.default_rng(seed)
    x = (1e-3 * rs.standard_normal(n)).astype(np.float32)
    x[rs.choice(n, 3, replace=False)] = np.float32(1e-2)
    return x


# (name, generator arguments, the (hi - lo) / wd the oracle's range gives them);
# every case holds elements above hi
CASES = [
    ("lo_eq_hi", (0, 4000, 1.0, 0.0, 1, 1), (0.0, 0.0)),
    ("lo_eq_hi_negative_mean", (0, 4000, -3.0, 0.0, 3, 2), (0.0, 0.0)),
    ("ratio_195", (0, 4000, 1.0, 0.0, 3, 2), (190.0, 200.0)),
    ("ratio_241", (0, 4000, 1.0, 0.0, 5, 10), (235.0, 245.0)),
    ("ratio_248_noisy", (0, 4000, 1.0, 0.3, 2, 6), (245.0, 250.0)),
    ("ratio_271_noisy", (0, 4000, -3.0, 1.0, 5, 10), (265.0, 275.0)),
]


def case_input(name, args):
    return ordinary(*args) if name == "ordinary" else mean_dominated(*args)
