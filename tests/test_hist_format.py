"""The encode pass's fixed-point bucket histogram, restated on the CPU with exact
arithmetic, on the inputs that stress its bounds.

The kernel adds, per element of bucket c, the bit pattern of
    y = fma(c, -2^s, fma(x_c, 2^s / wd, 2^52 + 2^44 + rint(-lo 2^s / wd) + bias))
to a 64-bit word per bucket: the low 44 bits sum the element's position inside
its bucket (units of wd 2^-s, offset by the bias), the top 20 bits count
elements in units of an odd constant.  The codebook stage takes the count back
with the constant's inverse mod 2^20 and forms lo + wd (c + mean position).

That only works while every position plus the bias stays in [0, 2^27).  An
element above hi is clipped to hi but coded from its own value; when lo and hi
round to fp32 steps coarser than the bucket width (a mean many orders above the
spread), (hi - lo) / wd falls below 255 and such an element lands in a bucket
above hi's, at a negative position.  The bias and the fraction bits s are
therefore chosen per (learner, tensor) from (hi - lo) / wd.  These tests restate
that choice and the addend, decode the sums, and check counts (exact) and
codebook entries (within one fp32 ulp of the oracle's fp64 bucket means) on
mean-dominated tensors, and that a single fixed bias of 2^13 would corrupt them.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.edge_inputs import CASES, case_input
from tests.parity import codebook_bound

K_POS_MAGIC = 2.0 ** 52 + 2.0 ** 44
K_POS_UNIT = 0x43301
K_POS_UNIT_INV = 0x4CD01
K_FRAC_BITS = 26
K_BIAS = 1 << 13
MASK44 = (1 << 44) - 1
MASK20 = (1 << 20) - 1


def hist_format(lo, hi, wd, per_tensor_bias=True):
    """(s, bias): the fraction bits and bias of one (learner, tensor)."""
    ext = (float(hi) - float(lo)) / float(wd) - 255.0
    top = max(ext, 1.0)
    neg = max(-ext, 0.0) if per_tensor_bias else 0.0
    s = K_FRAC_BITS
    while s > 0 and (top + neg) * float(1 << s) + 2.0 * K_BIAS >= float(1 << 27):
        s -= 1
    return s, float(K_BIAS) + math.ceil(neg * float(1 << s))


def fma(a, b, c):
    """fl64(a * b + c) with one rounding (round half to even)."""
    return float(Fraction(a) * Fraction(b) + Fraction(c))


def bits(y):
    return struct.unpack("<Q", struct.pack("<d", y))[0]


def packed_histogram(x, lo, hi, wd, per_tensor_bias=True):
    """The kernel's packed 64-bit bucket words for one block holding all of x,
    plus the encode parameters the decode needs."""
    s, bias = hist_format(lo, hi, wd, per_tensor_bias)
    scale = float(1 << s) / float(wd)
    b = -float(lo) * scale
    bi = float(round(b))  # round half to even, as rint
    magic = K_POS_MAGIC + (bi + bias)
    codes = oracle.encode(x, lo, wd).astype(np.int64)
    xc = np.minimum(np.maximum(x, np.float32(lo)), np.float32(hi)).astype(np.float64)
    words = [0] * 256
    for c, v in zip(codes, xc):
        y = fma(float(c), -float(1 << s), fma(float(v), scale, magic))
        words[c] = (words[c] + bits(y)) & ((1 << 64) - 1)
    return words, codes, dict(s=s, bias=bias, origin_frac=b - bi)


def decode(words, lo, wd, par):
    """Counts and codebook entries from the packed words (one block per tensor)."""
    counts = np.zeros(256, np.int64)
    cb = np.zeros(256, np.float32)
    for c, w in enumerate(words):
        n = ((w >> 44) * K_POS_UNIT_INV) & MASK20
        q = (w & MASK44) - n * int(par["bias"])
        counts[c] = n
        if n:
            frac = (q / n + par["origin_frac"]) / float(1 << par["s"])
            cb[c] = np.float32(float(lo) + float(wd) * (c + frac))
        else:
            cb[c] = np.float32(float(lo) + (c + 0.5) * float(wd))
    return counts, cb


@pytest.mark.parametrize("name,args,ratio_range", CASES + [("ordinary", (4, 4000), (255.5, 256.5))])
def test_counts_and_codebook_decode_exactly(name, args, ratio_range):
    x = case_input(name, args)
    mu, sd = oracle.tensor_stats(x)
    lo, hi, wd, _, degenerate = oracle.clip_range(mu, sd)
    assert not degenerate
    ratio = (float(hi) - float(lo)) / float(wd)
    assert ratio_range[0] <= ratio <= ratio_range[1], ratio
    assert np.any(x > hi), "the case must hold elements above hi"
    words, codes, par = packed_histogram(x, lo, hi, wd)
    counts, cb = decode(words, lo, wd, par)
    bs, bn = oracle.histogram(codes.astype(np.uint8), oracle.clip_values(x, lo, hi))
    np.testing.assert_array_equal(counts, bn)
    want = oracle.codebook(bs, bn, lo, wd)
    used = bn > 0
    err = np.abs(cb.astype(np.float64) - want.astype(np.float64))
    assert np.all(err[used] <= codebook_bound(want, wd)[used]), (name, err[used].max())
    np.testing.assert_array_equal(cb[~used], want[~used])
    # every addend fits the 44-bit field of one block
    assert par["bias"] >= K_BIAS


@pytest.mark.parametrize("name,args,ratio_range", [c for c in CASES if c[2][1] < 255.0])
def test_a_fixed_bias_would_corrupt_the_counts(name, args, ratio_range):
    """With the bias fixed at 2^13, elements above hi borrow from the count field."""
    x = case_input(name, args)
    mu, sd = oracle.tensor_stats(x)
    lo, hi, wd, _, _ = oracle.clip_range(mu, sd)
    words, codes, par = packed_histogram(x, lo, hi, wd, per_tensor_bias=False)
    counts, _ = decode(words, lo, wd, par)
    assert not np.array_equal(counts, np.bincount(codes, minlength=256))


def test_format_bounds():
    """s stays at 26 for ordinary ranges; the bias grows with how far (hi - lo) / wd
    falls below 255, and s drops just enough to keep the top position below 2^27."""
    assert hist_format(-1.0, 1.0, 2.0 / 256) == (26, float(K_BIAS))
    s, bias = hist_format(1.0, 1.0, 1e-9)  # lo == hi
    assert s == 18 and bias == K_BIAS + 255 * (1 << 18)
    assert (256 * (1 << s)) + 2 * K_BIAS < (1 << 27)
    for ratio in (0.0, 10.5, 100.0, 254.0, 254.99, 255.0, 256.0, 300.0, 5000.0):
        wd = 1.0 / 1024
        s, bias = hist_format(0.0, ratio * wd, wd)
        lo_pos = min(0.0, ratio - 255.0) * (1 << s) - (1 << 12) - 1
        hi_pos = max(1.0, ratio - 255.0) * (1 << s) + (1 << 12) + 1
        assert lo_pos + bias >= 0 and hi_pos + bias < (1 << 27), ratio
