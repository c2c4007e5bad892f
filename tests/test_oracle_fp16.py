"""Pins of the oracle's fp16 storage rounding against values IEEE 754 fixes
and against a brute-force nearest search over all finite binary16 values."""
import json
import os

import numpy as np

from oracle.fp16 import fp16_rne, fp16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp16_values.json")


def _all_finite_fp16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    ok = np.isfinite(vals)
    vals, bits = vals[ok], bits[ok]
    order = np.argsort(vals, kind="stable")
    vals, bits = vals[order], bits[order]
    # drop -0.0 duplicate of +0.0 (keep the +0 pattern)
    keep = np.ones(len(vals), bool)
    z = np.where(vals == 0)[0]
    keep[z[bits[z] == 0x8000]] = False
    return vals[keep], bits[keep]


def _brute(x, vals, bits):
    """Nearest finite fp16 value; ties go to the even significand (even bit pattern)."""
    out = np.empty_like(x)
    for i, xi in enumerate(x):
        xi = min(max(xi, -65504.0), 65504.0)
        d = np.abs(vals - xi)
        best = np.flatnonzero(d == d.min())
        if len(best) > 1:
            best = [b for b in best if bits[b] % 2 == 0]
        out[i] = vals[best[0]]
    return out


def test_golden_values():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        v = fp16_rne(np.array([c["x"]]))
        assert v[0] == c["value"], c
        assert int(fp16_bits(v)[0]) == int(c["bits"], 16), c


def test_brute_force_random():
    vals, bits = _all_finite_fp16()
    rng = np.random.default_rng(1234)
    x = np.concatenate([
        rng.standard_normal(400),
        rng.standard_normal(200) * 1e-5,     # subnormal range
        rng.standard_normal(200) * 3e4,      # near the top
        rng.uniform(-1, 1, 200) * 1e6,       # saturating
    ])
    np.testing.assert_array_equal(fp16_rne(x), _brute(x, vals, bits))


def test_exact_midpoints_tie_to_even():
    vals, bits = _all_finite_fp16()
    rng = np.random.default_rng(7)
    idx = rng.integers(0, len(vals) - 1, 300)
    mids = (vals[idx] + vals[idx + 1]) / 2.0   # exact in float64
    np.testing.assert_array_equal(fp16_rne(mids), _brute(mids, vals, bits))
    # direct check of the rule on the same points
    got_bits = fp16_bits(fp16_rne(mids)).astype(np.int64)
    pos = mids > 0
    assert np.all(got_bits[pos] % 2 == 0)


def test_saturation():
    x = np.array([65519.0, 65520.0, 1e30, -1e30, -65520.0])
    np.testing.assert_array_equal(fp16_rne(x), [65504.0, 65504.0, 65504.0, -65504.0, -65504.0])
