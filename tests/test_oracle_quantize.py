"""Pins of the oracle quantizer: closed forms on one-hot keys and on
integer-grid values, brute-force nearest reconstruction level, exact
rational parameters, unit norms after scaling, reconstruction error bounds,
degenerate groups, and the method's qualitative claims on synthetic keys."""
from fractions import Fraction

import numpy as np
import scipy.linalg

from oracle.fp16 import fp16_rne
from oracle.quantize import (quantize_keys, quantize_values, rotate_keys,
                             token_norms, scale_tokens)
from synthetic import bf16_bits_to_f64, keys_slice, values_slice, workload

# fp16 values worked out by hand: 1/sqrt(128) = 0.0883883476... lies in
# [2^-4, 2^-3) where the fp16 step is 2^-14: 1448.15 steps -> 1448 * 2^-14.
FP16_INV_SQRT128 = 1448 * 2.0 ** -14          # 0.08837890625
# (2/sqrt(128))/3 = 0.0589255651 lies in [2^-5, 2^-4), step 2^-15:
# 1930.87 steps -> 1931 * 2^-15.
FP16_TWO_THIRDS_INV_SQRT128 = 1931 * 2.0 ** -15   # 0.058929443359375


def _cfg0_keys():
    return bf16_bits_to_f64(keys_slice(workload(0), 0, 0))


def test_one_hot_group_closed_form():
    """Tokens 0..63 are a_t * e_i and tokens 64..127 are b_t * e_j (i != j).
    After rotation and scaling every token is column i or column j of the
    orthonormal Hadamard matrix, so each channel either holds one value
    (s16 = 0, codes 0, z16 = +-fp16(1/sqrt 128)) or two opposite values
    (z16 = -fp16(1/sqrt 128), s16 = fp16(2/(3 sqrt 128)), codes 0 / 3)."""
    i, j = 5, 77
    a = np.array([1.0, 1.5, 2.0, 3.0, 0.75, 6.0, 0.5, 4.0] * 8)
    b = np.array([2.0, 0.25, 5.0, 1.0] * 16)
    k = np.zeros((128, 128))
    k[np.arange(64), i] = a
    k[64 + np.arange(64), j] = b
    q = quantize_keys(k)
    np.testing.assert_array_equal(q["n16"], np.concatenate([a, b]))
    Hs = scipy.linalg.hadamard(128)
    same = Hs[:, i] == Hs[:, j]
    assert same.sum() == 64
    s16, z16 = q["s16"][0], q["z16"][0]
    np.testing.assert_array_equal(s16[same], 0.0)
    np.testing.assert_array_equal(z16[same], Hs[same, i] * FP16_INV_SQRT128)
    np.testing.assert_array_equal(s16[~same], FP16_TWO_THIRDS_INV_SQRT128)
    np.testing.assert_array_equal(z16[~same], -FP16_INV_SQRT128)
    codes = q["codes"]
    np.testing.assert_array_equal(codes[:, same], 0)
    expect = np.where(np.concatenate([np.tile(Hs[:, i], (64, 1)), np.tile(Hs[:, j], (64, 1))]) > 0, 3, 0)
    np.testing.assert_array_equal(codes[:, ~same], expect[:, ~same])


def test_codes_are_nearest_level_brute_force():
    k = _cfg0_keys()
    q = quantize_keys(k)
    u, s16, z16 = q["u"], q["s16"], q["z16"]
    g = np.arange(k.shape[0]) // 128
    levels = z16[g][:, :, None] + s16[g][:, :, None] * np.arange(4)[None, None, :]
    dist = np.abs(u[:, :, None] - levels)
    nearest = dist.argmin(axis=-1)
    # exclude exact ties between two levels (none expected on this data)
    srt = np.sort(dist, axis=-1)
    clear = srt[..., 1] - srt[..., 0] > 1e-12
    assert clear.mean() > 0.999
    np.testing.assert_array_equal(q["codes"][clear], nearest[clear])


def test_value_codes_nearest_level_brute_force():
    v = bf16_bits_to_f64(values_slice(workload(0), 0, 0))
    q = quantize_values(v)
    levels = q["vz16"][:, None, None] + q["vs16"][:, None, None] * np.arange(4)
    dist = np.abs(v[:, :, None] - levels)
    srt = np.sort(dist, axis=-1)
    clear = srt[..., 1] - srt[..., 0] > 1e-12
    np.testing.assert_array_equal(q["codes"][clear], dist.argmin(-1)[clear])


def test_value_params_exact_rational():
    """vs16 is the fp16 value nearest to the exact rational (max - min) / 3 of
    the bf16 inputs, and vz16 = fp16(min): no double rounding."""
    v = bf16_bits_to_f64(values_slice(workload(1), 0, 3))[:200]
    q = quantize_values(v)
    fp16_grid = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    fp16_grid = np.unique(fp16_grid[np.isfinite(fp16_grid)])
    for t in range(0, 200, 7):
        exact = (Fraction(v[t].max()) - Fraction(v[t].min())) / 3
        pos = np.searchsorted(fp16_grid, float(exact))
        cands = fp16_grid[max(pos - 2, 0):pos + 2]
        d = [abs(Fraction(c) - exact) for c in cands]
        best = cands[int(np.argmin(d))]
        assert q["vs16"][t] == best
        assert q["vz16"][t] == fp16_rne(v[t].min())


def test_value_integer_grid_closed_form():
    """Values on the grid -1.5 + 1.5 c (c = 0..3) with both ends present:
    vs16 = 1.5, vz16 = -1.5 and the codes are the grid indices."""
    rng = np.random.default_rng(11)
    c = rng.integers(0, 4, (32, 128))
    c[:, 0], c[:, 1] = 0, 3
    v = -1.5 + 1.5 * c
    q = quantize_values(v)
    np.testing.assert_array_equal(q["vs16"], 1.5)
    np.testing.assert_array_equal(q["vz16"], -1.5)
    np.testing.assert_array_equal(q["codes"], c)
    np.testing.assert_array_equal(q["r"], c)


def test_every_token_unit_norm_after_scaling():
    """Omni-Token Scaling: every token, the sink included, has unit norm up
    to the fp16 rounding of the stored norm."""
    k = _cfg0_keys()
    y = rotate_keys(k)
    n, n16 = token_norms(y)
    u = scale_tokens(y, n16)
    un = np.linalg.norm(u, axis=1)
    assert np.all(np.abs(un - 1) <= 2.0 ** -11 * (1 + 1e-9))
    # the synthetic sink is far below the median norm before scaling
    assert n[0] < 0.1 * np.median(n[1:])


def test_group_extremes_map_to_end_codes():
    k = _cfg0_keys()
    q = quantize_keys(k)
    codes = q["codes"].reshape(-1, 128, 128)
    nondeg = q["s16"] > 0
    assert nondeg.all()
    assert np.all(codes.min(axis=1)[nondeg] == 0)
    assert np.all(codes.max(axis=1)[nondeg] == 3)


def test_reconstruction_error_bound():
    """|u - (s16 c + z16)| <= s16 / 2 + fp16 endpoint slack, and the same
    bound times n16 in the rotated key space."""
    k = _cfg0_keys()
    q = quantize_keys(k)
    g = np.arange(k.shape[0]) // 128
    s16, z16 = q["s16"][g], q["z16"][g]
    deq = s16 * q["codes"] + z16
    slack = 2.0 ** -11 * (np.abs(z16) + 3 * s16) + 2.0 ** -24
    err = np.abs(q["u"] - deq)
    assert np.all(err <= s16 / 2 + slack)
    kerr = np.abs(q["y"] - q["n16"][:, None] * deq)
    assert np.all(kerr <= q["n16"][:, None] * (s16 / 2 + slack) + 1e-12)


def test_degenerate_constant_group_and_zero_token():
    k = np.tile(np.linspace(-1, 1, 128), (128, 1))
    q = quantize_keys(k)
    np.testing.assert_array_equal(q["s16"], 0.0)
    np.testing.assert_array_equal(q["codes"], 0)
    k2 = _cfg0_keys()[:128].copy()
    k2[10] = 0.0
    q2 = quantize_keys(k2)
    assert q2["n16"][10] == 0.0
    np.testing.assert_array_equal(q2["u"][10], 0.0)
    v = np.full((4, 128), 0.5)
    qv = quantize_values(v)
    np.testing.assert_array_equal(qv["vs16"], 0.0)
    np.testing.assert_array_equal(qv["codes"], 0)
    np.testing.assert_array_equal(qv["vz16"], 0.5)


def _per_channel_only(k):
    """Per-channel INT2 over 128-token groups without rotation or scaling."""
    kg = k.reshape(-1, 128, 128)
    mn, mx = kg.min(1, keepdims=True), kg.max(1, keepdims=True)
    s = (mx - mn) / 3
    c = np.clip(np.rint((kg - mn) / np.where(s > 0, s, 1)), 0, 3)
    return (s * c + mn).reshape(k.shape)


def test_sink_token_error_shrinks_with_scaling():
    """Method sanity (Token Norm Imbalance): the relative reconstruction error
    of the low-norm sink token is far smaller with rotation + per-token
    scaling than with per-channel INT2 alone."""
    k = _cfg0_keys()
    q = quantize_keys(k)
    g = np.arange(k.shape[0]) // 128
    y_hat = q["n16"][:, None] * (q["s16"][g] * q["codes"] + q["z16"][g])
    oscar_rel = np.linalg.norm(q["y"][0] - y_hat[0]) / np.linalg.norm(q["y"][0])
    base = _per_channel_only(k)
    base_rel = np.linalg.norm(k[0] - base[0]) / np.linalg.norm(k[0])
    assert oscar_rel < 0.25 * base_rel
