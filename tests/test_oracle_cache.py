"""Pins of the oracle's packed slice: the bytes decode back to the
quantizer's own dequantized values, and quantization is position
independent (prefill of n + 128 tokens = prefill of n, then one group)."""
import numpy as np

from oracle.cache import quantize_slice
from synthetic import bf16_bits_to_f64, keys_slice, values_slice, workload


def test_packed_slice_round_trip_and_position_independence():
    w = workload(0)
    k = bf16_bits_to_f64(keys_slice(w, 0, 0))
    v = bf16_bits_to_f64(values_slice(w, 0, 0))
    s = quantize_slice(k, v, 1024, keep_intermediates=True)
    k_hat, v_hat = s.dequantized()
    g = np.arange(1024) // 128
    expect_k = s.kq["n16"][:, None] * (s.kq["s16"][g] * s.kq["codes"] + s.kq["z16"][g])
    np.testing.assert_array_equal(k_hat, expect_k)
    np.testing.assert_array_equal(v_hat, s.vq["vs16"][:, None] * s.vq["codes"] + s.vq["vz16"][:, None])
    a = quantize_slice(k[:896], v[:896], 896)
    b = quantize_slice(k[896:], v[896:], 128)
    np.testing.assert_array_equal(np.concatenate([a.k_codes, b.k_codes]), s.k_codes)
    np.testing.assert_array_equal(np.concatenate([a.v_codes, b.v_codes]), s.v_codes)
    np.testing.assert_array_equal(np.concatenate([a.k_sz, b.k_sz]), s.k_sz)
    np.testing.assert_array_equal(np.concatenate([a.k_norm, b.k_norm]), s.k_norm)
    np.testing.assert_array_equal(np.concatenate([a.v_sz, b.v_sz]), s.v_sz)


def test_tail_and_empty():
    w = workload(0)
    k = bf16_bits_to_f64(keys_slice(w, 0, 0))[:300]
    v = bf16_bits_to_f64(values_slice(w, 0, 0))[:300]
    s = quantize_slice(k, v, 256)
    assert s.k_tail.shape == (44, 128)
    e = quantize_slice(k[:5], v[:5], 0)
    out = e.decode(np.ones((1, 128)), 0.1)
    assert out.shape == (1, 128)
    e0 = quantize_slice(k[:0], v[:0], 0)
    np.testing.assert_array_equal(e0.decode(np.ones((2, 128)), 0.1), 0.0)


def test_dequantized_bytes_within_quantization_bounds():
    """The packed bytes alone reproduce the rotated keys (rotation taken from
    scipy's Hadamard routine) and the values within half a quantization step
    plus fp16 endpoint slack."""
    import scipy.linalg
    w = workload(1)
    k = bf16_bits_to_f64(keys_slice(w, 0, 2))[:512]
    v = bf16_bits_to_f64(values_slice(w, 0, 2))[:512]
    s = quantize_slice(k, v, 512)
    k_hat, v_hat = s.dequantized()
    y = k @ (scipy.linalg.hadamard(128) / np.sqrt(128)).T
    n16 = s.k_norm.view(np.float16).astype(np.float64)
    s16 = s.k_sz[..., 0].view(np.float16).astype(np.float64)
    z16 = s.k_sz[..., 1].view(np.float16).astype(np.float64)
    g = np.arange(512) // 128
    bound_u = s16[g] / 2 + 2.0 ** -11 * (np.abs(z16[g]) + 3 * s16[g]) + 2.0 ** -24
    # y = n * u and n16 differs from n by <= 2^-11 relative
    bound_k = n16[:, None] * bound_u + 2.0 ** -10 * np.abs(y)
    assert np.all(np.abs(y - k_hat) <= bound_k)
    vs = s.v_sz[:, 0].view(np.float16).astype(np.float64)
    vz = s.v_sz[:, 1].view(np.float16).astype(np.float64)
    bound_v = vs[:, None] / 2 + 2.0 ** -11 * (np.abs(vz)[:, None] + 3 * vs[:, None]) + 2.0 ** -24
    assert np.all(np.abs(v - v_hat) <= bound_v)
