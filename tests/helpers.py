"""Test helpers: moving oracle results into GPU cache buffers and the parity
criteria, written once for the GPU tests, ``smoke()`` and ``bench.py``.

Parity criteria (the path's stated bar):
* packed INT2 codes are bit-exact, except codes whose oracle pre-round value
  r lies within 1e-4 of a .5 boundary, and those must be under 0.01% of the
  codes compared;
* fp16 scales, zero-points and norms agree within 1e-6 relative: the GPU's
  fp16 value must be the fp16 rounding of some x within 1e-6 relative of the
  oracle's float64 value before rounding (absolute floor 1e-6 * the group's
  scale for zero-points near 0);
* attention output: |out - ref| <= 1e-3 + 1e-3 * |ref| elementwise, the GPU
  decode running on the very bytes the oracle produced.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle.fp16 import fp16_rne

CODE_WINDOW = 1e-4
CODE_MAX_FRACTION = 1e-4
PARAM_RTOL = 1e-6
OUT_ATOL = 1e-3
OUT_RTOL = 1e-3


def bits_to_dev_bf16(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def token_rows(field: torch.Tensor, b: int, h: int, g0: int, ng: int) -> np.ndarray:
    """Rows of a per-token cache field ([B, H, G, 128, ...] view) for groups
    g0 .. g0+ng-1 of slice (b, h), with the group dimension folded into the
    token dimension, as a host array."""
    x = field[b, h, g0:g0 + ng].cpu().numpy()
    return x.reshape(ng * x.shape[1], *x.shape[2:])


def upload_slice(cache, b: int, h: int, s: "oracle.OracleSlice"):
    """Copy one oracle slice (packed bytes + bf16 tail) into a PackedCache."""
    n = s.n_quant
    dev = cache.k_codes.device
    if n:
        ng = n // 128
        cache.k_codes[b, h, :ng] = torch.from_numpy(s.k_codes.reshape(ng, 128, 32)).to(dev)
        cache.k_norm[b, h, :ng] = torch.from_numpy(s.k_norm.view(np.int16).reshape(ng, 128)).to(dev)
        cache.v_sz[b, h, :ng] = torch.from_numpy(s.v_sz.view(np.int16).reshape(ng, 128, 2)).to(dev)
        cache.k_sz[b, h, :ng] = torch.from_numpy(s.k_sz.view(np.int16)).to(dev)
        cache.v_codes[b, h, :ng] = torch.from_numpy(s.v_codes).to(dev)
    nt = s.k_tail.shape[0]
    if nt:
        from synthetic import f32_to_bf16_bits
        cache.k_tail[b, h, :nt] = bits_to_dev_bf16(f32_to_bf16_bits(s.k_tail.astype(np.float32)), dev)
        cache.v_tail[b, h, :nt] = bits_to_dev_bf16(f32_to_bf16_bits(s.v_tail.astype(np.float32)), dev)


def fp16_param_ok(gpu_bits: np.ndarray, pre: np.ndarray, abs_floor=None) -> np.ndarray:
    """Elementwise: is the GPU fp16 value the rounding of some x within
    PARAM_RTOL relative (or abs_floor) of the oracle's pre-rounding value?"""
    g = np.asarray(gpu_bits, np.uint16).view(np.float16).astype(np.float64)
    pre = np.asarray(pre, np.float64)
    tol = PARAM_RTOL * np.abs(pre)
    if abs_floor is not None:
        tol = np.maximum(tol, abs_floor)
    lo = fp16_rne(pre - tol)
    hi = fp16_rne(pre + tol)
    return (g >= lo) & (g <= hi)


def code_mismatch_report(gpu_codes: np.ndarray, ref_codes: np.ndarray, r: np.ndarray):
    """(n_mismatch, n_outside_window, n_total) for unpacked codes; r is the
    oracle's pre-round value (NaN where the scale is 0 and no decision is taken)."""
    diff = gpu_codes != ref_codes
    n_mis = int(np.count_nonzero(diff))
    near = np.abs((r - np.floor(r)) - 0.5) < CODE_WINDOW
    near = np.where(np.isnan(r), False, near)
    outside = int(np.count_nonzero(diff & ~near))
    return n_mis, outside, int(diff.size)


def assert_codes_ok(gpu_codes, ref_codes, r, what="codes"):
    n_mis, outside, total = code_mismatch_report(gpu_codes, ref_codes, r)
    assert outside == 0, f"{what}: {outside} mismatches outside the 1e-4 window (of {total})"
    assert n_mis <= CODE_MAX_FRACTION * total, f"{what}: {n_mis} mismatches of {total} exceed 0.01%"
    return n_mis


def check_quantized_slice(cache, b: int, h: int, ref: "oracle.OracleSlice", g0: int = 0, ng: int = None):
    """Compare GPU cache groups g0 .. g0+ng-1 of slice (b, h) with an oracle
    slice quantized with keep_intermediates=True over the same tokens.
    Returns a dict of counts (exact-bit matches included)."""
    ng = ref.n_quant // 128 if ng is None else ng
    kq, vq = ref.kq, ref.vq
    gk = token_rows(cache.k_codes, b, h, g0, ng)
    gn = token_rows(cache.k_norm, b, h, g0, ng).view(np.uint16)
    gks = cache.k_sz[b, h, g0:g0 + ng].cpu().numpy().view(np.uint16)
    gv = cache.v_codes[b, h, g0:g0 + ng].cpu().numpy()
    gvs = token_rows(cache.v_sz, b, h, g0, ng).view(np.uint16)

    assert fp16_param_ok(gn, kq["n"]).all(), "key norms outside tolerance"
    s_pre, z_pre = kq["s_pre"], kq["z_pre"]
    assert fp16_param_ok(gks[..., 0], s_pre).all(), "key scales outside tolerance"
    assert fp16_param_ok(gks[..., 1], z_pre, abs_floor=PARAM_RTOL * np.maximum(np.abs(z_pre), s_pre)).all(), \
        "key zero-points outside tolerance"
    assert fp16_param_ok(gvs[:, 0], vq["s_pre"]).all(), "value scales outside tolerance"
    assert fp16_param_ok(gvs[:, 1], vq["z_pre"],
                         abs_floor=PARAM_RTOL * np.maximum(np.abs(vq["z_pre"]), vq["s_pre"])).all(), \
        "value zero-points outside tolerance"
    from oracle.pack import unpack_k_codes, unpack_v_codes
    nk = assert_codes_ok(unpack_k_codes(gk), kq["codes"], kq["r"], "key codes")
    nv = assert_codes_ok(unpack_v_codes(gv), vq["codes"], vq["r"], "value codes")
    return dict(
        key_code_mismatch=nk, value_code_mismatch=nv,
        norm_bits_equal=bool(np.array_equal(gn, ref.k_norm)),
        key_param_bits_equal=bool(np.array_equal(gks, ref.k_sz)),
        value_param_bits_equal=bool(np.array_equal(gvs, ref.v_sz)),
        key_bytes_equal=bool(np.array_equal(gk, ref.k_codes)),
        value_bytes_equal=bool(np.array_equal(gv, ref.v_codes)),
    )


def assert_out_close(got: np.ndarray, ref: np.ndarray, what="out"):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    bound = OUT_ATOL + OUT_RTOL * np.abs(ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements outside 1e-3 + 1e-3|ref|; "
                           f"max err {err.max():.3e}")
    return float(err.max())
