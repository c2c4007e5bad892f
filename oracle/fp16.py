"""fp16 storage rounding used by the oracle (test infrastructure only).

The OScaR key path keeps each token's L2 norm in fp16, and the INT2 scale
and zero-point of keys and values are fp16 as well (OScaR abstract, arXiv
2605.19660; the fp16 norm is part of Omni-Token Scaling in the ai-papers.net
summary, section "OScaRの提案手法").  The pages do not state the rounding;
the reading used here is IEEE binary16 round-to-nearest-even, saturating to
+/-65504 instead of overflowing to infinity.  NaN inputs are not supported.

Pin: ``tests/test_oracle_fp16.py`` compares against a brute-force nearest
search over every finite binary16 value.
"""
import numpy as np

FP16_MAX = 65504.0


def fp16_rne(x):
    """Round float64 values to the nearest fp16 value (ties to even),
    saturating at +/-65504.  Returns float64 holding the fp16 values.

    numpy's float64 -> float16 cast rounds once, directly from the double
    bits, so no double rounding through float32 occurs.
    """
    x = np.clip(np.asarray(x, dtype=np.float64), -FP16_MAX, FP16_MAX)
    return x.astype(np.float16).astype(np.float64)


def fp16_bits(x):
    """IEEE binary16 bit patterns (uint16) of values already exact in fp16."""
    h = np.asarray(x, dtype=np.float64).astype(np.float16)
    if not np.array_equal(h.astype(np.float64), np.asarray(x, dtype=np.float64)):
        raise ValueError("fp16_bits: values are not exactly representable in fp16")
    return h.view(np.uint16)


def fp16_from_bits(b):
    """float64 values of uint16 fp16 bit patterns."""
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)
