"""The 128-point Hadamard matrix of Canalized Rotation (test infrastructure).

Canalized Rotation applies a Hadamard transform to each key so that the
energy of channel outliers is spread evenly over all channels (ai-papers.net
OScaR summary, section "OScaRの提案手法" and Fig. 4; OScaR abstract, arXiv
2605.19660).  The pages give neither the order nor the normalisation; the
reading used here is the Sylvester matrix in natural order, scaled to be
orthonormal, with no random signs:

    H[i, j] = (-1) ** popcount(i & j) / sqrt(n).

This is the closed form of the Sylvester construction written out entry by
entry.  Pin: ``tests/test_oracle_hadamard.py`` (scipy.linalg.hadamard,
H @ H.T = I, a recursive Kronecker construction).
"""
import numpy as np


def _popcount(a):
    a = np.asarray(a, dtype=np.uint64)
    count = np.zeros(a.shape, dtype=np.uint64)
    while np.any(a):
        count += a & np.uint64(1)
        a = a >> np.uint64(1)
    return count


def hadamard(n: int = 128) -> np.ndarray:
    """Orthonormal Sylvester Hadamard matrix of order n (a power of two)."""
    if n < 1 or (n & (n - 1)) != 0:
        raise ValueError("Hadamard order must be a power of two")
    i = np.arange(n, dtype=np.uint64)
    parity = _popcount(i[:, None] & i[None, :]) % np.uint64(2)
    return np.where(parity == 0, 1.0, -1.0) / np.sqrt(float(n))
