"""OScaR key and value quantization, step by step in float64 (test infrastructure).

Keys (OScaR abstract, arXiv 2605.19660; ai-papers.net OScaR summary, section
"OScaRの提案手法" and Fig. 4), in the order the pages give:

1. Canalized Rotation: y_t = H k_t with the orthonormal 128-point Hadamard H.
2. Omni-Token Scaling: n_t = ||y_t||_2, stored as n16_t = fp16(n_t);
   u_t = y_t / n16_t (every token then has unit norm up to fp16 rounding of
   the norm).  Reading: the divisor is the stored fp16 norm, so that encoder
   and decoder use the same number; u_t = 0 when n16_t = 0.
3. Per-channel INT2 over groups of 128 tokens (the per-channel key paradigm
   that OScaR builds on, abstract; KIVI's key-per-channel / value-per-token
   split is described on the Qiita NOVA-KV page, bandwidth section):
   for each group g and channel d, mn = min_t u_t[d], mx = max_t u_t[d],
   s16 = fp16((mx - mn) / 3), z16 = fp16(mn)  (asymmetric, float zero-point);
   r = (u_t[d] - z16) / s16, code = clamp(round_half_even(r), 0, 3);
   code = 0 when s16 = 0.

Values: no rotation or scaling.  Per token (one 128-channel group when
head_dim is 128): mn, mx over channels, vs16 = fp16((mx - mn) / 3),
vz16 = fp16(mn), codes as above.

Each step is its own function so tests can check them one at a time.
Pins: ``tests/test_oracle_quantize.py`` (brute-force nearest level, closed
forms on one-hot keys, unit norms, error bounds, degenerate groups).
"""
import numpy as np

from .fp16 import fp16_rne
from .hadamard import hadamard

HEAD_DIM = 128
GROUP = 128


def rotate_keys(k):
    """Canalized Rotation: y_t = H k_t for every row k_t of k [T, 128]."""
    k = np.asarray(k, dtype=np.float64)
    H = hadamard(k.shape[-1])
    return k @ H.T


def token_norms(y):
    """Per-token L2 norm n_t and its fp16 storage value n16_t."""
    n = np.sqrt(np.sum(np.asarray(y, dtype=np.float64) ** 2, axis=-1))
    return n, fp16_rne(n)


def scale_tokens(y, n16):
    """Omni-Token Scaling: u_t = y_t / n16_t (0 where the stored norm is 0)."""
    y = np.asarray(y, dtype=np.float64)
    n16 = np.asarray(n16, dtype=np.float64)
    safe = np.where(n16 > 0, n16, 1.0)
    return np.where(n16[..., None] > 0, y / safe[..., None], 0.0)


def key_group_params(u, group=GROUP):
    """Per (group, channel) asymmetric INT2 parameters of scaled keys.

    Returns (s_pre, z_pre, s16, z16), each [T // group, 128]; *_pre are the
    float64 values before fp16 rounding.
    """
    u = np.asarray(u, dtype=np.float64)
    T, D = u.shape
    if T % group:
        raise ValueError("key token count must be a multiple of the group size")
    ug = u.reshape(T // group, group, D)
    mn = ug.min(axis=1)
    mx = ug.max(axis=1)
    s_pre = (mx - mn) / 3.0
    z_pre = mn
    return s_pre, z_pre, fp16_rne(s_pre), fp16_rne(z_pre)


def _codes(x, s16, z16):
    """r = (x - z16) / s16 and code = clamp(rint(r), 0, 3); code 0 if s16 == 0.

    np.rint rounds half to even.  r is returned as NaN where s16 == 0 (no
    rounding decision is taken there).
    """
    s_safe = np.where(s16 > 0, s16, 1.0)
    r = (x - z16) / s_safe
    c = np.clip(np.rint(r), 0, 3)
    c = np.where(s16 > 0, c, 0)
    r = np.where(s16 > 0, r, np.nan)
    return r, c.astype(np.uint8)


def key_codes(u, s16, z16, group=GROUP):
    """INT2 key codes [T, 128] and the pre-round values r [T, 128]."""
    u = np.asarray(u, dtype=np.float64)
    T, D = u.shape
    g = np.arange(T) // group
    return _codes(u, np.asarray(s16)[g], np.asarray(z16)[g])


def quantize_keys(k, group=GROUP, rotate=True, scale=True):
    """Full key quantizer for k [T, 128] (T a multiple of 128, bf16-exact values).

    Returns a dict with every intermediate: y, n, n16, u, s_pre, z_pre, s16,
    z16, r, codes.

    rotate / scale switch the two OScaR steps off for the Token Norm
    Imbalance ablation (ai-papers.net OScaR summary, sections
    "TNIという根本課題の特定" and "OScaRの提案手法"): without the rotation
    y = k; without the scaling the stored norm is 1 (n = n16 = 1) and u = y,
    so that dequantization n16 (s16 c + z16) is the same formula for every
    variant.  Both on (the default) is the method.
    """
    y = rotate_keys(k) if rotate else np.asarray(k, dtype=np.float64)
    if scale:
        n, n16 = token_norms(y)
        u = scale_tokens(y, n16)
    else:
        n = n16 = np.ones(y.shape[0])
        u = y
    s_pre, z_pre, s16, z16 = key_group_params(u, group)
    r, codes = key_codes(u, s16, z16, group)
    return dict(y=y, n=n, n16=n16, u=u, s_pre=s_pre, z_pre=z_pre, s16=s16,
                z16=z16, r=r, codes=codes)


def value_params(v):
    """Per-token asymmetric INT2 parameters of values [T, 128]."""
    v = np.asarray(v, dtype=np.float64)
    mn = v.min(axis=-1)
    mx = v.max(axis=-1)
    s_pre = (mx - mn) / 3.0
    z_pre = mn
    return s_pre, z_pre, fp16_rne(s_pre), fp16_rne(z_pre)


def value_codes(v, vs16, vz16):
    """INT2 value codes [T, 128] and pre-round values r."""
    v = np.asarray(v, dtype=np.float64)
    return _codes(v, np.asarray(vs16)[:, None], np.asarray(vz16)[:, None])


def quantize_values(v):
    """Full value quantizer: dict with s_pre, z_pre, vs16, vz16, r, codes."""
    s_pre, z_pre, vs16, vz16 = value_params(v)
    r, codes = value_codes(v, vs16, vz16)
    return dict(s_pre=s_pre, z_pre=z_pre, vs16=vs16, vz16=vz16, r=r, codes=codes)
