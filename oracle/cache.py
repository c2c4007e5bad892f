"""One (sequence, KV-head) slice of the packed cache, built by the oracle
(test infrastructure).

``quantize_slice`` runs the oracle quantizer over the whole 128-token groups
of a slice and packs the result in the library's storage layout (see
``oracle.pack``), so that the very same bytes can be uploaded to the GPU and
the GPU decode can be compared with ``OracleSlice.decode`` on an identical
cache.  Storage formats: codes uint8, fp16 parameters as uint16 bit
patterns, key (s, z) interleaved per channel, value (s, z) interleaved per
token.
"""
import dataclasses

import numpy as np

from .attention import decode_slice, dequant_keys_rotated, dequant_values
from .hadamard import hadamard
from .fp16 import fp16_bits, fp16_from_bits
from .pack import pack_k_codes, pack_v_codes, unpack_k_codes, unpack_v_codes
from .quantize import quantize_keys, quantize_values

GROUP = 128


@dataclasses.dataclass
class OracleSlice:
    n_quant: int
    k_codes: np.ndarray   # uint8 [n_quant, 32]
    k_sz: np.ndarray      # uint16 [n_quant // 128, 128, 2] (s16, z16) bits
    k_norm: np.ndarray    # uint16 [n_quant] n16 bits
    v_codes: np.ndarray   # uint8 [n_quant // 128, 128, 32]
    v_sz: np.ndarray      # uint16 [n_quant, 2] (vs16, vz16) bits
    k_tail: np.ndarray    # float64 [n_tail, 128] (bf16-exact)
    v_tail: np.ndarray
    kq: dict = None       # key quantizer intermediates
    vq: dict = None       # value quantizer intermediates
    rotated: bool = True  # keys stored in the rotated domain (the method; False only for the ablation)

    def dequantized(self):
        """(k^ rotated, v^) recovered from the packed bytes alone."""
        kc = unpack_k_codes(self.k_codes)
        vc = unpack_v_codes(self.v_codes)
        n16 = fp16_from_bits(self.k_norm)
        s16 = fp16_from_bits(self.k_sz[..., 0])
        z16 = fp16_from_bits(self.k_sz[..., 1])
        vs16 = fp16_from_bits(self.v_sz[:, 0])
        vz16 = fp16_from_bits(self.v_sz[:, 1])
        return (dequant_keys_rotated(kc, n16, s16, z16, GROUP),
                dequant_values(vc, vs16, vz16))

    def decode(self, q, sm_scale):
        """Attention of q [G, 128] (bf16-exact) over this slice."""
        k_hat, v_hat = self.dequantized()
        if not self.rotated:
            # keys stored as they are: H^T brings them to the rotated domain
            # that decode_slice scores against (H is orthonormal)
            k_hat = k_hat @ hadamard(k_hat.shape[-1]).T
        return decode_slice(q, k_hat, v_hat, self.k_tail, self.v_tail, sm_scale)


def quantize_slice(k, v, n_quant, keep_intermediates=False, rotate=True, scale=True):
    """Quantize the first n_quant tokens (a multiple of 128) of one slice;
    the remaining tokens form the bf16 tail.  k, v: float64 [T, 128].
    rotate / scale: the key-quantizer variants of ``quantize_keys``."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if n_quant % GROUP:
        raise ValueError("n_quant must be a multiple of 128")
    kq = quantize_keys(k[:n_quant], rotate=rotate, scale=scale)
    vq = quantize_values(v[:n_quant])
    G = n_quant // GROUP
    k_sz = np.stack([fp16_bits(kq["s16"]), fp16_bits(kq["z16"])], axis=-1).reshape(G, 128, 2)
    v_sz = np.stack([fp16_bits(vq["vs16"]), fp16_bits(vq["vz16"])], axis=-1).reshape(n_quant, 2)
    return OracleSlice(
        n_quant=n_quant,
        k_codes=pack_k_codes(kq["codes"]) if n_quant else np.zeros((0, 32), np.uint8),
        k_sz=k_sz.astype(np.uint16),
        k_norm=fp16_bits(kq["n16"]).astype(np.uint16),
        v_codes=pack_v_codes(vq["codes"]) if n_quant else np.zeros((0, 128, 32), np.uint8),
        v_sz=v_sz.astype(np.uint16),
        k_tail=k[n_quant:], v_tail=v[n_quant:],
        kq=kq if keep_intermediates else None,
        vq=vq if keep_intermediates else None,
        rotated=rotate,
    )
