"""2-bit packing of INT2 codes (test infrastructure).

The pages say only that the cache is INT2 (OScaR abstract, arXiv
2605.19660; ai-papers.net OScaR summary, title and "OScaRの提案手法").  The
packed layout is this library's own reading, written here from its
specification and independently of the GPU code:

* four codes per byte, least-significant bits first:
  byte = c0 | c1 << 2 | c2 << 4 | c3 << 6;
* keys: token-major rows of 32 bytes, byte i of token t holds channels
  4i .. 4i+3 of that token (channels in the rotated domain);
* values: per 128-token group, channel-major rows of 32 bytes, byte j of
  channel d holds tokens 4j .. 4j+3 of the group for that channel.

Pins: ``tests/test_oracle_pack.py`` (literal bytes from the specification,
round trips, a pure-Python bit-by-bit packer on small inputs).
"""
import numpy as np

GROUP = 128


def _pack4(c):
    """Pack the last axis (length divisible by 4) of 2-bit codes, LSB first."""
    c = np.asarray(c, dtype=np.uint8)
    if np.any(c > 3):
        raise ValueError("codes must be in 0..3")
    c = c.reshape(c.shape[:-1] + (c.shape[-1] // 4, 4))
    return (c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)).astype(np.uint8)


def _unpack4(b):
    b = np.asarray(b, dtype=np.uint8)
    parts = [(b >> (2 * i)) & 3 for i in range(4)]
    return np.stack(parts, axis=-1).reshape(b.shape[:-1] + (b.shape[-1] * 4,))


def pack_k_codes(codes):
    """Key codes [T, 128] -> packed rows [T, 32]."""
    return _pack4(codes)


def unpack_k_codes(packed):
    """Packed key rows [T, 32] -> codes [T, 128]."""
    return _unpack4(packed)


def pack_v_codes(codes, group=GROUP):
    """Value codes [T, 128] (T a multiple of 128) -> [T // 128, 128, 32]."""
    codes = np.asarray(codes, dtype=np.uint8)
    T, D = codes.shape
    if T % group:
        raise ValueError("value token count must be a multiple of the group size")
    per_channel = codes.reshape(T // group, group, D).transpose(0, 2, 1)  # [G, D, tokens]
    return _pack4(per_channel)


def unpack_v_codes(packed):
    """[G, 128, 32] -> value codes [G * 128, 128]."""
    per_channel = _unpack4(packed)  # [G, D, tokens]
    G, D, tokens = per_channel.shape
    return per_channel.transpose(0, 2, 1).reshape(G * tokens, D)
