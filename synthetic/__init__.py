"""Seeded synthetic KV-cache workloads (inputs only).

This module produces the bf16 keys, values and queries that both the CPU
oracle and the HIP path consume.  It contains none of the quantization or
attention arithmetic: only random draws, the workload's outlier structure and
the fp32 -> bf16 rounding of the generated inputs.

Workload structure (Llama-3.1-8B layer shape: 32 query heads, 8 KV heads,
head_dim 128) follows the OScaR pages' setting: keys carry a few fixed
channels with large magnitude (channel outliers), per-token magnitudes vary
(lognormal), and token 0 is an attention-sink key with a very small L2 norm
(ai-papers.net OScaR summary, section "TNIという根本課題の特定"; arXiv
2605.19660 abstract, fugumt.com record).  Values and queries are plain
standard normal.

Seeding: every (config, sequence, kv-head) slice has its own numpy
``default_rng`` stream, so any slice can be regenerated alone (the full-size
parity tests recompute single slices on the host).

All tensors are returned as ``uint16`` arrays holding bf16 bit patterns, in
the layout ``[..., tokens, 128]`` with the channel index fastest.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

HEAD_DIM = 128
GROUP = 128
_SLICE_TAG = 0x05CA
_QUERY_TAG = 0xA11
_LEN_TAG = 0x1E7


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even), returned as uint16 bits.

    Inputs are finite by construction; NaN handling is not needed here.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One of the five seeded workloads.

    ``lengths[b]`` is the number of cached tokens of sequence b at the decode
    step (quantized groups plus bf16 tail).  ``append_steps`` > 0 means the
    last ``append_steps`` tokens of each sequence are fed one per decode step
    (the 32K group-append workload).
    """

    cfg: int
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    lengths: tuple
    append_steps: int = 0
    outlier_factors: tuple = (8.0,)

    @property
    def max_len(self) -> int:
        return max(self.lengths)

    def total_tokens(self, b: int) -> int:
        """Tokens generated for sequence b (prefix + appended steps)."""
        return self.lengths[b] + self.append_steps

    def outlier_factor(self, b: int) -> float:
        return self.outlier_factors[b % len(self.outlier_factors)]


def _cfg4_lengths() -> tuple:
    rng = np.random.default_rng([4, _LEN_TAG])
    return tuple(int(x) for x in rng.integers(98304, 131072, size=8, endpoint=True))


def workload(cfg: int) -> Workload:
    """The five workloads: tiny single head, 8K, 32K + 57-token tail with 128
    appended decode steps, 128K, and batch 8 with jittered 96K-128K lengths."""
    if cfg == 0:
        return Workload(0, "tiny-1kv-1q-1k", 1, 1, 1, (1024,))
    if cfg == 1:
        return Workload(1, "llama31-8b-layer-8k", 1, 32, 8, (8192,))
    if cfg == 2:
        return Workload(2, "llama31-8b-layer-32k+57-append128", 1, 32, 8,
                        (32768 + 57,), append_steps=128)
    if cfg == 3:
        return Workload(3, "llama31-8b-layer-128k", 1, 32, 8, (131072,))
    if cfg == 4:
        return Workload(4, "llama31-8b-layer-b8-96k-128k", 8, 32, 8,
                        _cfg4_lengths(), outlier_factors=(8.0, 16.0))
    raise ValueError(f"unknown workload {cfg}")


def custom_workload(batch: int, num_q_heads: int, num_kv_heads: int,
                    lengths: List[int], cfg_tag: int = 100,
                    append_steps: int = 0) -> Workload:
    """A workload with arbitrary shape, for ragged / edge-case tests."""
    assert len(lengths) == batch
    return Workload(cfg_tag, "custom", batch, num_q_heads, num_kv_heads,
                    tuple(int(x) for x in lengths), append_steps)


def keys_slice_f32(w: Workload, b: int, h: int, n_tokens: Optional[int] = None) -> np.ndarray:
    """fp32 keys of one (sequence, kv-head) slice before bf16 rounding.

    Draw order: N(0,1) [T,128]; four outlier channels (without replacement)
    multiplied by the workload's factor; a lognormal(0, 0.5) factor per
    token; token 0 rescaled so its L2 norm is 0.05 x the median norm of
    tokens 1..T-1.
    """
    T = w.total_tokens(b) if n_tokens is None else n_tokens
    rng = np.random.default_rng([w.cfg, b, h, _SLICE_TAG, 0])
    k = rng.standard_normal((T, HEAD_DIM), dtype=np.float32)
    ch = rng.choice(HEAD_DIM, size=4, replace=False)
    k[:, ch] *= np.float32(w.outlier_factor(b))
    tok = np.exp(rng.normal(0.0, 0.5, size=T)).astype(np.float32)
    k *= tok[:, None]
    if T > 1:
        norms = np.sqrt(np.einsum("td,td->t", k, k, dtype=np.float64))
        target = 0.05 * np.median(norms[1:])
        if norms[0] > 0:
            k[0] *= np.float32(target / norms[0])
    return k


def keys_slice(w: Workload, b: int, h: int) -> np.ndarray:
    """bf16 bits [T,128] of one key slice (all generated tokens)."""
    return f32_to_bf16_bits(keys_slice_f32(w, b, h))


def values_slice(w: Workload, b: int, h: int) -> np.ndarray:
    """bf16 bits [T,128] of one value slice: plain N(0,1)."""
    T = w.total_tokens(b)
    rng = np.random.default_rng([w.cfg, b, h, _SLICE_TAG, 1])
    return f32_to_bf16_bits(rng.standard_normal((T, HEAD_DIM), dtype=np.float32))


def query(w: Workload, b: int, step: int = 0) -> np.ndarray:
    """bf16 bits [Hq,128] of the query of sequence b at decode step ``step``."""
    rng = np.random.default_rng([w.cfg, b, _QUERY_TAG, step])
    return f32_to_bf16_bits(rng.standard_normal((w.num_q_heads, HEAD_DIM), dtype=np.float32))


def split_lengths(length: int) -> tuple:
    """(n_quant, n_tail) of a sequence of ``length`` cached tokens: whole
    128-token groups are quantized, the remainder stays in the bf16 tail."""
    n_quant = (length // GROUP) * GROUP
    return n_quant, length - n_quant
