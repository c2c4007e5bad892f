"""Decode-time bookkeeping of the packed cache: the group-append workflow.

The pages quantize a group of 128 tokens once it is complete and keep the
newest tokens unquantized until then (ai-papers.net OScaR summary, section
"OScaRの提案手法").  ``DecodeSession`` keeps, for every sequence of a batch,
the number of quantized tokens and of bf16 tail tokens, runs a decode step
that stores the step's own key and value in the tail inside the decode
launch (``oscar_decode_attn_append``), and quantizes a sequence's tail into
its next group (``oscar_quantize_kv``) after the step that fills it.

Host logic only: every step of the computation runs in the library's
kernels.  The counts of all steps are planned up front (``plan_steps``) and
kept on the device, so a run of steps launches nothing but the library's
kernels and can be captured in a HIP graph.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import torch

from . import binding as ob

GROUP = 128


@dataclasses.dataclass(frozen=True)
class StepPlan:
    """Counts of one decode step, per sequence: n_quant and n_tail as the
    decode sees them (n_tail counts the step's own token), and whether the
    tail is full after the step (then group n_quant / 128 is quantized)."""
    n_quant: List[int]
    n_tail: List[int]
    full: List[bool]

    @property
    def max_tokens(self) -> int:
        return max(q + t for q, t in zip(self.n_quant, self.n_tail))


def plan_steps(n_quant: Sequence[int], n_tail: Sequence[int], steps: int) -> List[StepPlan]:
    """Counts of `steps` decode steps that append one token per sequence,
    starting from n_quant[b] quantized tokens (a multiple of 128) and
    n_tail[b] tail tokens (0..127) per sequence."""
    nq, nt = [int(x) for x in n_quant], [int(x) for x in n_tail]
    for q, t in zip(nq, nt):
        if q < 0 or q % GROUP or not 0 <= t < GROUP:
            raise ValueError("n_quant must be a non-negative multiple of 128 and n_tail in [0, 127]")
    plans = []
    for _ in range(steps):
        nt = [t + 1 for t in nt]
        full = [t == GROUP for t in nt]
        plans.append(StepPlan(list(nq), list(nt), full))
        nq = [q + GROUP if f else q for q, f in zip(nq, full)]
        nt = [0 if f else t for t, f in zip(nt, full)]
    return plans


class DecodeSession:
    """A run of `steps` decode steps over `cache`, one new token per sequence
    and step.  ``step(s, ...)`` launches step s on the current stream (or
    `stream`); steps must be issued in order, once each.  The tail of the
    cache must hold the sequences' first n_tail[b] tail tokens."""

    def __init__(self, cache: "ob.PackedCache", n_quant: Sequence[int], n_tail: Sequence[int], num_q_heads: int,
                 steps: int, ws: Optional[torch.Tensor] = None):
        if len(n_quant) != cache.batch or len(n_tail) != cache.batch:
            raise ValueError("one n_quant and one n_tail per sequence")
        self.cache = cache
        self.plans = plan_steps(n_quant, n_tail, steps)
        last = self.plans[-1] if self.plans else None
        if last is not None and max(q + GROUP for q in last.n_quant) > cache.capacity:
            raise ValueError("the cache is too small for these steps (the tail's group must fit)")
        dev = cache.blocks.device
        i32 = lambda rows: torch.tensor(rows, dtype=torch.int32, device=dev)   # noqa: E731
        self.n_quant = i32([p.n_quant for p in self.plans])             # [steps, B]
        self.n_tail = i32([p.n_tail for p in self.plans])
        self.group_start = i32([[q // GROUP for q in p.n_quant] for p in self.plans])
        self.num_groups = i32([[int(f) for f in p.full] for p in self.plans])
        max_tokens = max((p.max_tokens for p in self.plans), default=0)
        self.ws = ws if ws is not None else ob.alloc_workspace(cache.batch, cache.num_kv_heads, num_q_heads,
                                                               max(max_tokens, 1), device=dev)

    def step(self, s: int, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, sm_scale: float,
             out: torch.Tensor, stream: Optional[torch.cuda.Stream] = None) -> None:
        """Decode step s: q bf16 [B, Hq, 128]; the step's key and value bf16
        [B, Hkv, 128]; out fp32 [B, Hq, 128]."""
        p = self.plans[s]
        ob.decode_attn_append(self.cache, self.n_quant[s], self.n_tail[s], p.max_tokens, q, k_new, v_new,
                              sm_scale, out, self.ws, stream=stream)
        if any(p.full):
            c = self.cache
            ob.quantize_kv(c, c.k_tail, c.v_tail, self.group_start[s], self.num_groups[s], 1, stream=stream)
