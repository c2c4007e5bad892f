"""Pins of the oracle attention: a pure-Python naive softmax on tiny inputs,
rotation invariance, T = 1 and q = 0 special cases, permutation invariance,
empty caches and partition merges of partial softmax states."""
import math

import numpy as np

from oracle.attention import (decode_bf16_slice, decode_slice, merge_states,
                              softmax_state)
from oracle.hadamard import hadamard


def _naive(q, k, v, sm):
    out = []
    for qi in q:
        logits = [sm * sum(a * b for a, b in zip(qi, kt)) for kt in k]
        w = [math.exp(x) for x in logits]     # tiny inputs: no overflow
        s = sum(w)
        out.append([sum(w[t] * v[t][d] for t in range(len(k))) / s for d in range(len(v[0]))])
    return np.array(out)


def test_naive_softmax_tiny():
    rng = np.random.default_rng(0)
    for T in (1, 2, 5, 16):
        q = rng.standard_normal((2, 128))
        k = rng.standard_normal((T, 128))
        v = rng.standard_normal((T, 128))
        sm = 1 / math.sqrt(128)
        ref = _naive(q.tolist(), k.tolist(), v.tolist(), sm)
        np.testing.assert_allclose(decode_bf16_slice(q, k, v, sm), ref, rtol=1e-12, atol=1e-12)
        # the same tokens as rotated quantized keys (k^ = H k) must give the
        # same result, because the query is rotated by the same orthonormal H
        H = hadamard(128)
        np.testing.assert_allclose(
            decode_slice(q, k @ H.T, v, np.zeros((0, 128)), np.zeros((0, 128)), sm),
            ref, rtol=1e-10, atol=1e-12)
        # and as bf16 tail tokens (unrotated path)
        np.testing.assert_allclose(
            decode_slice(q, np.zeros((0, 128)), np.zeros((0, 128)), k, v, sm),
            ref, rtol=1e-12, atol=1e-12)


def test_special_cases():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((9, 128))
    v = rng.standard_normal((9, 128))
    q = rng.standard_normal((3, 128))
    np.testing.assert_allclose(decode_bf16_slice(q, k[:1], v[:1], 0.1), np.tile(v[0], (3, 1)), atol=1e-15)
    np.testing.assert_allclose(decode_bf16_slice(np.zeros((1, 128)), k, v, 0.1), v.mean(0)[None], atol=1e-14)
    perm = rng.permutation(9)
    np.testing.assert_allclose(decode_bf16_slice(q, k[perm], v[perm], 0.1),
                               decode_bf16_slice(q, k, v, 0.1), rtol=1e-12, atol=1e-14)
    empty = decode_slice(q, np.zeros((0, 128)), np.zeros((0, 128)), np.zeros((0, 128)), np.zeros((0, 128)), 0.1)
    np.testing.assert_array_equal(empty, 0.0)


def test_partition_merge():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal(300) * 4
    values = rng.standard_normal((300, 128))
    p = np.exp(logits - logits.max())
    full = p @ values / p.sum()
    for parts in (1, 2, 7, 40):
        cuts = np.sort(rng.choice(np.arange(1, 300), parts - 1, replace=False)) if parts > 1 else []
        bounds = [0, *cuts, 300]
        states = [softmax_state(logits[a:b], values[a:b]) for a, b in zip(bounds[:-1], bounds[1:])]
        states.append(softmax_state(logits[:0], values[:0]))    # an empty part
        np.testing.assert_allclose(merge_states(states), full, rtol=1e-12, atol=1e-14)
