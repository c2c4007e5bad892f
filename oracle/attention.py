"""Single-query attention over the packed INT2 cache, in float64 (test infrastructure).

The decode step the OScaR efficiency numbers refer to (ai-papers.net OScaR
summary, section "実験結果"; OScaR abstract, arXiv 2605.19660) attends one
new query per head over the whole cache.  Written out plainly:

* dequantized key in the rotated domain: k^_t = n16_t * (s16_g * c_t + z16_g)
  (g = group of token t); the query is rotated by the same orthonormal H, so
  (H q) . k^_t approximates q . k_t;
* dequantized value: v^_t = vs16_t * cv_t + vz16_t;
* tokens still in the bf16 tail are used as stored, with the unrotated query;
* logits l_t = sm_scale * score_t; p = softmax(l) (max subtracted, two
  passes); out = sum_t p_t v_t.  An empty cache gives out = 0.

Reading: query head j uses KV head j // (Hq / Hkv) (grouped-query attention,
Llama convention); the output is float64 here and fp32 on the GPU.

``softmax_state`` / ``merge_states`` restate the partial-softmax algebra used
to split the token range across workgroups; tests use them to check that any
partition of the tokens merges to the same output.

Pins: ``tests/test_oracle_attention.py`` (pure-Python naive softmax on tiny
inputs, T = 1, q = 0, permutation invariance, partition merges).
"""
import numpy as np

from .hadamard import hadamard


def dequant_keys_rotated(codes, n16, s16, z16, group=128):
    """k^ [T, 128] in the rotated domain from codes [T,128], n16 [T],
    per-group s16 / z16 [T // group, 128]."""
    codes = np.asarray(codes, dtype=np.float64)
    g = np.arange(codes.shape[0]) // group
    return np.asarray(n16, np.float64)[:, None] * (
        np.asarray(s16, np.float64)[g] * codes + np.asarray(z16, np.float64)[g])


def dequant_values(codes, vs16, vz16):
    """v^ [T, 128] = vs16_t * c + vz16_t."""
    codes = np.asarray(codes, dtype=np.float64)
    return np.asarray(vs16, np.float64)[:, None] * codes + np.asarray(vz16, np.float64)[:, None]


def _attend(logits, values):
    """Two-pass max-subtracted softmax of logits [G, N] applied to values [N, D]."""
    if logits.shape[-1] == 0:
        return np.zeros((logits.shape[0], values.shape[-1]), dtype=np.float64)
    m = logits.max(axis=-1, keepdims=True)
    p = np.exp(logits - m)
    return (p @ values) / p.sum(axis=-1, keepdims=True)


def decode_slice(q, k_hat_rot, v_hat, k_tail, v_tail, sm_scale):
    """Attention of G query heads q [G,128] (bf16-exact) sharing one KV head.

    k_hat_rot / v_hat: dequantized quantized tokens [Nq, 128];
    k_tail / v_tail: bf16-exact tail tokens [Nt, 128].
    """
    q = np.asarray(q, dtype=np.float64)
    H = hadamard(q.shape[-1])
    q_rot = q @ H.T
    logits = np.concatenate([
        sm_scale * (q_rot @ np.asarray(k_hat_rot, np.float64).T),
        sm_scale * (q @ np.asarray(k_tail, np.float64).T),
    ], axis=-1)
    values = np.concatenate([np.asarray(v_hat, np.float64), np.asarray(v_tail, np.float64)], axis=0)
    return _attend(logits, values)


def decode_bf16_slice(q, k, v, sm_scale):
    """Plain attention of q [G,128] over bf16-exact keys/values [N,128]."""
    q = np.asarray(q, dtype=np.float64)
    logits = sm_scale * (q @ np.asarray(k, np.float64).T)
    return _attend(logits, np.asarray(v, np.float64))


def softmax_state(logits, values):
    """Partial softmax state (m, l, acc) of one token subset: m = max logit,
    l = sum exp(l_t - m), acc = sum exp(l_t - m) v_t.  Empty: (-inf, 0, 0)."""
    logits = np.asarray(logits, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if logits.size == 0:
        return -np.inf, 0.0, np.zeros(values.shape[-1])
    m = logits.max()
    p = np.exp(logits - m)
    return m, p.sum(), p @ values


def merge_states(states):
    """Merge partial states: M = max m_i, L = sum l_i e^(m_i - M),
    out = sum acc_i e^(m_i - M) / L (0 if every part is empty)."""
    ms = np.array([s[0] for s in states], dtype=np.float64)
    if not np.isfinite(ms).any():
        return np.zeros_like(states[0][2])
    M = ms.max()
    w = np.where(np.isfinite(ms), np.exp(ms - M), 0.0)
    L = sum(wi * s[1] for wi, s in zip(w, states))
    acc = sum(wi * s[2] for wi, s in zip(w, states))
    return acc / L
