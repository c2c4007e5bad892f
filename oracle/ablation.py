"""Token Norm Imbalance (TNI) ablation of the OScaR key pipeline, float64
(test infrastructure and a small study; nothing on the GPU path uses it).

The pages (ai-papers.net OScaR summary, sections "TNIという根本課題の特定"
and "OScaRの提案手法"; OScaR abstract) attribute the INT2 failure of
per-channel key quantization to tokens whose L2 norm is far below the
others (attention-sink tokens), and fix it in two steps: a Hadamard
rotation that spreads channel outliers, then a per-token L2 scaling that
equalises the norms before the per-channel quantizer.  This module
quantizes keys four ways, with the same per-channel asymmetric INT2 over
128-token groups each time, and measures what the pages argue about:

* ``per_channel`` - neither step (the KIVI-style key quantizer);
* ``rotation``    - the Hadamard rotation only (QuaRot-style);
* ``scaling``     - the per-token L2 scaling only;
* ``oscar``       - rotation, then scaling (the method).

Keys are dequantized back to the original (unrotated) basis, so every
variant is compared on k itself.  Values are quantized per token in every
variant (the method leaves them unchanged).
"""
import numpy as np

from .attention import decode_bf16_slice, dequant_values
from .fp16 import fp16_rne
from .hadamard import hadamard
from .quantize import key_group_params, key_codes, quantize_values, scale_tokens

VARIANTS = ("per_channel", "rotation", "scaling", "oscar")
GROUP = 128


def quantize_dequantize_keys(k, variant):
    """k [T, 128] (T a multiple of 128) -> the dequantized keys in k's basis."""
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant}")
    k = np.asarray(k, dtype=np.float64)
    rotate = variant in ("rotation", "oscar")
    scale = variant in ("scaling", "oscar")
    H = hadamard(k.shape[-1])
    y = k @ H.T if rotate else k
    if scale:
        n16 = fp16_rne(np.sqrt(np.sum(y * y, axis=-1)))
        u = scale_tokens(y, n16)
    else:
        n16 = np.ones(y.shape[0])
        u = y
    _, _, s16, z16 = key_group_params(u, GROUP)
    _, codes = key_codes(u, s16, z16, GROUP)
    g = np.arange(u.shape[0]) // GROUP
    u_hat = s16[g] * codes + z16[g]
    y_hat = u_hat * n16[:, None]
    return y_hat @ H if rotate else y_hat   # H is orthonormal and symmetric


def key_errors(k, variant):
    """Relative key reconstruction error ||k_t - k_hat_t|| / ||k_t|| per token."""
    k = np.asarray(k, dtype=np.float64)
    k_hat = quantize_dequantize_keys(k, variant)
    num = np.linalg.norm(k - k_hat, axis=-1)
    den = np.linalg.norm(k, axis=-1)
    return num / np.where(den > 0, den, 1.0)


def softmax_weights(logits):
    """Row-wise softmax of logits [G, N] (max subtracted), float64."""
    x = np.asarray(logits, dtype=np.float64)
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=-1, keepdims=True)


def tv_distance(p, p_hat):
    """Total-variation distance per row of two weight vectors [G, N]:
    1/2 sum_t |p_t - p_hat_t| (symmetric; 0 for equal weights, 1 for
    weights on disjoint tokens)."""
    return 0.5 * np.abs(np.asarray(p, np.float64) - np.asarray(p_hat, np.float64)).sum(axis=-1)


def rel_output_error(out, ref):
    """Relative error per row ||out - ref|| / ||ref||: the norm of the
    reference (exact attention) is the denominator, not the estimate's."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.linalg.norm(out - ref, axis=-1) / np.linalg.norm(ref, axis=-1)


def attention_tv(q, k, variant, sm_scale):
    """Max over query heads of the total-variation distance between the
    attention weights over the exact keys and over the variant's dequantized
    keys.  Values do not enter, so the number isolates the key quantizer."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    k_hat = quantize_dequantize_keys(k, variant)
    p = softmax_weights(sm_scale * q @ k.T)
    p_hat = softmax_weights(sm_scale * q @ k_hat.T)
    return float(np.max(tv_distance(p, p_hat)))


def output_error(q, k, v, variant, sm_scale):
    """Max over query heads of ||out - out_ref|| / ||out_ref|| with the
    variant's keys and per-token INT2 values against exact attention."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    k_hat = quantize_dequantize_keys(k, variant)
    vq = quantize_values(v)
    v_hat = dequant_values(vq["codes"], vq["vs16"], vq["vz16"])
    out = decode_bf16_slice(q, k_hat, v_hat, sm_scale)
    ref = decode_bf16_slice(q, k, v, sm_scale)
    return float(np.max(rel_output_error(out, ref)))


def study(workload=1, heads=(0, 1, 2, 3), sm_scale=1.0 / np.sqrt(128.0)):
    """Errors of every variant on the synthetic generator (sequence 0), as
    means over the given KV heads.  ``workload`` is a workload index or a
    ``synthetic.Workload``; its quantized tokens (whole groups) are used."""
    import synthetic as syn
    w = syn.workload(workload) if isinstance(workload, int) else workload
    G = w.num_q_heads // w.num_kv_heads
    n_quant = syn.split_lengths(w.total_tokens(0))[0]
    rows = {v: {"key_err_mean": [], "key_err_sink": [], "key_err_p99": [], "attn_tv": [], "out_err": []}
            for v in VARIANTS}
    for h in heads:
        k = syn.bf16_bits_to_f64(syn.keys_slice(w, 0, h))[:n_quant]
        val = syn.bf16_bits_to_f64(syn.values_slice(w, 0, h))[:n_quant]
        q = syn.bf16_bits_to_f64(syn.query(w, 0)[h * G:(h + 1) * G])
        for var in VARIANTS:
            e = key_errors(k, var)
            rows[var]["key_err_mean"].append(float(e.mean()))
            rows[var]["key_err_sink"].append(float(e[0]))
            rows[var]["key_err_p99"].append(float(np.percentile(e, 99)))
            rows[var]["attn_tv"].append(attention_tv(q, k, var, sm_scale))
            rows[var]["out_err"].append(output_error(q, k, val, var, sm_scale))
    return {v: {m: float(np.mean(x)) for m, x in r.items()} for v, r in rows.items()}


if __name__ == "__main__":
    import json
    import sys
    wl = int(sys.argv[1]) if len(sys.argv) > 1 else 1
    for var, r in study(wl).items():
        print(json.dumps({"variant": var, **{k: round(x, 5) for k, x in r.items()}}))
