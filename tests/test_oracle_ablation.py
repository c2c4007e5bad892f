"""Sanity pins of the TNI ablation (oracle/ablation.py): the full variant is
the oracle's own quantizer, per-channel INT2 without scaling destroys the
low-norm attention-sink token, and the per-token scaling equalises the
relative error across tokens (the two points the pages make about Token
Norm Imbalance: ai-papers.net OScaR summary, sections
"TNIという根本課題の特定" and "OScaRの提案手法")."""
import numpy as np

import oracle
import synthetic as syn
from oracle import ablation as A
from oracle.hadamard import hadamard


def _keys():
    w = syn.workload(0)
    return syn.bf16_bits_to_f64(syn.keys_slice(w, 0, 0))


def test_oscar_variant_is_the_oracle_quantizer():
    k = _keys()
    s = oracle.quantize_slice(k, np.zeros_like(k), k.shape[0])
    k_hat_rot, _ = s.dequantized()
    H = hadamard(128)
    np.testing.assert_allclose(A.quantize_dequantize_keys(k, "oscar"), k_hat_rot @ H, rtol=0, atol=1e-12)


def test_no_rotation_no_scaling_is_plain_per_channel_int2():
    k = _keys()[:256]
    k_hat = A.quantize_dequantize_keys(k, "per_channel")
    for g in range(2):
        blk, hat = k[128 * g:128 * (g + 1)], k_hat[128 * g:128 * (g + 1)]
        # every channel of a group dequantizes onto at most 4 levels inside [min, max] (+ fp16 slack)
        for d in range(0, 128, 17):
            assert len(np.unique(hat[:, d])) <= 4
            span = blk[:, d].max() - blk[:, d].min()
            assert hat[:, d].min() >= blk[:, d].min() - 1e-3 * (1 + abs(blk[:, d].min()))
            assert hat[:, d].max() <= blk[:, d].max() + 1e-3 * (1 + span)


def test_scaling_fixes_the_sink_token():
    k = _keys()
    e_pc = A.key_errors(k, "per_channel")
    e_os = A.key_errors(k, "oscar")
    # token 0 is the sink (norm 0.05 x the median): without scaling its relative
    # error is many times its own norm, with scaling it is like every other token's
    assert e_pc[0] > 10 * e_os[0]
    assert e_os[0] < 2 * np.median(e_os)
    # the scaled variants keep the relative error flat across tokens
    assert np.percentile(e_os, 99) < 1.5 * np.mean(e_os)
    assert np.percentile(e_pc, 99) > 2 * np.mean(e_pc)


def test_attention_weights_distance_is_a_distance():
    k = _keys()
    q = syn.bf16_bits_to_f64(syn.query(syn.workload(0), 0))
    for var in A.VARIANTS:
        tv = A.attention_tv(q, k, var, 1 / np.sqrt(128))
        assert 0.0 <= tv <= 1.0
