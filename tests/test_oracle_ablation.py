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


FLAGS = {"per_channel": (False, False), "rotation": (True, False), "scaling": (False, True), "oscar": (True, True)}


def test_quantizer_variants_closed_forms():
    """quantize_keys(rotate, scale): u is k itself, k / fp16(||k||), H k, or
    H k / fp16(||H k||); the stored norm is 1 whenever the scaling is off."""
    k = _keys()[:256]
    H = hadamard(128)
    for var, (rot, sc) in FLAGS.items():
        kq = oracle.quantize_keys(k, rotate=rot, scale=sc)
        y = k @ H.T if rot else k
        if sc:
            n16 = oracle.fp16_rne(np.linalg.norm(y, axis=1))
            np.testing.assert_allclose(kq["n16"], n16, rtol=0, atol=0)
            np.testing.assert_allclose(kq["u"], y / n16[:, None], rtol=1e-15, atol=0)
        else:
            assert np.all(kq["n16"] == 1.0) and np.all(kq["n"] == 1.0)
            np.testing.assert_array_equal(kq["u"], y)
        # min / max per group and channel land on levels 0 and 3
        codes = kq["codes"].reshape(2, 128, 128)
        assert codes.min() == 0 and codes.max() == 3


def test_variant_slices_decode_like_attention_over_their_dequantized_keys():
    """OracleSlice.decode of every variant equals plain attention (no
    Hadamard anywhere) of q over the variant's dequantized keys in k's basis
    and the dequantized values."""
    w = syn.workload(0)
    k = _keys()
    v = syn.bf16_bits_to_f64(syn.values_slice(w, 0, 0))
    q = syn.bf16_bits_to_f64(syn.query(w, 0))
    sm = 1 / np.sqrt(128)
    vq = oracle.quantize_values(v)
    v_hat = oracle.dequant_values(vq["codes"], vq["vs16"], vq["vz16"])
    for var, (rot, sc) in FLAGS.items():
        s = oracle.quantize_slice(k, v, k.shape[0], rotate=rot, scale=sc)
        ref = oracle.decode_bf16_slice(q, A.quantize_dequantize_keys(k, var), v_hat, sm)
        np.testing.assert_allclose(s.decode(q, sm), ref, rtol=0, atol=1e-12)
