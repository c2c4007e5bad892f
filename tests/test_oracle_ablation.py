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


def test_tv_distance_hand_worked():
    """1/2 sum |p - p_hat| on small weight vectors worked by hand."""
    assert A.tv_distance([[0.5, 0.5]], [[1.0, 0.0]])[0] == 0.5
    np.testing.assert_allclose(A.tv_distance([[0.2, 0.3, 0.5]], [[0.5, 0.3, 0.2]]), [0.3], rtol=0, atol=1e-15)
    # identical weights: 0; weights on disjoint tokens: 1; one value per row
    np.testing.assert_array_equal(A.tv_distance([[0.25, 0.75], [1.0, 0.0]], [[0.25, 0.75], [0.0, 1.0]]), [0.0, 1.0])


def test_softmax_weights_hand_worked():
    # logits (0, ln 3): weights 1/4 and 3/4, whatever constant is added
    np.testing.assert_allclose(A.softmax_weights([[0.0, np.log(3.0)], [7.0, 7.0 + np.log(3.0)]]),
                               [[0.25, 0.75], [0.25, 0.75]], rtol=0, atol=1e-15)


def test_rel_output_error_uses_the_reference_norm():
    # out - ref = (0, 4): 4 / ||ref|| = 4 / 3 (dividing by ||out|| = 5 would give 0.8)
    np.testing.assert_allclose(A.rel_output_error([[3.0, 4.0]], [[3.0, 0.0]]), [4.0 / 3.0], rtol=0, atol=1e-15)


def _ladder_keys(moved=1.25):
    """128 tokens; channel 0 of token t holds t mod 4 (the INT2 levels of s = 1,
    z = 0), except token 5, which holds `moved`; every other channel is 0.
    Per-channel INT2 keeps every key but token 5, whose channel 0 becomes
    round(moved)."""
    k = np.zeros((128, 128))
    k[:, 0] = np.arange(128) % 4
    k[5, 0] = moved
    return k


def test_attention_tv_closed_form_one_token_moved():
    """Only token 5's logit changes (x -> x_hat), so the TV distance is
    |p_5 - p_hat_5| with p_5 = e^x / (R + e^x), R the sum over the other
    tokens: 32 (1 + e^c + e^2c + e^3c) - e^c for logits c k_t0."""
    k = _ladder_keys(1.25)
    np.testing.assert_array_equal(A.quantize_dequantize_keys(k, "per_channel")[5, 0], 1.0)
    a, sm = 2.0, 0.375
    q = np.zeros((1, 128))
    q[0, 0] = a
    c = a * sm
    rest = 32 * (1 + np.exp(c) + np.exp(2 * c) + np.exp(3 * c)) - np.exp(c)
    p5 = np.exp(1.25 * c) / (rest + np.exp(1.25 * c))
    p5_hat = np.exp(c) / (rest + np.exp(c))
    np.testing.assert_allclose(A.attention_tv(q, k, "per_channel", sm), abs(p5 - p5_hat), rtol=1e-12, atol=0)
    # keys on the levels exactly: the weights do not move
    assert A.attention_tv(q, _ladder_keys(1.0), "per_channel", sm) == 0.0


def test_attention_tv_is_the_max_over_heads():
    k = _ladder_keys(1.25)
    q = np.zeros((3, 128))
    q[1, 0] = 2.0     # head 1 sees token 5 move; heads 0 and 2 (q = 0, q on channel 1) do not
    q[2, 1] = 5.0
    sm = 0.375
    c = 0.75
    rest = 32 * (1 + np.exp(c) + np.exp(2 * c) + np.exp(3 * c)) - np.exp(c)
    expect = abs(np.exp(1.25 * c) / (rest + np.exp(1.25 * c)) - np.exp(c) / (rest + np.exp(c)))
    np.testing.assert_allclose(A.attention_tv(q, k, "per_channel", sm), expect, rtol=1e-12, atol=0)


def test_output_error_closed_form():
    """Zero keys quantize to zero in every variant (s = 0, or n = 0), so the
    weights are uniform and out is the mean value.  Every token holds
    v = (0, 1, 2, 3, 1.4, 0, ...): per-token INT2 has s = 1, z = 0 and maps
    1.4 to 1, so the error is 0.4 / ||v|| = 0.4 / sqrt(15.96)."""
    k = np.zeros((128, 128))
    v = np.zeros((128, 128))
    v[:, :5] = [0.0, 1.0, 2.0, 3.0, 1.4]
    q = syn.bf16_bits_to_f64(syn.query(syn.workload(0), 0))
    for var in A.VARIANTS:
        np.testing.assert_array_equal(A.quantize_dequantize_keys(k, var), 0.0)
        np.testing.assert_allclose(A.output_error(q, k, v, var, 1 / np.sqrt(128)), 0.4 / np.sqrt(15.96),
                                   rtol=1e-12, atol=0)
        v_exact = v.copy()
        v_exact[:, 4] = 1.0
        assert A.output_error(q, k, v_exact, var, 1 / np.sqrt(128)) == 0.0


def test_study_rows_on_a_tiny_workload():
    """study() averages, per variant, the pinned per-head metrics over the
    KV heads, each head with its own G query heads."""
    w = syn.custom_workload(1, 4, 2, [256 + 17], cfg_tag=77)
    sm = 1 / np.sqrt(128)
    res = A.study(w, heads=(0, 1), sm_scale=sm)
    assert set(res) == set(A.VARIANTS)
    per_head = {v: [] for v in A.VARIANTS}
    for h in (0, 1):
        k = syn.bf16_bits_to_f64(syn.keys_slice(w, 0, h))[:256]
        val = syn.bf16_bits_to_f64(syn.values_slice(w, 0, h))[:256]
        q = syn.bf16_bits_to_f64(syn.query(w, 0))[2 * h:2 * h + 2]
        for var in A.VARIANTS:
            e = A.key_errors(k, var)
            per_head[var].append((e.mean(), e[0], np.percentile(e, 99), A.attention_tv(q, k, var, sm),
                                  A.output_error(q, k, val, var, sm)))
    names = ("key_err_mean", "key_err_sink", "key_err_p99", "attn_tv", "out_err")
    for var in A.VARIANTS:
        assert set(res[var]) == set(names)
        mean = np.mean(np.array(per_head[var]), axis=0)
        for i, name in enumerate(names):
            assert np.isfinite(res[var][name])
            np.testing.assert_allclose(res[var][name], mean[i], rtol=1e-14, atol=0)
    # the two heads differ, so a study over one head is not the mean over two
    assert A.study(w, heads=(1,), sm_scale=sm)["oscar"]["attn_tv"] != res["oscar"]["attn_tv"]


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
