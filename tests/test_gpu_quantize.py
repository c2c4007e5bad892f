"""GPU parity of oscar_quantize_kv against the CPU oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from tests.helpers import bits_to_dev_bf16, check_quantized_slice

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _quantize_workload_on_gpu(ob, w, n_quant_per_b, capacity, dev):
    """Generate every slice, stack into [B, H, T, 128] bf16 and quantize the
    first n_quant_per_b[b] tokens of each sequence in one call."""
    B, H = w.batch, w.num_kv_heads
    T = max(w.total_tokens(b) for b in range(B))
    k = np.zeros((B, H, T, 128), np.uint16)
    v = np.zeros((B, H, T, 128), np.uint16)
    for b in range(B):
        for h in range(H):
            n = w.total_tokens(b)
            k[b, h, :n] = syn.keys_slice(w, b, h)
            v[b, h, :n] = syn.values_slice(w, b, h)
    cache = ob.PackedCache(B, H, capacity, device=dev)
    kd, vd = bits_to_dev_bf16(k, dev), bits_to_dev_bf16(v, dev)
    starts = torch.zeros(B, dtype=torch.int32, device=dev)
    ng = torch.tensor([n // 128 for n in n_quant_per_b], dtype=torch.int32, device=dev)
    ob.quantize_kv(cache, kd, vd, starts, ng, max(n_quant_per_b) // 128)
    torch.cuda.synchronize()
    return cache, k, v


@pytest.mark.parametrize("cfg", [0, 1])
def test_quantize_matches_oracle(gpu_lib, cfg):
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    w = syn.workload(cfg)
    nq = [syn.split_lengths(w.lengths[b])[0] for b in range(w.batch)]
    _say(f"quantize cfg {cfg}: B={w.batch} H={w.num_kv_heads} n_quant={nq}")
    cache, k, v = _quantize_workload_on_gpu(ob, w, nq, max(nq), dev)
    exact = 0
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            ref = oracle.quantize_slice(syn.bf16_bits_to_f64(k[b, h]), syn.bf16_bits_to_f64(v[b, h]), nq[b],
                                        keep_intermediates=True)
            rep = check_quantized_slice(cache, b, h, ref)
            exact += all(rep[key] for key in rep if key.endswith("equal"))
    _say(f"slices bit-identical to the oracle: {exact} of {w.batch * w.num_kv_heads}")
    # the codes are decided in fp64 like the oracle's, with the correctly
    # rounded quotient near a half-way point: every slice is bit-identical
    assert exact == w.batch * w.num_kv_heads


def test_quantize_strided_offsets_and_ragged_groups(gpu_lib):
    """Token-major source layout [B, T, H, 128] (non-contiguous view),
    per-sequence destination offsets, ragged group counts including 0; groups
    that are not written keep their previous contents."""
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    w = syn.custom_workload(3, 6, 3, [512, 384, 256], cfg_tag=101)
    ngroups = [3, 0, 2]
    starts = [1, 0, 5]
    capacity = 1024
    B, H = w.batch, w.num_kv_heads
    T = 512
    k = np.zeros((B, T, H, 128), np.uint16)
    v = np.zeros((B, T, H, 128), np.uint16)
    for b in range(B):
        for h in range(H):
            n = w.total_tokens(b)
            k[b, :n, h] = syn.keys_slice(w, b, h)
            v[b, :n, h] = syn.values_slice(w, b, h)
    kd = bits_to_dev_bf16(k, dev).permute(0, 2, 1, 3)   # [B, H, T, 128] view, strides (T*H*128, 128, H*128, 1)
    vd = bits_to_dev_bf16(v, dev).permute(0, 2, 1, 3)
    cache = ob.PackedCache(B, H, capacity, device=dev)
    for t in (cache.k_codes, cache.v_codes):
        t.fill_(0xA5)
    cache.k_norm.fill_(0x1234)
    _say("quantize strided: ragged groups [3, 0, 2], starts [1, 0, 5]")
    ob.quantize_kv(cache, kd, vd, torch.tensor(starts, dtype=torch.int32, device=dev),
                   torch.tensor(ngroups, dtype=torch.int32, device=dev), 4)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            n = ngroups[b] * 128
            if n:
                ref = oracle.quantize_slice(syn.bf16_bits_to_f64(k[b, :n, h]), syn.bf16_bits_to_f64(v[b, :n, h]), n,
                                            keep_intermediates=True)
                check_quantized_slice(cache, b, h, ref, g0=starts[b], ng=ngroups[b])
            written = set(range(starts[b], starts[b] + ngroups[b]))
            for g in range(capacity // 128):
                if g not in written:
                    assert int(cache.k_codes[b, h, g].eq(0xA5).all()) == 1
                    assert int(cache.v_codes[b, h, g].eq(0xA5).all()) == 1
                    assert int(cache.k_norm[b, h, g].eq(0x1234).all()) == 1


def test_quantize_degenerate_inputs(gpu_lib):
    """Constant groups (scale 0), zero tokens (norm 0), very large values
    (saturating fp16 norm) and mixed magnitudes."""
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(77)
    k = rng.standard_normal((4 * 128, 128)).astype(np.float32)
    v = rng.standard_normal((4 * 128, 128)).astype(np.float32)
    k[0:128] = np.linspace(-2, 2, 128, dtype=np.float32)[None]   # identical tokens: scale 0
    k[130] = 0.0                                                  # zero token: norm 0
    k[200] = 30000.0                                              # norm far above 65504: saturates
    k[256:384] *= np.exp(rng.normal(0, 4, (128, 1))).astype(np.float32)   # wide magnitude spread
    v[0:128] = 0.25                                               # constant value tokens
    v[300] = 1e-30
    kb = syn.f32_to_bf16_bits(k)
    vb = syn.f32_to_bf16_bits(v)
    cache = ob.PackedCache(1, 1, 512, device=dev)
    _say("quantize degenerate inputs")
    ob.quantize_kv(cache, bits_to_dev_bf16(kb, dev)[None, None], bits_to_dev_bf16(vb, dev)[None, None],
                   torch.zeros(1, dtype=torch.int32, device=dev), torch.full((1,), 4, dtype=torch.int32, device=dev), 4)
    torch.cuda.synchronize()
    ref = oracle.quantize_slice(syn.bf16_bits_to_f64(kb), syn.bf16_bits_to_f64(vb), 512, keep_intermediates=True)
    check_quantized_slice(cache, 0, 0, ref)
    assert int(cache.k_norm[0, 0, 1, 72].item()) & 0xFFFF == 0x7BFF   # saturated at 65504
    assert int(cache.k_norm[0, 0, 1, 2].item()) == 0


def test_quantize_is_deterministic(gpu_lib):
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    w = syn.workload(0)
    cache_a, k, v = _quantize_workload_on_gpu(ob, w, [1024], 1024, dev)
    cache_b, _, _ = _quantize_workload_on_gpu(ob, w, [1024], 1024, dev)
    assert torch.equal(cache_a.blocks, cache_b.blocks)


def test_quantize_exact_half_way_values(gpu_lib):
    """Values and keys exactly half-way between two code levels, where the
    quantizer decides the code from the correctly rounded quotient instead
    of the reciprocal product: every value token and every key channel holds
    levels 0 and 3 (z = 0, s an exact power of two) and otherwise levels
    from {0, 0.5, 1, ..., 3} times that power, so (x - z) / s lands exactly
    on 0.5, 1.5 and 2.5 (round half to even: codes 0, 2, 2).  Keys are
    quantized without rotation and scaling, the variant in which the codes
    see the keys as given; the bytes must equal the oracle's bit for bit."""
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(4242)
    T = 256
    levels = np.arange(7, dtype=np.float64) / 2.0               # 0, 0.5, ..., 3
    lk = levels[rng.integers(0, 7, (T, 128))]
    lv = levels[rng.integers(0, 7, (T, 128))]
    for g in range(T // 128):                                    # per key group: each channel spans 0..3
        lk[128 * g] = 0.0
        lk[128 * g + 1] = 3.0
    lv[:, 0] = 0.0                                               # per value token: 0..3
    lv[:, 1] = 3.0
    k = lk * np.exp2(rng.integers(-6, 4, (1, 128)))               # per-channel power of two
    v = lv * np.exp2(rng.integers(-6, 4, (T, 1)))                 # per-token power of two
    assert np.isin(lk, [0.5, 1.5, 2.5]).sum() > 1000 and np.isin(lv, [0.5, 1.5, 2.5]).sum() > 1000
    kb, vb = syn.f32_to_bf16_bits(k.astype(np.float32)), syn.f32_to_bf16_bits(v.astype(np.float32))
    assert np.array_equal(syn.bf16_bits_to_f64(kb), k) and np.array_equal(syn.bf16_bits_to_f64(vb), v)
    flags = ob.KEYS_UNROTATED | ob.KEYS_UNSCALED
    cache = ob.PackedCache(1, 1, T, device=dev, flags=flags)
    _say("quantize exact half-way values (keys unrotated and unscaled)")
    ob.quantize_kv(cache, bits_to_dev_bf16(kb, dev)[None, None], bits_to_dev_bf16(vb, dev)[None, None],
                   torch.zeros(1, dtype=torch.int32, device=dev), torch.full((1,), T // 128, dtype=torch.int32,
                                                                             device=dev), T // 128)
    torch.cuda.synchronize()
    ref = oracle.quantize_slice(syn.bf16_bits_to_f64(kb), syn.bf16_bits_to_f64(vb), T, keep_intermediates=True,
                                rotate=False, scale=False)
    rep = check_quantized_slice(cache, 0, 0, ref)
    assert rep["key_code_mismatch"] == 0 and rep["value_code_mismatch"] == 0, rep
    assert all(rep[key] for key in rep if key.endswith("equal")), rep
