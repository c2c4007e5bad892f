"""GPU parity on the full-size workloads, through the C ABI, in the launch
configuration the benchmark uses:

* 32K context + 57-token bf16 tail, then 128 decode steps that append one
  token each; the tail fills after 71 steps and its group is quantized by
  oscar_quantize_kv (group append);
* 128K context, batch 1 (the benchmark workload): prefill quantize and one
  decode step, checked on sampled KV heads;
* batch 8 with jittered 96K-128K lengths: checked on sampled (sequence,
  KV head) slices.

Sampling keeps the float64 oracle to seconds: each sampled slice is
quantized and decoded by the oracle in full, and compared with the GPU's
bytes (bit for bit) and outputs (1e-3 + 1e-3|ref|).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from tests.helpers import assert_out_close, bits_to_dev_bf16, check_quantized_slice, token_rows

pytestmark = pytest.mark.gpu

SM = 1.0 / np.sqrt(128.0)


def _say(msg):
    print(msg, flush=True)


def _dev_bf16(bits):
    return bits_to_dev_bf16(bits, torch.device("cuda:0"))


def _i32(vals):
    return torch.tensor(vals, dtype=torch.int32, device="cuda:0")


def _assert_bytes_equal(cache, b, h, ref, g0=0):
    """The GPU's packed bytes of slice (b, h) from group g0 on equal the oracle's."""
    ng = ref.n_quant // 128
    assert np.array_equal(token_rows(cache.k_codes, b, h, g0, ng), ref.k_codes)
    assert np.array_equal(token_rows(cache.k_norm, b, h, g0, ng).view(np.uint16), ref.k_norm)
    assert np.array_equal(token_rows(cache.v_sz, b, h, g0, ng).view(np.uint16), ref.v_sz)
    assert np.array_equal(cache.k_sz[b, h, g0:g0 + ng].cpu().numpy().view(np.uint16), ref.k_sz)
    assert np.array_equal(cache.v_codes[b, h, g0:g0 + ng].cpu().numpy(), ref.v_codes)


def test_32k_group_append_over_128_steps(gpu_lib):
    from kv_cache_int2_fwht_amd import binding as ob
    w = syn.workload(2)
    B, H, Hq = w.batch, w.num_kv_heads, w.num_q_heads
    G = Hq // H
    L0 = w.lengths[0]                      # 32768 + 57 tokens before the first step
    n_q0, tail0 = syn.split_lengths(L0)    # 32768, 57
    steps = w.append_steps
    total = w.total_tokens(0)
    cap = ((total + 127) // 128) * 128
    _say(f"32K append: prefix {L0}, steps {steps}, capacity {cap}")
    k_bits = np.stack([syn.keys_slice(w, 0, h) for h in range(H)])[None]      # [1, H, total, 128]
    v_bits = np.stack([syn.values_slice(w, 0, h) for h in range(H)])[None]
    k_dev, v_dev = _dev_bf16(k_bits), _dev_bf16(v_bits)

    cache = ob.PackedCache(B, H, cap)
    ob.quantize_kv(cache, k_dev, v_dev, _i32([0]), _i32([n_q0 // 128]), n_q0 // 128)
    cache.k_tail[0, :, :tail0] = k_dev[0, :, n_q0:L0]
    cache.v_tail[0, :, :tail0] = v_dev[0, :, n_q0:L0]
    ws = ob.alloc_workspace(B, H, Hq, cap)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda:0")

    check = {0: None, 1: None, 69: None, 70: None, 71: None, steps - 1: None}
    n_quant, n_tail = n_q0, tail0
    appended_at = None
    for s in range(steps):
        t = L0 + s                             # the token this step appends
        cache.k_tail[0, :, n_tail] = k_dev[0, :, t]
        cache.v_tail[0, :, n_tail] = v_dev[0, :, t]
        n_tail += 1
        if n_tail == 128:                      # the tail group is complete: quantize it
            ob.quantize_kv(cache, cache.k_tail, cache.v_tail, _i32([n_quant // 128]), _i32([1]), 1)
            n_quant += 128
            n_tail = 0
            appended_at = s
        q = syn.query(w, 0, s)[None]
        ob.decode_attn(cache, _i32([n_quant]), _i32([n_tail]), n_quant + n_tail, _dev_bf16(q), SM, out, ws)
        if s in check:
            torch.cuda.synchronize()
            check[s] = (out.cpu().numpy().copy(), q, n_quant, n_tail)
    torch.cuda.synchronize()
    assert appended_at == 128 - tail0 - 1

    k64 = syn.bf16_bits_to_f64(k_bits[0])
    v64 = syn.bf16_bits_to_f64(v_bits[0])
    g_app = n_q0 // 128
    for h in range(H):
        # prefill groups and the appended group: packed bytes equal the oracle's
        pre = oracle.quantize_slice(k64[h, :n_q0], v64[h, :n_q0], n_q0)
        _assert_bytes_equal(cache, 0, h, pre)
        app = oracle.quantize_slice(k64[h, n_q0:n_q0 + 128], v64[h, n_q0:n_q0 + 128], 128,
                                    keep_intermediates=True)
        rep = check_quantized_slice(cache, 0, h, app, g0=g_app, ng=1)
        assert rep["key_bytes_equal"] and rep["value_bytes_equal"], rep
        full = oracle.quantize_slice(k64[h, :n_q0 + 128], v64[h, :n_q0 + 128], n_q0 + 128)
        for s, (got, q, nq, nt) in check.items():
            L = nq + nt
            base = pre if nq == n_q0 else full
            sl = dataclasses.replace(base, k_tail=k64[h, nq:L], v_tail=v64[h, nq:L])
            ref = sl.decode(syn.bf16_bits_to_f64(q[0, h * G:(h + 1) * G]), SM)
            assert_out_close(got[0, h * G:(h + 1) * G], ref, f"step {s} head {h}")
    _say(f"  group appended at step {appended_at}; steps {sorted(check)} match the oracle")


def test_128k_prefill_and_decode_all_heads(gpu_lib):
    """The benchmark workload at full size: all 8 KV heads quantized and
    decoded on the GPU and checked against the oracle (all 1024 groups of
    every head bit for bit, and all 32 query heads' outputs)."""
    from kv_cache_int2_fwht_amd import binding as ob
    w = syn.workload(3)
    B, H, Hq, T = w.batch, w.num_kv_heads, w.num_q_heads, w.lengths[0]
    G = Hq // H
    sample = tuple(range(H))
    _say(f"128K: B={B} Hq={Hq} Hkv={H} T={T}, oracle on KV heads {sample}")
    k_dev = torch.empty((B, H, T, 128), dtype=torch.bfloat16, device="cuda:0")
    v_dev = torch.empty_like(k_dev)
    bits = {}
    for h in range(H):
        kb, vb = syn.keys_slice(w, 0, h), syn.values_slice(w, 0, h)
        k_dev[0, h] = _dev_bf16(kb)
        v_dev[0, h] = _dev_bf16(vb)
        if h in sample:
            bits[h] = (kb, vb)
    cache = ob.PackedCache(B, H, T)
    ob.quantize_kv(cache, k_dev, v_dev, _i32([0]), _i32([T // 128]), T // 128)
    q = syn.query(w, 0)[None]
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda:0")
    ws = ob.alloc_workspace(B, H, Hq, T)
    ob.decode_attn(cache, _i32([T]), _i32([0]), T, _dev_bf16(q), SM, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for h in sample:
        kb, vb = bits[h]
        ref_slice = oracle.quantize_slice(syn.bf16_bits_to_f64(kb), syn.bf16_bits_to_f64(vb), T)
        _assert_bytes_equal(cache, 0, h, ref_slice)
        ref = ref_slice.decode(syn.bf16_bits_to_f64(q[0, h * G:(h + 1) * G]), SM)
        assert_out_close(got[0, h * G:(h + 1) * G], ref, f"128K head {h}")
    _say("  every head: bytes identical, outputs within tolerance")


def test_batch8_jittered_lengths_one_slice_per_sequence(gpu_lib):
    """Batch 8, lengths uniform in [98304, 131072] (quantized groups plus a
    bf16 tail), two outlier regimes.  One slice of every sequence, KV head
    (3 b + 1) mod 8 of sequence b, carries its generated data and is checked
    against the oracle; the sequence's other heads hold copies of it, so the
    grid, lengths and traffic are those of the full workload."""
    from kv_cache_int2_fwht_amd import binding as ob
    w = syn.workload(4)
    B, H, Hq = w.batch, w.num_kv_heads, w.num_q_heads
    G = Hq // H
    lens = [w.total_tokens(b) for b in range(B)]
    nqs = [syn.split_lengths(n)[0] for n in lens]
    cap = max(((n + 127) // 128) * 128 for n in lens)
    sample = [(b, (3 * b + 1) % H) for b in range(B)]
    _say(f"batch 8: lengths {lens}, sampled slices {sample}")
    cache = ob.PackedCache(B, H, cap)
    gen, gen_dev = {}, {}
    for b, h in sample:
        gen[b, h] = (syn.keys_slice(w, b, h), syn.values_slice(w, b, h))
        gen_dev[b, h] = (_dev_bf16(gen[b, h][0]), _dev_bf16(gen[b, h][1]))
    # per sequence: a bf16 source [1, H, cap, 128] whose heads all hold the
    # sequence's generated slice
    for b in range(B):
        k_dev = torch.zeros((1, H, cap, 128), dtype=torch.bfloat16, device="cuda:0")
        v_dev = torch.zeros_like(k_dev)
        for h in range(H):
            kd, vd = gen_dev[sample[b]]
            n = min(lens[b], kd.shape[0])
            k_dev[0, h, :n] = kd[:n]
            v_dev[0, h, :n] = vd[:n]
        sub = ob.PackedCache(1, H, cap)
        ob.quantize_kv(sub, k_dev, v_dev, _i32([0]), _i32([nqs[b] // 128]), nqs[b] // 128)
        cache.blocks[b].copy_(sub.blocks[0])
        nt = lens[b] - nqs[b]
        cache.k_tail[b, :, :nt] = k_dev[0, :, nqs[b]:lens[b]]
        cache.v_tail[b, :, :nt] = v_dev[0, :, nqs[b]:lens[b]]
        del sub, k_dev, v_dev
    q = np.stack([syn.query(w, b) for b in range(B)])
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda:0")
    mt = max(lens)
    ws = ob.alloc_workspace(B, H, Hq, mt)
    ob.decode_attn(cache, _i32(nqs), _i32([n - m for n, m in zip(lens, nqs)]), mt, _dev_bf16(q), SM, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b, h in sample:
        kb, vb = gen[b, h]
        ref_slice = oracle.quantize_slice(syn.bf16_bits_to_f64(kb), syn.bf16_bits_to_f64(vb), nqs[b])
        _assert_bytes_equal(cache, b, h, ref_slice)
        ref = ref_slice.decode(syn.bf16_bits_to_f64(q[b, h * G:(h + 1) * G]), SM)
        assert_out_close(got[b, h * G:(h + 1) * G], ref, f"batch8 slice ({b}, {h})")
    _say("  sampled slices: bytes identical, outputs within tolerance")
