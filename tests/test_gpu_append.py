"""oscar_decode_attn_append on the 32K group-append workload (32768
quantized tokens + a 57-token bf16 tail, 128 steps of one new token each),
through the C ABI: the step's own key and value go into the tail inside the
decode launch.  Against the same loop written with separate tail copies and
oscar_decode_attn: identical outputs at every step where the tail is not
full, identical cache bytes at the end; at the step that fills the tail (128
bf16 tokens, attended before the group is quantized) against the oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from tests.helpers import assert_out_close, bits_to_dev_bf16

pytestmark = pytest.mark.gpu

SM = 1.0 / np.sqrt(128.0)


def test_32k_append_inside_the_decode_launch(gpu_lib):
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    w = syn.workload(2)
    B, H, Hq = w.batch, w.num_kv_heads, w.num_q_heads
    G = Hq // H
    L0 = w.lengths[0]
    n_q0, tail0 = syn.split_lengths(L0)
    steps = w.append_steps
    cap = ((w.total_tokens(0) + 127) // 128) * 128
    print(f"append in the decode launch: {L0} tokens + {steps} steps", flush=True)
    k_bits = np.stack([syn.keys_slice(w, 0, h) for h in range(H)])[None]
    v_bits = np.stack([syn.values_slice(w, 0, h) for h in range(H)])[None]
    k_dev, v_dev = bits_to_dev_bf16(k_bits, dev), bits_to_dev_bf16(v_bits, dev)
    i32 = lambda x: torch.tensor([x], dtype=torch.int32, device=dev)   # noqa: E731

    def fresh():
        c = ob.PackedCache(B, H, cap, device=dev)
        ob.quantize_kv(c, k_dev, v_dev, i32(0), i32(n_q0 // 128), n_q0 // 128)
        c.k_tail[0, :, :tail0] = k_dev[0, :, n_q0:L0]
        c.v_tail[0, :, :tail0] = v_dev[0, :, n_q0:L0]
        return c

    ws = ob.alloc_workspace(B, H, Hq, cap, device=dev)
    # separate copies + oscar_decode_attn (the group is quantized before the
    # step that completes it attends)
    ca, outs_a = fresh(), []
    nq, nt = n_q0, tail0
    for s in range(steps):
        ca.k_tail[0, :, nt] = k_dev[0, :, L0 + s]
        ca.v_tail[0, :, nt] = v_dev[0, :, L0 + s]
        nt += 1
        if nt == 128:
            ob.quantize_kv(ca, ca.k_tail, ca.v_tail, i32(nq // 128), i32(1), 1)
            nq, nt = nq + 128, 0
        o = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
        ob.decode_attn(ca, i32(nq), i32(nt), nq + nt, bits_to_dev_bf16(syn.query(w, 0, s)[None], dev), SM, o, ws)
        outs_a.append(o)
    # the append inside the decode launch, driven by a DecodeSession (the full
    # tail is attended as bf16, then quantized after the step)
    from kv_cache_int2_fwht_amd.session import DecodeSession
    cb, outs_b = fresh(), []
    session = DecodeSession(cb, [n_q0], [tail0], Hq, steps, ws=ws)
    full_step = None
    for s in range(steps):
        o = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
        k_new = k_dev[0, :, L0 + s][None].contiguous()
        v_new = v_dev[0, :, L0 + s][None].contiguous()
        session.step(s, bits_to_dev_bf16(syn.query(w, 0, s)[None], dev), k_new, v_new, SM, o)
        outs_b.append(o)
        if session.plans[s].full[0]:
            full_step = s
    torch.cuda.synchronize()
    assert full_step == 128 - tail0 - 1
    for s in range(steps):
        if s != full_step:
            assert torch.equal(outs_a[s], outs_b[s]), f"step {s}"
    assert torch.equal(ca.blocks, cb.blocks)
    ntail = tail0 + steps - 128
    assert torch.equal(ca.k_tail[:, :, :ntail], cb.k_tail[:, :, :ntail])
    assert torch.equal(ca.v_tail[:, :, :ntail], cb.v_tail[:, :, :ntail])
    # the step with a full bf16 tail against the oracle
    got = outs_b[full_step][0].cpu().numpy()
    k64, v64 = syn.bf16_bits_to_f64(k_bits[0]), syn.bf16_bits_to_f64(v_bits[0])
    q = syn.query(w, 0, full_step)
    for h in range(H):
        pre = oracle.quantize_slice(k64[h, :n_q0], v64[h, :n_q0], n_q0)
        sl = dataclasses.replace(pre, k_tail=k64[h, n_q0:n_q0 + 128], v_tail=v64[h, n_q0:n_q0 + 128])
        ref = sl.decode(syn.bf16_bits_to_f64(q[h * G:(h + 1) * G]), SM)
        assert_out_close(got[h * G:(h + 1) * G], ref, f"full tail, head {h}")


@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("n_tail", [1, 64, 65, 127, 128])
def test_append_with_non_finite_rows_past_the_tail(gpu_lib, n_tail, G):
    """Tail rows past the appended token hold NaN (never written: the ABI does
    not ask the caller to initialise them).  Each tail wave reads masked
    tokens from a row of its own part, which at n_tail = 65 is the very row
    the other wave stores the new token into; none of it may reach the
    output.  Two sequences of 512 quantized tokens, two KV heads of G query
    heads each (G = 8: two row groups of the tail's matrix operand), against
    the oracle."""
    from kv_cache_int2_fwht_amd import binding as ob
    from tests.helpers import upload_slice
    dev = torch.device("cuda:0")
    Hkv = 2
    Hq = G * Hkv
    nq = 512
    w = syn.custom_workload(2, Hq, Hkv, [nq + n_tail, nq + n_tail], cfg_tag=120 + n_tail + (0 if G == 4 else 1000 * G))
    print(f"append with NaN past the tail: n_tail {n_tail}, G {G}", flush=True)
    cache = ob.PackedCache(2, Hkv, nq + 128, device=dev)
    refs, k_new, v_new = {}, [], []
    for b in range(2):
        kn, vn = [], []
        for h in range(Hkv):
            k64 = syn.bf16_bits_to_f64(syn.keys_slice(w, b, h))
            v64 = syn.bf16_bits_to_f64(syn.values_slice(w, b, h))
            s = oracle.quantize_slice(k64, v64, nq)
            refs[b, h] = s
            upload_slice(cache, b, h, dataclasses.replace(s, k_tail=s.k_tail[:n_tail - 1], v_tail=s.v_tail[:n_tail - 1]))
            kn.append(syn.keys_slice(w, b, h)[nq + n_tail - 1])
            vn.append(syn.values_slice(w, b, h)[nq + n_tail - 1])
        k_new.append(np.stack(kn))
        v_new.append(np.stack(vn))
    nan = torch.tensor(float("nan"), dtype=torch.bfloat16, device=dev)
    cache.k_tail[:, :, n_tail - 1:] = nan
    cache.v_tail[:, :, n_tail - 1:] = nan
    i32 = lambda x: torch.tensor(x, dtype=torch.int32, device=dev)   # noqa: E731
    q_bits = np.stack([syn.query(w, b) for b in range(2)])
    out = torch.empty((2, Hq, 128), dtype=torch.float32, device=dev)
    ws = ob.alloc_workspace(2, Hkv, Hq, nq + 128, device=dev)
    ob.decode_attn_append(cache, i32([nq, nq]), i32([n_tail, n_tail]), nq + n_tail,
                          bits_to_dev_bf16(q_bits, dev), bits_to_dev_bf16(np.stack(k_new), dev),
                          bits_to_dev_bf16(np.stack(v_new), dev), SM, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    for b in range(2):
        for h in range(Hkv):
            ref = refs[b, h].decode(syn.bf16_bits_to_f64(q_bits[b, h * G:(h + 1) * G]), SM)
            assert_out_close(got[b, h * G:(h + 1) * G], ref, f"n_tail {n_tail}, G {G}, sequence {b}, head {h}")
    # the stored tail rows are exactly the appended tokens
    np.testing.assert_array_equal(cache.k_tail[:, :, n_tail - 1].view(torch.int16).cpu().numpy().view(np.uint16),
                                  np.stack(k_new))


@pytest.mark.parametrize("n_tail", [1, 65])
def test_decode_with_non_finite_rows_past_the_tail(gpu_lib, n_tail):
    """oscar_decode_attn with NaN in every tail row at or past n_tail."""
    from kv_cache_int2_fwht_amd import binding as ob
    from tests.helpers import upload_slice
    dev = torch.device("cuda:0")
    Hkv, Hq, nq = 1, 4, 256
    w = syn.custom_workload(1, Hq, Hkv, [nq + n_tail], cfg_tag=140 + n_tail)
    print(f"decode with NaN past the tail: n_tail {n_tail}", flush=True)
    k64 = syn.bf16_bits_to_f64(syn.keys_slice(w, 0, 0))
    v64 = syn.bf16_bits_to_f64(syn.values_slice(w, 0, 0))
    s = oracle.quantize_slice(k64, v64, nq)
    cache = ob.PackedCache(1, Hkv, nq + 128, device=dev)
    upload_slice(cache, 0, 0, s)
    nan = torch.tensor(float("nan"), dtype=torch.bfloat16, device=dev)
    cache.k_tail[:, :, n_tail:] = nan
    cache.v_tail[:, :, n_tail:] = nan
    i32 = lambda x: torch.tensor([x], dtype=torch.int32, device=dev)   # noqa: E731
    q_bits = syn.query(w, 0)
    out = torch.empty((1, Hq, 128), dtype=torch.float32, device=dev)
    ws = ob.alloc_workspace(1, Hkv, Hq, nq + 128, device=dev)
    ob.decode_attn(cache, i32(nq), i32(n_tail), nq + n_tail, bits_to_dev_bf16(q_bits[None], dev), SM, out, ws)
    torch.cuda.synchronize()
    got = out[0].cpu().numpy()
    assert np.isfinite(got).all()
    assert_out_close(got, s.decode(syn.bf16_bits_to_f64(q_bits), SM), f"n_tail {n_tail}")
