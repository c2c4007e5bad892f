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
    # the append inside the decode launch (the full tail is attended as bf16,
    # then quantized after the step)
    cb, outs_b = fresh(), []
    nq, nt = n_q0, tail0
    full_step = None
    for s in range(steps):
        nt += 1
        o = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
        k_new = k_dev[0, :, L0 + s][None].contiguous()
        v_new = v_dev[0, :, L0 + s][None].contiguous()
        ob.decode_attn_append(cb, i32(nq), i32(nt), nq + nt, bits_to_dev_bf16(syn.query(w, 0, s)[None], dev),
                              k_new, v_new, SM, o, ws)
        outs_b.append(o)
        if nt == 128:
            full_step = s
            ob.quantize_kv(cb, cb.k_tail, cb.v_tail, i32(nq // 128), i32(1), 1)
            nq, nt = nq + 128, 0
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
