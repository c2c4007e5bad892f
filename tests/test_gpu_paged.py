"""GPU parity of the paged cache layout (a block table over a pool of pages).

A cache whose groups live in shuffled pages of a larger pool must behave
exactly like the contiguous cache holding the same data: oscar_quantize_kv
writes the same block bytes (and no other page of the pool), and
oscar_decode_attn / oscar_decode_attn_append give the same outputs bit for
bit, which also match the CPU oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from tests.helpers import assert_out_close, bits_to_dev_bf16, upload_slice

pytestmark = pytest.mark.gpu

SM = 1.0 / np.sqrt(128.0)


def _say(msg):
    print(msg, flush=True)


def _pair(ob, w, dev, extra_pages=5, seed=0):
    """A contiguous cache and a paged one with a shuffled table (distinct
    pages, some pages of the pool never referenced)."""
    B, H = w.batch, w.num_kv_heads
    lens = [w.total_tokens(b) for b in range(B)]
    cap = max(128, max(((n + 127) // 128) * 128 for n in lens))
    gc = cap // 128
    pages = B * gc + extra_pages
    table = np.random.default_rng(seed).permutation(pages)[:B * gc].reshape(B, gc).astype(np.int32)
    contig = ob.PackedCache(B, H, cap, device=dev)
    paged = ob.PackedCache(B, H, cap, device=dev, num_pages=pages, block_table=torch.from_numpy(table))
    return contig, paged, table, lens


def _sources(w, dev, cap):
    B, H = w.batch, w.num_kv_heads
    k = np.zeros((B, H, cap, 128), np.uint16)
    v = np.zeros((B, H, cap, 128), np.uint16)
    for b in range(B):
        n = w.total_tokens(b)
        for h in range(H):
            k[b, h, :n] = syn.keys_slice(w, b, h)
            v[b, h, :n] = syn.values_slice(w, b, h)
    return bits_to_dev_bf16(k, dev), bits_to_dev_bf16(v, dev)


QUANT_CASES = {
    "cfg1_8k": lambda: syn.workload(1),
    "ragged_g4": lambda: syn.custom_workload(4, 8, 2, [0, 77, 128, 1000 + 5], cfg_tag=131),
    "g8": lambda: syn.custom_workload(2, 16, 2, [1, 4096 + 64], cfg_tag=132),
}


@pytest.mark.parametrize("case", list(QUANT_CASES))
def test_paged_quantize_writes_the_contiguous_bytes(gpu_lib, case):
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    w = QUANT_CASES[case]()
    _say(f"paged quantize {case}: B={w.batch} Hkv={w.num_kv_heads} lens={w.lengths}")
    contig, paged, table, lens = _pair(ob, w, dev)
    k, v = _sources(w, dev, contig.capacity)
    ngroups = [n // 128 for n in lens]
    start = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    num = torch.tensor(ngroups, dtype=torch.int32, device=dev)
    for c in (contig, paged):
        ob.quantize_kv(c, k, v, start, num, max(ngroups))
    torch.cuda.synchronize()
    got = paged.group_blocks().cpu().numpy()
    ref = contig.blocks.cpu().numpy()
    pool = paged.blocks.cpu().numpy()
    used = set()
    for b in range(w.batch):
        g = ngroups[b]
        assert np.array_equal(got[b, :, :g], ref[b, :, :g]), f"sequence {b}"
        used.update(int(p) for p in table[b, :g])
    untouched = [p for p in range(pool.shape[0]) if p not in used]
    assert not pool[untouched].any(), "the quantizer wrote a page no quantized group maps to"


DECODE_CASES = {
    "ragged_g4": lambda: syn.custom_workload(4, 8, 2, [0, 77, 128, 1000 + 5], cfg_tag=133),
    "g1_tail": lambda: syn.custom_workload(2, 3, 3, [300, 2048 + 127], cfg_tag=134),
    "g8_tail100": lambda: syn.custom_workload(1, 8, 1, [640 + 100], cfg_tag=135),
    "cfg1_8k": lambda: syn.workload(1),
}


@pytest.mark.parametrize("case", list(DECODE_CASES))
def test_paged_decode_equals_contiguous_and_oracle(gpu_lib, case):
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    w = DECODE_CASES[case]()
    B, H, Hq = w.batch, w.num_kv_heads, w.num_q_heads
    G = Hq // H
    _say(f"paged decode {case}: B={B} Hq={Hq} Hkv={H} lens={w.lengths}")
    contig, paged, table, lens = _pair(ob, w, dev, seed=1)
    nq = [syn.split_lengths(n)[0] for n in lens]
    ref = np.zeros((B, Hq, 128))
    q = np.stack([syn.query(w, b) for b in range(B)])
    for b in range(B):
        for h in range(H):
            s = oracle.quantize_slice(syn.bf16_bits_to_f64(syn.keys_slice(w, b, h)),
                                      syn.bf16_bits_to_f64(syn.values_slice(w, b, h)), nq[b])
            upload_slice(contig, b, h, s)
            ref[b, h * G:(h + 1) * G] = s.decode(syn.bf16_bits_to_f64(q[b, h * G:(h + 1) * G]), SM)
    # the same bytes, page by page, and the same tails
    for b in range(B):
        for g in range(contig.capacity // 128):
            paged.blocks[int(table[b, g])] = contig.blocks[b, :, g]
    paged.k_tail.copy_(contig.k_tail)
    paged.v_tail.copy_(contig.v_tail)
    mt = max(lens)
    qd = bits_to_dev_bf16(q, dev)
    nq_d = torch.tensor(nq, dtype=torch.int32, device=dev)
    nt_d = torch.tensor([n - m for n, m in zip(lens, nq)], dtype=torch.int32, device=dev)
    outs = []
    for c in (contig, paged):
        out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device=dev)
        ws = ob.alloc_workspace(B, H, Hq, mt, device=dev)
        ob.decode_attn(c, nq_d, nt_d, mt, qd, SM, out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]), "paged decode differs from the contiguous decode"
    err = assert_out_close(outs[1].cpu().numpy(), ref, case)
    _say(f"  bit-identical to the contiguous cache; max abs err vs oracle {err:.2e}")


def test_paged_decode_append_equals_contiguous(gpu_lib):
    """oscar_decode_attn_append on a paged cache: the same output and the
    same tail contents as on the contiguous cache, over 80 steps that cross
    a group boundary (the full tail is then quantized into its page)."""
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    w = syn.custom_workload(2, 8, 2, [1024 + 90, 384 + 10], cfg_tag=136, append_steps=80)
    B, H, Hq = w.batch, w.num_kv_heads, w.num_q_heads
    contig, paged, table, _ = _pair(ob, w, dev, seed=2)
    k, v = _sources(w, dev, contig.capacity)
    lens = list(w.lengths)
    nq = [syn.split_lengths(n)[0] for n in lens]
    start = torch.zeros(B, dtype=torch.int32, device=dev)
    num = torch.tensor([n // 128 for n in nq], dtype=torch.int32, device=dev)
    for c in (contig, paged):
        ob.quantize_kv(c, k, v, start, num, max(n // 128 for n in nq))
        for b in range(B):
            c.k_tail[b, :, :lens[b] - nq[b]] = k[b, :, nq[b]:lens[b]]
            c.v_tail[b, :, :lens[b] - nq[b]] = v[b, :, nq[b]:lens[b]]
    cap = contig.capacity
    ws = [ob.alloc_workspace(B, H, Hq, cap, device=dev) for _ in range(2)]
    for step in range(w.append_steps):
        tail = [lens[b] - nq[b] + 1 for b in range(B)]     # the appended token is the tail's last
        nq_d = torch.tensor(nq, dtype=torch.int32, device=dev)
        nt_d = torch.tensor(tail, dtype=torch.int32, device=dev)
        q = bits_to_dev_bf16(np.stack([syn.query(w, b, step) for b in range(B)]), dev)
        k_new = torch.stack([k[b, :, lens[b]] for b in range(B)]).contiguous()
        v_new = torch.stack([v[b, :, lens[b]] for b in range(B)]).contiguous()
        outs = []
        for c, wsi in zip((contig, paged), ws):
            out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
            ob.decode_attn_append(c, nq_d, nt_d, max(n + 1 for n in lens), q, k_new, v_new, 1.0 / np.sqrt(128.0),
                                  out, wsi)
            outs.append(out)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1]), f"step {step}"
        assert torch.equal(contig.k_tail, paged.k_tail) and torch.equal(contig.v_tail, paged.v_tail), f"step {step}"
        lens = [n + 1 for n in lens]
        full = [b for b in range(B) if lens[b] - nq[b] == 128]
        if full:   # quantize the completed tail group into its page
            st = torch.tensor([nq[b] // 128 if b in full else 0 for b in range(B)], dtype=torch.int32, device=dev)
            cnt = torch.tensor([1 if b in full else 0 for b in range(B)], dtype=torch.int32, device=dev)
            for c in (contig, paged):
                ob.quantize_kv(c, c.k_tail, c.v_tail, st, cnt, 1)
            for b in full:
                nq[b] += 128
    torch.cuda.synchronize()
    ng = [n // 128 for n in nq]
    got = paged.group_blocks().cpu().numpy()
    ref = contig.blocks.cpu().numpy()
    for b in range(B):
        assert np.array_equal(got[b, :, :ng[b]], ref[b, :, :ng[b]])
    _say(f"  80 append steps bit-identical; groups now {ng}")


def test_paged_128k_layer_equals_contiguous(gpu_lib):
    """The 128K-token Llama-3.1-8B layer (8 KV heads, 32 query heads) in the
    launch configuration the benchmark times: quantized straight into
    shuffled pages of a larger pool it gives the contiguous cache's bytes,
    and its decode output equals the contiguous decode bit for bit."""
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    w = syn.workload(3)
    B, H, Hq, T = w.batch, w.num_kv_heads, w.num_q_heads, w.lengths[0]
    _say(f"paged 128K layer: B={B} Hq={Hq} Hkv={H} T={T}")
    k = torch.stack([bits_to_dev_bf16(syn.keys_slice(w, 0, h), dev) for h in range(H)])[None]
    v = torch.stack([bits_to_dev_bf16(syn.values_slice(w, 0, h), dev) for h in range(H)])[None]
    gc = T // 128
    table = np.random.default_rng(7).permutation(gc + 64)[:gc].astype(np.int32)[None]
    contig = ob.PackedCache(B, H, T, device=dev)
    paged = ob.PackedCache(B, H, T, device=dev, num_pages=gc + 64, block_table=torch.from_numpy(table))
    zero = torch.zeros(B, dtype=torch.int32, device=dev)
    ng = torch.full((B,), gc, dtype=torch.int32, device=dev)
    for c in (contig, paged):
        ob.quantize_kv(c, k, v, zero, ng, gc)
    torch.cuda.synchronize()
    assert torch.equal(paged.group_blocks(), contig.blocks)
    q = bits_to_dev_bf16(syn.query(w, 0), dev)[None].contiguous()
    nq = torch.full((B,), T, dtype=torch.int32, device=dev)
    outs = []
    for c in (contig, paged):
        out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
        ob.decode_attn(c, nq, zero, T, q, SM, out, ob.alloc_workspace(B, H, Hq, T, device=dev))
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
