"""GPU parity of oscar_decode_attn (on the oracle's packed bytes) and of
oscar_decode_attn_bf16 against the CPU oracle, through the C ABI."""
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


def _build(ob, w, dev, capacity=None):
    """Oracle slices of every (b, h), uploaded into a PackedCache, plus the
    raw bf16 K/V (for the bf16 kernel) and the queries."""
    B, H, Hq = w.batch, w.num_kv_heads, w.num_q_heads
    lens = [w.total_tokens(b) for b in range(B)]
    nq = [syn.split_lengths(n)[0] for n in lens]
    cap = capacity or max(128, max(((n + 127) // 128) * 128 for n in lens))
    cache = ob.PackedCache(B, H, cap, device=dev)
    kraw = np.zeros((B, H, cap, 128), np.uint16)
    vraw = np.zeros((B, H, cap, 128), np.uint16)
    slices = {}
    for b in range(B):
        for h in range(H):
            kb, vb = syn.keys_slice(w, b, h), syn.values_slice(w, b, h)
            kraw[b, h, :lens[b]] = kb
            vraw[b, h, :lens[b]] = vb
            s = oracle.quantize_slice(syn.bf16_bits_to_f64(kb), syn.bf16_bits_to_f64(vb), nq[b])
            upload_slice(cache, b, h, s)
            slices[b, h] = s
    q = np.stack([syn.query(w, b) for b in range(B)])
    return cache, slices, kraw, vraw, q, lens, nq


def _oracle_out(w, slices, q, lens, sm=SM):
    G = w.num_q_heads // w.num_kv_heads
    out = np.zeros((w.batch, w.num_q_heads, 128))
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            qq = syn.bf16_bits_to_f64(q[b, h * G:(h + 1) * G])
            out[b, h * G:(h + 1) * G] = slices[b, h].decode(qq, sm)
    return out


def _run_int2(ob, cache, q, lens, nq, dev, max_tokens=None, sm=SM):
    B, Hq = q.shape[0], q.shape[1]
    mt = max(lens) if max_tokens is None else max_tokens
    qd = bits_to_dev_bf16(q, dev)
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device=dev)
    ws = ob.alloc_workspace(B, cache.num_kv_heads, Hq, mt, device=dev)
    ob.decode_attn(cache, torch.tensor(nq, dtype=torch.int32, device=dev),
                   torch.tensor([n - m for n, m in zip(lens, nq)], dtype=torch.int32, device=dev),
                   mt, qd, sm, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ws


CASES = {
    "cfg0": lambda: syn.workload(0),
    "cfg1": lambda: syn.workload(1),
    "ragged_g4": lambda: syn.custom_workload(4, 8, 2, [0, 77, 128, 1000 + 5], cfg_tag=102),
    "g1_tail": lambda: syn.custom_workload(2, 3, 3, [300, 2048 + 127], cfg_tag=103),
    "g2": lambda: syn.custom_workload(1, 4, 2, [5000], cfg_tag=104),
    "g8": lambda: syn.custom_workload(2, 16, 2, [1, 4096 + 64], cfg_tag=105),
    # tails longer than 64 tokens are scored by two waves (both row groups at G = 8)
    "g8_tail100": lambda: syn.custom_workload(1, 8, 1, [640 + 100], cfg_tag=106),
    # a sequence made of a tail only (no quantized group), and a long tail after groups
    "g2_tail90": lambda: syn.custom_workload(2, 4, 2, [90, 1280 + 90], cfg_tag=107),
}


@pytest.mark.parametrize("case", list(CASES))
def test_int2_decode_matches_oracle(gpu_lib, case):
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    w = CASES[case]()
    _say(f"int2 decode {case}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} lens={w.lengths}")
    cache, slices, _, _, q, lens, nq = _build(ob, w, dev)
    got, _ = _run_int2(ob, cache, q, lens, nq, dev)
    err = assert_out_close(got, _oracle_out(w, slices, q, lens), case)
    _say(f"  max abs err {err:.2e}")


@pytest.mark.parametrize("sm", [4.0, 1e-3])
def test_int2_and_bf16_decode_sharp_and_flat_softmax(gpu_lib, sm):
    """A softmax scale 45x the usual one (logits spread over hundreds of
    units: the weights of most groups, and of whole early groups once a
    later maximum appears, underflow to zero) and one 88x smaller (nearly
    uniform weights, the output close to the mean value): both kernels stay
    within the output tolerance of the oracle, quantized groups and bf16
    tails alike."""
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    w = syn.custom_workload(2, 8, 2, [3000 + 40, 700], cfg_tag=150)
    _say(f"int2/bf16 decode, sm_scale {sm}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} lens={w.lengths}")
    cache, slices, kraw, vraw, q, lens, nq = _build(ob, w, dev)
    got, _ = _run_int2(ob, cache, q, lens, nq, dev, sm=sm)
    err = assert_out_close(got, _oracle_out(w, slices, q, lens, sm=sm), f"int2 sm {sm}")
    B, H, Hq = w.batch, w.num_kv_heads, w.num_q_heads
    G = Hq // H
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
    ws = ob.alloc_workspace(B, H, Hq, max(lens), device=dev)
    ob.decode_attn_bf16(bits_to_dev_bf16(kraw, dev), bits_to_dev_bf16(vraw, dev),
                        torch.tensor(lens, dtype=torch.int32, device=dev), max(lens),
                        bits_to_dev_bf16(q, dev), sm, out, ws)
    torch.cuda.synchronize()
    ref = np.zeros((B, Hq, 128))
    for b in range(B):
        for h in range(H):
            ref[b, h * G:(h + 1) * G] = oracle.decode_bf16_slice(
                syn.bf16_bits_to_f64(q[b, h * G:(h + 1) * G]), syn.bf16_bits_to_f64(kraw[b, h, :lens[b]]),
                syn.bf16_bits_to_f64(vraw[b, h, :lens[b]]), sm)
    err_bf = assert_out_close(out.cpu().numpy(), ref, f"bf16 sm {sm}")
    _say(f"  max abs err int2 {err:.2e}, bf16 {err_bf:.2e}")


def test_int2_decode_grid_larger_than_lengths(gpu_lib):
    """max_tokens far above the real lengths: extra splits see no tokens."""
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    w = syn.custom_workload(2, 8, 2, [700, 129], cfg_tag=106)
    cache, slices, _, _, q, lens, nq = _build(ob, w, dev, capacity=8192)
    got, _ = _run_int2(ob, cache, q, lens, nq, dev, max_tokens=8192)
    assert_out_close(got, _oracle_out(w, slices, q, lens), "oversized grid")


def test_int2_decode_empty_and_deterministic(gpu_lib):
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    w = syn.custom_workload(2, 4, 1, [0, 3000], cfg_tag=107)
    cache, slices, _, _, q, lens, nq = _build(ob, w, dev)
    a, ws = _run_int2(ob, cache, q, lens, nq, dev)
    b, _ = _run_int2(ob, cache, q, lens, nq, dev)
    assert np.array_equal(a, b)
    assert np.all(a[0] == 0.0)


def test_int2_decode_reused_workspace_sees_fresh_partials(gpu_lib):
    """One workspace, many calls with different data: the split merge must
    read this call's partial records, never a stale copy of an earlier call's."""
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    ws = None
    for tag in range(108, 113):
        w = syn.custom_workload(1, 32, 8, [6000 + 37 * (tag - 108)], cfg_tag=tag)
        cache, slices, _, _, q, lens, nq = _build(ob, w, dev, capacity=6400)
        if ws is None:
            ws = ob.alloc_workspace(1, 8, 32, 6400, device=dev)
        out = torch.empty((1, 32, 128), dtype=torch.float32, device=dev)
        ob.decode_attn(cache, torch.tensor(nq, dtype=torch.int32, device=dev),
                       torch.tensor([lens[0] - nq[0]], dtype=torch.int32, device=dev), 6400,
                       bits_to_dev_bf16(q, dev), SM, out, ws)
        torch.cuda.synchronize()
        assert_out_close(out.cpu().numpy(), _oracle_out(w, slices, q, lens), f"reuse {tag}")


def test_workspace_shared_across_shapes_and_kernels(gpu_lib):
    """One workspace for calls of different shapes, INT2 and bf16 in turn:
    each call, whatever its (batch, KV heads) and split count, must merge
    exactly the partial records it wrote itself."""
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    shapes = [(1, 8, 2, [9000], 113), (3, 64, 8, [700, 2500, 129], 114), (1, 2, 1, [40], 115),
              (2, 16, 4, [5000, 1], 116), (3, 8, 8, [300, 0, 8000], 117)]
    n = max(ob.decode_workspace_bytes(B, hkv, hq, max(lens)) for B, hq, hkv, lens, _ in shapes)
    ws = torch.zeros(n, dtype=torch.uint8, device=dev)
    for B, hq, hkv, lens, tag in shapes:
        w = syn.custom_workload(B, hq, hkv, lens, cfg_tag=tag)
        _say(f"shared workspace: B={B} Hq={hq} Hkv={hkv} lens={lens}")
        cache, slices, kraw, vraw, q, lens_, nq = _build(ob, w, dev)
        mt = max(lens_)
        out = torch.full((B, hq, 128), float("nan"), dtype=torch.float32, device=dev)
        ob.decode_attn(cache, torch.tensor(nq, dtype=torch.int32, device=dev),
                       torch.tensor([n - m for n, m in zip(lens_, nq)], dtype=torch.int32, device=dev),
                       mt, bits_to_dev_bf16(q, dev), SM, out, ws)
        torch.cuda.synchronize()
        assert_out_close(out.cpu().numpy(), _oracle_out(w, slices, q, lens_), f"int2 {tag}")
        out_bf = torch.full((B, hq, 128), float("nan"), dtype=torch.float32, device=dev)
        ob.decode_attn_bf16(bits_to_dev_bf16(kraw, dev), bits_to_dev_bf16(vraw, dev),
                            torch.tensor(lens_, dtype=torch.int32, device=dev), mt,
                            bits_to_dev_bf16(q, dev), SM, out_bf, ws)
        torch.cuda.synchronize()
        G = hq // hkv
        ref = np.zeros((B, hq, 128))
        for b in range(B):
            for h in range(hkv):
                ref[b, h * G:(h + 1) * G] = oracle.decode_bf16_slice(
                    syn.bf16_bits_to_f64(q[b, h * G:(h + 1) * G]), syn.bf16_bits_to_f64(kraw[b, h, :lens_[b]]),
                    syn.bf16_bits_to_f64(vraw[b, h, :lens_[b]]), SM)
        assert_out_close(out_bf.cpu().numpy(), ref, f"bf16 {tag}")


@pytest.mark.parametrize("case", ["cfg0", "cfg1", "ragged_g4", "g8"])
def test_bf16_decode_matches_oracle(gpu_lib, case):
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    w = CASES[case]()
    _say(f"bf16 decode {case}")
    B, H, Hq = w.batch, w.num_kv_heads, w.num_q_heads
    lens = [w.total_tokens(b) for b in range(B)]
    cap = max(128, max(lens))
    k = np.zeros((B, H, cap, 128), np.uint16)
    v = np.zeros((B, H, cap, 128), np.uint16)
    for b in range(B):
        for h in range(H):
            k[b, h, :lens[b]] = syn.keys_slice(w, b, h)
            v[b, h, :lens[b]] = syn.values_slice(w, b, h)
    q = np.stack([syn.query(w, b) for b in range(B)])
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
    ws = ob.alloc_workspace(B, H, Hq, max(lens), device=dev)
    ob.decode_attn_bf16(bits_to_dev_bf16(k, dev), bits_to_dev_bf16(v, dev),
                        torch.tensor(lens, dtype=torch.int32, device=dev), max(lens),
                        bits_to_dev_bf16(q, dev), SM, out, ws)
    torch.cuda.synchronize()
    G = Hq // H
    ref = np.zeros((B, Hq, 128))
    for b in range(B):
        for h in range(H):
            ref[b, h * G:(h + 1) * G] = oracle.decode_bf16_slice(
                syn.bf16_bits_to_f64(q[b, h * G:(h + 1) * G]), syn.bf16_bits_to_f64(k[b, h, :lens[b]]),
                syn.bf16_bits_to_f64(v[b, h, :lens[b]]), SM)
    assert_out_close(out.cpu().numpy(), ref, case)


def test_workspace_too_small_is_an_error(gpu_lib):
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    cache = ob.PackedCache(1, 1, 1024, device=dev)
    q = torch.zeros((1, 1, 128), dtype=torch.bfloat16, device=dev)
    out = torch.zeros((1, 1, 128), dtype=torch.float32, device=dev)
    ws = torch.zeros(16, dtype=torch.uint8, device=dev)
    z = torch.zeros(1, dtype=torch.int32, device=dev)
    with pytest.raises(ob.OscarError) as e:
        ob.decode_attn(cache, z, z, 1024, q, SM, out, ws)
    assert e.value.status == ob.OSCAR_EWORKSPACE


def test_splits_then_merge_equals_decode(gpu_lib):
    """oscar_decode_attn_splits + oscar_decode_merge give oscar_decode_attn's
    output bit for bit, and the records are softmax states whose merge (by
    the oracle's algebra, in float64) is the oracle's attention output."""
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    w = syn.custom_workload(2, 16, 4, [2500, 700 + 45], cfg_tag=118)
    cache, slices, _, _, q, lens, nq = _build(ob, w, dev)
    mt = max(lens)
    full, ws = _run_int2(ob, cache, q, lens, nq, dev)
    S = ob.decode_num_splits(w.batch, w.num_kv_heads, mt)
    assert S >= 1
    ob.decode_attn_splits(cache, torch.tensor(nq, dtype=torch.int32, device=dev),
                          torch.tensor([n - m for n, m in zip(lens, nq)], dtype=torch.int32, device=dev),
                          mt, bits_to_dev_bf16(q, dev), SM, ws)
    rec = ob.split_records(ws, w.batch, w.num_q_heads, S)
    out = torch.full((w.batch, w.num_q_heads, 128), float("nan"), dtype=torch.float32, device=dev)
    ob.decode_merge(rec, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), full)
    r = rec.cpu().numpy().astype(np.float64)
    ref = _oracle_out(w, slices, q, lens)
    ln2 = np.log(2.0)
    for b in range(w.batch):
        for j in range(w.num_q_heads):
            states = [(r[b, j, s, 0] * ln2, r[b, j, s, 1], r[b, j, s, 4:]) for s in range(S)]
            got = oracle.merge_states(states)
            assert_out_close(got[None, None], ref[b:b + 1, j:j + 1], f"records b={b} head={j}")


def test_merge_of_records_from_two_token_shards(gpu_lib):
    """A sequence held as two caches (tokens [0, 1024) and [1024, n), the
    second with the bf16 tail): the records of both, concatenated along the
    split axis and merged once, give attention over the whole sequence."""
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    n = 3000 + 37
    w = syn.custom_workload(1, 8, 2, [n], cfg_tag=119)
    B, H, Hq = 1, 2, 8
    n_q_full = syn.split_lengths(n)[0]
    parts = [(0, 1024), (1024, n)]
    recs = []
    full_slices = {}
    qd = bits_to_dev_bf16(np.stack([syn.query(w, 0)]), dev)
    for lo, hi in parts:
        m = hi - lo
        nq = syn.split_lengths(m)[0]
        cache = ob.PackedCache(B, H, max(128, ((m + 127) // 128) * 128), device=dev)
        for h in range(H):
            kb = syn.bf16_bits_to_f64(syn.keys_slice(w, 0, h))
            vb = syn.bf16_bits_to_f64(syn.values_slice(w, 0, h))
            upload_slice(cache, 0, h, oracle.quantize_slice(kb[lo:hi], vb[lo:hi], nq))
            if (lo, hi) == parts[0]:
                full_slices[0, h] = oracle.quantize_slice(kb, vb, n_q_full)
        ws = ob.alloc_workspace(B, H, Hq, m, device=dev)
        ob.decode_attn_splits(cache, torch.tensor([nq], dtype=torch.int32, device=dev),
                              torch.tensor([m - nq], dtype=torch.int32, device=dev), m, qd, SM, ws)
        S = ob.decode_num_splits(B, H, m)
        recs.append(ob.split_records(ws, B, Hq, S).clone())
    allrec = torch.cat(recs, dim=2).contiguous()
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device=dev)
    ob.decode_merge(allrec, out)
    torch.cuda.synchronize()
    q = np.stack([syn.query(w, 0)])
    assert_out_close(out.cpu().numpy(), _oracle_out(w, full_slices, q, [n]), "two shards")


@pytest.mark.parametrize("G", [4, 8])
@pytest.mark.parametrize("max_tokens", [600, 1000, 1030])
def test_int2_decode_max_tokens_cuts_the_sequences(gpu_lib, G, max_tokens):
    """max_tokens below a sequence's length: only its first max_tokens
    tokens are attended (quantized ones first, then the tail), so the cut can
    fall inside a quantized group (the group's later tokens masked) or inside
    the tail.  Sequence 0: 1024 quantized + 50 tail tokens; sequence 1: 512 +
    100.  Reference: the oracle's dequantized tokens, truncated."""
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    Hkv = 2
    w = syn.custom_workload(2, G * Hkv, Hkv, [1024 + 50, 512 + 100], cfg_tag=170 + G)
    cache, slices, _, _, q, lens, nq = _build(ob, w, dev)
    _say(f"max_tokens {max_tokens}, G {G}, lengths {lens}")
    got, _ = _run_int2(ob, cache, q, lens, nq, dev, max_tokens=max_tokens)
    assert np.isfinite(got).all()
    for b in range(2):
        m = min(max_tokens, lens[b])
        for h in range(Hkv):
            s = slices[b, h]
            k_hat, v_hat = s.dequantized()
            mq = min(m, s.n_quant)
            ref = oracle.decode_slice(syn.bf16_bits_to_f64(q[b, h * G:(h + 1) * G]), k_hat[:mq], v_hat[:mq],
                                      s.k_tail[:m - mq], s.v_tail[:m - mq], SM)
            assert_out_close(got[b, h * G:(h + 1) * G], ref, f"max_tokens {max_tokens}, sequence {b}, head {h}")


@pytest.mark.parametrize("max_tokens", [600, 1000, 1030])
def test_bf16_decode_max_tokens_cuts_the_sequences(gpu_lib, max_tokens):
    """The bf16 reference kernel with max_tokens below a sequence's length
    (a cut inside a 32-token piece): only the first max_tokens tokens are
    attended."""
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    B, H, G = 2, 2, 4
    w = syn.custom_workload(B, G * H, H, [1024 + 50, 512 + 100], cfg_tag=180)
    lens = [w.total_tokens(b) for b in range(B)]
    cap = max(lens)
    k = np.zeros((B, H, cap, 128), np.uint16)
    v = np.zeros((B, H, cap, 128), np.uint16)
    for b in range(B):
        for h in range(H):
            k[b, h, :lens[b]] = syn.keys_slice(w, b, h)
            v[b, h, :lens[b]] = syn.values_slice(w, b, h)
    q = np.stack([syn.query(w, b) for b in range(B)])
    _say(f"bf16 decode, max_tokens {max_tokens}, lengths {lens}")
    out = torch.empty((B, G * H, 128), dtype=torch.float32, device=dev)
    ws = ob.alloc_workspace(B, H, G * H, max_tokens, device=dev)
    ob.decode_attn_bf16(bits_to_dev_bf16(k, dev), bits_to_dev_bf16(v, dev),
                        torch.tensor(lens, dtype=torch.int32, device=dev), max_tokens,
                        bits_to_dev_bf16(q, dev), SM, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(B):
        m = min(max_tokens, lens[b])
        for h in range(H):
            ref = oracle.decode_bf16_slice(syn.bf16_bits_to_f64(q[b, h * G:(h + 1) * G]),
                                           syn.bf16_bits_to_f64(k[b, h, :m]), syn.bf16_bits_to_f64(v[b, h, :m]), SM)
            assert_out_close(got[b, h * G:(h + 1) * G], ref, f"bf16, max_tokens {max_tokens}, sequence {b}, head {h}")
