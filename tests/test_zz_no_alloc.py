"""oscar_decode_attn_noalloc through the C ABI against oscar_decode_attn on
the same inputs: the same kernels with the split records in the library's
own device array instead of a workspace, so the outputs must be equal bit
for bit.  Two calls in a row, the second with a smaller shape (fewer
splits, fewer query heads), so that the second reads none of the first's
records."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from tests.helpers import assert_out_close, bits_to_dev_bf16, upload_slice

pytestmark = pytest.mark.gpu

SM = 1.0 / np.sqrt(128.0)


def _case(dev, B, Hq, Hkv, lengths, tag):
    from kv_cache_int2_fwht_amd import binding as ob
    w = syn.custom_workload(B, Hq, Hkv, lengths, cfg_tag=tag)
    cap = ((max(lengths) + 127) // 128) * 128 + 128
    cache = ob.PackedCache(B, Hkv, cap, device=dev)
    refs = {}
    for b in range(B):
        nq = syn.split_lengths(lengths[b])[0]
        for h in range(Hkv):
            s = oracle.quantize_slice(syn.bf16_bits_to_f64(syn.keys_slice(w, b, h)),
                                      syn.bf16_bits_to_f64(syn.values_slice(w, b, h)), nq)
            upload_slice(cache, b, h, s)
            refs[b, h] = s
    nq = torch.tensor([syn.split_lengths(x)[0] for x in lengths], dtype=torch.int32, device=dev)
    nt = torch.tensor([syn.split_lengths(x)[1] for x in lengths], dtype=torch.int32, device=dev)
    q_bits = np.stack([syn.query(w, b) for b in range(B)])
    return cache, nq, nt, max(lengths), bits_to_dev_bf16(q_bits, dev), q_bits, refs


def _check(dev, B, Hq, Hkv, lengths, tag):
    from kv_cache_int2_fwht_amd import binding as ob
    cache, nq, nt, mt, q, q_bits, refs = _case(dev, B, Hq, Hkv, lengths, tag)
    print(f"noalloc decode: B {B}, Hq {Hq}, Hkv {Hkv}, lengths {lengths}", flush=True)
    out_ws = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device=dev)
    out_na = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device=dev)
    ws = ob.alloc_workspace(B, Hkv, Hq, mt, device=dev)
    ob.decode_attn(cache, nq, nt, mt, q, SM, out_ws, ws)
    ob.decode_attn_noalloc(cache, nq, nt, mt, q, SM, out_na)
    torch.cuda.synchronize()
    assert torch.equal(out_ws, out_na)
    got = out_na.cpu().numpy()
    G = Hq // Hkv
    for (b, h), s in refs.items():
        ref = s.decode(syn.bf16_bits_to_f64(q_bits[b, h * G:(h + 1) * G]), SM)
        assert_out_close(got[b, h * G:(h + 1) * G], ref, f"noalloc, sequence {b}, head {h}")
    return ob.decode_num_splits(B, Hkv, mt)


def test_noalloc_equals_the_workspace_call_twice_in_a_row(gpu_lib):
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    s1 = _check(dev, 2, 16, 4, [4096 + 37, 2048 + 128 * 3 + 5], 160)
    s2 = _check(dev, 1, 4, 1, [1024 + 11], 161)
    assert s2 < s1


def test_noalloc_refuses_a_shape_beyond_its_array(gpu_lib):
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    cache = ob.PackedCache(1024, 8, 128, device=dev)
    i32 = torch.zeros(1024, dtype=torch.int32, device=dev)
    q = torch.zeros((1024, 64, 128), dtype=torch.bfloat16, device=dev)
    out = torch.zeros((1024, 64, 128), dtype=torch.float32, device=dev)
    with pytest.raises(ob.OscarError) as e:
        ob.decode_attn_noalloc(cache, i32, i32, 128, q, SM, out)
    assert e.value.status == 3
    assert torch.count_nonzero(out).item() == 0
