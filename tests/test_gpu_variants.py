"""GPU parity of the key-quantizer variants of the Token Norm Imbalance
ablation (cache flags OSCAR_KEYS_UNROTATED / OSCAR_KEYS_UNSCALED) against
the oracle's quantize_keys(rotate, scale), through the C ABI: packed bytes to
the quantizer's bar, and the decode over the oracle's bytes to the output
bar (ai-papers.net OScaR summary, sections "TNIという根本課題の特定" and
"OScaRの提案手法")."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from tests.helpers import assert_out_close, bits_to_dev_bf16, check_quantized_slice, upload_slice

pytestmark = pytest.mark.gpu

SM = 1.0 / np.sqrt(128.0)
# variant -> (rotate, scale)
VARIANTS = {"per_channel": (False, False), "rotation": (True, False), "scaling": (False, True), "oscar": (True, True)}


def _flags(ob, rot, sc):
    return (0 if rot else ob.KEYS_UNROTATED) | (0 if sc else ob.KEYS_UNSCALED)


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("G", [4, 8])
def test_variant_quantize_and_decode_match_oracle(gpu_lib, variant, G):
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    rot, sc = VARIANTS[variant]
    flags = _flags(ob, rot, sc)
    H = 2
    w = syn.custom_workload(1, G * H, H, [1024 + 45], cfg_tag=140 + G)
    nq, nt = syn.split_lengths(w.lengths[0])
    print(f"variant {variant} G={G} flags={flags}", flush=True)
    kb = [syn.keys_slice(w, 0, h) for h in range(H)]
    vb = [syn.values_slice(w, 0, h) for h in range(H)]
    q_bits = syn.query(w, 0)

    # quantizer: GPU bytes against the oracle variant
    cache = ob.PackedCache(1, H, 1024 + 128, device=dev, flags=flags)
    k_dev = torch.stack([bits_to_dev_bf16(x, dev) for x in kb])[None]
    v_dev = torch.stack([bits_to_dev_bf16(x, dev) for x in vb])[None]
    ob.quantize_kv(cache, k_dev, v_dev, torch.zeros(1, dtype=torch.int32, device=dev),
                   torch.full((1,), nq // 128, dtype=torch.int32, device=dev), nq // 128)
    torch.cuda.synchronize()
    refs = []
    for h in range(H):
        ref = oracle.quantize_slice(syn.bf16_bits_to_f64(kb[h]), syn.bf16_bits_to_f64(vb[h]), nq,
                                    keep_intermediates=True, rotate=rot, scale=sc)
        check_quantized_slice(cache, 0, h, ref)
        refs.append(ref)

    # decode over the oracle's bytes, with the variant's flags
    oc = ob.PackedCache(1, H, 1024 + 128, device=dev, flags=flags)
    for h in range(H):
        upload_slice(oc, 0, h, refs[h])
    out = torch.empty((1, G * H, 128), dtype=torch.float32, device=dev)
    ws = ob.alloc_workspace(1, H, G * H, nq + nt, device=dev)
    ob.decode_attn(oc, torch.full((1,), nq, dtype=torch.int32, device=dev),
                   torch.full((1,), nt, dtype=torch.int32, device=dev), nq + nt,
                   bits_to_dev_bf16(q_bits, dev)[None], SM, out, ws)
    torch.cuda.synchronize()
    got = out[0].cpu().numpy()
    for h in range(H):
        ref_out = refs[h].decode(syn.bf16_bits_to_f64(q_bits[h * G:(h + 1) * G]), SM)
        assert_out_close(got[h * G:(h + 1) * G], ref_out, f"{variant} G={G} head {h}")
