"""The 32K group-append workload (128 decode steps, one group append) captured
in a HIP graph through torch.cuda.CUDAGraph and replayed: every replay must
give the eager run's outputs bit for bit.  Replays are separated by eager
work and synchronizations, and the packed cache is restored from a snapshot
before each replay (the loop appends to it)."""
import numpy as np
import pytest
import torch

import synthetic as syn
from tests.helpers import bits_to_dev_bf16

pytestmark = pytest.mark.gpu

SM = 1.0 / np.sqrt(128.0)
STATE = ("blocks", "k_tail", "v_tail")


def _say(msg):
    print(msg, flush=True)


def test_32k_append_loop_graph_replay_matches_eager(gpu_lib):
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    w = syn.workload(2)
    B, H, Hq = w.batch, w.num_kv_heads, w.num_q_heads
    L0 = w.lengths[0]
    n_q0, tail0 = syn.split_lengths(L0)
    steps = w.append_steps
    cap = ((w.total_tokens(0) + 127) // 128) * 128
    _say(f"graph capture of {steps} decode steps at {L0} tokens")
    k_dev = bits_to_dev_bf16(np.stack([syn.keys_slice(w, 0, h) for h in range(H)])[None], dev)
    v_dev = bits_to_dev_bf16(np.stack([syn.values_slice(w, 0, h) for h in range(H)])[None], dev)
    cache = ob.PackedCache(B, H, cap, device=dev)
    ob.quantize_kv(cache, k_dev, v_dev, torch.zeros(1, dtype=torch.int32, device=dev),
                   torch.full((1,), n_q0 // 128, dtype=torch.int32, device=dev), n_q0 // 128)
    cache.k_tail[0, :, :tail0] = k_dev[0, :, n_q0:L0]
    cache.v_tail[0, :, :tail0] = v_dev[0, :, n_q0:L0]
    torch.cuda.synchronize()
    snapshot = {n: getattr(cache, n).clone() for n in STATE}

    # every per-step input is on the device before capture
    plan, n_quant, n_tail = [], n_q0, tail0
    for s in range(steps):
        slot = n_tail
        n_tail += 1
        append = n_tail == 128
        if append:
            n_quant, n_tail = n_quant + 128, 0
        plan.append((slot, append, n_quant, n_tail))
    nq_dev = torch.tensor([[p[2]] for p in plan], dtype=torch.int32, device=dev)
    nt_dev = torch.tensor([[p[3]] for p in plan], dtype=torch.int32, device=dev)
    q_dev = bits_to_dev_bf16(np.stack([syn.query(w, 0, s)[None] for s in range(steps)]), dev)
    start = torch.full((1,), n_q0 // 128, dtype=torch.int32, device=dev)
    one = torch.ones(1, dtype=torch.int32, device=dev)
    outs = torch.zeros((steps, B, Hq, 128), dtype=torch.float32, device=dev)
    ws = ob.alloc_workspace(B, H, Hq, cap, device=dev)

    def loop():
        for s, (slot, append, nq, nt) in enumerate(plan):
            cache.k_tail[0, :, slot] = k_dev[0, :, L0 + s]
            cache.v_tail[0, :, slot] = v_dev[0, :, L0 + s]
            if append:
                ob.quantize_kv(cache, cache.k_tail, cache.v_tail, start, one, 1)
            ob.decode_attn(cache, nq_dev[s], nt_dev[s], nq + nt, q_dev[s], SM, outs[s], ws)

    def restore():
        for n in STATE:
            getattr(cache, n).copy_(snapshot[n])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # eager warm-up on the capture stream
        loop()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = outs.clone()
    assert torch.isfinite(eager).all()

    restore()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loop()
    torch.cuda.synchronize()
    for rep in range(3):
        restore()
        outs.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs, eager), f"replay {rep} differs from the eager run"
        _ = (k_dev.float().sum() + 1).item()   # eager work between replays
    _say("  3 replays equal the eager run")


def test_32k_append_in_decode_loop_graph_replay_matches_eager(gpu_lib):
    """The same workload with the token written inside the decode launch
    (oscar_decode_attn_append): the tail reaches 128 tokens at step 70 and
    is quantized after that step.  Replays equal the eager run bit for bit,
    and the cache ends in the same state."""
    from kv_cache_int2_fwht_amd import binding as ob
    dev = torch.device("cuda:0")
    w = syn.workload(2)
    B, H, Hq = w.batch, w.num_kv_heads, w.num_q_heads
    L0 = w.lengths[0]
    n_q0, tail0 = syn.split_lengths(L0)
    steps = w.append_steps
    cap = ((w.total_tokens(0) + 127) // 128) * 128
    _say(f"graph capture of {steps} append-in-decode steps at {L0} tokens")
    k_dev = bits_to_dev_bf16(np.stack([syn.keys_slice(w, 0, h) for h in range(H)])[None], dev)
    v_dev = bits_to_dev_bf16(np.stack([syn.values_slice(w, 0, h) for h in range(H)])[None], dev)
    cache = ob.PackedCache(B, H, cap, device=dev)
    ob.quantize_kv(cache, k_dev, v_dev, torch.zeros(1, dtype=torch.int32, device=dev),
                   torch.full((1,), n_q0 // 128, dtype=torch.int32, device=dev), n_q0 // 128)
    cache.k_tail[0, :, :tail0] = k_dev[0, :, n_q0:L0]
    cache.v_tail[0, :, :tail0] = v_dev[0, :, n_q0:L0]
    torch.cuda.synchronize()
    snapshot = {n: getattr(cache, n).clone() for n in STATE}

    # the per-step counts live on the device before capture (DecodeSession)
    from kv_cache_int2_fwht_amd.session import DecodeSession
    session = DecodeSession(cache, [n_q0], [tail0], Hq, steps)
    assert [s for s, p in enumerate(session.plans) if p.full[0]] == [70]
    q_dev = bits_to_dev_bf16(np.stack([syn.query(w, 0, s)[None] for s in range(steps)]), dev)
    new_k = k_dev[0, :, L0:L0 + steps].transpose(0, 1).contiguous()[:, None]   # [steps, 1, H, 128]
    new_v = v_dev[0, :, L0:L0 + steps].transpose(0, 1).contiguous()[:, None]
    outs = torch.zeros((steps, B, Hq, 128), dtype=torch.float32, device=dev)

    def loop():
        for s in range(steps):
            session.step(s, q_dev[s], new_k[s], new_v[s], SM, outs[s])

    def restore():
        for n in STATE:
            getattr(cache, n).copy_(snapshot[n])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        loop()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = outs.clone()
    final = {n: getattr(cache, n).clone() for n in STATE}
    assert torch.isfinite(eager).all()
    restore()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loop()
    torch.cuda.synchronize()
    for rep in range(3):
        restore()
        outs.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs, eager), f"replay {rep} differs from the eager run"
        for n in STATE:
            assert torch.equal(getattr(cache, n), final[n]), f"replay {rep}: cache {n} differs"
        _ = (k_dev.float().sum() + 1).item()   # eager work between replays
    _say("  3 replays equal the eager run")
