"""Host bookkeeping of the group-append workflow (kv_cache_int2_fwht_amd.session):
the per-step counts a run of decode steps uses, checked against the rule
that a sequence's tail is quantized once it holds 128 tokens (ai-papers.net
OScaR summary, section "OScaRの提案手法")."""
import pytest

from kv_cache_int2_fwht_amd.session import plan_steps


def test_32k_workload_plan():
    # 32768 quantized tokens and a 57-token tail: the tail fills at step 70
    # (57 + 71 = 128), after which the next group starts empty
    plans = plan_steps([32768], [57], 128)
    full = [s for s, p in enumerate(plans) if p.full[0]]
    assert full == [70]
    assert plans[0].n_quant == [32768] and plans[0].n_tail == [58]
    assert plans[70].n_quant == [32768] and plans[70].n_tail == [128]
    assert plans[71].n_quant == [32896] and plans[71].n_tail == [1]
    assert plans[127].n_quant == [32896] and plans[127].n_tail == [57]
    assert plans[70].max_tokens == 32768 + 128


def test_batch_tails_fill_independently():
    plans = plan_steps([0, 128, 256], [127, 0, 100], 300)
    for b, (nq0, nt0) in enumerate([(0, 127), (128, 0), (256, 100)]):
        # total tokens after step s are nq0 + nt0 + s + 1, split into whole
        # groups plus a tail of 1..128 tokens
        for s, p in enumerate(plans):
            total = nq0 + nt0 + s + 1
            assert p.n_quant[b] + p.n_tail[b] == total
            assert p.n_quant[b] % 128 == 0 and 1 <= p.n_tail[b] <= 128
            assert p.full[b] == (p.n_tail[b] == 128)
    assert plans[0].full == [True, False, False]


@pytest.mark.parametrize("nq, nt", [(-128, 0), (100, 0), (0, 128), (0, -1)])
def test_invalid_counts(nq, nt):
    with pytest.raises(ValueError):
        plan_steps([nq], [nt], 4)
