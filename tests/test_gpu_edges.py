"""GPU edge cases of the run calls: empty batches (nothing launched, outputs untouched),
requests that all have empty token sets (the merge identity), the largest page size, one very
long sequence split across the whole chip, and shapes whose offsets would not fit in 32 bits
(rejected before any launch)."""

import pytest
import torch

from oracle import attention as oatt
from paged_kv_cascade_amd import workloads
from tests.gpu_helpers import PoolView, check_state, gpu, host, needs_gpu, say

pytestmark = [gpu, needs_gpu]


@pytest.fixture(scope="module")
def api():
    from paged_kv_cascade_amd import api as _api
    return _api


def test_empty_batch_launches_nothing(api):
    say("case: batch of 0 requests (decode, plan-driven decode, cascade, prefill)")
    q = torch.empty(0, 4, 128, dtype=torch.float16, device="cuda")
    k = torch.zeros(2, 16, 4, 128, dtype=torch.float16, device="cuda")
    bt = torch.zeros(0, 1, dtype=torch.int32, device="cuda")
    lens = torch.zeros(0, dtype=torch.int32, device="cuda")
    o = torch.full((0, 4, 128), 7.0, dtype=torch.float16, device="cuda")
    lse = torch.full((0, 4), 7.0, device="cuda")
    api.batch_decode_paged(q, k, k, bt, lens, out=o, lse=lse)
    params = api.make_params(0, 4, 4, 128, 16, num_ctas=8, level_ctas=2)
    ws = api.Workspace(params)
    info = api.plan(params, [], workspace=ws)
    api.batch_decode_paged(q, k, k, bt, lens, plan_info=info, out=o, lse=lse)
    info2, ws2, qi = api.prefill_plan([], [], 4, 4, 128, 16)
    api.batch_prefill_paged(info2, q, k, k, bt, torch.zeros(1, dtype=torch.int32, device="cuda"), lens)
    torch.cuda.synchronize()


def test_all_requests_empty_give_the_identity_state(api):
    """Every request has zero tokens: O = 0 and LSE = -inf (the merge identity), through the
    plain kernel, the split plan and a cascade whose levels cover nobody's tokens."""
    say("case: every request empty")
    B, H, D, P = 9, 4, 64, 16
    q = torch.randn(B, H, D, device="cuda").half()
    k = torch.full((3, P, H, D), float("nan"), device="cuda").half()
    bt = torch.full((B, 2), -1, dtype=torch.int32, device="cuda")
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    o, lse = api.batch_decode_paged(q, k, k, bt, lens)
    params = api.make_params(B, H, H, D, P, num_ctas=5)
    ws = api.Workspace(params)
    info = api.plan(params, [0] * B, workspace=ws)
    o2, lse2 = api.batch_decode_paged(q, k, k, bt, lens, plan_info=info)
    levels = [{"qo_indptr": [0, 4, 9], "kv_lens": [0, 0], "kv_page_indptr": [0, 0, 0], "kv_page_indices": []}]
    params3 = api.make_params(B, H, H, D, P, num_ctas=5, level_ctas=3)
    host_levels = [{"qo_indptr": lv["qo_indptr"], "kv_lens": lv["kv_lens"]} for lv in levels]
    ws3 = api.Workspace(params3, host_levels)
    info3 = api.plan(params3, [0] * B, host_levels, workspace=ws3)
    d, keep = api.level_dev(levels[0])
    o3, lse3 = api.cascade_decode(info3, q, k, k, [d], bt, lens)
    torch.cuda.synchronize()
    for oo, ll in ((o, lse), (o2, lse2), (o3, lse3)):
        assert torch.all(oo == 0) and torch.all(torch.isneginf(ll))


def test_largest_page_size(api):
    """Page size 1024 (the largest the plan accepts): a page holds whole wave steps."""
    say("case: decode with 1024-token pages, fp16, D=128, g=4")
    w = workloads.paged_decode(batch=6, heads=16, kv_heads=4, kv_len=2500, page_size=1024, seed=91,
                               device="cuda")
    o, lse = api.batch_decode_paged(w.q, w.k_pool, w.v_pool, w.block_table, w.cache_seqlens,
                                    sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    O, L = oatt.batch_decode(host(w.q), PoolView(w.k_pool), PoolView(w.v_pool), w.block_table.cpu().numpy(),
                             w.cache_seqlens.cpu().numpy(), 1024, w.sm_scale)
    check_state(o, lse, O, L, torch.float16, "page 1024")


def test_one_long_sequence_split_over_the_chip(api):
    """One request of 262144 tokens (32 KV heads x 128, bf16) split by the plan over 2 x CUs
    CTAs and merged; sampled heads against the oracle."""
    say("case: one 262144-token request, plan split over 2 x CUs, bf16")
    w = workloads.paged_decode(batch=1, heads=32, kv_len=262144, page_size=16, dtype=torch.bfloat16,
                               seed=92, device="cuda")
    cus = api.device_info(0)["num_cus"]
    params = api.make_params(1, 32, 32, 128, 16, num_ctas=2 * cus)
    ws = api.Workspace(params)
    info = api.plan(params, [262144], workspace=ws)
    assert info.num_merge == 1 and info.dec_items > cus
    o, lse = api.batch_decode_paged(w.q, w.k_pool, w.v_pool, w.block_table, w.cache_seqlens,
                                    sm_scale=w.sm_scale, plan_info=info)
    torch.cuda.synchronize()
    heads = [0, 13, 31]
    O, L = oatt.batch_decode(host(w.q), PoolView(w.k_pool), PoolView(w.v_pool), w.block_table.cpu().numpy(),
                             w.cache_seqlens.cpu().numpy(), 16, w.sm_scale, heads=heads)
    check_state(o, lse, O, L, torch.bfloat16, "262144 tokens")


def test_offsets_past_32_bits_are_rejected(api):
    say("case: block-table span past int32 rejected before launch")
    q = torch.zeros(1, 4, 64, dtype=torch.float16, device="cuda")
    k = torch.zeros(1, 16, 4, 64, dtype=torch.float16, device="cuda")
    wide = torch.empty(1, (1 << 31) // 16 + 1, dtype=torch.int32, device="cuda")
    lens = torch.ones(1, dtype=torch.int32, device="cuda")
    with pytest.raises(api.PkcError):
        api.batch_decode_paged(q, k, k, wide, lens)
