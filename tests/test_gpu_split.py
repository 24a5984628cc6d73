"""GPU parity of plan-driven split-KV decode (load-balancing plan + partial states +
merge) against the fp64 oracle, and bit-exactness of the work-to-workgroup map the
device walks against the host plan."""

import math
import random

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import plan as oplan
from paged_kv_cascade_amd import workloads
from tests.gpu_helpers import FULL_SIZE_HEADS, HostPool, PoolView, check_state, gpu, host, needs_gpu, say

pytestmark = [gpu, needs_gpu]


@pytest.fixture(scope="module")
def api():
    from paged_kv_cascade_amd import api as _api
    return _api


def _check_trace(api, info, stage_lists, stage):
    max_items = max([1] + [len(c) for c in stage_lists])
    tr = api.debug_cta_trace(info, stage, max_items).cpu().numpy()
    for c, recs in enumerate(stage_lists):
        for k in range(max_items):
            exp = recs[k] if k < len(recs) else [-1] * 8
            assert tr[c, k].tolist() == list(exp), f"stage {stage} CTA {c} item {k}"


def test_gqa_split_full_size(api):
    """32 q / 8 kv heads, bf16, 256 requests with log-uniform lengths in [128, 32768],
    plan over #CTA = 2 x compute units, alpha = beta = 1."""
    say("case: GQA split-KV b256 hq32 hkv8 d128 bf16 log-uniform lengths, plan #CTA = 2 x CUs")
    w = workloads.gqa_split(device="cuda")
    cus = api.device_info(0)["num_cus"]
    lens = w.cache_seqlens.cpu().tolist()
    api.validate_block_table(w.block_table.cpu(), w.cache_seqlens.cpu(), w.page_size, w.num_pages)
    params = api.make_params(w.batch, 32, 8, 128, 16, num_ctas=2 * cus, alpha=1, beta=1)
    ws = api.Workspace(params)
    info = api.plan(params, lens, workspace=ws)
    o, lse = api.batch_decode_paged(w.q, w.k_pool, w.v_pool, w.block_table, w.cache_seqlens,
                                    sm_scale=w.sm_scale, plan_info=info)
    o2, lse2 = api.batch_decode_paged(w.q, w.k_pool, w.v_pool, w.block_table, w.cache_seqlens,
                                      sm_scale=w.sm_scale, plan_info=info)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "repeat run differs"
    say(f"  plan: L_kv={info.dec_kv_chunk} items={info.dec_items} slots={info.dec_slots} merged={info.num_merge}")
    # device walk of the plan == host plan == oracle plan
    arr = api.read_plan_arrays(info, ws.host)
    _check_trace(api, info, arr["decode"], 0)
    o_plan = oplan.cascade_plan(w.batch, [], lens, num_ctas=2 * cus, level_ctas=1, level_tile_q=[])
    for c, recs in enumerate(arr["decode"]):
        assert [r[7] for r in recs] == o_plan.suffix.cta_items[c]
    # every request on query heads 0, 13, 31 (kv heads 0, 3, 7): every decode workgroup's items
    O, L = oatt.batch_decode(host(w.q), HostPool(w.k_pool), HostPool(w.v_pool),
                             w.block_table.cpu().numpy(), np.array(lens), 16, w.sm_scale, heads=FULL_SIZE_HEADS)
    check_state(o, lse, O, L, torch.bfloat16, "GQA split-KV")


@pytest.mark.parametrize("seed", range(6))
def test_split_ragged_random(api, seed):
    rng = random.Random(seed)
    dtype = [torch.float16, torch.bfloat16, torch.float32][seed % 3]
    D = [128, 64][seed % 2]
    g = [1, 4, 8, 2, 1, 4][seed]
    P = [16, 4, 32, 1, 8, 16][seed]
    hkv = 2
    B = rng.randint(5, 30)
    lens = [rng.choice([0, 1, P, rng.randint(1, 3000)]) for _ in range(B)]
    ctas = rng.choice([1, 3, 64, 512])
    align = rng.choice([1, 16])
    split = seed != 5
    say(f"case: split ragged seed={seed} {dtype} D={D} g={g} P={P} B={B} ctas={ctas} align={align} split={split}")
    npg = [-(-n // P) for n in lens]
    num_pages = sum(npg) + 3
    perm = torch.randperm(num_pages, generator=torch.Generator().manual_seed(seed)).tolist()
    bt = torch.full((B, max(npg) + 2), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(npg):
        bt[b, :n] = torch.tensor(perm[off:off + n], dtype=torch.int32)
        off += n
    gen = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn(B, hkv * g, D, generator=gen, device="cuda").to(dtype)
    k = torch.randn(num_pages, P, hkv, D, generator=gen, device="cuda").to(dtype)
    v = torch.randn(num_pages, P, hkv, D, generator=gen, device="cuda").to(dtype)
    api.validate_block_table(bt, torch.tensor(lens, dtype=torch.int32), P, num_pages)
    params = api.make_params(B, hkv * g, hkv, D, P, num_ctas=ctas, chunk_align=align, enable_split=split)
    ws = api.Workspace(params)
    info = api.plan(params, lens, workspace=ws)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, lse = api.batch_decode_paged(q, k, v, bt.cuda(), sl, sm_scale=0.3, plan_info=info)
    o_ref, l_ref = api.batch_decode_paged(q, k, v, bt.cuda(), sl, sm_scale=0.3)
    torch.cuda.synchronize()
    arr = api.read_plan_arrays(info, ws.host)
    _check_trace(api, info, arr["decode"], 0)
    O, L = oatt.batch_decode(host(q), PoolView(k), PoolView(v), bt.numpy(), np.array(lens), P, 0.3)
    check_state(o, lse, O, L, dtype, "split plan", rounding_allowance=True)
    check_state(o_ref, l_ref, O, L, dtype, "no plan", rounding_allowance=True)


def test_plan_reuse_across_steps(api):
    """The workspace is sized from upper bounds: successive steps with new lengths re-plan
    into the same buffers (fixed pointers) and stay correct."""
    say("case: re-plan into the same workspace across steps")
    B, P, D = 12, 16, 128
    w = workloads.paged_decode(batch=B, heads=8, kv_heads=2, kv_len=2048, page_size=P, seed=9, device="cuda")
    params = api.make_params(B, 8, 2, D, P, num_ctas=40)
    ws = api.Workspace(params)
    rng = random.Random(1)
    for step in range(3):
        lens = [rng.randint(0, 2048) for _ in range(B)]
        info = api.plan(params, lens, workspace=ws)
        sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
        o, lse = api.batch_decode_paged(w.q, w.k_pool, w.v_pool, w.block_table, sl, sm_scale=w.sm_scale,
                                        plan_info=info)
        torch.cuda.synchronize()
        O, L = oatt.batch_decode(host(w.q), PoolView(w.k_pool), PoolView(w.v_pool), w.block_table.cpu().numpy(),
                                 np.array(lens), P, w.sm_scale)
        check_state(o, lse, O, L, torch.float16, f"step {step}")
