"""Allocation-free split-KV decode (pkc_batch_decode_paged_noalloc): the plan is built on the
host (pkc_plan_host) and the workspace is the library's fixed device array.  Two calls in a row,
the second with a smaller input; each must equal pkc_batch_decode_paged with a caller workspace
and the same plan bitwise, and match the oracle within |dO| <= 2e-3, |dLSE| <= 1e-3 (bf16 inputs,
fp32 accumulation).  A plan larger than the array is refused before any launch."""

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from paged_kv_cascade_amd import workloads
from tests.gpu_helpers import FULL_SIZE_HEADS, HostPool, check_state, gpu, host, needs_gpu, say

pytestmark = [gpu, needs_gpu]


def _one_call(api, w, num_ctas, label):
    lens = w.cache_seqlens.cpu().tolist()
    params = api.make_params(w.batch, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                             num_ctas=num_ctas, level_ctas=1)
    hb, _ = api.plan_buffer_sizes(params)
    host_buf = torch.zeros(max(hb, 16), dtype=torch.uint8, pin_memory=True)
    info_h, _ = api.plan_host(params, lens, host_buf=host_buf)
    assert info_h.num_merge > 0, "the plan should split some requests"
    assert info_h.dev_bytes <= api.NOALLOC_SCRATCH_BYTES
    out = torch.full_like(w.q, float("nan"))
    lse = torch.full((w.batch, w.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
    api.batch_decode_paged_noalloc(info_h, host_buf, w.q, w.k_pool, w.v_pool, w.block_table, w.cache_seqlens,
                                   sm_scale=w.sm_scale, out=out, lse=lse)
    # the existing entry point with a caller workspace and the same plan
    ws = api.Workspace(params)
    info = api.plan(params, lens, workspace=ws)
    ref_o, ref_l = api.batch_decode_paged(w.q, w.k_pool, w.v_pool, w.block_table, w.cache_seqlens,
                                          sm_scale=w.sm_scale, plan_info=info)
    torch.cuda.synchronize()
    say(f"  {label}: items={info_h.dec_items} merged requests={info_h.num_merge} "
        f"workspace bytes={info_h.dev_bytes}")
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"{label}: differs from the workspace call"
    O, L = oatt.batch_decode(host(w.q), HostPool(w.k_pool), HostPool(w.v_pool), w.block_table.cpu().numpy(),
                             np.array(lens), w.page_size, w.sm_scale, heads=FULL_SIZE_HEADS)
    check_state(out, lse, O, L, w.dtype, label)


def test_noalloc_decode_matches_workspace_call_twice():
    from paged_kv_cascade_amd import api
    say("case: allocation-free split-KV decode, b96 hq32 hkv8 d128 bf16 log-uniform 128..8192, #CTA 256; "
        "then b20 log-uniform 128..2000, #CTA 64")
    w1 = workloads.gqa_split(batch=96, lo=128, hi=8192, seed=1104, device="cuda")
    _one_call(api, w1, 256, "first call")
    w2 = workloads.gqa_split(batch=20, lo=128, hi=2000, seed=1105, device="cuda")
    _one_call(api, w2, 64, "second call (smaller)")


def test_noalloc_refuses_a_plan_larger_than_its_array():
    from paged_kv_cascade_amd import api
    say("case: allocation-free decode refuses a plan whose workspace exceeds the array")
    B = 4096
    params = api.make_params(B, 32, 32, 128, 16, num_ctas=B, level_ctas=1)
    info, hb = api.plan_host(params, [64] * B)
    assert info.dev_bytes > api.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, 32, 128, dtype=torch.float16, device="cuda")
    pool = torch.zeros(4, 16, 32, 128, dtype=torch.float16, device="cuda")
    bt = torch.zeros(B, 4, dtype=torch.int32, device="cuda")
    lens = torch.full((B,), 64, dtype=torch.int32, device="cuda")
    with pytest.raises(api.PkcError) as e:
        api.batch_decode_paged_noalloc(info, hb, q, pool, pool, bt, lens)
    assert e.value.status == 3 and "allocation-free" in str(e.value)
