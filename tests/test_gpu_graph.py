"""The cascade run captured in a HIP graph and replayed (fixed pointers: the plan is rebuilt
on the CPU into the same pinned buffer and device workspace between replays, as the
FlashInfer paper's appendix D describes for CUDA graphs).  Every replay is checked against
the eager run of the same plan, with eager work and synchronisations between replays."""

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from paged_kv_cascade_amd import workloads
from tests.gpu_helpers import PoolView, check_state, gpu, host, needs_gpu, say

pytestmark = [gpu, needs_gpu]


def test_captured_cascade_replays_with_new_plans():
    from paged_kv_cascade_amd import api
    say("case: cascade_decode captured in a graph, replayed under three plans (b16 prefix1500 suffix<=300 fp16)")
    w = workloads.cascade_two_level(batch=16, prefix_len=1500, suffix_len=300, device="cuda", seed=31)
    levels = [{"qo_indptr": lv["qo_indptr"], "kv_lens": lv["kv_lens"]} for lv in w.levels]
    d, keep = api.level_dev(w.levels[0])
    # Fixed launch structure for replays: decode waves fixed, no split-KV (so no merge launch).
    params = api.make_params(w.batch, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                             num_ctas=16, level_ctas=4, enable_split=False, decode_waves=4)
    ws = api.Workspace(params, levels)
    out = torch.empty_like(w.q)
    lse = torch.empty(w.batch, w.num_qo_heads, dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(3)
    lens_seq = [[300] * 16, rng.integers(260, 301, 16).tolist(), rng.integers(257, 301, 16).tolist()]

    def plan(lens):
        w.cache_seqlens.copy_(torch.tensor(lens, dtype=torch.int32))
        info = api.plan(params, lens, levels, workspace=ws)
        torch.cuda.synchronize()
        return info

    def run(info):
        api.cascade_decode(info, w.q, w.k_pool, w.v_pool, [d], w.block_table, w.cache_seqlens,
                           sm_scale=w.sm_scale, out=out, lse=lse)

    info0 = plan(lens_seq[0])
    run(info0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            run(info0)
    torch.cuda.synchronize()
    sig0 = (info0.dec_waves, info0.num_merge > 0)
    scratch = torch.zeros(1 << 20, device="cuda")
    for k, lens in enumerate(lens_seq):
        info = plan(lens)
        assert (info.dec_waves, info.num_merge > 0) == sig0, "plan changed the launch structure"
        run(info)
        torch.cuda.synchronize()
        ref_o, ref_l = out.clone(), lse.clone()
        for r in range(3):
            out.fill_(float("nan"))
            scratch.add_(1.0)                       # eager work between replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"plan {k} replay {r} differs"
        O, L = oatt.cascade_decode(host(w.q), PoolView(w.k_pool), PoolView(w.v_pool), w.page_size, w.sm_scale,
                                   w.levels, w.block_table.cpu().numpy(), w.cache_seqlens.cpu().numpy())
        check_state(out, lse, O, L, torch.float16, f"graph replay, plan {k}")
