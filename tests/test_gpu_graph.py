"""Runs captured in a HIP graph and replayed after re-planning (FlashInfer paper summary, section
A3: the plan runs on the CPU outside the graph, the run is captured once; appendix D: fixed
pointers).  The plan is rebuilt into the same pinned buffer and device workspace between
replays, with split-KV on: the sequence of plans goes from no split request to split requests
and back, so the merge pass and the fold change what they do but not what is launched.  Every
replay is checked bitwise against the eager run of the same plan, with eager work and
synchronisations between replays, and against the oracle."""

import numpy as np
import torch

from oracle import attention as oatt
from paged_kv_cascade_amd import workloads
from tests.gpu_helpers import PoolView, check_state, gpu, host, needs_gpu, say

pytestmark = [gpu, needs_gpu]


def _capture(run):
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            run()
    torch.cuda.synchronize()
    return graph


def _replay_and_compare(graph, run, out, lse, label):
    """Eager run of the current plan, then three replays with eager work in between; every
    replay must equal the eager result bitwise."""
    run()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    scratch = torch.zeros(1 << 20, device="cuda")
    for r in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        scratch.add_(1.0)                       # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"{label}: replay {r} differs"


def test_captured_cascade_replays_across_split_and_unsplit_plans():
    from paged_kv_cascade_amd import api
    say("case: cascade_decode captured once, replayed under plans with and without split requests "
        "(b16 prefix1500 suffix<=300 fp16, split-KV on)")
    w = workloads.cascade_two_level(batch=16, prefix_len=1500, suffix_len=300, device="cuda", seed=31)
    levels = [{"qo_indptr": lv["qo_indptr"], "kv_lens": lv["kv_lens"]} for lv in w.levels]
    d, keep = api.level_dev(w.levels[0])
    params = api.make_params(w.batch, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                             num_ctas=16, level_ctas=4, enable_split=True)
    ws = api.Workspace(params, levels)
    out = torch.empty_like(w.q)
    lse = torch.empty(w.batch, w.num_qo_heads, dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(3)
    skew = rng.integers(1, 60, 16).tolist()
    skew[3], skew[9] = 300, 0                   # one long request (split), one with no own KV
    lens_seq = [[300] * 16, skew, rng.integers(257, 301, 16).tolist(), [300] * 16]

    def plan(lens):
        w.cache_seqlens.copy_(torch.tensor(lens, dtype=torch.int32))
        info = api.plan(params, lens, levels, workspace=ws)
        torch.cuda.synchronize()
        return info

    def run_with(info):
        return lambda: api.cascade_decode(info, w.q, w.k_pool, w.v_pool, [d], w.block_table, w.cache_seqlens,
                                          sm_scale=w.sm_scale, out=out, lse=lse)

    info0 = plan(lens_seq[0])
    assert info0.num_merge == 0
    graph = _capture(run_with(info0))
    merged = []
    for k, lens in enumerate(lens_seq):
        info = plan(lens)
        merged.append(info.num_merge)
        say(f"  plan {k}: L_kv={info.dec_kv_chunk} items={info.dec_items} merged requests={info.num_merge}")
        _replay_and_compare(graph, run_with(info), out, lse, f"cascade plan {k}")
        O, L = oatt.cascade_decode(host(w.q), PoolView(w.k_pool), PoolView(w.v_pool), w.page_size, w.sm_scale,
                                   w.levels, w.block_table.cpu().numpy(), w.cache_seqlens.cpu().numpy())
        check_state(out, lse, O, L, torch.float16, f"graph replay, plan {k}")
    assert merged[0] == 0 and merged[1] > 0, "the plans should go from no split to split requests"


def test_captured_split_decode_replays_across_plans():
    from paged_kv_cascade_amd import api
    say("case: batch_decode_paged (split-KV plan) captured once, replayed under plans with and without "
        "split requests (b24 h8/2 d128 bf16)")
    B, P = 24, 16
    w = workloads.paged_decode(batch=B, heads=8, kv_heads=2, kv_len=2048, page_size=P, dtype=torch.bfloat16,
                               seed=37, device="cuda")
    params = api.make_params(B, 8, 2, 128, P, num_ctas=24)
    ws = api.Workspace(params)
    out = torch.empty_like(w.q)
    lse = torch.empty(B, 8, dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(5)
    uneven = rng.integers(0, 300, B).tolist()
    uneven[0] = 2048
    lens_seq = [[2048] * B, uneven, rng.integers(1500, 2049, B).tolist()]

    def plan(lens):
        w.cache_seqlens.copy_(torch.tensor(lens, dtype=torch.int32))
        info = api.plan(params, lens, workspace=ws)
        torch.cuda.synchronize()
        return info

    def run_with(info):
        return lambda: api.batch_decode_paged(w.q, w.k_pool, w.v_pool, w.block_table, w.cache_seqlens,
                                              sm_scale=w.sm_scale, plan_info=info, out=out, lse=lse)

    info0 = plan(lens_seq[0])
    graph = _capture(run_with(info0))
    merged = []
    for k, lens in enumerate(lens_seq):
        info = plan(lens)
        merged.append(info.num_merge)
        say(f"  plan {k}: L_kv={info.dec_kv_chunk} items={info.dec_items} merged requests={info.num_merge}")
        _replay_and_compare(graph, run_with(info), out, lse, f"decode plan {k}")
        O, L = oatt.batch_decode(host(w.q), PoolView(w.k_pool), PoolView(w.v_pool), w.block_table.cpu().numpy(),
                                 np.array(lens), P, w.sm_scale)
        check_state(out, lse, O, L, torch.bfloat16, f"graph replay, decode plan {k}")
    assert merged[0] == 0 and merged[1] > 0, "the plans should go from no split to split requests"
