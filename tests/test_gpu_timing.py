"""Per-kernel timing hooks (pkc_timing_*): every timed launch is bracketed by a pair of events on
its stream, launches are counted per kernel kind, the measured durations are consistent with the
wall time of the runs, and a run captured into a graph while timing is on is captured without
events and replays as the eager run does (its replays are not counted)."""

import time

import torch

from paged_kv_cascade_amd import workloads
from tests.gpu_helpers import gpu, needs_gpu, say

pytestmark = [gpu, needs_gpu]

KIND_DECODE, KIND_PREFIX, KIND_MERGE_PLAN = 0, 1, 2


def _cascade(api, batch=24, prefix_len=2000, suffix_len=200):
    w = workloads.cascade_two_level(batch=batch, prefix_len=prefix_len, suffix_len=suffix_len,
                                    device="cuda", seed=7)
    levels = [{"qo_indptr": lv["qo_indptr"], "kv_lens": lv["kv_lens"]} for lv in w.levels]
    d, keep = api.level_dev(w.levels[0])
    params = api.make_params(w.batch, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size)
    ws = api.Workspace(params, levels)
    info = api.plan(params, w.cache_seqlens.cpu().tolist(), levels, workspace=ws)
    out = torch.empty_like(w.q)
    lse = torch.empty(w.batch, w.num_qo_heads, dtype=torch.float32, device="cuda")

    def run():
        api.cascade_decode(info, w.q, w.k_pool, w.v_pool, [d], w.block_table, w.cache_seqlens,
                           sm_scale=w.sm_scale, out=out, lse=lse)
    return run, out, lse, (w, d, keep, ws)


def test_timing_counts_launches_and_durations_fit_the_wall_time():
    from paged_kv_cascade_amd import api
    say("case: timing of 40 cascade runs (b24 prefix2000 suffix200 fp16)")
    run, out, lse, _keep = _cascade(api)
    for _ in range(5):
        run()
    torch.cuda.synchronize()
    n = 40
    api.timing_reset()
    api.timing_enable(True)
    try:
        t0 = time.perf_counter()
        for _ in range(n):
            run()
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3
        n_pre, ms_pre = api.timing_read(KIND_PREFIX)
        n_dec, ms_dec = api.timing_read(KIND_DECODE)
    finally:
        api.timing_enable(False)
    say(f"  prefix {n_pre} launches {ms_pre / max(n_pre, 1) * 1e3:.1f} us, decode {n_dec} launches "
        f"{ms_dec / max(n_dec, 1) * 1e3:.1f} us, wall {wall_ms / n * 1e3:.1f} us per run")
    assert n_pre == n and n_dec == n
    assert ms_pre > 0 and ms_dec > 0
    # The kernels of a run execute one after the other on one stream, so their measured times
    # add up to at most the wall time of the runs.
    assert ms_pre + ms_dec <= wall_ms * 1.02
    # Disabled: nothing more is counted.
    run()
    torch.cuda.synchronize()
    assert api.timing_read(KIND_PREFIX)[0] == n
    api.timing_reset()
    assert api.timing_read(KIND_PREFIX) == (0, 0.0)


def test_capture_with_timing_on_records_no_events_and_replays_equal_the_eager_run():
    from paged_kv_cascade_amd import api
    say("case: cascade run captured into a graph with timing on (b24 prefix2000 suffix200 fp16)")
    run, out, lse, _keep = _cascade(api)
    run()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    api.timing_reset()
    api.timing_enable(True)
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                run()
        torch.cuda.synchronize()
        assert api.timing_read(KIND_PREFIX)[0] == 0 and api.timing_read(KIND_DECODE)[0] == 0
        scratch = torch.zeros(1 << 20, device="cuda")
        for r in range(3):
            out.fill_(float("nan"))
            lse.fill_(float("nan"))
            scratch.add_(1.0)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {r} differs"
        assert api.timing_read(KIND_PREFIX)[0] == 0
        # An eager run after the capture is timed again.
        run()
        torch.cuda.synchronize()
        assert api.timing_read(KIND_PREFIX)[0] == 1 and api.timing_read(KIND_DECODE)[0] == 1
    finally:
        api.timing_enable(False)
        api.timing_reset()
