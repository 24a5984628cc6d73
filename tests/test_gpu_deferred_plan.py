"""Plans built with defer_upload = 1: pkc_plan enqueues no copy, and the run brings the plan
over from its page-locked host buffer (a cascade's, prefix attention's or batch prefill's
first level kernel reads its own items from the host buffer and copies the plan into the
workspace; the batch decode and the debug trace enqueue the copy first).  Before each
deferred run the workspace's copy of the integer arrays is zeroed (an all-zero plan is an
empty work list), so a run that read the workspace instead of the host buffer, or a copy that
missed words, shows in the results.  Every result must equal, bit for bit, the run of the same
plan copied by pkc_plan."""

import random

import pytest
import torch

from paged_kv_cascade_amd import workloads
from tests.gpu_helpers import gpu, needs_gpu, say
from tests.test_gpu_cascade import _small_cascade
from tests.test_gpu_prefill import _case as _prefill_case

pytestmark = [gpu, needs_gpu]


@pytest.fixture(scope="module")
def api():
    from paged_kv_cascade_amd import api as _api
    return _api


def _zero_plan_copy(ws, info):
    ws.device[:info.int_bytes].zero_()


def _levels(api, w):
    host_levels = [{"qo_indptr": lv["qo_indptr"], "kv_lens": lv["kv_lens"]} for lv in w.levels]
    devs, keep = [], []
    for lv in w.levels:
        d, k = api.level_dev(lv)
        devs.append(d)
        keep.append(k)
    return host_levels, devs, keep


def _cascade(api, w, info, devs, seqlens):
    o, lse = api.cascade_decode(info, w.q, w.k_pool, w.v_pool, devs, w.block_table, seqlens,
                                sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    return o, lse


def _same(a, b, label):
    assert torch.equal(a[0], b[0]), f"{label}: O differs"
    assert torch.equal(a[1], b[1]), f"{label}: LSE differs"


@pytest.mark.parametrize("seed", range(6))
def test_cascade_deferred_plan(api, seed):
    """Random small cascades, default and small grids; then a second step whose suffixes are
    shorter, planned into a second host buffer over the same workspace."""
    dtype = [torch.float16, torch.bfloat16][seed % 2]
    D = [128, 64][(seed // 2) % 2]
    g = [1, 4, 2][seed % 3]
    P = [16, 4, 32][(seed + 1) % 3]
    w = _small_cascade(300 + seed, dtype, D, g, P)
    host_levels, devs, keep = _levels(api, w)
    lens = w.cache_seqlens.cpu().tolist()
    lens2 = [n // 2 for n in lens]
    sl2 = torch.tensor(lens2, dtype=torch.int32, device="cuda")
    say(f"case: deferred plan, small cascade seed={300 + seed} {dtype} D={D} g={g} P={P} B={w.batch} "
        f"levels={len(w.levels)}")
    for kw in (dict(), dict(num_ctas=7, level_ctas=3)):
        shape = (w.batch, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size)
        p0 = api.make_params(*shape, **kw)
        p1 = api.make_params(*shape, **kw, defer_upload=True)
        ws0 = api.Workspace(p0, host_levels)
        ref1 = _cascade(api, w, api.plan(p0, lens, host_levels, workspace=ws0), devs, w.cache_seqlens)
        ref2 = _cascade(api, w, api.plan(p0, lens2, host_levels, workspace=ws0), devs, sl2)
        wa = api.Workspace(p1, host_levels)
        wb = api.Workspace(p1, host_levels)
        wb.device = wa.device
        info = api.plan(p1, lens, host_levels, workspace=wa)
        assert info.host_src == wa.host.data_ptr()
        _zero_plan_copy(wa, info)
        _same(_cascade(api, w, info, devs, w.cache_seqlens), ref1, f"{kw} step 1")
        info = api.plan(p1, lens2, host_levels, workspace=wb)
        _zero_plan_copy(wb, info)
        _same(_cascade(api, w, info, devs, sl2), ref2, f"{kw} step 2")
        # the same plan run twice (the second run copies it again)
        _same(_cascade(api, w, info, devs, sl2), ref2, f"{kw} step 2 again")


def test_headline_cascade_deferred_plan(api):
    say("case: deferred plan, two-level cascade prefix32768 suffix256 b128 h32 d128 p16 fp16")
    w = workloads.cascade_two_level(device="cuda")
    host_levels, devs, keep = _levels(api, w)
    lens = w.cache_seqlens.cpu().tolist()
    shape = (w.batch, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size)
    p0 = api.make_params(*shape)
    p1 = api.make_params(*shape, defer_upload=True)
    ws0 = api.Workspace(p0, host_levels)
    ref = _cascade(api, w, api.plan(p0, lens, host_levels, workspace=ws0), devs, w.cache_seqlens)
    ws1 = api.Workspace(p1, host_levels)
    info = api.plan(p1, lens, host_levels, workspace=ws1)
    _zero_plan_copy(ws1, info)
    _same(_cascade(api, w, info, devs, w.cache_seqlens), ref, "headline cascade")


def test_split_decode_deferred_plan(api):
    """Batch decode with a split plan: the decode call enqueues the copy before its kernel."""
    B, P = 48, 16
    say("case: deferred plan, split batch decode b48 hq8 hkv2 d128 fp16")
    w = workloads.paged_decode(batch=B, heads=8, kv_heads=2, kv_len=3000, page_size=P, seed=23, device="cuda")
    rng = random.Random(9)
    lens = [rng.choice([0, 7, rng.randint(1, 3000)]) for _ in range(B)]
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    outs = []
    for defer in (False, True):
        p = api.make_params(B, 8, 2, 128, P, num_ctas=40, defer_upload=defer)
        ws = api.Workspace(p)
        info = api.plan(p, lens, workspace=ws)
        assert info.num_merge > 0 and (info.host_src != 0) == defer
        if defer:
            _zero_plan_copy(ws, info)
        o, lse = api.batch_decode_paged(w.q, w.k_pool, w.v_pool, w.block_table, sl, sm_scale=w.sm_scale,
                                        plan_info=info)
        torch.cuda.synchronize()
        outs.append((o, lse))
    _same(outs[1], outs[0], "split decode")


def test_prefix_attention_and_trace_deferred_plan(api):
    say("case: deferred plan, prefix_attention of each level and the CTA trace")
    w = _small_cascade(101, torch.float16, 128, 1, 16)
    host_levels, devs, keep = _levels(api, w)
    lens = w.cache_seqlens.cpu().tolist()
    shape = (w.batch, w.num_qo_heads, w.num_kv_heads, 128, 16)
    p0 = api.make_params(*shape, num_ctas=8, level_ctas=5)
    p1 = api.make_params(*shape, num_ctas=8, level_ctas=5, defer_upload=True)
    ws0 = api.Workspace(p0, host_levels)
    info0 = api.plan(p0, lens, host_levels, workspace=ws0)
    ws1 = api.Workspace(p1, host_levels)
    for l in range(len(w.levels)):
        ref = api.prefix_attention(info0, l, w.q, w.k_pool, w.v_pool, devs[l], sm_scale=w.sm_scale)
        info1 = api.plan(p1, lens, host_levels, workspace=ws1)
        _zero_plan_copy(ws1, info1)
        got = api.prefix_attention(info1, l, w.q, w.k_pool, w.v_pool, devs[l], sm_scale=w.sm_scale)
        torch.cuda.synchronize()
        _same(got, ref, f"level {l}")
    for stage in range(len(w.levels) + 1):
        t0 = api.debug_cta_trace(info0, stage, 64)
        info1 = api.plan(p1, lens, host_levels, workspace=ws1)
        _zero_plan_copy(ws1, info1)
        t1 = api.debug_cta_trace(info1, stage, 64)
        torch.cuda.synchronize()
        assert torch.equal(t0, t1), f"stage {stage}: CTA trace differs"


@pytest.mark.parametrize("level_ctas", [1, 3])
def test_prefill_deferred_plan(api, level_ctas):
    """Causal ragged prefill; with one or three level CTAs the plan holds more words than the
    level grid has threads, so the kernel copies the rest after its items."""
    lq, lkv = [300, 33, 130, 2], [300, 40, 600, 2]
    say(f"case: deferred plan, causal prefill lq={lq} lkv={lkv} fp16 D128 g1 P16 level_ctas={level_ctas}")
    q, k, v, bt = _prefill_case(77, lq, lkv, torch.float16, 128, 1, 16, hkv=2)
    qi_d = None
    outs = []
    for defer in (False, True):
        info, ws, qi = api.prefill_plan(lq, lkv, 2, 2, 128, 16, level_ctas=level_ctas, defer_upload=defer)
        if defer:
            assert info.int_bytes // 4 > level_ctas * 2 * 512, "the plan should exceed the grid's threads"
            _zero_plan_copy(ws, info)
        qi_d = torch.tensor(qi, dtype=torch.int32, device="cuda")
        kv_d = torch.tensor(lkv, dtype=torch.int32, device="cuda")
        o, lse = api.batch_prefill_paged(info, q, k, v, bt.cuda(), qi_d, kv_d, causal=True,
                                         sm_scale=128 ** -0.5)
        torch.cuda.synchronize()
        outs.append((o, lse))
    _same(outs[1], outs[0], "prefill")


def test_deferred_plan_needs_pinned_host_buffer(api):
    p = api.make_params(4, 8, 2, 128, 16, num_ctas=4, defer_upload=True)
    ws = api.Workspace(p)
    ws.host = torch.zeros(ws.host.numel(), dtype=torch.uint8)   # pageable
    with pytest.raises(api.PkcError) as e:
        api.plan(p, [5, 0, 17, 300], workspace=ws)
    assert e.value.status == 1


def test_alternating_host_buffers_deferred_plan(api):
    """Four steps over two host buffers (A, B, A, B), each with other suffix lengths: every run
    reads the plan its buffer holds now, not what the buffer held two steps before."""
    say("case: deferred plan, host buffers A B A B with a different plan each step")
    w = _small_cascade(411, torch.float16, 128, 1, 16)
    host_levels, devs, keep = _levels(api, w)
    lens0 = w.cache_seqlens.cpu().tolist()
    shape = (w.batch, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size)
    p0 = api.make_params(*shape, num_ctas=7, level_ctas=3)
    p1 = api.make_params(*shape, num_ctas=7, level_ctas=3, defer_upload=True)
    ws0 = api.Workspace(p0, host_levels)
    bufs = [api.Workspace(p1, host_levels) for _ in range(2)]
    bufs[1].device = bufs[0].device
    for step, div in enumerate((1, 2, 3, 5)):
        lens = [n // div for n in lens0]
        sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
        ref = _cascade(api, w, api.plan(p0, lens, host_levels, workspace=ws0), devs, sl)
        ws = bufs[step % 2]
        info = api.plan(p1, lens, host_levels, workspace=ws)
        _zero_plan_copy(ws, info)
        _same(_cascade(api, w, info, devs, sl), ref, f"step {step}")


@pytest.mark.parametrize("seed", range(3))
def test_fp8_cascade_deferred_plan(api, seed):
    """Cascades over E4M3 pools: the FP8 level kernel brings a deferred plan over the same way."""
    qdt = [torch.float16, torch.bfloat16, torch.float16][seed]
    D, g, P = [(128, 1, 16), (64, 4, 4), (128, 2, 32)][seed]
    w = _small_cascade(520 + seed, qdt, D, g, P)
    k8 = workloads.fp8_e4m3_pool(w.k_pool, 0.5)
    v8 = workloads.fp8_e4m3_pool(w.v_pool, 0.25)
    host_levels, devs, keep = _levels(api, w)
    lens = w.cache_seqlens.cpu().tolist()
    say(f"case: deferred plan, fp8 small cascade seed={520 + seed} q {qdt} D={D} g={g} P={P} B={w.batch}")
    shape = (w.batch, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size)
    outs = []
    for defer in (False, True):
        p = api.make_params(*shape, num_ctas=9, level_ctas=2, defer_upload=defer)
        ws = api.Workspace(p, host_levels)
        info = api.plan(p, lens, host_levels, workspace=ws)
        if defer:
            _zero_plan_copy(ws, info)
        o, lse = api.cascade_decode_fp8(info, w.q, k8, v8, devs, w.block_table, w.cache_seqlens,
                                        k_scale=0.5, v_scale=0.25, sm_scale=w.sm_scale)
        torch.cuda.synchronize()
        outs.append((o, lse))
    _same(outs[1], outs[0], "fp8 cascade")
