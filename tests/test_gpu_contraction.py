"""Attention and contraction in one launch (FlashInfer paper summary, section A3: the partial
outputs of split KV are contracted by the same persistent kernel, with a grid fixed by the
parameters).  With contraction = 1 the decode kernel merges every split request itself (the
workgroup whose partial state arrives last) and also writes the requests that have no decode
item; with contraction = 2 a merge pass follows.  Both use the same merge arithmetic in the
same order, so their outputs must agree bit for bit; each is also checked against the oracle.
Runs are repeated, since the arrival counters must be back at zero after every run."""

import random

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from paged_kv_cascade_amd import workloads
from tests.gpu_helpers import FULL_SIZE_HEADS, HostPool, PoolView, check_state, gpu, host, needs_gpu, say
from tests.test_gpu_cascade import _oracle, _small_cascade
from tests.test_gpu_fp8 import _oracle as _fp8_oracle

pytestmark = [gpu, needs_gpu]


@pytest.fixture(scope="module")
def api():
    from paged_kv_cascade_amd import api as _api
    return _api


def _decode_both(api, run, params_kw, lens):
    """Runs `run(info)` under both contraction modes (three times in-kernel) and returns the
    in-kernel result after checking the two modes agree bitwise."""
    outs = {}
    for mode in (1, 2):
        params = api.make_params(**params_kw, contraction=mode)
        ws = api.Workspace(params)
        info = api.plan(params, lens, workspace=ws)
        assert info.dec_contraction == mode
        reps = 3 if mode == 1 else 1
        res = []
        for _ in range(reps):
            o, lse = run(info)
            torch.cuda.synchronize()
            res.append((o.clone(), lse.clone()))
        for r in res[1:]:
            assert torch.equal(r[0], res[0][0]) and torch.equal(r[1], res[0][1]), "repeat run differs"
        outs[mode] = res[0]
        outs["info"] = info
    (o1, l1), (o2, l2) = outs[1], outs[2]
    assert torch.equal(o1, o2), f"in-kernel vs pass: max |dO| {float((o1.float() - o2.float()).abs().max())}"
    assert torch.equal(l1, l2), "in-kernel vs pass: LSE differs"
    return o1, l1, outs["info"]


@pytest.mark.parametrize("seed", range(6))
def test_split_decode_contraction_modes(api, seed):
    rng = random.Random(100 + seed)
    dtype = [torch.float16, torch.bfloat16, torch.float32][seed % 3]
    D = [128, 64][seed % 2]
    g = [1, 4, 8, 2, 1, 4][seed]
    P = [16, 4, 32, 1, 8, 16][seed]
    hkv = 2
    B = rng.randint(5, 40)
    lens = [rng.choice([0, 1, P, rng.randint(1, 3000), rng.randint(2000, 5000)]) for _ in range(B)]
    lens[0] = 0                      # a request with no decode item (written by the kernel)
    lens[-1] = 4000                  # and one that is split
    ctas = rng.choice([3, 16, 64])
    say(f"case: contraction modes, split decode seed={seed} {dtype} D={D} g={g} P={P} B={B} ctas={ctas}")
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
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    btd = bt.cuda()
    kw = dict(batch=B, num_qo_heads=hkv * g, num_kv_heads=hkv, head_dim=D, page_size=P, num_ctas=ctas)
    o, lse, info = _decode_both(api, lambda info: api.batch_decode_paged(q, k, v, btd, sl, sm_scale=0.3,
                                                                          plan_info=info), kw, lens)
    say(f"  plan: L_kv={info.dec_kv_chunk} items={info.dec_items} merged={info.num_merge}")
    assert info.num_merge > 0
    O, L = oatt.batch_decode(host(q), PoolView(k), PoolView(v), bt.numpy(), np.array(lens), P, 0.3)
    check_state(o, lse, O, L, dtype, "in-kernel contraction", rounding_allowance=True)


def test_gqa_split_full_size_contraction_modes(api):
    say("case: contraction modes, GQA split-KV b256 hq32 hkv8 d128 bf16, plan #CTA = 2 x CUs")
    w = workloads.gqa_split(device="cuda")
    cus = api.device_info(0)["num_cus"]
    lens = w.cache_seqlens.cpu().tolist()
    kw = dict(batch=w.batch, num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16, num_ctas=2 * cus)
    o, lse, info = _decode_both(api, lambda info: api.batch_decode_paged(
        w.q, w.k_pool, w.v_pool, w.block_table, w.cache_seqlens, sm_scale=w.sm_scale, plan_info=info), kw, lens)
    say(f"  plan: L_kv={info.dec_kv_chunk} items={info.dec_items} merged={info.num_merge}")
    O, L = oatt.batch_decode(host(w.q), HostPool(w.k_pool), HostPool(w.v_pool), w.block_table.cpu().numpy(),
                             np.array(lens), 16, w.sm_scale, heads=FULL_SIZE_HEADS)
    check_state(o, lse, O, L, torch.bfloat16, "GQA split-KV, in-kernel contraction")


def test_fp8_split_contraction_modes(api):
    say("case: contraction modes, fp8 split decode b48 hq8 hkv2 d128 fp16 q")
    B, P = 48, 16
    w = workloads.paged_decode(batch=B, heads=8, kv_heads=2, kv_len=3000, page_size=P, seed=21, device="cuda")
    k8 = workloads.fp8_e4m3_pool(w.k_pool, 0.5)
    v8 = workloads.fp8_e4m3_pool(w.v_pool, 0.5)
    rng = random.Random(4)
    lens = [rng.choice([0, 7, rng.randint(1, 3000)]) for _ in range(B)]
    lens[1] = 3000
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    kw = dict(batch=B, num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=P, num_ctas=40)
    o, lse, info = _decode_both(api, lambda info: api.batch_decode_paged_fp8(
        w.q, k8, v8, w.block_table, sl, k_scale=0.5, v_scale=0.5, sm_scale=w.sm_scale, plan_info=info), kw, lens)
    assert info.num_merge > 0
    O, L = _fp8_oracle(w.q, k8, v8, 0.5, 0.5, w.block_table, sl, P, w.sm_scale)
    check_state(o, lse, O, L, torch.float16, "fp8 in-kernel contraction")


@pytest.mark.parametrize("seed", range(8))
def test_cascade_contraction_modes(api, seed):
    """Random small cascades (some requests with no own KV, some split suffixes, some with no
    level): both contraction modes bitwise, then the oracle."""
    dtype = [torch.float16, torch.bfloat16][seed % 2]
    D = [128, 64][(seed // 2) % 2]
    g = [1, 4, 2, 8][(seed // 4) % 4]
    P = [16, 4, 32][seed % 3]
    w = _small_cascade(200 + seed, dtype, D, g, P)
    host_levels = [{"qo_indptr": lv["qo_indptr"], "kv_lens": lv["kv_lens"]} for lv in w.levels]
    devs, keep = [], []
    for lv in w.levels:
        d, kk = api.level_dev(lv)
        devs.append(d)
        keep.append(kk)
    say(f"case: contraction modes, small cascade seed={200 + seed} {dtype} D={D} g={g} P={P} B={w.batch} "
        f"levels={len(w.levels)}")
    outs = {}
    for mode in (1, 2):
        params = api.make_params(w.batch, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                                 num_ctas=7, level_ctas=3, contraction=mode)
        ws = api.Workspace(params, host_levels)
        info = api.plan(params, w.cache_seqlens.cpu().tolist(), host_levels, workspace=ws)
        res = []
        for _ in range(2 if mode == 1 else 1):
            o, lse = api.cascade_decode(info, w.q, w.k_pool, w.v_pool, devs, w.block_table, w.cache_seqlens,
                                        sm_scale=w.sm_scale)
            torch.cuda.synchronize()
            res.append((o, lse))
        if mode == 1:
            assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1]), "repeat run differs"
            say(f"  plan: suffix items={info.dec_items} merged={info.num_merge}")
        outs[mode] = res[0]
    assert torch.equal(outs[1][0], outs[2][0]) and torch.equal(outs[1][1], outs[2][1]), "in-kernel vs pass differ"
    O, L = _oracle(w)
    check_state(outs[1][0], outs[1][1], O, L, dtype, f"cascade {seed}, in-kernel contraction",
                rounding_allowance=True)
