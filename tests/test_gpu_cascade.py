"""GPU parity of the cascade: MFMA multi-query prefix kernel per level, suffix decode,
and the final merge, against the oracle's single softmax over each request's union
of token sets."""

import math
import random

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from paged_kv_cascade_amd import workloads
from tests.gpu_helpers import FULL_SIZE_HEADS, HostPool, PoolView, check_state, gpu, host, needs_gpu, say

pytestmark = [gpu, needs_gpu]


@pytest.fixture(scope="module")
def api():
    from paged_kv_cascade_amd import api as _api
    return _api


def _run_cascade(api, w, level_ctas=0, num_ctas=0, enable_split=True, tile_q=0):
    params = api.make_params(w.batch, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                             num_ctas=num_ctas, level_ctas=level_ctas, level_tile_q=tile_q,
                             enable_split=enable_split)
    host_levels = [{"qo_indptr": lv["qo_indptr"], "kv_lens": lv["kv_lens"]} for lv in w.levels]
    ws = api.Workspace(params, host_levels)
    info = api.plan(params, w.cache_seqlens.cpu().tolist(), host_levels, workspace=ws)
    devs, keep = [], []
    for lv in w.levels:
        d, k = api.level_dev(lv)
        devs.append(d)
        keep.append(k)
    o, lse = api.cascade_decode(info, w.q, w.k_pool, w.v_pool, devs, w.block_table, w.cache_seqlens,
                                sm_scale=w.sm_scale)
    return o, lse, info, ws, devs, keep


def _oracle(w, requests=None, heads=None, pools=None):
    kp, vp = pools if pools is not None else (PoolView(w.k_pool), PoolView(w.v_pool))
    return oatt.cascade_decode(host(w.q), kp, vp, w.page_size, w.sm_scale,
                               w.levels, w.block_table.cpu().numpy(), w.cache_seqlens.cpu().numpy(),
                               requests=requests, heads=heads)


def _level_grid(api, grid, hkv):
    """level_ctas of a grid choice: the default (one 8-wave workgroup per compute unit) or two
    4-wave workgroups per compute unit."""
    return 0 if grid == "default" else 2 * api.device_info(0)["num_cus"] // hkv


@pytest.mark.parametrize("grid", ["default", "two_per_cu"])
def test_two_level_cascade_full_size(api, grid):
    """Shared prefix 32768 tokens (pages 0..2047) + 256 unique tokens per request in
    permuted pages, batch 128, 32 heads x 128, fp16."""
    say(f"case: two-level cascade prefix32768 suffix256 b128 h32 d128 p16 fp16 level grid {grid} "
        "(full size, every request on heads 0, 13, 31)")
    w = workloads.cascade_two_level(device="cuda")
    api.validate_block_table(w.block_table.cpu(), w.cache_seqlens.cpu(), w.page_size, w.num_pages)
    lc = _level_grid(api, grid, w.num_kv_heads)
    o, lse, info, ws, devs, keep = _run_cascade(api, w, level_ctas=lc)
    o2, lse2, *_ = _run_cascade(api, w, level_ctas=lc)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "repeat run differs"
    say(f"  plan: level chunk={info.lvl_kv_chunk[0]} level items={info.lvl_items[0]} "
        f"suffix items={info.dec_items} rows={info.state_rows}")
    O, L = _oracle(w, heads=FULL_SIZE_HEADS, pools=(HostPool(w.k_pool), HostPool(w.v_pool)))
    check_state(o, lse, O, L, torch.float16, "cascade 32K prefix")


@pytest.mark.parametrize("grid", ["default", "two_per_cu"])
def test_multi_level_cascade_full_size(api, grid):
    """Global prefix 16384 + 4 groups x 4096 + 512 per request, batch 128, fp16."""
    say(f"case: three-level cascade 16384 + 4x4096 + 512, b128 h32 d128 fp16 level grid {grid} "
        "(full size, every request on heads 0, 13, 31)")
    w = workloads.cascade_multi_level(device="cuda")
    o, lse, info, *_ = _run_cascade(api, w, level_ctas=_level_grid(api, grid, w.num_kv_heads))
    torch.cuda.synchronize()
    O, L = _oracle(w, heads=FULL_SIZE_HEADS, pools=(HostPool(w.k_pool), HostPool(w.v_pool)))
    check_state(o, lse, O, L, torch.float16, "cascade 3 levels")


def _small_cascade(seed, dtype, D, g, P, hkv=2):
    rng = random.Random(seed)
    B = rng.randint(3, 70)
    n_lv = rng.randint(1, 3)
    levels_spec = []
    for _ in range(n_lv):
        G = rng.randint(1, 4)
        cuts = sorted(set([0, B] + rng.sample(range(1, B), min(G - 1, B - 1))))
        if rng.random() < 0.3:
            cuts = cuts[:-1] + [max(cuts[-2], B - rng.randint(0, 2))]   # leave some requests uncovered
        kv = [rng.choice([0, 1, P + 1, 63, 64, 65, rng.randint(1, 900)]) for _ in range(len(cuts) - 1)]
        levels_spec.append((cuts, kv))
    suffix = [rng.choice([0, 1, rng.randint(1, 300)]) for _ in range(B)]
    # page placement: every level group's run and every suffix get distinct pages
    need = sum(-(-n // P) for _, kv in levels_spec for n in kv) + sum(-(-n // P) for n in suffix) + 4
    perm = torch.randperm(need, generator=torch.Generator().manual_seed(seed)).tolist()
    pos = 0
    levels = []
    used = torch.zeros(need, P, dtype=torch.bool)
    for cuts, kv in levels_spec:
        runs = []
        for n in kv:
            k = -(-n // P)
            runs.append(perm[pos:pos + k])
            for t in range(n):
                used[runs[-1][t // P], t % P] = True
            pos += k
        lv = workloads._level(cuts, runs, kv)
        levels.append(lv)
    spg = [-(-n // P) for n in suffix]
    bt = torch.full((B, max(spg) + 1), -1, dtype=torch.int32)
    for b, k in enumerate(spg):
        bt[b, :k] = torch.tensor(perm[pos:pos + k], dtype=torch.int32)
        for t in range(suffix[b]):
            used[int(bt[b, t // P]), t % P] = True
        pos += k
    gen = torch.Generator(device="cuda").manual_seed(seed)
    q = (torch.randn(B, hkv * g, D, generator=gen, device="cuda") * 0.5).to(dtype)
    k = (torch.randn(need, P, hkv, D, generator=gen, device="cuda") * 0.5).to(dtype)
    v = (torch.randn(need, P, hkv, D, generator=gen, device="cuda") * 0.5).to(dtype)
    k[~used.cuda()] = float("nan")
    v[~used.cuda()] = float("nan")
    return workloads.Workload(f"small_cascade_{seed}", B, hkv * g, hkv, D, P, dtype, 1.0 / math.sqrt(D),
                              q, k, v, bt.cuda(), torch.tensor(suffix, dtype=torch.int32, device="cuda"),
                              None, levels, seed)


@pytest.mark.parametrize("seed", range(12))
def test_small_cascades(api, seed):
    dtype = [torch.float16, torch.bfloat16][seed % 2]
    D = [128, 64][(seed // 2) % 2]
    g = [1, 4, 2, 8][(seed // 4) % 4]
    P = [16, 4, 32][seed % 3]
    w = _small_cascade(seed, dtype, D, g, P)
    lctas = [1, 3, 8][seed % 3]
    tile_q = [0, 16 // g if g < 16 else 1, 128 // g][seed % 3]
    say(f"case: small cascade seed={seed} {dtype} D={D} g={g} P={P} B={w.batch} levels={len(w.levels)} "
        f"level_ctas={lctas} tile_q={tile_q}")
    o, lse, info, ws, devs, keep = _run_cascade(api, w, level_ctas=lctas, num_ctas=13, tile_q=tile_q)
    torch.cuda.synchronize()
    arr = api.read_plan_arrays(info, ws.host)
    for l in range(info.num_levels):
        lists = arr["levels"][l]
        mx = max([1] + [len(c) for c in lists])
        tr = api.debug_cta_trace(info, l, mx).cpu().numpy()
        for c, recs in enumerate(lists):
            for kk in range(mx):
                assert tr[c, kk].tolist() == (list(recs[kk]) if kk < len(recs) else [-1] * 8)
    O, L = _oracle(w)
    check_state(o, lse, O, L, dtype, f"small cascade {seed}", rounding_allowance=True)


def test_prefix_attention_standalone(api):
    say("case: prefix_attention of each level vs the oracle's level states")
    w = _small_cascade(100, torch.float16, 128, 1, 16)
    host_levels = [{"qo_indptr": lv["qo_indptr"], "kv_lens": lv["kv_lens"]} for lv in w.levels]
    params = api.make_params(w.batch, w.num_qo_heads, w.num_kv_heads, 128, 16, num_ctas=8, level_ctas=5)
    ws = api.Workspace(params, host_levels)
    info = api.plan(params, w.cache_seqlens.cpu().tolist(), host_levels, workspace=ws)
    for l, lv in enumerate(w.levels):
        d, keep = api.level_dev(lv)
        o, lse = api.prefix_attention(info, l, w.q, w.k_pool, w.v_pool, d, sm_scale=w.sm_scale)
        torch.cuda.synchronize()
        O, L = oatt.level_prefix_states(host(w.q), PoolView(w.k_pool), PoolView(w.v_pool), 16, w.sm_scale,
                                        lv, w.batch)
        covered = ~np.isnan(L[:, 0])
        Lf = np.where(covered[:, None], L, -np.inf)
        Of = np.where(covered[:, None, None], O, 0.0)
        check_state(o, lse, Of, Lf, torch.float16, f"level {l}")


def test_cascade_equals_flat_decode(api):
    """The cascade and a plain paged decode over a table that lists the prefix pages then
    the suffix pages give the same attention (page-aligned prefix)."""
    say("case: cascade vs flat decode over the concatenated block table")
    w = workloads.cascade_two_level(batch=16, prefix_len=1024, suffix_len=100, device="cuda", seed=5)
    o, lse, *_ = _run_cascade(api, w)
    ppg = 1024 // 16
    flat = torch.cat([torch.arange(ppg, dtype=torch.int32, device="cuda").repeat(16, 1), w.block_table], 1)
    o2, lse2 = api.batch_decode_paged(w.q, w.k_pool, w.v_pool, flat.contiguous(), w.cache_seqlens + 1024,
                                      sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    O, L = _oracle(w)
    check_state(o, lse, O, L, torch.float16, "cascade")
    check_state(o2, lse2, O, L, torch.float16, "flat decode")


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_cascade_growing_and_spiking_scores(api, dtype):
    """Scores whose maximum keeps rising along the prefix (by ~32 in log2 units) plus one
    spike in a middle tile: the prefix kernel's running reference maximum must move on
    later tiles, not only on the first one."""
    say(f"case: cascade with rising prefix scores and a spike, {dtype}")
    w = workloads.cascade_two_level(batch=24, prefix_len=3000, suffix_len=70, device="cuda", seed=21,
                                    dtype=dtype)
    D, P = w.head_dim, w.page_size
    gen = torch.Generator(device="cuda").manual_seed(77)
    u = torch.ones(D, device="cuda") / math.sqrt(D)
    # token t of the pool (prefix pages are the run 0..: t = page * P + slot) gets a key along u
    # with amplitude rising from -8 to 8 over the prefix; one token in the middle gets 20.
    npg = w.k_pool.shape[0]
    t = torch.arange(npg * P, device="cuda", dtype=torch.float32).view(npg, P)
    amp = -8.0 + 16.0 * t / 3000.0
    amp[(t >= 3000)] = 0.5
    amp.view(-1)[1543] = 20.0
    noise = torch.randn(npg, P, w.num_kv_heads, D, generator=gen, device="cuda") * 0.05
    k = amp[:, :, None, None] * u + noise
    keep_nan = torch.isnan(w.k_pool)
    w.k_pool.copy_(k.to(dtype))
    w.k_pool[keep_nan] = float("nan")
    q = 16.0 * u + torch.randn(w.batch, w.num_qo_heads, D, generator=gen, device="cuda") * 0.05
    w.q.copy_(q.to(dtype))
    o, lse, *_ = _run_cascade(api, w, level_ctas=3)
    torch.cuda.synchronize()
    O, L = _oracle(w)
    check_state(o, lse, O, L, dtype, "rising scores")
