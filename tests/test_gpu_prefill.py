"""GPU parity of ragged multi-token queries (prefill / append attention over the paged cache)
against the fp64 oracle.

The run is the multi-query level kernel over each request's block-table row (query tiles of
T_q rows, KV chunks from the load-balancing plan, the causal limit applied per query column)
followed by the merge of every query row's chunk states.  Covers the "Paged attention" page's
varlen example lengths (query lengths [10, 3, 1], key lengths [0, 1, 7]: empty and partly
visible rows), a matrix of random ragged batches over dtype, head_dim, group size, page size,
causal mask, level #CTA and query tile, a long prefill at LLaMA2-7B head shape (sampled rows),
and single-token requests against the batch decode kernel.
"""

import math
import random

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from tests.gpu_helpers import PoolView, check_state, gpu, host, needs_gpu, say

pytestmark = [gpu, needs_gpu]


@pytest.fixture(scope="module")
def api():
    from paged_kv_cascade_amd import api as _api
    return _api


def _case(seed, lq, lkv, dtype, D, g, P, hkv=2, scale=1.0):
    """Packed queries for the given lengths, each request's KV in its own permuted pages
    (block-table rows padded with -1), rows no request reads NaN."""
    B = len(lq)
    npg = [-(-n // P) for n in lkv]
    num_pages = sum(npg) + 3
    perm = torch.randperm(num_pages, generator=torch.Generator().manual_seed(seed)).tolist()
    bt = torch.full((B, max(npg + [0]) + 1), -1, dtype=torch.int32)
    used = torch.zeros(num_pages, P, dtype=torch.bool)
    off = 0
    for b, n in enumerate(npg):
        bt[b, :n] = torch.tensor(perm[off:off + n], dtype=torch.int32)
        off += n
        for t in range(lkv[b]):
            used[int(bt[b, t // P]), t % P] = True
    gen = torch.Generator(device="cuda").manual_seed(seed)
    T = sum(lq)
    q = (torch.randn(T, hkv * g, D, generator=gen, device="cuda") * scale).to(dtype)
    k = (torch.randn(num_pages, P, hkv, D, generator=gen, device="cuda") * scale).to(dtype)
    v = (torch.randn(num_pages, P, hkv, D, generator=gen, device="cuda") * scale).to(dtype)
    k[~used.cuda()] = float("nan")
    v[~used.cuda()] = float("nan")
    return q, k, v, bt


def _run(api, q, k, v, bt, lq, lkv, causal, level_ctas=0, tile_q=0, write_through=True):
    T, Hq, D = q.shape
    P, Hkv = k.shape[1], k.shape[2]
    info, ws, qi = api.prefill_plan(lq, lkv, Hq, Hkv, D, P, level_ctas=level_ctas, level_tile_q=tile_q,
                                    causal=causal, write_through=write_through)
    qi_d = torch.tensor(qi, dtype=torch.int32, device="cuda")
    kv_d = torch.tensor(lkv, dtype=torch.int32, device="cuda")
    o, lse = api.batch_prefill_paged(info, q, k, v, bt.cuda(), qi_d, kv_d, causal=causal,
                                     sm_scale=1.0 / math.sqrt(D))
    torch.cuda.synchronize()
    return o, lse, qi, info


def _oracle(q, k, v, bt, qi, lkv, causal, rows=None):
    D = q.shape[2]
    return oatt.batch_prefill(host(q), qi, PoolView(k), PoolView(v), bt.numpy(), lkv, k.shape[1],
                              1.0 / math.sqrt(D), causal, rows=rows)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("P", [4, 16])
def test_varlen_example_lengths(api, causal, P):
    lq, lkv = [10, 3, 1], [0, 1, 7]
    say(f"case: prefill varlen example lengths q{lq} kv{lkv} causal={causal} P={P} fp16 D64 g2")
    q, k, v, bt = _case(70 + P, lq, lkv, torch.float16, 64, 2, P)
    o, lse, qi, _ = _run(api, q, k, v, bt, lq, lkv, causal, level_ctas=3, tile_q=8)
    O, L = _oracle(q, k, v, bt, qi, lkv, causal)
    check_state(o, lse, O, L, torch.float16, f"varlen example causal={causal}")
    # Request 0 sees no key: its rows are the empty state.
    assert torch.all(torch.isneginf(lse[:10])) and torch.all(o[:10] == 0)


@pytest.mark.parametrize("seed", range(16))
def test_random_ragged_prefill(api, seed):
    rng = random.Random(seed)
    dtype = [torch.float16, torch.bfloat16][seed % 2]
    D = [128, 64][(seed // 2) % 2]
    g = [1, 2, 4, 8][(seed // 4) % 4]
    P = [16, 4, 32, 8][seed % 4]
    causal = seed % 3 != 2
    B = rng.randint(1, 6)
    lq = [rng.choice([1, 2, 5, 33, 130, 300]) for _ in range(B)]
    lkv = [max(0, n + rng.choice([0, 1, 17, 500, -3])) for n in lq]
    lctas = rng.choice([0, 1, 3, 8])
    tile_q = rng.choice([0, 16 // g, 128 // g])
    say(f"case: prefill seed={seed} {dtype} D={D} g={g} P={P} causal={causal} lq={lq} lkv={lkv} "
        f"level_ctas={lctas} tile_q={tile_q}")
    q, k, v, bt = _case(900 + seed, lq, lkv, dtype, D, g, P)
    o, lse, qi, _ = _run(api, q, k, v, bt, lq, lkv, causal, level_ctas=lctas, tile_q=tile_q)
    O, L = _oracle(q, k, v, bt, qi, lkv, causal)
    check_state(o, lse, O, L, dtype, f"prefill seed {seed}", rounding_allowance=True)


def test_long_causal_prefill_sampled(api):
    """4 requests x 512 new tokens over 2048-token sequences, 32 heads x 128, fp16, causal."""
    lq, lkv = [512] * 4, [2048, 1500, 512, 2048]
    say(f"case: long causal prefill lq={lq} lkv={lkv} h32 d128 fp16 P16")
    q, k, v, bt = _case(4242, lq, lkv, torch.float16, 128, 1, 16, hkv=32, scale=0.5)
    o, lse, qi, info = _run(api, q, k, v, bt, lq, lkv, True)
    rows = sorted({qi[b] + i for b in range(4) for i in (0, 1, 255, 510, 511)})
    O, L = _oracle(q, k, v, bt, qi, lkv, True, rows=rows)
    check_state(o, lse, O, L, torch.float16, "long causal prefill", rows=rows)


def test_single_token_requests_match_decode(api):
    lq, lkv = [1] * 9, [1, 2, 15, 16, 17, 100, 333, 700, 1]
    say("case: prefill with one query per request vs the batch decode kernel")
    q, k, v, bt = _case(31, lq, lkv, torch.bfloat16, 128, 4, 16)
    o, lse, qi, _ = _run(api, q, k, v, bt, lq, lkv, True)
    od, lsed = api.batch_decode_paged(q, k, v, bt.cuda(), torch.tensor(lkv, dtype=torch.int32, device="cuda"),
                                      sm_scale=1.0 / math.sqrt(128))
    torch.cuda.synchronize()
    O, L = _oracle(q, k, v, bt, qi, lkv, True)
    # one- and two-token requests give |O| near 1: bf16 output rounding alone exceeds 2e-3
    check_state(o, lse, O, L, torch.bfloat16, "prefill l_q = 1", rounding_allowance=True)
    check_state(od, lsed, O, L, torch.bfloat16, "decode", rounding_allowance=True)


def test_prefill_rejects_plan_of_other_shape(api):
    say("case: prefill with a plan of another shape is rejected before any launch")
    q, k, v, bt = _case(5, [3, 2], [4, 9], torch.float16, 64, 1, 4)
    info, ws, qi = api.prefill_plan([3, 2], [4, 9], 2, 2, 64, 4)
    qi_d = torch.tensor(qi, dtype=torch.int32, device="cuda")
    kv_d = torch.tensor([4, 9], dtype=torch.int32, device="cuda")
    with pytest.raises(api.PkcError):   # three requests against a plan of two
        api.batch_prefill_paged(info, q, k, v, torch.cat([bt, bt[:1]]).cuda(), qi_d, kv_d)
    with pytest.raises(api.PkcError):   # fp32 queries
        api.batch_prefill_paged(info, q.float(), k.float(), v.float(), bt.cuda(), qi_d, kv_d)
    with pytest.raises(api.PkcError):   # a causal plan run without the mask
        api.batch_prefill_paged(info, q, k, v, bt.cuda(), qi_d, kv_d, causal=False)


@pytest.mark.parametrize("causal", [False, True])
def test_write_through_and_merged_rows_agree(api, causal):
    """Tiles whose KV is one chunk write their rows' output from the level kernel; the same
    batch planned without write-through sends every row through the merge pass.  Both match
    the oracle, and the write-through plan merges fewer rows."""
    lq, lkv = [300, 5, 130, 1, 64], [300, 900, 17, 0, 2000]
    say(f"case: prefill write-through vs merged, causal={causal}, bf16 D128 g2 P16 lq={lq} lkv={lkv}")
    q, k, v, bt = _case(77, lq, lkv, torch.bfloat16, 128, 2, 16)
    res = {}
    for wt in (True, False):
        res[wt] = _run(api, q, k, v, bt, lq, lkv, causal, level_ctas=8, write_through=wt)
    info_wt, info_m = res[True][3], res[False][3]
    assert info_wt.lvl_write_through > 0 and info_m.lvl_write_through == 0
    assert info_wt.num_merge < info_m.num_merge == sum(lq)
    O, L = _oracle(q, k, v, bt, res[True][2], lkv, causal)
    for wt in (True, False):
        # causal first rows see one or two tokens (|O| near 1; bf16 output rounding)
        check_state(res[wt][0], res[wt][1], O, L, torch.bfloat16, f"write_through={wt}", rounding_allowance=True)


def test_write_through_plan_runs_only_as_prefill(api):
    say("case: a level write-through plan is rejected by prefix_attention before any launch")
    lq, lkv = [3, 2], [4, 9]
    q, k, v, bt = _case(5, lq, lkv, torch.float16, 64, 1, 4)
    info, ws, qi = api.prefill_plan(lq, lkv, 2, 2, 64, 4, level_ctas=2)
    assert info.lvl_write_through > 0
    d, keep = api.level_dev({"kv_page_indptr": [0, 1, 2], "kv_page_indices": [0, 1]})
    with pytest.raises(api.PkcError):
        api.prefix_attention(info, 0, q, k, v, d)


# --- tree (speculative) decoding masks ------------------------------------------------------------

def _tree_masks(rng, lq):
    """Per request: each new token sees itself and its chain of parents in a random tree, plus
    random bytes above the diagonal (which the causal limit must ignore)."""
    masks = []
    for n in lq:
        parent = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
        m = np.zeros((n, n), dtype=bool)
        for i in range(n):
            j = i
            while j >= 0:
                m[i, j] = True
                j = parent[j]
        m |= np.triu(rng.random((n, n)) < 0.5, k=1)
        masks.append(m)
    return masks


def _run_tree(api, q, k, v, bt, lq, lkv, masks, level_ctas=0):
    T, Hq, D = q.shape
    P, Hkv = k.shape[1], k.shape[2]
    info, ws, qi = api.prefill_plan(lq, lkv, Hq, Hkv, D, P, level_ctas=level_ctas, causal=True)
    flat = np.concatenate([m.astype(np.uint8).ravel() for m in masks] + [np.zeros(1, np.uint8)])
    offs = np.concatenate([[0], np.cumsum([m.size for m in masks])[:-1]]).astype(np.int32)
    o, lse = api.batch_prefill_paged_tree(info, q, k, v, bt.cuda(), torch.tensor(qi, dtype=torch.int32, device="cuda"),
                                          torch.tensor(lkv, dtype=torch.int32, device="cuda"),
                                          torch.from_numpy(flat).cuda(), torch.from_numpy(offs).cuda(),
                                          sm_scale=1.0 / math.sqrt(D))
    torch.cuda.synchronize()
    return o, lse, qi


@pytest.mark.parametrize("seed", range(8))
def test_tree_masked_prefill(api, seed):
    rng = np.random.default_rng(2200 + seed)
    dtype = [torch.float16, torch.bfloat16][seed % 2]
    D = [128, 64][(seed // 2) % 2]
    g = [1, 2, 4, 8][seed % 4]
    P = [16, 4][seed % 2]
    lq = [int(x) for x in rng.choice([1, 4, 7, 33, 64], size=4)]
    lkv = [n + int(x) for n, x in zip(lq, rng.choice([0, 5, 100, 700], size=4))]
    lctas = int(rng.choice([0, 3, 8]))
    say(f"case: tree-masked prefill seed={seed} {dtype} D={D} g={g} P={P} lq={lq} lkv={lkv} level_ctas={lctas}")
    masks = _tree_masks(rng, lq)
    q, k, v, bt = _case(2300 + seed, lq, lkv, dtype, D, g, P)
    o, lse, qi = _run_tree(api, q, k, v, bt, lq, lkv, masks, level_ctas=lctas)
    O, L = oatt.batch_prefill(host(q), qi, PoolView(k), PoolView(v), bt.numpy(), lkv, P, 1.0 / math.sqrt(D), True,
                              tree_masks=masks)
    # tree rows see few tokens (|O| near 1): bf16 output rounding alone exceeds 2e-3
    check_state(o, lse, O, L, dtype, f"tree prefill seed {seed}", rounding_allowance=dtype == torch.bfloat16)


def test_tree_mask_of_ones_is_the_causal_prefill(api):
    lq, lkv = [5, 40], [30, 40]
    say("case: all-ones tree masks vs the causal prefill, fp16 D128 g2 P16")
    q, k, v, bt = _case(2400, lq, lkv, torch.float16, 128, 2, 16)
    o, lse, qi = _run_tree(api, q, k, v, bt, lq, lkv, [np.ones((n, n), dtype=bool) for n in lq])
    o2, lse2, _, _ = _run(api, q, k, v, bt, lq, lkv, True)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_tree_mask_needs_a_causal_plan(api):
    say("case: tree-masked prefill with a non-causal plan is rejected before any launch")
    lq, lkv = [3, 2], [4, 9]
    q, k, v, bt = _case(5, lq, lkv, torch.float16, 64, 1, 4)
    info, ws, qi = api.prefill_plan(lq, lkv, 2, 2, 64, 4, causal=False)
    with pytest.raises(api.PkcError):
        api.batch_prefill_paged_tree(info, q, k, v, bt.cuda(), torch.tensor(qi, dtype=torch.int32, device="cuda"),
                                     torch.tensor(lkv, dtype=torch.int32, device="cuda"),
                                     torch.ones(13, dtype=torch.uint8, device="cuda"),
                                     torch.tensor([0, 9], dtype=torch.int32, device="cuda"))
