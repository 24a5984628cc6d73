"""GPU parity of the FP8 (OCP E4M3) KV decode against the fp64 oracle.

FlashInfer paper summary, appendix F: queries and outputs stay 16-bit while the KV
pools hold fp8 codes.  The oracle decodes the codes itself (oracle.fp8, pinned to the
format on the CPU) and attends over the dequantised pools; the kernel converts codes
with the gfx950 conversion instructions.  Covers every byte value through a single-token
decode (bit-exact outputs, which also pins the byte order within a lane's load), a matrix
of small ragged cases over query dtype, head_dim, group size and page size with NaN codes
in every row no request reads, the LLaMA2-7B-shaped decode at full size (sampled
requests) and the plan-driven split path with its merge.  Cascades over FP8 pools (the
matrix-core level kernel on converted tiles, then the FP8 suffix decode with its fold): the
two- and three-level workloads at full size (sampled), small random cascades, and each
level's states alone with 4- and 8-wave workgroups.
"""

import math
import random

import numpy as np
import pytest
import torch

from oracle import fp8 as ofp8
from paged_kv_cascade_amd import workloads
from tests.gpu_helpers import FULL_SIZE_HEADS, CodeView, HostCodeView, check_state, gpu, host, needs_gpu, say

pytestmark = [gpu, needs_gpu]

NAN_CODES = (0x7F, 0xFF)


@pytest.fixture(scope="module")
def api():
    from paged_kv_cascade_amd import api as _api
    return _api


def _oracle(q, k8, v8, k_scale, v_scale, bt, lens, P, sm_scale, kv_start=None, requests=None,
            heads=None, host_copy=False):
    view = HostCodeView if host_copy else CodeView
    return ofp8.batch_decode_fp8(host(q), view(k8), view(v8), k_scale, v_scale,
                                 bt.cpu().numpy(), lens.cpu().numpy(), P, sm_scale,
                                 kv_start=None if kv_start is None else kv_start.cpu().numpy(),
                                 requests=requests, heads=heads)


@pytest.mark.parametrize("qdt", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("D", [64, 128])
def test_every_code_decodes_exactly(api, qdt, D):
    """256 requests of one token each.  Request b's key row is zero except code b at column
    b % D and its query is the unit vector there, so LSE_b = e4m3(b) (sm_scale = k_scale = 1);
    its value row holds codes (b * D + d) mod 256, so O = 2 * e4m3(code), exact in the
    16-bit output (v_scale = 2).  NaN codes are replaced by zero; the other 15 slots of every
    page hold NaN codes and must never be read."""
    say(f"case: fp8 every code, q {qdt}, D={D}, P=16")
    n, P = 256, 16
    k = torch.full((n, P, 1, D), 0x7F, dtype=torch.uint8)
    v = torch.full((n, P, 1, D), 0x7F, dtype=torch.uint8)
    q = torch.zeros(n, 1, D)
    for b in range(n):
        k[b, 0, 0, :] = 0
        k[b, 0, 0, b % D] = 0 if b in NAN_CODES else b
        q[b, 0, b % D] = 1.0
        codes = [(b * D + d) % 256 for d in range(D)]
        v[b, 0, 0, :] = torch.tensor([0 if c in NAN_CODES else c for c in codes], dtype=torch.uint8)
    k8 = k.cuda().view(torch.float8_e4m3fn)
    v8 = v.cuda().view(torch.float8_e4m3fn)
    qd = q.to(qdt).cuda()
    bt = torch.arange(n, dtype=torch.int32).view(n, 1).cuda()
    lens = torch.ones(n, dtype=torch.int32).cuda()
    o, lse = api.batch_decode_paged_fp8(qd, k8, v8, bt, lens, k_scale=1.0, v_scale=2.0, sm_scale=1.0)
    torch.cuda.synchronize()
    O, L = _oracle(qd, k8, v8, 1.0, 2.0, bt, lens, P, 1.0)
    assert o.dtype == qdt
    # Outputs are exact: every 2 * e4m3 value is representable in fp16 and bf16.
    assert np.array_equal(host(o), O), "decoded value rows differ"
    got = lse.cpu().double().numpy()
    err = np.abs(got - L)
    assert np.all(err <= 2e-6 * np.maximum(1.0, np.abs(L))), f"key codes: max |dLSE| {err.max()}"


def _ragged_fp8_case(qdt, D, g, P, seed, hkv=2, with_start=False):
    rng = random.Random(seed)
    B = 7
    lens = [0, 1, P - 1 if P > 1 else 2, P, P + 1, rng.randint(100, 700), rng.randint(1, 300)]
    npg = [-(-n // P) for n in lens]
    num_pages = sum(npg) + 5
    perm = torch.randperm(num_pages, generator=torch.Generator().manual_seed(seed)).tolist()
    maxb = max(npg) + 1
    bt = torch.full((B, maxb), -1, dtype=torch.int32)
    used = torch.zeros(num_pages, P, dtype=torch.bool)
    off = 0
    for b, n in enumerate(npg):
        bt[b, :n] = torch.tensor(perm[off:off + n], dtype=torch.int32)
        off += n
        for t in range(lens[b]):
            used[int(bt[b, t // P]), t % P] = True
    gen = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn(B, hkv * g, D, generator=gen, device="cuda").to(qdt)
    k = torch.randn(num_pages, P, hkv, D, generator=gen, device="cuda")
    v = torch.randn(num_pages, P, hkv, D, generator=gen, device="cuda")
    k[~used.cuda()] = float("nan")
    v[~used.cuda()] = float("nan")
    k_scale, v_scale = rng.choice([(1.0, 1.0), (0.37, 1.9), (2.5, 0.05)])
    k8 = workloads.fp8_e4m3_pool(k, k_scale)
    v8 = workloads.fp8_e4m3_pool(v, v_scale)
    ks = None
    if with_start:
        ks = torch.tensor([min(n, rng.randint(0, n)) for n in lens], dtype=torch.int32)
    return q, k8, v8, k_scale, v_scale, bt, torch.tensor(lens, dtype=torch.int32), ks


@pytest.mark.parametrize("qdt", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("g", [1, 2, 4, 8])
@pytest.mark.parametrize("P", [1, 4, 16, 64])
def test_fp8_ragged_matrix(api, qdt, D, g, P):
    seed = (1 if qdt == torch.float16 else 2) * 20000 + D * 10 + g * 1000 + P
    with_start = (D + g + P) % 2 == 0
    q, k8, v8, ksc, vsc, bt, lens, ks = _ragged_fp8_case(qdt, D, g, P, seed, with_start=with_start)
    say(f"case: fp8 ragged q {qdt} D={D} g={g} P={P} kv_start={with_start} scales=({ksc}, {vsc})")
    assert int((k8.view(torch.uint8) == 0x7F).sum()) > 0, "no poisoned rows"
    api.validate_block_table(bt, lens, P, k8.shape[0], kv_start=ks)
    btd, ld = bt.cuda(), lens.cuda()
    ksd = ks.cuda() if ks is not None else None
    sm = 1.0 / math.sqrt(D)
    o, lse = api.batch_decode_paged_fp8(q, k8, v8, btd, ld, k_scale=ksc, v_scale=vsc, kv_start=ksd,
                                        sm_scale=sm)
    torch.cuda.synchronize()
    O, L = _oracle(q, k8, v8, ksc, vsc, btd, ld, P, sm, kv_start=ksd)
    check_state(o, lse, O, L, qdt, f"fp8 ragged {qdt} D{D} g{g} P{P}", rounding_allowance=True)


def test_fp8_llama_shape_full_size(api):
    """LLaMA2-7B decode shape: 64 requests x 4096 tokens, 32 heads x 128, page 16; fp16
    queries; pools quantised with k_scale 0.25 and v_scale 0.125; every request on heads 0, 13,
    31."""
    say("case: fp8 paged decode b64 h32 d128 len4096 p16, fp16 q")
    w = workloads.paged_decode(batch=64, kv_len=4096, page_size=16, dtype=torch.float16, device="cuda")
    k8 = workloads.fp8_e4m3_pool(w.k_pool, 0.25)
    v8 = workloads.fp8_e4m3_pool(w.v_pool, 0.125)
    o, lse = api.batch_decode_paged_fp8(w.q, k8, v8, w.block_table, w.cache_seqlens, k_scale=0.25,
                                        v_scale=0.125, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    O, L = _oracle(w.q, k8, v8, 0.25, 0.125, w.block_table, w.cache_seqlens, 16, w.sm_scale,
                   heads=FULL_SIZE_HEADS, host_copy=True)
    check_state(o, lse, O, L, torch.float16, "fp8 llama shape")


def test_fp8_split_plan(api):
    """Plan-driven split-KV decode over FP8 pools: 32 q / 8 kv heads, bf16 queries, 256
    requests with log-uniform lengths in [128, 32768], plan over 2 x compute units."""
    say("case: fp8 GQA split-KV b256 hq32 hkv8 d128 bf16 q, plan #CTA = 2 x CUs")
    w = workloads.gqa_split(device="cuda")
    k8 = workloads.fp8_e4m3_pool(w.k_pool, 0.5)
    v8 = workloads.fp8_e4m3_pool(w.v_pool, 0.5)
    cus = api.device_info(0)["num_cus"]
    lens = w.cache_seqlens.cpu().tolist()
    params = api.make_params(w.batch, 32, 8, 128, 16, num_ctas=2 * cus, alpha=1, beta=1)
    ws = api.Workspace(params)
    info = api.plan(params, lens, workspace=ws)
    assert info.num_merge > 0, "the plan should split some requests"
    o, lse = api.batch_decode_paged_fp8(w.q, k8, v8, w.block_table, w.cache_seqlens, k_scale=0.5,
                                        v_scale=0.5, sm_scale=w.sm_scale, plan_info=info)
    o2, lse2 = api.batch_decode_paged_fp8(w.q, k8, v8, w.block_table, w.cache_seqlens, k_scale=0.5,
                                          v_scale=0.5, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    O, L = _oracle(w.q, k8, v8, 0.5, 0.5, w.block_table, w.cache_seqlens, 16, w.sm_scale,
                   heads=FULL_SIZE_HEADS, host_copy=True)
    check_state(o, lse, O, L, torch.bfloat16, "fp8 split plan")
    check_state(o2, lse2, O, L, torch.bfloat16, "fp8 no plan")


def test_fp8_argument_errors(api):
    """Rejected before any launch: fp32 queries, non-positive or non-finite scales."""
    say("case: fp8 argument errors")
    q = torch.zeros(2, 4, 64, dtype=torch.float16, device="cuda")
    k8 = torch.zeros(4, 16, 4, 64, dtype=torch.uint8, device="cuda")
    bt = torch.zeros(2, 1, dtype=torch.int32, device="cuda")
    lens = torch.ones(2, dtype=torch.int32, device="cuda")
    with pytest.raises(api.PkcError):
        api.batch_decode_paged_fp8(q.float(), k8, k8, bt, lens)
    for ks, vs in ((0.0, 1.0), (1.0, -2.0), (math.inf, 1.0), (1.0, math.nan)):
        with pytest.raises(api.PkcError):
            api.batch_decode_paged_fp8(q, k8, k8, bt, lens, k_scale=ks, v_scale=vs)
    o, lse = api.batch_decode_paged_fp8(q, k8, k8, bt, lens)   # valid: all-zero codes
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.allclose(lse, torch.zeros_like(lse))


# --- cascades over FP8 pools: MFMA level kernel on converted tiles + FP8 suffix decode ----------

def _fp8_cascade_run(api, w, k8, v8, ksc, vsc, level_ctas=0, num_ctas=0, tile_q=0):
    params = api.make_params(w.batch, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                             num_ctas=num_ctas, level_ctas=level_ctas, level_tile_q=tile_q)
    host_levels = [{"qo_indptr": lv["qo_indptr"], "kv_lens": lv["kv_lens"]} for lv in w.levels]
    ws = api.Workspace(params, host_levels)
    info = api.plan(params, w.cache_seqlens.cpu().tolist(), host_levels, workspace=ws)
    devs, keep = [], []
    for lv in w.levels:
        d, k = api.level_dev(lv)
        devs.append(d)
        keep.append(k)
    o, lse = api.cascade_decode_fp8(info, w.q, k8, v8, devs, w.block_table, w.cache_seqlens,
                                    k_scale=ksc, v_scale=vsc, sm_scale=w.sm_scale)
    return o, lse, info, ws, devs, keep


def _fp8_cascade_oracle(w, k8, v8, ksc, vsc, requests=None, heads=None, host_copy=False):
    view = HostCodeView if host_copy else CodeView
    return ofp8.cascade_decode_fp8(host(w.q), view(k8), view(v8), ksc, vsc, w.page_size,
                                   w.sm_scale, w.levels, w.block_table.cpu().numpy(),
                                   w.cache_seqlens.cpu().numpy(), requests=requests, heads=heads)


@pytest.mark.parametrize("grid", ["default", "two_per_cu"])
def test_fp8_two_level_cascade_full_size(api, grid):
    """The cascade workload (32768-token shared prefix + 256 tokens per request, batch 128,
    32 heads x 128, page 16) with fp16 queries over E4M3 pools (k_scale 0.25, v_scale 0.125),
    on the default level grid (one 8-wave workgroup per compute unit) and on two 4-wave
    workgroups per compute unit."""
    say(f"case: fp8 two-level cascade prefix32768 suffix256 b128 h32 d128 p16, fp16 q, level grid {grid} "
        "(every request on heads 0, 13, 31)")
    w = workloads.cascade_two_level(device="cuda")
    k8 = workloads.fp8_e4m3_pool(w.k_pool, 0.25)
    v8 = workloads.fp8_e4m3_pool(w.v_pool, 0.125)
    lc = 0 if grid == "default" else 2 * api.device_info(0)["num_cus"] // w.num_kv_heads
    o, lse, info, *_ = _fp8_cascade_run(api, w, k8, v8, 0.25, 0.125, level_ctas=lc)
    o2, lse2, *_ = _fp8_cascade_run(api, w, k8, v8, 0.25, 0.125, level_ctas=lc)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "repeat run differs"
    O, L = _fp8_cascade_oracle(w, k8, v8, 0.25, 0.125, heads=FULL_SIZE_HEADS, host_copy=True)
    check_state(o, lse, O, L, torch.float16, "fp8 cascade 32K prefix")


def test_fp8_multi_level_cascade_full_size(api):
    """Global prefix 16384 + 4 groups x 4096 + 512 per request, batch 128, bf16 queries over
    E4M3 pools."""
    say("case: fp8 three-level cascade 16384 + 4x4096 + 512, b128 h32 d128, bf16 q (every request on "
        "heads 0, 13, 31)")
    w = workloads.cascade_multi_level(device="cuda", dtype=torch.bfloat16)
    k8 = workloads.fp8_e4m3_pool(w.k_pool, 0.5)
    v8 = workloads.fp8_e4m3_pool(w.v_pool, 0.5)
    o, lse, *_ = _fp8_cascade_run(api, w, k8, v8, 0.5, 0.5)
    torch.cuda.synchronize()
    O, L = _fp8_cascade_oracle(w, k8, v8, 0.5, 0.5, heads=FULL_SIZE_HEADS, host_copy=True)
    check_state(o, lse, O, L, torch.bfloat16, "fp8 cascade 3 levels")


@pytest.mark.parametrize("seed", range(8))
def test_fp8_small_cascades(api, seed):
    from tests.test_gpu_cascade import _small_cascade
    qdt = [torch.float16, torch.bfloat16][seed % 2]
    D = [128, 64][(seed // 2) % 2]
    g = [1, 4, 2, 8][seed % 4]
    P = [16, 4, 32][seed % 3]
    w = _small_cascade(500 + seed, qdt, D, g, P)
    ksc, vsc = [(1.0, 1.0), (0.3, 2.0), (1.7, 0.4)][seed % 3]
    k8 = workloads.fp8_e4m3_pool(w.k_pool, ksc)
    v8 = workloads.fp8_e4m3_pool(w.v_pool, vsc)
    lctas = [1, 3, 8][seed % 3]
    tile_q = [0, 16 // g, 128 // g][seed % 3]
    say(f"case: fp8 small cascade seed={seed} q {qdt} D={D} g={g} P={P} B={w.batch} levels={len(w.levels)} "
        f"level_ctas={lctas} tile_q={tile_q} scales=({ksc}, {vsc})")
    o, lse, *_ = _fp8_cascade_run(api, w, k8, v8, ksc, vsc, level_ctas=lctas, num_ctas=13, tile_q=tile_q)
    torch.cuda.synchronize()
    O, L = _fp8_cascade_oracle(w, k8, v8, ksc, vsc)
    check_state(o, lse, O, L, qdt, f"fp8 small cascade {seed}", rounding_allowance=True)


@pytest.mark.parametrize("streams", ["1", "2"])
def test_fp8_prefix_attention_standalone(api, streams):
    """Each level's states alone (the level kernel over converted tiles, then its merge), with
    4-wave and 8-wave workgroups."""
    from tests.test_gpu_cascade import _small_cascade
    say(f"case: fp8 prefix_attention per level vs the oracle's level states, streams={streams}")
    w = _small_cascade(600, torch.float16, 128, 2, 16)
    k8 = workloads.fp8_e4m3_pool(w.k_pool, 0.6)
    v8 = workloads.fp8_e4m3_pool(w.v_pool, 1.5)
    host_levels = [{"qo_indptr": lv["qo_indptr"], "kv_lens": lv["kv_lens"]} for lv in w.levels]
    params = api.make_params(w.batch, w.num_qo_heads, w.num_kv_heads, 128, 16, num_ctas=8, level_ctas=5,
                             level_streams=int(streams))
    ws = api.Workspace(params, host_levels)
    info = api.plan(params, w.cache_seqlens.cpu().tolist(), host_levels, workspace=ws)
    assert info.lvl_streams == int(streams)
    for l, lv in enumerate(w.levels):
        d, keep = api.level_dev(lv)
        o, lse = api.prefix_attention_fp8(info, l, w.q, k8, v8, d, k_scale=0.6, v_scale=1.5,
                                          sm_scale=w.sm_scale)
        torch.cuda.synchronize()
        O, L = ofp8.level_prefix_states_fp8(host(w.q), CodeView(k8), CodeView(v8), 0.6, 1.5, 16,
                                            w.sm_scale, lv, w.batch)
        covered = ~np.isnan(L[:, 0])
        Lf = np.where(covered[:, None], L, -np.inf)
        Of = np.where(covered[:, None, None], O, 0.0)
        check_state(o, lse, Of, Lf, torch.float16, f"fp8 level {l}")


# --- ragged multi-token queries over FP8 pools -------------------------------------------------

@pytest.mark.parametrize("seed", range(8))
def test_fp8_ragged_prefill(api, seed):
    from tests.test_gpu_prefill import _case
    rng = random.Random(700 + seed)
    qdt = [torch.float16, torch.bfloat16][seed % 2]
    D = [128, 64][(seed // 2) % 2]
    g = [1, 8, 2, 4][seed % 4]
    P = [16, 4][seed % 2]
    causal = seed % 3 != 1
    B = rng.randint(1, 5)
    lq = [rng.choice([1, 3, 40, 130]) for _ in range(B)]
    lkv = [max(0, n + rng.choice([0, 2, 90, -2])) for n in lq]
    ksc, vsc = [(1.0, 1.0), (0.4, 1.7)][seed % 2]
    say(f"case: fp8 prefill seed={seed} q {qdt} D={D} g={g} P={P} causal={causal} lq={lq} lkv={lkv}")
    q, k, v, bt = _case(800 + seed, lq, lkv, qdt, D, g, P)
    k8, v8 = workloads.fp8_e4m3_pool(k, ksc), workloads.fp8_e4m3_pool(v, vsc)
    info, ws, qi = api.prefill_plan(lq, lkv, q.shape[1], k.shape[2], D, P, level_ctas=rng.choice([0, 3]),
                                    causal=causal)
    qi_d = torch.tensor(qi, dtype=torch.int32, device="cuda")
    kv_d = torch.tensor(lkv, dtype=torch.int32, device="cuda")
    o, lse = api.batch_prefill_paged_fp8(info, q, k8, v8, bt.cuda(), qi_d, kv_d, k_scale=ksc, v_scale=vsc,
                                         causal=causal, sm_scale=1.0 / math.sqrt(D))
    torch.cuda.synchronize()
    O, L = ofp8.batch_prefill_fp8(host(q), qi, CodeView(k8), CodeView(v8), ksc, vsc, bt.numpy(), lkv, P,
                                  1.0 / math.sqrt(D), causal)
    check_state(o, lse, O, L, qdt, f"fp8 prefill seed {seed}", rounding_allowance=True)


def test_fp8_grouped_decode_through_matrix_cores(api):
    """One query per request with 8 query heads per KV head: the prefill path (matrix cores)
    and the vector-ALU decode kernel give the same decode."""
    say("case: fp8 GQA g8 decode through the prefill path vs the decode kernel")
    w = workloads.gqa_split(batch=24, heads=32, kv_heads=4, lo=16, hi=3000, device="cuda")
    k8 = workloads.fp8_e4m3_pool(w.k_pool, 0.5)
    v8 = workloads.fp8_e4m3_pool(w.v_pool, 0.5)
    lens = w.cache_seqlens.cpu().tolist()
    info, ws, qi = api.prefill_plan([1] * w.batch, lens, 32, 4, 128, 16, causal=False)
    qi_d = torch.tensor(qi, dtype=torch.int32, device="cuda")
    o, lse = api.batch_prefill_paged_fp8(info, w.q, k8, v8, w.block_table, qi_d, w.cache_seqlens,
                                         k_scale=0.5, v_scale=0.5, causal=False, sm_scale=w.sm_scale)
    o2, lse2 = api.batch_decode_paged_fp8(w.q, k8, v8, w.block_table, w.cache_seqlens, k_scale=0.5,
                                          v_scale=0.5, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    reqs = [0, 5, 11, 23]
    O, L = _oracle(w.q, k8, v8, 0.5, 0.5, w.block_table, w.cache_seqlens, 16, w.sm_scale, requests=reqs)
    check_state(o, lse, O, L, torch.bfloat16, "fp8 g8 decode, matrix cores", rows=reqs)
    check_state(o2, lse2, O, L, torch.bfloat16, "fp8 g8 decode, vector ALU", rows=reqs)
