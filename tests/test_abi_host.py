"""Host-side checks of the C-ABI library (CPU only, no GPU work is launched).

* libpkc.so loads and exports every function include/pkc.h declares;
* the C++ plan (pkc_plan_host) equals the oracle plan bit for bit: work items,
  their CTA assignment and order, partial-state rows, merge lists and
  write-through flags, for plain split-KV decode and for cascades.  The oracle
  plan follows appendix D's write-through rule; the library also finishes a
  request whose merge list is its level states plus one own chunk in that
  chunk's decode item, so the comparison is against ``fused_fold`` of the
  oracle plan (tests/plan_transform.py);
* argument validation rejects bad shapes before any HIP call;
* the host block-table validator on the "Paged attention" worked example.
"""

import ctypes
import json
import os
import random
import re

import pytest
import torch

from oracle import plan as oplan
from plan_transform import fused_fold

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkc.h")


@pytest.fixture(scope="module")
def api():
    from paged_kv_cascade_amd import api as _api
    return _api


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkc_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function(api):
    names = _declared_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(api.lib, n), f"{n} not exported"
        assert n in api.SIGNATURES, f"{n} has no binding signature"
    assert set(api.SIGNATURES) == set(names)


def test_abi_struct_sizes(api):
    sizes = [ctypes.c_size_t() for _ in range(4)]
    api.lib.pkc_abi_struct_sizes(*[ctypes.byref(s) for s in sizes])
    assert [s.value for s in sizes] == [ctypes.sizeof(api.PlanParams), ctypes.sizeof(api.LevelHost),
                                        ctypes.sizeof(api.LevelDev), ctypes.sizeof(api.PlanInfo)]
    assert api.lib.pkc_status_string(3).decode() == "PKC_ERR_WORKSPACE_TOO_SMALL"


def _compare_plan(api, info, hb, o, levels, tile_q):
    o = fused_fold(o)
    arr = api.read_plan_arrays(info, hb)
    # decode stage
    for c, recs in enumerate(arr["decode"]):
        exp = o.suffix.cta_items[c]
        got = [(r[7], r[0], r[3], r[4]) for r in recs]
        assert got == [(w, o.suffix.items[w].req, o.suffix.items[w].kv_begin,
                        o.suffix.items[w].kv_end) for w in exp], f"decode CTA {c}"
        for r in recs:
            slot = o.suffix.slots[r[7]]
            assert r[5] == (-1 if slot < 0 else info.dec_row_base + slot)
            assert r[1] == r[0] and r[2] == 1
    assert info.dec_kv_chunk == o.suffix.kv_chunk
    # levels
    for l, st in enumerate(o.levels):
        qi = levels[l]["qo_indptr"]
        assert info.lvl_kv_chunk[l] == st.kv_chunk
        for c, recs in enumerate(arr["levels"][l]):
            exp = st.cta_items[c]
            assert [(r[7], r[0], r[6], r[3], r[4]) for r in recs] == \
                [(w, st.items[w].req, st.items[w].tile, st.items[w].kv_begin, st.items[w].kv_end) for w in exp]
            for r in recs:
                it = st.items[r[7]]
                slot = st.slots[it.w]
                assert r[5] == (-1 if slot < 0 else info.lvl_row_base[l] + slot * tile_q)
                assert r[1] == qi[it.req] + it.tile * tile_q and r[2] == it.lq
    # merge lists and flags
    nl = len(levels)
    for b in range(info.batch):
        ptr = arr["merge_ptr"][b]
        for l in range(nl + 1):
            got = arr["merge_rows"][ptr[l]:ptr[l + 1]]
            want = []
            for (stage, slot, row) in o.merge[b]:
                if stage == "suffix" and l == nl:
                    want.append(info.dec_row_base + slot)
                elif stage == l:
                    want.append(info.lvl_row_base[l] + slot * tile_q + row)
            assert got == want, f"request {b} stage {l}"
            if l < nl:
                # {first row, count}: the same rows, as first + c * T_q
                first, cnt = arr["req_levels"][b][l]
                assert cnt == len(want)
                assert want == [first + c * tile_q for c in range(cnt)]
        assert arr["req_flags"][b] == (1 if o.write_through[b] else 0)
    assert info.num_merge == sum(1 for w in o.write_through if not w)


@pytest.mark.parametrize("seed", range(20))
def test_decode_plan_matches_oracle(api, seed):
    rng = random.Random(seed)
    B = rng.randint(1, 60)
    kv = [rng.choice([0, 1, 7, 16, 300, rng.randint(0, 40000)]) for _ in range(B)]
    ctas = rng.choice([1, 3, 16, 512])
    align = rng.choice([1, 1, 16])
    alpha, beta = rng.randint(0, 2), rng.randint(1, 3)
    split = rng.random() < 0.8
    p = api.make_params(B, 8, 2, 128, 16, num_ctas=ctas, level_ctas=1, chunk_align=align,
                        enable_split=split, alpha=alpha, beta=beta)
    info, hb = api.plan_host(p, kv)
    o = oplan.cascade_plan(B, [], kv, num_ctas=ctas, level_ctas=1, level_tile_q=[], alpha=alpha,
                           beta=beta, chunk_align=align, enable_split=split)
    _compare_plan(api, info, hb, o, [], 0)
    # appendix-D bound on partial states of a plain decode: at most 2 * #CTA
    assert info.dec_slots <= 2 * ctas


@pytest.mark.parametrize("seed", range(20))
def test_cascade_plan_matches_oracle(api, seed):
    rng = random.Random(1000 + seed)
    B = rng.randint(1, 70)
    levels = []
    for _ in range(rng.randint(1, 3)):
        G = rng.randint(1, 5)
        cuts = sorted(rng.sample(range(0, B + 1), min(G + 1, B + 1)))
        G = len(cuts) - 1
        if G < 1:
            cuts, G = [0, B], 1
        levels.append({"qo_indptr": cuts, "kv_lens": [rng.choice([0, 5, 64, rng.randint(1, 9000)]) for _ in range(G)]})
    kv = [rng.choice([0, 3, 256, rng.randint(0, 2000)]) for _ in range(B)]
    g = rng.choice([1, 4])
    tile_q = rng.choice([1, 4, 128 // g])
    ctas, lctas = rng.choice([2, 64, 512]), rng.choice([1, 8, 16])
    p = api.make_params(B, 8 * g, 8, 128, 16, num_ctas=ctas, level_ctas=lctas, level_tile_q=tile_q)
    info, hb = api.plan_host(p, kv, levels)
    o = oplan.cascade_plan(B, levels, kv, num_ctas=ctas, level_ctas=lctas,
                           level_tile_q=[tile_q] * len(levels), alpha=1, beta=1)
    _compare_plan(api, info, hb, o, levels, tile_q)


@pytest.mark.parametrize("seed", range(12))
def test_causal_prefill_plan_matches_oracle(api, seed):
    """Plans of ragged multi-token queries (one level whose groups are the requests, causal
    tile extents, one plan request per query row), bit for bit against the oracle."""
    rng = random.Random(3000 + seed)
    B = rng.randint(1, 6)
    qo = [rng.choice([1, 2, 9, 40, 130]) for _ in range(B)]
    kv = [max(0, q + rng.choice([-5, 0, 3, 200])) for q in qo]
    qi = [0]
    for q in qo:
        qi.append(qi[-1] + q)
    T = qi[-1]
    g = rng.choice([1, 2, 4])
    tile_q = rng.choice([0, 4, 16 // g])
    lctas = rng.choice([1, 5, 32])
    levels = [{"qo_indptr": qi, "kv_lens": kv, "causal": seed % 4 != 3}]
    wt = seed % 3 != 0
    p = api.make_params(T, 4 * g, 4, 128, 16, num_ctas=1, level_ctas=lctas, level_tile_q=tile_q,
                        level_write_through=wt)
    info, hb = api.plan_host(p, [0] * T, levels)
    tq = tile_q or 128 // g
    o = oplan.cascade_plan(T, levels, [0] * T, num_ctas=1, level_ctas=lctas, level_tile_q=[tq], alpha=1, beta=1,
                           level_write_through=wt)
    _compare_plan(api, info, hb, o, levels, tq)
    n_wt = sum(1 for s in o.levels[0].slots if s < 0)
    assert info.lvl_write_through == n_wt and (wt or n_wt == 0)


def test_standard_workload_plans_match_oracle(api):
    """The plans of the GQA split-KV workload (256 requests, log-uniform
    128..32768, #CTA = 512) and of both cascades, bit for bit."""
    from paged_kv_cascade_amd import workloads
    g = torch.Generator().manual_seed(1004)
    lens = workloads.loguniform_lengths(256, 128, 32768, g)
    p = api.make_params(256, 32, 8, 128, 16, num_ctas=512, level_ctas=16)
    info, hb = api.plan_host(p, lens)
    o = oplan.cascade_plan(256, [], lens, num_ctas=512, level_ctas=16, level_tile_q=[])
    _compare_plan(api, info, hb, o, [], 0)
    assert info.dec_slots <= 2 * 512
    lv2 = [{"qo_indptr": [0, 128], "kv_lens": [32768]}]
    p = api.make_params(128, 32, 32, 128, 16, num_ctas=512, level_ctas=16, level_tile_q=128)
    info, hb = api.plan_host(p, [256] * 128, lv2)
    o = oplan.cascade_plan(128, lv2, [256] * 128, num_ctas=512, level_ctas=16, level_tile_q=[128])
    _compare_plan(api, info, hb, o, lv2, 128)
    lv3 = [{"qo_indptr": [0, 128], "kv_lens": [16384]},
           {"qo_indptr": [0, 32, 64, 96, 128], "kv_lens": [4096] * 4}]
    info, hb = api.plan_host(p, [512] * 128, lv3)
    o = oplan.cascade_plan(128, lv3, [512] * 128, num_ctas=512, level_ctas=16, level_tile_q=[128, 128])
    _compare_plan(api, info, hb, o, lv3, 128)


def test_plan_buffer_sizes_bound_every_plan(api):
    rng = random.Random(5)
    for _ in range(20):
        B = rng.randint(1, 50)
        levels = [{"qo_indptr": [0, B], "kv_lens": [rng.randint(0, 5000)]}]
        p = api.make_params(B, 4, 4, 64, 8, num_ctas=rng.randint(1, 40), level_ctas=rng.randint(1, 9),
                            level_tile_q=rng.choice([1, 8, 128]))
        hb, db = api.plan_buffer_sizes(p, levels)
        info, _ = api.plan_host(p, [rng.randint(0, 3000) for _ in range(B)], levels)
        assert info.int_bytes <= hb and info.dev_bytes <= db
        assert info.state_rows * 4 * 64 * 4 <= info.off_state_lse - info.off_state_o


def test_validation_errors_before_any_launch(api):
    lib = api.lib
    # head_dim 96 is not built
    assert lib.pkc_batch_decode_paged(None, None, None, None, 0, None, 0, None, None, 1, 4, 4, 96, 16,
                                      1, 1.0, None, None, None, 0, None) == 2
    # Hq not a multiple of Hkv
    assert lib.pkc_batch_decode_paged(None, None, None, None, 0, None, 0, None, None, 1, 6, 4, 128, 16,
                                      1, 1.0, None, None, None, 0, None) == 1
    # page size not a power of two
    assert lib.pkc_batch_decode_paged(None, None, None, None, 0, None, 0, None, None, 1, 4, 4, 128, 12,
                                      1, 1.0, None, None, None, 0, None) == 2
    # non-positive scale
    assert lib.pkc_batch_decode_paged(None, None, None, None, 0, None, 0, None, None, 1, 4, 4, 128, 16,
                                      1, -1.0, None, None, None, 0, None) == 1
    # NULL tensors
    assert lib.pkc_batch_decode_paged(None, None, None, None, 0, None, 0, None, None, 1, 4, 4, 128, 16,
                                      1, 1.0, None, None, None, 0, None) == 1
    assert "NULL" in lib.pkc_last_error().decode()
    # cascade without a plan; prefix with fp32
    assert lib.pkc_cascade_decode(None, None, None, None, 0, None, 0, None, 0, None, 1, 4, 4, 128, 16,
                                  1, 1.0, None, None, None, 0, None) == 1
    # a host-only plan was never copied to a workspace: run calls refuse it (the plan check
    # fails before any launch, so the dummy non-NULL pointers are never dereferenced)
    p = api.make_params(2, 4, 4, 128, 16, num_ctas=4, level_ctas=1)
    info, _ = api.plan_host(p, [10, 20])
    d = ctypes.c_void_p(0x1000)
    assert lib.pkc_batch_decode_paged(ctypes.byref(info), d, d, d, 1, d, 0, d, None, 2, 4,
                                      4, 128, 16, 1, 1.0, d, d, None, 0, None) == 4
    assert "workspace" in lib.pkc_last_error().decode()
    info.magic = 0
    assert lib.pkc_batch_decode_paged(ctypes.byref(info), d, d, d, 1, d, 0, d, None, 2, 4,
                                      4, 128, 16, 1, 1.0, d, d, None, 0, None) == 4
    assert lib.pkc_batch_decode_paged(None, d, d, d, 1, d, 0, None, None, 2, 4, 4, 128, 16, 1, 1.0,
                                      d, d, None, 0, None) == 1   # no cache_seqlens without a plan
    # an empty pool: masked lanes could not read row 0 of page 0
    assert lib.pkc_batch_decode_paged(None, d, d, d, 0, d, 0, d, None, 2, 4, 4, 128, 16, 1, 1.0,
                                      d, d, None, 0, None) == 1
    # merge: bad head_dim, dense range beyond the states
    assert lib.pkc_merge_states(None, 1, None, 4, None, None, 1, 2, 4, 80, None, 1, None, None) == 2
    assert lib.pkc_merge_states(None, 1, None, 4, None, None, 3, 2, 4, 64, None, 1, None, None) == 1
    # plan: bad parameters
    bad = api.make_params(2, 4, 4, 128, 16, num_ctas=0, level_ctas=1)
    with pytest.raises(api.PkcError):
        api.plan_host(bad, [1, 2])
    bad = api.make_params(2, 32, 1, 128, 16, num_ctas=4, level_ctas=1)
    with pytest.raises(api.PkcError) as e:
        api.plan_host(bad, [1, 2])
    assert e.value.status == 2
    with pytest.raises(api.PkcError):
        api.plan_host(api.make_params(2, 4, 4, 128, 16, num_ctas=4, level_ctas=1), [1, -2])
    with pytest.raises(api.PkcError):
        api.plan_host(api.make_params(2, 4, 4, 128, 16, num_ctas=4, level_ctas=1), [1, 2],
                      [{"qo_indptr": [0, 3], "kv_lens": [5]}])
    # host buffer too small
    info = api.PlanInfo()
    small = torch.zeros(16, dtype=torch.uint8)
    kl = (ctypes.c_int32 * 2)(1, 2)
    assert lib.pkc_plan_host(ctypes.byref(api.make_params(2, 4, 4, 128, 16, num_ctas=4, level_ctas=1)),
                             kl, None, 0, ctypes.c_void_p(small.data_ptr()), 16, ctypes.byref(info)) == 3


def test_validate_block_table_worked_example(api):
    with open(os.path.join(ROOT, "tests", "golden", "hf_paged_decode_example.json")) as f:
        g = json.load(f)
    bt = torch.tensor(g["block_table"], dtype=torch.int32)
    sl = torch.tensor(g["cache_seqlens"], dtype=torch.int32)
    api.validate_block_table(bt, sl, g["page_size"], 8)
    with pytest.raises(api.PkcError) as e:
        api.validate_block_table(bt, torch.tensor([40, 32, 70], dtype=torch.int32), g["page_size"], 8)
    assert "request 0" in str(e.value)
    with pytest.raises(api.PkcError):
        api.validate_block_table(bt, sl, g["page_size"], 6)   # page 6 of sequence 2 out of range
    # starting past the unallocated block makes it legal again
    api.validate_block_table(bt, torch.tensor([30, 32, 70], dtype=torch.int32), g["page_size"], 8,
                             kv_start=torch.tensor([0, 0, 0], dtype=torch.int32))


def test_append_and_tree_validation_before_any_launch(api):
    """Argument errors of the multi-token append and of the tree-masked prefill are reported
    before any HIP call (dummy non-NULL pointers are never dereferenced)."""
    lib = api.lib
    d = ctypes.c_void_p(0x1000)
    e = ctypes.c_void_p(0x2000)
    # ragged append: too many requests for the grid, unsupported head_dim, aliased lengths
    assert lib.pkc_append_kv_ragged(d, d, 4, d, d, d, 8, d, 2, d, e, 70000, 2, 128, 16, 1, None) == 1
    assert lib.pkc_append_kv_ragged(d, d, 4, d, d, d, 8, d, 2, d, e, 2, 2, 96, 16, 1, None) == 2
    assert lib.pkc_append_kv_ragged(d, d, 4, d, d, d, 8, d, 2, d, d, 2, 2, 128, 16, 1, None) == 1
    assert "alias" in lib.pkc_last_error().decode()
    assert lib.pkc_append_kv_ragged(d, d, 4, None, d, d, 8, d, 2, d, e, 2, 2, 128, 16, 1, None) == 1
    # tree-masked prefill without a mask
    assert lib.pkc_batch_prefill_paged_tree(None, d, d, d, 8, d, 2, d, d, None, d, 4, 2, 4, 2, 2, 128, 16,
                                            1, 1.0, d, d, None, 0, None) == 1
    # a plan with level write-through is refused by the level-only call before any launch
    p = api.make_params(3, 2, 2, 64, 4, num_ctas=1, level_ctas=2, level_write_through=True)
    info, _ = api.plan_host(p, [0, 0, 0], [{"qo_indptr": [0, 2, 3], "kv_lens": [4, 9], "causal": True}])
    assert info.lvl_write_through > 0
    p2 = api.make_params(2, 4, 4, 128, 16, num_ctas=1, level_ctas=1, level_write_through=True)
    p2.level_write_through = 3
    with pytest.raises(api.PkcError):
        api.plan_host(p2, [1, 2])


def test_noalloc_decode_refuses_oversized_plans_before_any_hip_call(api):
    """The allocation-free decode checks the plan against its fixed array before touching the
    device (dummy non-NULL pointers are never dereferenced), and refuses plans with levels."""
    lib = api.lib
    d = ctypes.c_void_p(0x1000)
    B = 4096
    info, hb = api.plan_host(api.make_params(B, 32, 32, 128, 16, num_ctas=B, level_ctas=1), [64] * B)
    assert info.dev_bytes > api.NOALLOC_SCRATCH_BYTES
    st = lib.pkc_batch_decode_paged_noalloc(ctypes.byref(info), ctypes.c_void_p(hb.data_ptr()), hb.numel(),
                                            d, d, d, 4, d, 4, d, None, B, 32, 32, 128, 16, 1, 0.1, d, d, None)
    assert st == 3 and "allocation-free" in lib.pkc_last_error().decode()
    # a host buffer smaller than the plan's integer arrays
    small, hb2 = api.plan_host(api.make_params(8, 4, 4, 128, 16, num_ctas=4, level_ctas=1), [100] * 8)
    assert lib.pkc_batch_decode_paged_noalloc(ctypes.byref(small), ctypes.c_void_p(hb2.data_ptr()), 16,
                                              d, d, d, 4, d, 8, d, None, 8, 4, 4, 128, 16, 1, 0.1, d, d,
                                              None) == 1
    # a plan with levels
    lv = [{"qo_indptr": [0, 8], "kv_lens": [64]}]
    info3, hb3 = api.plan_host(api.make_params(8, 4, 4, 128, 16, num_ctas=4, level_ctas=1), [10] * 8, lv)
    assert lib.pkc_batch_decode_paged_noalloc(ctypes.byref(info3), ctypes.c_void_p(hb3.data_ptr()), hb3.numel(),
                                              d, d, d, 4, d, 8, d, None, 8, 4, 4, 128, 16, 1, 0.1, d, d,
                                              None) == 4


def test_contraction_mode_and_counter_region(api):
    """The contraction parameter selects where split requests are merged (1: inside the decode
    kernel; 2: a merge pass; 0: 1 when #CTA <= B, else 2), and the plan's arrival counters (uint32 [B, Hkv],
    inside the integer arrays) are zero in every plan, also when the host buffer held other
    values before."""
    rng = random.Random(7)
    for mode, ctas, want in ((0, 24, 1), (0, 37, 1), (0, 38, 2), (1, 80, 1), (2, 24, 2)):
        B, hkv = 37, 4
        lens = [rng.randint(0, 5000) for _ in range(B)]
        p = api.make_params(B, 16, hkv, 128, 16, num_ctas=ctas, level_ctas=2, contraction=mode)
        nb = api.plan_buffer_sizes(p)[0]
        hb = torch.full((nb,), 0x5A, dtype=torch.uint8)
        info, hb = api.plan_host(p, lens, host_buf=hb)
        assert info.dec_contraction == want
        assert info.off_counters + B * hkv * 4 <= info.int_bytes
        assert info.off_counters >= info.off_req_levels
        ctr = hb.numpy().view("uint32")[info.off_counters // 4: info.off_counters // 4 + B * hkv]
        assert not ctr.any(), "counters must be zero in every plan"
        assert info.num_merge > 0
    with pytest.raises(api.PkcError) as e:
        api.plan_host(api.make_params(2, 4, 4, 128, 16, num_ctas=4, level_ctas=1, contraction=3), [1, 2])
    assert e.value.status == 1


def test_defer_upload_parameter(api):
    """defer_upload is 0 or 1; a host-only plan never carries a pending host source."""
    p = api.make_params(5, 8, 2, 128, 16, num_ctas=4, level_ctas=1, defer_upload=True)
    info, _ = api.plan_host(p, [3, 70, 0, 16, 900])
    assert info.host_src == 0
    bad = api.make_params(5, 8, 2, 128, 16, num_ctas=4, level_ctas=1)
    bad.defer_upload = 2
    with pytest.raises(api.PkcError) as e:
        api.plan_host(bad, [3, 70, 0, 16, 900])
    assert e.value.status == 1
