"""Pins of the oracle's load-balancing plan (CPU only).

Hand-worked examples (tests/golden/plan_hand_examples.json), the structural
invariants that the scheduler's steps imply, the appendix-D workspace bound,
and Graham's LPT makespan bound against a brute-forced optimum on tiny inputs.
"""

import itertools
import json
import os
import random

import pytest

from oracle import plan

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _examples():
    with open(os.path.join(GOLDEN, "plan_hand_examples.json")) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("ex", _examples())
def test_hand_examples(ex):
    n = len(ex["kv_lens"])
    st = plan.lpt_plan([1] * n, ex["kv_lens"], 1, ex["num_ctas"], ex["alpha"], ex["beta"])
    assert st.kv_chunk == ex["kv_chunk"]
    assert [[it.w, it.req, it.kv_begin, it.kv_end] for it in st.items] == ex["items"]
    assert st.order == ex["sorted_order"]
    assert st.cta_items == ex["cta_items"]
    assert st.cta_cost == ex["cta_cost"]
    slots = plan.assign_slots(st, lambda r: True)
    assert slots == ex["slots"]
    wt = sorted({st.items[w].req for w, s in enumerate(slots) if s < 0})
    assert wt == ex["write_through_requests"]


def _random_case(rng, tile_q=1):
    n = rng.randint(1, 40)
    kv = [rng.choice([0, 1, 2, 5, 16, 100, rng.randint(0, 5000)]) for _ in range(n)]
    qo = [1] * n if tile_q == 1 else [rng.randint(0, 9) for _ in range(n)]
    return qo, kv, rng.randint(1, 64), rng.choice([1, 1, 4, 16])


@pytest.mark.parametrize("seed", range(30))
@pytest.mark.parametrize("tile_q", [1, 4])
def test_invariants(seed, tile_q):
    rng = random.Random(seed)
    qo, kv, ctas, align = _random_case(rng, tile_q)
    alpha, beta = rng.randint(0, 3), rng.randint(0, 3)
    st = plan.lpt_plan(qo, kv, tile_q, ctas, alpha, beta, align)
    L = st.kv_chunk
    S = sum(plan.ceil_div(a, tile_q) * b for a, b in zip(qo, kv))
    assert L % align == 0 and L >= max(1, plan.ceil_div(S, ctas))
    assert L < max(1, plan.ceil_div(S, ctas)) + align
    # chunks of every tile partition [0, l_kv) exactly, ceil(l/L) of them, at most L long
    by_tile = {}
    for it in st.items:
        by_tile.setdefault((it.req, it.tile), []).append(it)
        assert 0 < it.length <= L
    for i, (lqo, lkv) in enumerate(zip(qo, kv)):
        for j in range(plan.ceil_div(lqo, tile_q)):
            ch = by_tile.get((i, j), [])
            assert len(ch) == plan.ceil_div(lkv, L)
            assert [c.kv_begin for c in ch] == [k * L for k in range(len(ch))]
            if ch:
                assert ch[-1].kv_end == lkv
                assert all(a.kv_end == b.kv_begin for a, b in zip(ch, ch[1:]))
            assert all(c.lq == min(tile_q, lqo - j * tile_q) for c in ch)
    # enumeration order and sorted order
    assert [it.w for it in st.items] == list(range(len(st.items)))
    lens = [st.items[w].length for w in st.order]
    assert lens == sorted(lens, reverse=True)
    for a, b in zip(st.order, st.order[1:]):
        if st.items[a].length == st.items[b].length:
            assert a < b
    # every item assigned once; costs add up
    flat = sorted(w for c in st.cta_items for w in c)
    assert flat == list(range(len(st.items)))
    for c, ws in enumerate(st.cta_items):
        assert st.cta_cost[c] == sum(alpha * st.items[w].lq + beta * st.items[w].length for w in ws)
    # item count bound and the appendix-D workspace bound
    n_tiles = sum(plan.ceil_div(a, tile_q) for a in qo)
    assert len(st.items) <= ctas + n_tiles
    slots = plan.assign_slots(st, lambda r: True)
    n_slots = sum(1 for s in slots if s >= 0)
    assert n_slots <= 2 * ctas
    assert sorted(s for s in slots if s >= 0) == list(range(n_slots))


def test_queue_ties_go_to_smaller_cta():
    st = plan.lpt_plan([1] * 4, [5, 5, 5, 5], 1, 4, enable_split=False)
    assert st.cta_items == [[0], [1], [2], [3]]
    st = plan.lpt_plan([1] * 5, [5, 5, 5, 5, 5], 1, 2, enable_split=False)
    assert st.cta_items == [[0, 2, 4], [1, 3]]


def test_empty_and_degenerate():
    st = plan.lpt_plan([1, 1], [0, 0], 1, 8)
    assert st.items == [] and st.kv_chunk == 1 and st.cta_cost == [0] * 8
    st = plan.lpt_plan([], [], 1, 3)
    assert st.items == []
    st = plan.lpt_plan([1], [1], 1, 1000)
    assert len(st.items) == 1 and st.kv_chunk == 1
    st = plan.lpt_plan([1, 1], [100, 3], 1, 4, enable_split=False)
    assert [it.length for it in st.items] == [100, 3]
    with pytest.raises(ValueError):
        plan.lpt_plan([1], [-1], 1, 4)


def _opt_makespan(costs, m):
    best = None
    for assign in itertools.product(range(m), repeat=len(costs)):
        loads = [0] * m
        for c, a in zip(costs, assign):
            loads[a] += c
        mk = max(loads)
        best = mk if best is None else min(best, mk)
    return best


@pytest.mark.parametrize("seed", range(25))
def test_lpt_graham_bound(seed):
    """With one query per request every item costs alpha + beta * length, so
    sorting by length is sorting by cost and the plan is Graham's LPT rule:
    makespan <= (4/3 - 1/(3m)) * OPT."""
    rng = random.Random(seed)
    m = rng.randint(2, 3)
    n = rng.randint(2, 6)
    kv = [rng.randint(1, 30) for _ in range(n)]
    st = plan.lpt_plan([1] * n, kv, 1, m, 1, 1, enable_split=rng.random() < 0.5)
    if len(st.items) > 8:
        pytest.skip("too many items for brute force")
    costs = [1 + it.length for it in st.items]
    opt = _opt_makespan(costs, m)
    assert plan.makespan(st) * 3 * m <= (4 * m - 1) * opt


def test_cascade_plan_merge_lists():
    """Level states first (levels in order, chunks ascending), then the
    request's own chunks; write-through (appendix D) only for an item that is
    its request's only state: one own chunk and no level covering the request.
    Worked by hand from the scheduler's steps."""
    levels = [{"qo_indptr": [0, 4], "kv_lens": [40]},
              {"qo_indptr": [0, 2, 3], "kv_lens": [10, 0]}]
    cp = plan.cascade_plan(5, levels, [8, 0, 30, 3, 4], num_ctas=4, level_ctas=2,
                           level_tile_q=[2, 1], alpha=1, beta=1)
    # level 0: 2 tiles of 2 queries x 40 tokens -> S = 80, L = 40 -> one chunk per tile
    assert [(it.req, it.tile, it.kv_begin, it.kv_end) for it in cp.levels[0].items] == [(0, 0, 0, 40), (0, 1, 0, 40)]
    assert cp.levels[0].slots == [0, 1]
    # level 1 (T_q = 1): group 0 has 2 one-query tiles of 10 tokens, group 1 has no KV
    # -> S = 2 * 10 = 20, L = 10 -> one chunk per tile
    assert [(it.req, it.tile, it.kv_begin, it.kv_end) for it in cp.levels[1].items] == \
        [(0, 0, 0, 10), (0, 1, 0, 10)]
    assert cp.levels[1].slots == [0, 1]
    # suffix: S = 45, L = 12
    assert cp.suffix.kv_chunk == 12
    assert [(it.req, it.kv_begin, it.kv_end) for it in cp.suffix.items] == \
        [(0, 0, 8), (2, 0, 12), (2, 12, 24), (2, 24, 30), (3, 0, 3), (4, 0, 4)]
    # requests 0..3 are covered by level 0, so their own chunks are partial states even when
    # single (requests 0 and 3); request 4 (no level, one chunk) writes through
    assert cp.suffix.slots == [0, 1, 2, 3, 4, -1]
    assert cp.write_through == [False, False, False, False, True]
    assert cp.merge[0] == [(0, 0, 0), (1, 0, 0), ("suffix", 0, 0)]
    assert cp.merge[1] == [(0, 0, 1), (1, 1, 0)]
    assert cp.merge[2] == [(0, 1, 0), ("suffix", 1, 0), ("suffix", 2, 0), ("suffix", 3, 0)]
    assert cp.merge[3] == [(0, 1, 1), ("suffix", 4, 0)]
    assert cp.merge[4] == []


def test_fused_fold_transform_hand_example():
    """The library finishes a request whose merge list is its level states plus one own chunk
    in that chunk's decode item (the item folds the level states in): the transform of the
    appendix-D plan above makes requests 0 and 3 write-through, drops their own chunk from
    their merge lists and renumbers the remaining partial slots densely in ascending w."""
    from plan_transform import fused_fold
    levels = [{"qo_indptr": [0, 4], "kv_lens": [40]},
              {"qo_indptr": [0, 2, 3], "kv_lens": [10, 0]}]
    cp = plan.cascade_plan(5, levels, [8, 0, 30, 3, 4], num_ctas=4, level_ctas=2,
                           level_tile_q=[2, 1], alpha=1, beta=1)
    f = fused_fold(cp)
    assert f.suffix.slots == [-1, 0, 1, 2, -1, -1]
    assert f.write_through == [True, False, False, True, True]
    assert f.merge[0] == [(0, 0, 0), (1, 0, 0)]
    assert f.merge[1] == [(0, 0, 1), (1, 1, 0)]
    assert f.merge[2] == [(0, 1, 0), ("suffix", 0, 0), ("suffix", 1, 0), ("suffix", 2, 0)]
    assert f.merge[3] == [(0, 1, 1)]
    assert f.merge[4] == []
    # the appendix-D plan itself is unchanged
    assert cp.suffix.slots == [0, 1, 2, 3, 4, -1]


@pytest.mark.parametrize("seed", range(30))
def test_fused_fold_keeps_items_and_states(seed):
    """The fold moves no work: the same items on the same CTAs in the same order, level slots
    unchanged, and per request the same set of states combined (a folded request's own chunk
    is the finishing item itself instead of a merge-list entry)."""
    from plan_transform import fused_fold
    rng = random.Random(seed)
    B = rng.randint(1, 40)
    levels = []
    for _ in range(rng.randint(0, 3)):
        cuts = sorted(rng.sample(range(0, B + 1), min(rng.randint(2, 5), B + 1)))
        if len(cuts) < 2:
            cuts = [0, B]
        levels.append({"qo_indptr": cuts, "kv_lens": [rng.choice([0, 7, rng.randint(1, 900)])
                                                       for _ in range(len(cuts) - 1)]})
    kv = [rng.choice([0, 3, 64, rng.randint(0, 700)]) for _ in range(B)]
    tq = [rng.choice([1, 2, 8]) for _ in levels]
    cp = plan.cascade_plan(B, levels, kv, num_ctas=rng.choice([1, 4, 16]), level_ctas=rng.choice([1, 3]),
                           level_tile_q=tq, enable_split=rng.random() < 0.8)
    f = fused_fold(cp)
    assert [it.w for it in f.suffix.items] == [it.w for it in cp.suffix.items]
    assert f.suffix.cta_items == cp.suffix.cta_items
    assert [st.slots for st in f.levels] == [st.slots for st in cp.levels]
    n_slots = sum(1 for s in f.suffix.slots if s >= 0)
    assert sorted(s for s in f.suffix.slots if s >= 0) == list(range(n_slots))
    own = {}
    for it in cp.suffix.items:
        own.setdefault(it.req, []).append(it.w)
    for b in range(B):
        lv_a = [e for e in cp.merge[b] if e[0] != "suffix"]
        lv_b = [e for e in f.merge[b] if e[0] != "suffix"]
        assert lv_a == lv_b
        states_a = sorted(cp.suffix.slots.index(e[1]) for e in cp.merge[b] if e[0] == "suffix")
        states_b = sorted(f.suffix.slots.index(e[1]) for e in f.merge[b] if e[0] == "suffix")
        if f.write_through[b] and not cp.write_through[b]:
            assert len(own.get(b, [])) == 1 and states_b == [] and states_a == own[b]
            assert f.suffix.slots[own[b][0]] == -1
        else:
            assert states_a == states_b and f.write_through[b] == cp.write_through[b]


# --- causal query tiles (ragged multi-token queries) -----------------------------------------

def test_causal_hand_example():
    """One request of 5 queries over 7 tokens, T_q = 2, two CTAs, alpha = beta = 1 (worked by
    hand): tile extents 7-5+2 = 4, 7-5+4 = 6, 7-5+5 = 7, S = 17, L_kv = 9, one chunk each;
    sorted w2 (7), w1 (6), w0 (4); CTA0 <- w2 (1+7), CTA1 <- w1 (2+6), tie -> CTA0 <- w0 (2+4)."""
    st = plan.lpt_plan([5], [7], 2, 2, 1, 1, causal=True)
    assert st.kv_chunk == 9
    assert [[it.w, it.tile, it.lq, it.kv_begin, it.kv_end] for it in st.items] == \
        [[0, 0, 2, 0, 4], [1, 1, 2, 0, 6], [2, 2, 1, 0, 7]]
    assert st.order == [2, 1, 0]
    assert st.cta_items == [[2, 0], [1]]
    assert st.cta_cost == [14, 8]


def test_causal_tiles_that_see_nothing_get_no_item():
    """4 queries over 2 tokens, T_q = 2, three CTAs: the first tile's queries see nothing
    (extent 2-4+2 = 0); the second sees 2 tokens, S = 2, L_kv = 1: two chunks."""
    st = plan.lpt_plan([4], [2], 2, 3, 1, 1, causal=True)
    assert [[it.tile, it.kv_begin, it.kv_end] for it in st.items] == [[1, 0, 1], [1, 1, 2]]


@pytest.mark.parametrize("seed", range(10))
def test_causal_extent_is_the_last_querys_visible_length(seed):
    """The chunks of every causal tile cover exactly [0, n) where n is the number of tokens the
    tile's last query sees by the attention oracle's definition (and nothing for tiles whose
    queries see none); non-causal tiles cover [0, l_kv)."""
    from oracle.attention import prefill_limit
    rng = random.Random(seed)
    qo = [rng.randint(0, 40) for _ in range(rng.randint(1, 6))]
    kv = [max(0, q + rng.randint(-10, 60)) for q in qo]
    tq = rng.choice([1, 3, 8, 16])
    for causal in (False, True):
        st = plan.lpt_plan(qo, kv, tq, rng.randint(1, 9), causal=causal, enable_split=rng.random() < 0.7)
        cover = {}
        for it in st.items:
            cover.setdefault((it.req, it.tile), []).append((it.kv_begin, it.kv_end))
        for i, (lq, lkv) in enumerate(zip(qo, kv)):
            for j in range(plan.ceil_div(lq, tq)):
                last = min((j + 1) * tq, lq) - 1
                n = prefill_limit(lq, lkv, last, causal)
                segs = sorted(cover.get((i, j), []))
                if n == 0:
                    assert segs == []
                else:
                    assert segs[0][0] == 0 and segs[-1][1] == n
                    assert all(a[1] == b[0] for a, b in zip(segs, segs[1:]))


def test_level_write_through_hand_example():
    """Prefill-shaped plan (one level, no own KV): query lengths [3, 1], KV lengths [3, 40],
    T_q = 2, #CTA = 2.  S = 2 * 3 + 1 * 40 = 46, L = 23: request 0's two tiles are one chunk
    each and write through; request 1's tile is cut into [0, 23) and [23, 40), whose states
    take slots 0 and 1 and are merged.  Worked by hand from the scheduler's steps."""
    levels = [{"qo_indptr": [0, 3, 4], "kv_lens": [3, 40]}]
    o = plan.cascade_plan(4, levels, [0] * 4, num_ctas=1, level_ctas=2, level_tile_q=[2],
                          level_write_through=True)
    st = o.levels[0]
    assert st.kv_chunk == 23
    assert [(it.req, it.tile, it.kv_begin, it.kv_end) for it in st.items] == \
        [(0, 0, 0, 3), (0, 1, 0, 3), (1, 0, 0, 23), (1, 0, 23, 40)]
    assert st.slots == [-1, -1, 0, 1]
    assert o.write_through == [True, True, True, False]
    assert o.merge == [[], [], [], [(0, 0, 0), (0, 1, 0)]]
    # Without the flag, or with a second level, or with own KV in the group, nothing writes
    # through at the level.
    o2 = plan.cascade_plan(4, levels, [0] * 4, num_ctas=1, level_ctas=2, level_tile_q=[2])
    assert o2.levels[0].slots == [0, 1, 2, 3] and not any(o2.write_through)
    o3 = plan.cascade_plan(4, levels, [0, 0, 5, 0], num_ctas=1, level_ctas=2, level_tile_q=[2],
                           level_write_through=True)
    assert o3.levels[0].slots == [0, 1, 2, 3]
