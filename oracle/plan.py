"""CPU load-balancing plan (oracle; test infrastructure only).

Follows the FlashInfer paper summary, section A3 "Dynamic-aware runtime --
load-balancing scheduling", and appendix D (memory management):

1. Input: per-request query and KV lengths {l_qo(i), l_kv(i)} and a query
   tile size T_q.
2. Cost of a tile with l_q query rows and l_kv KV tokens:
   alpha * l_q + beta * l_kv.
3. Maximum KV chunk length: L_kv = (sum_i ceil(l_qo(i) / T_q) * l_kv(i)) / #CTA.
4. Every query tile's KV is cut into chunks of at most L_kv; each chunk is a
   work item w with length l_kv(w).
5. The work list W is sorted by length, longest first.
6. A priority queue Q holds (CTA, cost) with every cost 0.
7. While W is not empty: take the CTA with the smallest cost from Q and the
   next item from W, give the item to that CTA, and push the CTA back with
   its cost increased by the item's cost.
Appendix D: only tiles whose KV was actually split write partial states to
the workspace; unsplit tiles write straight to the final output
(write-through).  The partial-output workspace is bounded by
2 * #CTA * T_q * H_qo * (D + 1) floats.

Readings where the pages are silent (each one is listed in the design notes):
* R10 all lengths are tokens; decode uses T_q = 1 and l_q = 1;
* R11 L_kv = max(1, ceil(S / #CTA)), then rounded up to a multiple of
  ``chunk_align``;
* R12 chunks are cut greedily from the front, the last one shorter; a tile
  with l_kv = 0 yields no item;
* R13 the sort is stable (equal lengths keep ascending w);
* R14 queue ties go to the smaller CTA index;
* R15 costs are integers, alpha and beta non-negative integers;
* R16 a CTA runs its items in assignment order;
* R17 partial slots are numbered densely in ascending w over the items that
  do not write through.
``enable_split=False`` makes L_kv the longest KV length, i.e. one chunk per
tile.
"""

from __future__ import annotations

import heapq
from dataclasses import dataclass, field


@dataclass(frozen=True)
class WorkItem:
    w: int          # work index, enumeration order of step 4
    req: int        # request (decode) or group (cascade level) index i
    tile: int       # query tile j of that request
    lq: int         # query rows in the tile
    kv_begin: int   # chunk [kv_begin, kv_end) of the tile's KV, in tokens
    kv_end: int

    @property
    def length(self) -> int:
        return self.kv_end - self.kv_begin


@dataclass
class StagePlan:
    kv_chunk: int                       # L_kv
    items: list                         # WorkItem, index == w
    order: list                         # W after the sort of step 5 (list of w)
    cta_items: list                     # per CTA: list of w in assignment order
    cta_cost: list                      # final cost of every CTA
    slots: list = field(default_factory=list)   # per w: partial slot or -1


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def tile_extent(lqo, lkv, tile_q, j, causal):
    """KV tokens query tile j of a request needs: all l_kv, or with the causal mask (the
    request's l_qo queries are its last tokens) the tokens its last query sees, reading R28:
    l_kv - l_qo + min((j + 1) T_q, l_qo), clamped to [0, l_kv]."""
    if not causal:
        return lkv
    return min(lkv, max(0, lkv - lqo + min((j + 1) * tile_q, lqo)))


def lpt_plan(qo_lens, kv_lens, tile_q, num_ctas, alpha=1, beta=1,
             chunk_align=1, enable_split=True, causal=False) -> StagePlan:
    """Steps 1-7 of the scheduler for one stage.  With ``causal`` every query tile's KV is
    its causal extent (``tile_extent``) in steps 3 and 4."""
    if tile_q < 1 or num_ctas < 1 or chunk_align < 1:
        raise ValueError("tile_q, num_ctas and chunk_align must be >= 1")
    if alpha < 0 or beta < 0:
        raise ValueError("alpha and beta must be non-negative")
    qo_lens = [int(x) for x in qo_lens]
    kv_lens = [int(x) for x in kv_lens]
    if len(qo_lens) != len(kv_lens) or any(x < 0 for x in qo_lens + kv_lens):
        raise ValueError("bad lengths")

    # Step 3: maximum chunk length.
    if enable_split:
        total = sum(tile_extent(lqo, lkv, tile_q, j, causal)
                    for lqo, lkv in zip(qo_lens, kv_lens) for j in range(ceil_div(lqo, tile_q)))
        L = max(1, ceil_div(total, num_ctas))
    else:
        L = max([1] + kv_lens)
    L = ceil_div(L, chunk_align) * chunk_align

    # Step 4: chunk every query tile's KV; w follows (request, tile, chunk).
    items = []
    for i, (lqo, lkv) in enumerate(zip(qo_lens, kv_lens)):
        for j in range(ceil_div(lqo, tile_q)):
            lq = min(tile_q, lqo - j * tile_q)
            ext = tile_extent(lqo, lkv, tile_q, j, causal)
            for c in range(ceil_div(ext, L)):
                items.append(WorkItem(len(items), i, j, lq, c * L, min((c + 1) * L, ext)))

    # Step 5: longest first (stable).
    order = [it.w for it in sorted(items, key=lambda it: -it.length)]

    # Steps 6-7: min-cost CTA first, ties to the smaller CTA index.
    queue = [(0, c) for c in range(num_ctas)]
    heapq.heapify(queue)
    cta_items = [[] for _ in range(num_ctas)]
    cta_cost = [0] * num_ctas
    for w in order:
        cost, c = heapq.heappop(queue)
        cta_items[c].append(w)
        it = items[w]
        cost += alpha * it.lq + beta * it.length
        cta_cost[c] = cost
        heapq.heappush(queue, (cost, c))
    return StagePlan(L, items, order, cta_items, cta_cost)


def assign_slots(stage: StagePlan, may_write_through) -> list:
    """Appendix D write-through: an item writes to the final output (slot -1)
    when its tile has exactly one chunk and ``may_write_through(req)`` holds;
    every other item gets the next partial slot in ascending w."""
    chunks = {}
    for it in stage.items:
        chunks[(it.req, it.tile)] = chunks.get((it.req, it.tile), 0) + 1
    slots, n = [], 0
    for it in stage.items:
        if chunks[(it.req, it.tile)] == 1 and may_write_through(it.req):
            slots.append(-1)
        else:
            slots.append(n)
            n += 1
    stage.slots = slots
    return slots


@dataclass
class CascadePlan:
    levels: list        # StagePlan per cascade level (prefix stages)
    level_tile_q: list  # T_q of every level
    suffix: StagePlan   # decode stage over every request's own KV
    merge: list         # per request: ordered list of (stage, slot, row)
    write_through: list  # per request: True when the decode stage wrote it


def cascade_plan(batch, levels, suffix_kv_lens, num_ctas, level_ctas,
                 level_tile_q, alpha=1, beta=1, chunk_align=1,
                 enable_split=True, level_write_through=False) -> CascadePlan:
    """Plan of a cascade step (or of a plain batch decode when ``levels`` is
    empty).

    ``levels``: list of dicts with host ``qo_indptr`` [G+1] and ``kv_lens`` [G];
    the requests of group g are qo_indptr[g] <= b < qo_indptr[g+1] (reading R19).
    Each level is one stage: the query tile of a group is T_q consecutive
    requests of the group, its KV is the group's shared run.  Level items
    always write partial states.  The decode stage has one query per request
    (T_q = 1).  Appendix D's write-through rule: an item writes the final
    output only when it is its request's only state, i.e. the request's own
    KV is one chunk and no level covers the request; every other request is
    finished by the merge pass over its merge list.

    Merge order (reading R9): levels in order, chunks ascending, then the
    request's own chunks ascending.  A merge entry is (stage, slot, row):
    stage is the level index or 'suffix', row the query's index inside its
    tile.

    ``level_write_through`` (batch prefill, reading R30): with a single
    level, the appendix D write-through rule also applies to the level, for
    the groups none of whose requests has own KV: a tile with one chunk
    writes its rows' final output, and those requests are not merged.
    """
    lvl_plans = []
    covered = [False] * batch   # some level holds a state of the request
    for li, lv in enumerate(levels):
        qi = [int(x) for x in lv["qo_indptr"]]
        qo_lens = [qi[g + 1] - qi[g] for g in range(len(qi) - 1)]
        st = lpt_plan(qo_lens, lv["kv_lens"], level_tile_q[li], level_ctas, alpha,
                      beta, chunk_align, enable_split, causal=bool(lv.get("causal", False)))
        if level_write_through and len(levels) == 1:
            no_own_kv = [all(int(suffix_kv_lens[b]) == 0 for b in range(qi[g], qi[g + 1]))
                         for g in range(len(qo_lens))]
            assign_slots(st, lambda g: no_own_kv[g])
        else:
            assign_slots(st, lambda g: False)
        for it in st.items:
            b0 = qi[it.req] + it.tile * level_tile_q[li]
            for b in range(b0, b0 + it.lq):
                covered[b] = True
        lvl_plans.append(st)

    suf = lpt_plan([1] * batch, suffix_kv_lens, 1, num_ctas, alpha, beta,
                   chunk_align, enable_split)
    assign_slots(suf, lambda r: not covered[r])

    merge = [[] for _ in range(batch)]
    wt = [False] * batch
    for li, (lv, st) in enumerate(zip(levels, lvl_plans)):
        qi = [int(x) for x in lv["qo_indptr"]]
        tq = level_tile_q[li]
        for it in st.items:          # ascending w == ascending chunk per tile
            b0 = qi[it.req] + it.tile * tq
            for r in range(it.lq):
                if st.slots[it.w] < 0:
                    wt[b0 + r] = True
                else:
                    merge[b0 + r].append((li, st.slots[it.w], r))
    for it in suf.items:
        if suf.slots[it.w] < 0:
            wt[it.req] = True
        else:
            merge[it.req].append(("suffix", suf.slots[it.w], 0))
    return CascadePlan(lvl_plans, list(level_tile_q), suf, merge, wt)


def makespan(stage: StagePlan) -> int:
    return max(stage.cta_cost) if stage.cta_cost else 0
