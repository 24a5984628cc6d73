"""fp64 attention states by definition (oracle; test infrastructure only).

Definitions followed (same on three pages):

* "Attention States and Recursive Attention" (FlashInfer tutorial), the
  definitions of the generalised score and value:  s(I) is the log of the
  sum over i in I of exp(s_i);  v(I) is the exp(s_i)-weighted sum of v_i
  divided by exp(s(I));  the state of I is the pair (v(I), s(I)).  The
  generalised score is the log-sum-exp (LSE).
* "Cascade Inference" blog, "Recursive attention" section: the same pair,
  with the remark that the maximum is subtracted in practice for stability.
* FlashInfer paper summary, section A2 "Attention composition": O(T) and
  LSE(T) of a query over an index set T.

The pages write the pre-softmax score as the plain product q . k_i; every
kernel here scales it first, so s_i = sm_scale * (q . k_i) and LSE is defined
on the scaled scores (reading R1).  Natural logarithm throughout.

The batch decode and cascade results below are computed as ONE softmax over
the union of each request's token sets.  They never use the merge operator,
so they check the cascade's decomposition instead of repeating it.
"""

from __future__ import annotations

import math

import numpy as np

from .indexing import token_pages

NEG_INF = -math.inf


def attention_state(q, keys, values, sm_scale):
    """State of query rows over one token set.

    q: [R, D] (R query rows that share the token set) or [D];
    keys: [n, D]; values: [n, Dv].
    Returns (O [R, Dv], LSE [R]) in float64.  An empty token set gives the
    identity state (O = 0, LSE = -inf).
    """
    q = np.asarray(q, dtype=np.float64)
    single = q.ndim == 1
    q2 = q[None, :] if single else q
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    n = keys.shape[0]
    rows = q2.shape[0]
    if n == 0:
        o = np.zeros((rows, values.shape[1]))
        lse = np.full(rows, NEG_INF)
    else:
        s = float(sm_scale) * (q2 @ keys.T)          # [R, n] scaled scores s_i
        m = s.max(axis=1, keepdims=True)             # subtract the max (stability)
        lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))   # s(I)
        p = np.exp(s - lse[:, None])                 # exp(s_i) / exp(s(I))
        o = p @ values                               # v(I)
    if single:
        return o[0], float(lse[0])
    return o, lse


def _gather(pool, pages, slots, kv_head):
    """Rows pool[page, slot, kv_head] as float64 [n, D] (exact upcast)."""
    return np.asarray(pool[pages, slots, kv_head], dtype=np.float64)


def _state_over_rows(q, k_pool, v_pool, pages, slots, sm_scale, heads):
    """O [Hq, D] and LSE [Hq] of one query token over gathered rows.
    GQA head map: query head h reads kv head h // g (reading R3).
    One kv head is gathered at a time to bound memory."""
    hq, d = q.shape
    hkv = k_pool.shape[2]
    g = hq // hkv
    o = np.full((hq, d), np.nan)
    lse = np.full(hq, np.nan)
    for kh in sorted({h // g for h in heads}):
        K = _gather(k_pool, pages, slots, kh)
        V = _gather(v_pool, pages, slots, kh)
        for h in heads:
            if h // g == kh:
                o[h], lse[h] = attention_state(q[h], K, V, sm_scale)
    return o, lse


def batch_decode(q, k_pool, v_pool, block_table, cache_seqlens, page_size,
                 sm_scale, kv_start=None, requests=None, heads=None):
    """Paged batch decode: request b attends over tokens
    [kv_start[b], cache_seqlens[b]) gathered through block_table[b]
    ("Paged attention" page, decode path).

    q: [B, Hq, D]; k_pool / v_pool: [num_pages, P, Hkv, D] (anything that
    supports ``pool[pages, slots]`` and converts to float64).
    ``requests`` / ``heads`` restrict the work (sampled parity); entries that
    are not computed are NaN.  Returns (O [B, Hq, D], LSE [B, Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    O = np.full((B, Hq, D), np.nan)
    L = np.full((B, Hq), np.nan)
    reqs = range(B) if requests is None else requests
    hs = list(range(Hq)) if heads is None else list(heads)
    for b in reqs:
        start = 0 if kv_start is None else int(kv_start[b])
        pages, slots = token_pages(block_table[b], start, int(cache_seqlens[b]), page_size)
        O[b], L[b] = _state_over_rows(q[b], k_pool, v_pool, pages, slots, sm_scale, hs)
    return O, L


def group_of(qo_indptr, b):
    """Group g of a cascade level with qo_indptr[g] <= b < qo_indptr[g+1],
    or None when the level does not cover request b."""
    for g in range(len(qo_indptr) - 1):
        if qo_indptr[g] <= b < qo_indptr[g + 1]:
            return g
    return None


def cascade_token_rows(b, levels, suffix_block_table, suffix_seqlens, page_size):
    """The disjoint union of request b's token sets over all cascade levels
    (shared prefix, group prefixes ...) and its unique suffix, in that order.

    Each level is a dict with ``qo_indptr`` [G+1] (requests of each group),
    ``kv_page_indptr`` [G+1], ``kv_page_indices`` (pages of each group's KV
    run, BSR column indices) and ``kv_lens`` [G] (tokens).  This is the
    composable-format view (paper summary, A3): a shared prefix is a dense
    block of the KV sparse matrix addressed by its own indptr/indices, with no
    data moved.  Returns (pages, slots) int64 arrays.
    """
    all_p, all_s = [], []
    for lv in levels:
        g = group_of(lv["qo_indptr"], b)
        if g is None:
            continue
        lo, hi = int(lv["kv_page_indptr"][g]), int(lv["kv_page_indptr"][g + 1])
        p, s = token_pages(list(lv["kv_page_indices"][lo:hi]), 0, int(lv["kv_lens"][g]), page_size)
        all_p.append(p)
        all_s.append(s)
    if suffix_block_table is not None:
        p, s = token_pages(suffix_block_table[b], 0, int(suffix_seqlens[b]), page_size)
        all_p.append(p)
        all_s.append(s)
    if not all_p:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    return np.concatenate(all_p), np.concatenate(all_s)


def cascade_decode(q, k_pool, v_pool, page_size, sm_scale, levels,
                   suffix_block_table, suffix_seqlens, requests=None, heads=None):
    """Exact result of cascade decoding: the attention of each request's query
    over the union of its level token sets and its suffix, as one softmax
    ("Cascade Inference" blog, algorithm section: the three steps only
    reorganise this computation).  Returns (O [B, Hq, D], LSE [B, Hq])."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    O = np.full((B, Hq, D), np.nan)
    L = np.full((B, Hq), np.nan)
    reqs = range(B) if requests is None else requests
    hs = list(range(Hq)) if heads is None else list(heads)
    for b in reqs:
        pages, slots = cascade_token_rows(b, levels, suffix_block_table, suffix_seqlens, page_size)
        O[b], L[b] = _state_over_rows(q[b], k_pool, v_pool, pages, slots, sm_scale, hs)
    return O, L


def level_prefix_states(q, k_pool, v_pool, page_size, sm_scale, level, num_requests):
    """State of every covered request's query over its group's KV run at one
    level (the multi-query step of the cascade).  Uncovered rows are NaN."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    O = np.full((B, Hq, D), np.nan)
    L = np.full((B, Hq), np.nan)
    for b in range(num_requests):
        if group_of(level["qo_indptr"], b) is None:
            continue
        pages, slots = cascade_token_rows(b, [level], None, None, page_size)
        O[b], L[b] = _state_over_rows(q[b], k_pool, v_pool, pages, slots, sm_scale, range(Hq))
    return O, L


def prefill_limit(lq, lkv, i, causal):
    """Number of KV tokens query i of a request with lq queries and lkv KV tokens sees: the
    queries are the request's last lq tokens, so query i sits at position lkv - lq + i and,
    with the causal mask, sees tokens 0 .. lkv - lq + i (none when that is negative); without
    it, all lkv tokens."""
    if not causal:
        return lkv
    return max(0, min(lkv, lkv - lq + i + 1))


def batch_prefill(q, qo_indptr, k_pool, v_pool, block_table, kv_lens, page_size, sm_scale,
                  causal, rows=None, heads=None, tree_masks=None):
    """Ragged multi-token queries over a paged KV cache.

    q: [total_q, Hq, D], packed without padding: request b's queries are rows
    qo_indptr[b] .. qo_indptr[b+1]-1 (the cu_seq_lens_q indexing of the "Paged attention"
    page's varlen path; the paper summary's ragged query tensors, section A3).  Request b's
    KV is its block-table row over kv_lens[b] tokens (decode-path indexing), already holding
    the new tokens.  Query i of request b attends over the first prefill_limit(...) tokens.
    ``rows`` restricts the work to some query rows (sampled parity); other rows are NaN.
    ``tree_masks`` (tree / speculative decoding: the paper summary's logits mask, section A2
    and the JIT variant functors of A3; reading R32): per request None or an [lq, lq] boolean
    matrix over its new tokens.  Query i then sees the tokens before the new ones and new token
    j only where mask[i][j] holds, inside its causal limit.
    Returns (O [total_q, Hq, D], LSE [total_q, Hq])."""
    q = np.asarray(q, dtype=np.float64)
    T, Hq, D = q.shape
    O = np.full((T, Hq, D), np.nan)
    L = np.full((T, Hq), np.nan)
    want = None if rows is None else set(int(r) for r in rows)
    hs = list(range(Hq)) if heads is None else list(heads)
    B = len(qo_indptr) - 1
    for b in range(B):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        lq, lkv = q1 - q0, int(kv_lens[b])
        for i in range(lq):
            r = q0 + i
            if want is not None and r not in want:
                continue
            n = prefill_limit(lq, lkv, i, causal)
            pages, slots = token_pages(block_table[b], 0, n, page_size)
            tm = None if tree_masks is None else tree_masks[b]
            if tm is not None:
                base = lkv - lq   # position of the first new token
                keep = np.array([t < base or bool(tm[i][t - base]) for t in range(n)], dtype=bool)
                pages, slots = np.asarray(pages)[keep], np.asarray(slots)[keep]
            O[r], L[r] = _state_over_rows(q[r], k_pool, v_pool, pages, slots, sm_scale, hs)
    return O, L
