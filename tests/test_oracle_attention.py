"""Pins of the fp64 oracle's attention, merge and indexing (CPU only).

Each test checks the oracle against something other than itself: the merge
operator's closed form and algebra stated on the pages, the singleton case,
closed forms of uniform scores, a dominant key, torch's CPU attention routine,
mpmath brute force, and the worked examples printed on the Hugging Face
"Paged attention" page (fixtures under tests/golden/).
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import attention, indexing, merge

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(seed, n, d, dv=None):
    rng = np.random.default_rng(seed)
    return rng.normal(size=d), rng.normal(size=(n, d)), rng.normal(size=(n, dv or d))


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(1e-300, float(np.max(np.abs(b)))))


# --- Π1: the merge operator's closed form (binary and n-ary) --------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_merge_of_partition_equals_state_of_union(seed):
    """State of the union == merge of the states of a partition, for contiguous
    and scattered partitions ("Attention States and Recursive Attention",
    binary and n-ary merge equations)."""
    q, K, V = _rand(seed, 97, 24)
    scale = 0.37
    o_all, l_all = attention.attention_state(q, K, V, scale)
    rng = np.random.default_rng(100 + seed)
    for parts in (2, 3, 7):
        for scattered in (False, True):
            if scattered:
                lab = rng.integers(0, parts, size=97)
            else:
                cuts = np.sort(rng.choice(np.arange(1, 97), size=parts - 1, replace=False))
                lab = np.searchsorted(cuts, np.arange(97), side="right")
            os_, ls_ = [], []
            for p in range(parts):
                idx = np.nonzero(lab == p)[0]
                o, l = attention.attention_state(q, K[idx], V[idx], scale)
                os_.append(o)
                ls_.append(l)
            om, lm = merge.merge_many(os_, ls_)
            assert _rel(om, o_all) < 1e-12
            assert abs(lm - l_all) < 1e-12 * max(1.0, abs(l_all))
            ob, lb = os_[0], ls_[0]
            for o, l in zip(os_[1:], ls_[1:]):
                ob, lb = merge.merge_pair(ob, lb, o, l)
            assert _rel(ob, o_all) < 1e-12
            assert abs(lb - l_all) < 1e-12 * max(1.0, abs(l_all))


def test_binary_merge_matches_printed_formula_without_max_trick():
    """With moderate scores the max-subtracted merge equals the formula exactly
    as printed: (v_I e^{s_I} + v_J e^{s_J}) / (e^{s_I} + e^{s_J}),
    log(e^{s_I} + e^{s_J})."""
    rng = np.random.default_rng(7)
    va, vb = rng.normal(size=5), rng.normal(size=5)
    sa, sb = 0.3, -1.2
    o, l = merge.merge_pair(va, sa, vb, sb)
    ea, eb = math.exp(sa), math.exp(sb)
    assert np.allclose(o, (va * ea + vb * eb) / (ea + eb), rtol=1e-14, atol=0)
    assert abs(l - math.log(ea + eb)) < 1e-15


def test_merge_huge_scores_stay_finite():
    """Subtracting the max (noted on both merge pages) keeps scores of 1e4 finite."""
    o, l = merge.merge_pair(np.ones(3), 1.0e4, 2 * np.ones(3), 1.0e4)
    assert np.all(np.isfinite(o)) and np.allclose(o, 1.5) and abs(l - (1.0e4 + math.log(2))) < 1e-9


# --- Π2: commutativity and associativity ------------------------------------------------------

@pytest.mark.parametrize("seed", range(4))
def test_merge_commutative_associative(seed):
    """Any order and bracketing gives the same state ("Cascade Inference" blog,
    recursive attention section and Fig. 2)."""
    q, K, V = _rand(seed, 40, 8)
    states = [attention.attention_state(q, K[i::5], V[i::5], 0.5) for i in range(5)]
    ref_o, ref_l = merge.merge_many([s[0] for s in states], [s[1] for s in states])
    rng = np.random.default_rng(seed)
    for _ in range(10):
        perm = rng.permutation(5)
        o, l = states[perm[0]]
        for i in perm[1:]:
            o, l = merge.merge_pair(o, l, *states[i])
        assert _rel(o, ref_o) < 1e-12 and abs(l - ref_l) < 1e-12
    # bracketing: (a+b)+(c+(d+e)) vs a+(b+(c+(d+e)))
    a, b, c, d, e = states
    x = merge.merge_pair(*merge.merge_pair(*a, *b), *merge.merge_pair(*c, *merge.merge_pair(*d, *e)))
    y = merge.merge_pair(*a, *merge.merge_pair(*b, *merge.merge_pair(*c, *merge.merge_pair(*d, *e))))
    assert _rel(x[0], y[0]) < 1e-12 and abs(x[1] - y[1]) < 1e-12
    # binary merge is symmetric bit for bit
    o1, l1 = merge.merge_pair(*a, *b)
    o2, l2 = merge.merge_pair(*b, *a)
    assert np.array_equal(o1, o2) and l1 == l2


# --- Π3: the singleton case -------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(5))
def test_singleton_state_is_exact(seed):
    """s({i}) = s_i and v({i}) = v_i ("Cascade Inference" blog, recursive
    attention section) -- exactly, in fp64."""
    q, K, V = _rand(seed, 1, 16)
    o, l = attention.attention_state(q, K, V, 0.125)
    s = 0.125 * float(K[0] @ q)
    assert l == s
    assert np.array_equal(o, V[0])


# --- Π4: identity element and empty sets -------------------------------------------------------

def test_identity_and_empty_sets():
    q, K, V = _rand(3, 10, 4)
    o, l = attention.attention_state(q, K[:0], V[:0], 1.0)
    assert np.array_equal(o, np.zeros(4)) and l == -math.inf
    x = attention.attention_state(q, K, V, 1.0)
    y = merge.merge_pair(x[0], x[1], np.zeros(4), -math.inf)
    assert np.array_equal(y[0], x[0]) and y[1] == x[1]
    y = merge.merge_pair(np.zeros(4), -math.inf, x[0], x[1])
    assert np.array_equal(y[0], x[0]) and y[1] == x[1]
    z = merge.merge_many([np.zeros(4), np.zeros(4)], [-math.inf, -math.inf])
    assert np.array_equal(z[0], np.zeros(4)) and z[1] == -math.inf
    z = merge.merge_many(np.zeros((0, 4)), np.zeros(0))
    assert np.array_equal(z[0], np.zeros(4)) and z[1] == -math.inf


def test_varlen_request_with_zero_keys_gets_identity():
    """The varlen example has a request (r0) with zero key tokens; its state is
    the merge identity, never NaN."""
    g = _golden("hf_varlen_example.json")
    cu_k = indexing.cu_seq_lens(g["key_lens"])
    rng = np.random.default_rng(0)
    K = rng.normal(size=(cu_k[-1], 8))
    V = rng.normal(size=(cu_k[-1], 8))
    o, l = attention.attention_state(rng.normal(size=8), K[cu_k[0]:cu_k[1]], V[cu_k[0]:cu_k[1]], 1.0)
    assert np.array_equal(o, np.zeros(8)) and l == -math.inf


# --- Π5: uniform scores ------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 17, 4096])
def test_uniform_scores_closed_form(n):
    """q = 0 makes every score 0: LSE = ln n and O = mean of the values."""
    _, K, V = _rand(n, n, 8)
    o, l = attention.attention_state(np.zeros(8), K, V, 1.0)
    assert abs(l - math.log(n)) < 1e-12 * max(1, math.log(n))
    assert _rel(o, V.mean(axis=0)) < 1e-12


def test_equal_keys_closed_form():
    """All keys equal: LSE = s + ln n, O = mean of the values."""
    rng = np.random.default_rng(9)
    q = rng.normal(size=8)
    k = rng.normal(size=8)
    K = np.tile(k, (33, 1))
    V = rng.normal(size=(33, 8))
    o, l = attention.attention_state(q, K, V, 0.7)
    assert abs(l - (0.7 * float(q @ k) + math.log(33))) < 1e-12
    assert _rel(o, V.mean(axis=0)) < 1e-12


# --- Π6: a dominant key shows which row was gathered ------------------------------------------

def test_dominant_key():
    rng = np.random.default_rng(11)
    K = rng.normal(size=(50, 8)) * 0.01
    V = rng.normal(size=(50, 8))
    q = np.zeros(8)
    q[0] = 1.0
    K[23, 0] = 100.0
    o, l = attention.attention_state(q, K, V, 1.0)
    assert np.max(np.abs(o - V[23])) < 1e-12 * 10
    assert abs(l - 100.0) < 1e-12 * 100


# --- Π7: textbook routine ----------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(3))
def test_identity_block_table_equals_torch_sdpa(seed):
    """Pages in order (identity block table), one query per request: the
    paged decode equals torch's scaled_dot_product_attention on contiguous
    K/V (CPU, float64), and LSE equals torch.logsumexp of the scaled scores."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, D, P, npg = 3, 4, 2, 16, 8, 5
    L = [40, 17, 1]
    k_pool = rng.normal(size=(B * npg, P, Hkv, D))
    v_pool = rng.normal(size=(B * npg, P, Hkv, D))
    q = rng.normal(size=(B, Hq, D))
    bt = np.arange(B * npg).reshape(B, npg)
    scale = 1 / math.sqrt(D)
    O, LSE = attention.batch_decode(q, k_pool, v_pool, bt, L, P, scale)
    for b in range(B):
        K = k_pool[bt[b]].reshape(npg * P, Hkv, D)[: L[b]]
        V = v_pool[bt[b]].reshape(npg * P, Hkv, D)[: L[b]]
        Kt = torch.from_numpy(np.repeat(K, Hq // Hkv, axis=1)).permute(1, 0, 2)   # [Hq, n, D]
        Vt = torch.from_numpy(np.repeat(V, Hq // Hkv, axis=1)).permute(1, 0, 2)
        qt = torch.from_numpy(q[b])[:, None, :]                                     # [Hq, 1, D]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)[:, 0, :]
        assert _rel(O[b], ref.numpy()) < 1e-12
        lse_ref = torch.logsumexp(scale * (qt @ Kt.transpose(1, 2))[:, 0, :], dim=-1)
        assert np.max(np.abs(LSE[b] - lse_ref.numpy())) < 1e-12


# --- Π8: brute force at 50 digits --------------------------------------------------------------

@pytest.mark.parametrize("seed", range(4))
def test_mpmath_brute_force(seed):
    mp = pytest.importorskip("mpmath")
    mp.mp.dps = 50
    rng = np.random.default_rng(seed)
    n, d = int(rng.integers(1, 9)), int(rng.integers(1, 5))
    q = rng.normal(size=d) * 3
    K = rng.normal(size=(n, d)) * 3
    V = rng.normal(size=(n, d))
    scale = 0.9
    o, l = attention.attention_state(q, K, V, scale)
    s = [mp.mpf(scale) * mp.fsum(mp.mpf(q[j]) * mp.mpf(K[i, j]) for j in range(d)) for i in range(n)]
    tot = mp.fsum(mp.e ** si for si in s)
    lse = mp.log(tot)
    assert abs(l - float(lse)) < 1e-14 * max(1.0, abs(float(lse)))
    for j in range(d):
        oj = mp.fsum(mp.e ** si * mp.mpf(V[i, j]) for i, si in enumerate(s)) / tot
        assert abs(o[j] - float(oj)) < 1e-14 * max(1.0, abs(float(oj)))


# --- Π9: the worked examples of the "Paged attention" page -------------------------------------

def test_varlen_cu_seq_lens_example():
    g = _golden("hf_varlen_example.json")
    cu_q = indexing.cu_seq_lens(g["query_lens"])
    cu_k = indexing.cu_seq_lens(g["key_lens"])
    assert cu_q == g["cu_seq_lens_q"]
    assert cu_k == g["cu_seq_lens_k"]
    assert indexing.max_length(g["query_lens"]) == g["max_length_q"]
    assert indexing.max_length(g["key_lens"]) == g["max_length_k"]
    assert cu_q[-1] == g["q_total"] and cu_k[-1] == g["k_total"]
    assert indexing.request_index(cu_q) == g["q_request_index"]
    assert indexing.request_index(cu_k) == g["k_request_index"]


def test_block_table_example_reads():
    g = _golden("hf_paged_decode_example.json")
    P = g["page_size"]
    for b, row in enumerate(g["block_table"]):
        pages, slots = indexing.token_pages(row, 0, g["cache_seqlens"][b], P)
        assert sorted(set(pages.tolist()), key=pages.tolist().index) == g["read_pages"][b]
        for page, (lo, hi) in g["read_slots"][b].items():
            got = slots[pages == int(page)]
            assert got.tolist() == list(range(lo, hi + 1))
        # every allocated block holding a cached token is read, pre-allocated ones are not
        assert set(g["read_pages"][b]) <= set(g["allocated_blocks"][b])
    used = indexing.referenced_pages(g["block_table"], g["cache_seqlens"], P)
    assert sorted(set(range(8)) - used) == g["unreferenced_pages"]


def test_block_table_example_next_token():
    g = _golden("hf_paged_decode_example.json")
    for b, row in enumerate(g["block_table"]):
        j, page, slot = indexing.next_token_slot(row, g["cache_seqlens"][b], g["page_size"])
        exp = g["next_token"][b]
        assert (j, page, slot) == (exp["block"], exp["page"], exp["slot"])
        assert (page >= 0) == exp["fits_in_allocated"]


def test_append_writes_the_example_next_token_slots():
    """In-place append on the worked example: each sequence's new row lands at the printed
    next-token (page, slot), nothing else changes, lengths grow by one; afterwards the token
    is read (q = 0 and V = row id: O is the mean row id of the first length+1 tokens)."""
    g = _golden("hf_paged_decode_example.json")
    P = g["page_size"]
    k_pool = np.random.default_rng(2).normal(size=(8, P, 1, 4))
    v_pool = np.arange(8 * P, dtype=np.float64).reshape(8, P, 1, 1).repeat(4, axis=3)
    k_new = np.full((3, 1, 4), 7.0)
    v_new = np.full((3, 1, 4), -1000.0) - np.arange(3).reshape(3, 1, 1)
    tg = indexing.append_targets(g["block_table"], g["cache_seqlens"], P)
    assert tg == [(e["page"], e["slot"]) for e in g["next_token"]]
    k2, v2, lens = indexing.append_kv(k_pool, v_pool, k_new, v_new, g["block_table"], g["cache_seqlens"], P)
    assert lens == [n + 1 for n in g["cache_seqlens"]]
    changed = np.argwhere(np.any(v2 != v_pool, axis=(2, 3)))
    assert sorted(map(tuple, changed.tolist())) == sorted((e["page"], e["slot"]) for e in g["next_token"])
    assert np.array_equal(np.delete(k2.reshape(8 * P, -1), [e["page"] * P + e["slot"] for e in g["next_token"]], 0),
                          np.delete(k_pool.reshape(8 * P, -1), [e["page"] * P + e["slot"] for e in g["next_token"]], 0))
    q = np.zeros((3, 1, 4))
    O, L = attention.batch_decode(q, k2, v2, g["block_table"], lens, P, 1.0)
    for b in range(3):
        pages, slots = indexing.token_pages(g["block_table"][b], 0, lens[b], P)
        ids = (pages * P + slots).astype(np.float64)
        ids[-1] = -1000.0 - b            # the appended row's value
        assert abs(L[b, 0] - math.log(lens[b])) < 1e-12
        assert np.allclose(O[b, 0], ids.mean(), rtol=0, atol=1e-9)


def test_append_to_unallocated_block_writes_nothing():
    P = 4
    bt = [[3, -1], [1, 2]]
    k = np.zeros((4, P, 1, 2))
    k2, v2, lens = indexing.append_kv(k, k, np.ones((2, 1, 2)), np.ones((2, 1, 2)), bt, [4, 8], P)
    # request 0's next token needs block 1 (-1); request 1's needs block 2 (outside its row)
    assert lens == [4, 8] and not k2.any()
    assert indexing.append_targets(bt, [4, 8], P) == [None, None]


def test_unallocated_block_inside_length_raises():
    g = _golden("hf_paged_decode_example.json")
    with pytest.raises(ValueError):
        indexing.token_pages(g["block_table"][0], 0, 40, g["page_size"])
    with pytest.raises(IndexError):
        indexing.token_pages(g["block_table"][2], 0, 129, g["page_size"])


def test_block_table_example_token_id_values():
    """q = 0 and V[page, slot] = its physical row id make O the mean row id of
    exactly the tokens each sequence reads, and LSE = ln(cache_seqlens)."""
    g = _golden("hf_paged_decode_example.json")
    P = g["page_size"]
    k_pool = np.random.default_rng(1).normal(size=(8, P, 1, 4))
    v_pool = np.zeros((8, P, 1, 4))
    v_pool[:, :, 0, 0] = (np.arange(8)[:, None] * P + np.arange(P)[None, :])
    v_pool[..., 1] = 1.0
    O, LSE = attention.batch_decode(np.zeros((3, 1, 4)), k_pool, v_pool, g["block_table"],
                                    g["cache_seqlens"], P, 1.0)
    for b in range(3):
        rows = []
        for page, (lo, hi) in g["read_slots"][b].items():
            rows += [int(page) * P + s for s in range(lo, hi + 1)]
        assert abs(O[b, 0, 0] - np.mean(rows)) < 1e-9
        assert abs(O[b, 0, 1] - 1.0) < 1e-14
        assert abs(LSE[b, 0] - math.log(g["cache_seqlens"][b])) < 1e-13


def test_kv_start_restricts_token_set():
    """Tokens [kv_start, len) only: two chunks of a sequence merge back to the
    whole (the split used for the two-chunk check of the tiny example)."""
    g = _golden("hf_paged_decode_example.json")
    P = g["page_size"]
    rng = np.random.default_rng(5)
    k_pool = rng.normal(size=(8, P, 2, 8))
    v_pool = rng.normal(size=(8, P, 2, 8))
    q = rng.normal(size=(3, 2, 8))
    lens = g["cache_seqlens"]
    cuts = [7, 31, 33]
    full = attention.batch_decode(q, k_pool, v_pool, g["block_table"], lens, P, 0.3)
    a = attention.batch_decode(q, k_pool, v_pool, g["block_table"], cuts, P, 0.3)
    bb = attention.batch_decode(q, k_pool, v_pool, g["block_table"], lens, P, 0.3, kv_start=cuts)
    o, l = merge.merge_pair(a[0], a[1], bb[0], bb[1])
    assert _rel(o, full[0]) < 1e-12 and np.max(np.abs(l - full[1])) < 1e-12
    o, l = merge.merge_pair(bb[0], bb[1], a[0], a[1])
    assert _rel(o, full[0]) < 1e-12


# --- the cascade's union ---------------------------------------------------------------------

def _tiny_cascade(seed=0):
    rng = np.random.default_rng(seed)
    P, B, H, D = 4, 6, 2, 8
    num_pages = 40
    perm = rng.permutation(num_pages)
    glob = perm[:5].tolist()                  # 18 tokens (last page partial)
    grp = [perm[5:8].tolist(), perm[8:10].tolist()]   # 11 and 5 tokens
    suf = perm[10:].reshape(B, 5)
    lv0 = {"qo_indptr": [0, 6], "kv_page_indptr": [0, 5], "kv_page_indices": glob, "kv_lens": [18]}
    lv1 = {"qo_indptr": [0, 4, 6], "kv_page_indptr": [0, 3, 5],
           "kv_page_indices": grp[0] + grp[1], "kv_lens": [11, 5]}
    lens = [3, 20, 0, 7, 9, 1]
    k_pool = rng.normal(size=(num_pages, P, H, D))
    v_pool = rng.normal(size=(num_pages, P, H, D))
    q = rng.normal(size=(B, H, D))
    return q, k_pool, v_pool, P, [lv0, lv1], suf, lens


def test_cascade_equals_decode_over_concatenated_table():
    """With page-aligned levels the cascade's union is the same token set as
    a plain block table listing level pages then suffix pages."""
    rng = np.random.default_rng(2)
    P, B, H, D = 4, 3, 2, 8
    k_pool = rng.normal(size=(30, P, H, D))
    v_pool = rng.normal(size=(30, P, H, D))
    q = rng.normal(size=(B, H, D))
    lv = {"qo_indptr": [0, 3], "kv_page_indptr": [0, 2], "kv_page_indices": [7, 3], "kv_lens": [8]}
    suf = np.array([[1, 2, -1], [4, 5, 6], [9, 10, 11]])
    lens = [5, 12, 9]
    O, L = attention.cascade_decode(q, k_pool, v_pool, P, 0.4, [lv], suf, lens)
    bt = np.concatenate([np.tile([7, 3], (3, 1)), suf], axis=1)
    O2, L2 = attention.batch_decode(q, k_pool, v_pool, bt, [8 + n for n in lens], P, 0.4)
    assert _rel(O, O2) < 1e-12 and np.max(np.abs(L - L2)) < 1e-12


def test_cascade_uniform_scores_count_every_level():
    """q = 0: LSE = ln(prefix + group prefix + suffix tokens) per request."""
    q, k_pool, v_pool, P, levels, suf, lens = _tiny_cascade()
    O, L = attention.cascade_decode(np.zeros_like(q), k_pool, v_pool, P, 1.0, levels, suf, lens)
    group_len = [11, 11, 11, 11, 5, 5]
    for b in range(6):
        assert abs(L[b, 0] - math.log(18 + group_len[b] + lens[b])) < 1e-12


def test_cascade_equals_merge_of_level_states():
    """The three-step cascade (level states, suffix state, merge) reaches the
    one-softmax result ("Cascade Inference" blog, algorithm section)."""
    q, k_pool, v_pool, P, levels, suf, lens = _tiny_cascade(1)
    O, L = attention.cascade_decode(q, k_pool, v_pool, P, 0.5, levels, suf, lens)
    s0 = attention.level_prefix_states(q, k_pool, v_pool, P, 0.5, levels[0], 6)
    s1 = attention.level_prefix_states(q, k_pool, v_pool, P, 0.5, levels[1], 6)
    s2 = attention.batch_decode(q, k_pool, v_pool, suf, lens, P, 0.5)
    om, lm = merge.merge_many([s0[0], s1[0], s2[0]], [s0[1], s1[1], s2[1]])
    assert _rel(om, O) < 1e-12 and np.max(np.abs(lm - L)) < 1e-12


def test_gqa_head_map_is_contiguous():
    """Query head h reads kv head h // g (reading R3): with g = 2, heads 0 and 1
    see kv head 0, heads 2 and 3 see kv head 1."""
    rng = np.random.default_rng(4)
    P = 4
    k_pool = rng.normal(size=(2, P, 2, 4))
    v_pool = np.zeros((2, P, 2, 4))
    v_pool[:, :, 0, 0] = 1.0
    v_pool[:, :, 1, 0] = 2.0
    O, _ = attention.batch_decode(rng.normal(size=(1, 4, 4)), k_pool, v_pool, [[0, 1]], [7], P, 1.0)
    assert np.allclose(O[0, :, 0], [1, 1, 2, 2], atol=1e-14)


def test_ragged_append_of_one_token_each_equals_the_one_token_append():
    g = _golden("hf_paged_decode_example.json")
    P = g["page_size"]
    rng = np.random.default_rng(5)
    k_pool = rng.normal(size=(8, P, 1, 4))
    v_pool = rng.normal(size=(8, P, 1, 4))
    k_new = rng.normal(size=(3, 1, 4))
    v_new = rng.normal(size=(3, 1, 4))
    a = indexing.append_kv(k_pool, v_pool, k_new, v_new, g["block_table"], g["cache_seqlens"], P)
    b = indexing.append_kv_ragged(k_pool, v_pool, k_new, v_new, [0, 1, 2, 3], g["block_table"],
                                  g["cache_seqlens"], P)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


def test_ragged_append_on_the_worked_example():
    """Sequence 0 (30 tokens in page 2, block 1 unallocated) appends 2 tokens: slots 30 and 31
    of page 2.  Sequence 1 (32 tokens, pre-allocated block 1 = page 1) appends 3: page 1 slots
    0..2.  Sequence 2 (70 tokens over pages 3, 5, 6) appends 1: page 6 slot 6.  A third token
    for sequence 0 would need block 1 (-1): then sequence 0 writes nothing."""
    g = _golden("hf_paged_decode_example.json")
    P = g["page_size"]
    k_pool = np.zeros((8, P, 1, 2))
    ids = np.arange(1, 7, dtype=np.float64)
    k_new = np.stack([np.full((1, 2), x) for x in ids])
    k2, _, lens = indexing.append_kv_ragged(k_pool, k_pool, k_new, k_new, [0, 2, 5, 6], g["block_table"],
                                            g["cache_seqlens"], P)
    assert lens == [32, 35, 71]
    assert [tuple(x) for x in np.argwhere(k2[..., 0, 0] != 0).tolist()] == \
        [(1, 0), (1, 1), (1, 2), (2, 30), (2, 31), (6, 6)]
    assert [k2[2, 30, 0, 0], k2[2, 31, 0, 0], k2[1, 0, 0, 0], k2[1, 2, 0, 0], k2[6, 6, 0, 0]] == [1, 2, 3, 5, 6]
    k3, _, lens3 = indexing.append_kv_ragged(k_pool, k_pool, np.ones((4, 1, 2)), np.ones((4, 1, 2)),
                                             [0, 3, 3, 4], g["block_table"], g["cache_seqlens"], P)
    assert lens3 == [30, 32, 71] and not k3[2].any() and k3[6, 6].all()


def test_ragged_append_then_attention_sees_every_new_token():
    """Brute force: after the append, walking each request's first new-length tokens through
    the block table gives the old rows followed by exactly the new rows, in order."""
    rng = np.random.default_rng(9)
    P, B = 4, 5
    bt = np.full((B, 6), -1, dtype=np.int32)
    perm = rng.permutation(30)
    lens = [3, 0, 8, 5, 1]
    new = [6, 2, 0, 9, 3]
    for b in range(B):
        n = -(-(lens[b] + new[b]) // P)
        bt[b, :n] = perm[6 * b: 6 * b + n]
    k_pool = rng.normal(size=(30, P, 2, 2))
    indptr = np.concatenate([[0], np.cumsum(new)])
    k_new = rng.normal(size=(int(indptr[-1]), 2, 2))
    k2, _, lens2 = indexing.append_kv_ragged(k_pool, k_pool, k_new, k_new, indptr, bt, lens, P)
    assert lens2 == [lens[b] + new[b] for b in range(B)]
    for b in range(B):
        rows = [k2[bt[b, t // P], t % P] for t in range(lens2[b])]
        old = [k_pool[bt[b, t // P], t % P] for t in range(lens[b])]
        assert all(np.array_equal(x, y) for x, y in zip(rows[:lens[b]], old))
        assert all(np.array_equal(rows[lens[b] + i], k_new[indptr[b] + i]) for i in range(new[b]))
