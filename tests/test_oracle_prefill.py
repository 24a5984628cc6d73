"""Pins of the oracle's ragged multi-token query attention (prefill / append over a paged
KV cache), CPU only.

Checked against: the decode oracle when every request has one query (the causal limit of
the last query is the whole sequence), a dense masked softmax written independently (a
lower-triangular mask built with numpy over contiguous K/V), torch's CPU attention routine
with its causal flag where the two alignments coincide (as many queries as keys), and the
visible-token counts of the "Paged attention" page's varlen example (query lengths
[10, 3, 1], key lengths [0, 1, 7]) through uniform scores, where LSE = ln(count).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(seed, lq, lkv, hkv=2, g=2, D=8, P=4):
    rng = np.random.default_rng(seed)
    B = len(lq)
    qo = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
    npg = [-(-n // P) for n in lkv]
    num_pages = sum(npg) + 3
    perm = rng.permutation(num_pages)
    bt = np.full((B, max(npg + [1]) + 1), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(npg):
        bt[b, :n] = perm[off:off + n]
        off += n
    q = rng.normal(size=(int(qo[-1]), hkv * g, D))
    k = rng.normal(size=(num_pages, P, hkv, D))
    v = rng.normal(size=(num_pages, P, hkv, D))
    return q, qo, k, v, bt, np.array(lkv), P


@pytest.mark.parametrize("causal", [False, True])
def test_one_query_per_request_equals_decode(causal):
    q, qo, k, v, bt, lkv, P = _case(1, [1, 1, 1, 1], [0, 1, 7, 13])
    O, L = attention.batch_prefill(q, qo, k, v, bt, lkv, P, 0.4, causal)
    Od, Ld = attention.batch_decode(q, k, v, bt, lkv, P, 0.4)
    assert np.array_equal(np.isneginf(L), np.isneginf(Ld))
    assert np.array_equal(O, Od) and np.array_equal(L[~np.isneginf(L)], Ld[~np.isneginf(Ld)])


@pytest.mark.parametrize("causal", [False, True])
def test_matches_dense_masked_softmax(causal):
    """Independent formulation: contiguous K/V per request (rows gathered by page * P + slot
    arithmetic, not by the oracle's gather), scores for all (query, key) pairs, a lower-
    triangular mask aligned to the bottom-right corner, softmax over the unmasked entries."""
    lq, lkv = [5, 3, 1, 4, 6], [9, 3, 0, 2, 6]
    q, qo, k, v, bt, lkv_a, P = _case(2, lq, lkv)
    Hq, D = q.shape[1], q.shape[2]
    hkv = k.shape[2]
    g = Hq // hkv
    O, L = attention.batch_prefill(q, qo, k, v, bt, lkv_a, P, 0.3, causal)
    for b in range(len(lq)):
        n = lkv[b]
        rows_k = np.array([k[bt[b, t // P], t % P] for t in range(n)]).reshape(n, hkv, D)
        rows_v = np.array([v[bt[b, t // P], t % P] for t in range(n)]).reshape(n, hkv, D)
        for h in range(Hq):
            Q = q[qo[b]:qo[b + 1], h]                                  # [lq, D]
            S = 0.3 * Q @ rows_k[:, h // g].T if n else np.zeros((lq[b], 0))
            mask = np.ones_like(S, dtype=bool)
            if causal:
                mask = np.tril(mask, k=n - lq[b])
            for i in range(lq[b]):
                r = qo[b] + i
                s = S[i][mask[i]]
                if s.size == 0:
                    assert np.isneginf(L[r, h]) and np.all(O[r, h] == 0)
                    continue
                m = s.max()
                lse = m + math.log(np.exp(s - m).sum())
                w = np.exp(S[i] - lse) * mask[i]
                assert abs(L[r, h] - lse) < 1e-12
                assert np.allclose(O[r, h], w @ rows_v[:, h // g], rtol=1e-11, atol=1e-13)


def test_square_causal_matches_torch_sdpa():
    """As many queries as keys: bottom-right and top-left causal alignment coincide, so
    torch's scaled_dot_product_attention with is_causal gives the same outputs."""
    lq = [7, 12]
    q, qo, k, v, bt, lkv, P = _case(3, lq, lq, hkv=1, g=3)
    O, L = attention.batch_prefill(q, qo, k, v, bt, lkv, P, 0.25, True)
    for b, n in enumerate(lq):
        kk = np.array([k[bt[b, t // P], t % P, 0] for t in range(n)])
        vv = np.array([v[bt[b, t // P], t % P, 0] for t in range(n)])
        Q = torch.tensor(q[qo[b]:qo[b + 1]].transpose(1, 0, 2))   # [Hq, n, D]
        K = torch.tensor(kk)[None].expand(Q.shape[0], -1, -1)
        V = torch.tensor(vv)[None].expand(Q.shape[0], -1, -1)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=0.25)
        assert np.allclose(O[qo[b]:qo[b + 1]], ref.numpy().transpose(1, 0, 2), rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_example_visible_counts(causal):
    """The varlen worked example's lengths with zero queries (uniform scores): LSE of each query
    row is ln(number of keys it sees), -inf when it sees none."""
    with open(os.path.join(GOLDEN, "hf_varlen_example.json")) as f:
        ex = json.load(f)
    lq, lkv = ex["query_lens"], ex["key_lens"]
    q, qo, k, v, bt, lkv_a, P = _case(4, lq, lkv)
    assert list(qo) == ex["cu_seq_lens_q"]
    q = np.zeros_like(q)
    O, L = attention.batch_prefill(q, qo, k, v, bt, lkv_a, P, 1.0, causal)
    if causal:
        counts = [0] * 10 + [0, 0, 1] + [7]
    else:
        counts = [0] * 10 + [1, 1, 1] + [7]
    assert [int(x) for x in ex["q_request_index"]] == [b for b in range(3) for _ in range(lq[b])]
    for r, c in enumerate(counts):
        for h in range(q.shape[1]):
            if c == 0:
                assert np.isneginf(L[r, h]) and np.all(O[r, h] == 0)
            else:
                assert abs(L[r, h] - math.log(c)) < 1e-14


def test_prefill_limit_cases():
    assert attention.prefill_limit(3, 10, 0, True) == 8
    assert attention.prefill_limit(3, 10, 2, True) == 10
    assert attention.prefill_limit(3, 1, 1, True) == 0
    assert attention.prefill_limit(3, 1, 2, True) == 1
    assert attention.prefill_limit(4, 0, 3, True) == 0
    assert attention.prefill_limit(3, 10, 0, False) == 10


def test_tree_mask_of_ones_is_the_causal_mask():
    """A tree mask that lets every new token see every new token refines nothing: within the
    causal limit the result is the causal prefill."""
    lq, lkv = [4, 6], [9, 6]
    q, qo, k, v, bt, lkv_a, P = _case(11, lq, lkv)
    masks = [np.ones((n, n), dtype=bool) for n in lq]
    O1, L1 = attention.batch_prefill(q, qo, k, v, bt, lkv_a, P, 0.3, True, tree_masks=masks)
    O2, L2 = attention.batch_prefill(q, qo, k, v, bt, lkv_a, P, 0.3, True)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_tree_mask_matches_dense_masked_softmax():
    """Independent formulation: contiguous K/V per request, a dense [lq, lkv] visibility matrix
    built with numpy (all old tokens, then the tree mask restricted to the lower triangle over
    the new tokens), softmax over the visible entries.  The masks are random ancestor sets of a
    random tree (each new token sees itself and its chain of parents)."""
    rng = np.random.default_rng(12)
    lq, lkv = [5, 7, 1], [12, 7, 3]
    q, qo, k, v, bt, lkv_a, P = _case(13, lq, lkv)
    masks = []
    for n in lq:
        parent = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
        m = np.zeros((n, n), dtype=bool)
        for i in range(n):
            j = i
            while j >= 0:
                m[i, j] = True
                j = parent[j]
        masks.append(m)
    O, L = attention.batch_prefill(q, qo, k, v, bt, lkv_a, P, 0.5, True, tree_masks=masks)
    Hq, D = q.shape[1], q.shape[2]
    hkv = k.shape[2]
    g = Hq // hkv
    for b in range(len(lq)):
        n = lkv[b]
        rows_k = np.array([k[bt[b, t // P], t % P] for t in range(n)])
        rows_v = np.array([v[bt[b, t // P], t % P] for t in range(n)])
        vis = np.ones((lq[b], n), dtype=bool)
        vis[:, n - lq[b]:] = np.tril(masks[b])
        for h in range(Hq):
            S = 0.5 * q[qo[b]:qo[b + 1], h] @ rows_k[:, h // g].T
            for i in range(lq[b]):
                s = S[i][vis[i]]
                m = s.max()
                lse = m + math.log(np.exp(s - m).sum())
                w = np.exp(S[i] - lse) * vis[i]
                assert abs(L[qo[b] + i, h] - lse) < 1e-12
                assert np.allclose(O[qo[b] + i, h], w @ rows_v[:, h // g], rtol=1e-11, atol=1e-13)


def test_tree_mask_identity_sees_prefix_and_itself():
    """Uniform scores (q = 0) with an identity tree mask: each new token sees the old tokens and
    itself, so LSE = ln(lkv - lq + 1) for every query."""
    lq, lkv = [3, 2], [10, 2]
    q, qo, k, v, bt, lkv_a, P = _case(14, lq, lkv)
    q = np.zeros_like(q)
    masks = [np.eye(n, dtype=bool) for n in lq]
    O, L = attention.batch_prefill(q, qo, k, v, bt, lkv_a, P, 1.0, True, tree_masks=masks)
    for b in range(2):
        for i in range(lq[b]):
            assert np.all(np.abs(L[qo[b] + i] - math.log(lkv[b] - lq[b] + 1)) < 1e-14)
