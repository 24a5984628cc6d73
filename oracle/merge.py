"""The merge operator on attention states (oracle; test infrastructure only).

Follows "Attention States and Recursive Attention" (FlashInfer tutorial) and
the "Recursive attention" section of the "Cascade Inference" blog:

* binary merge: the merged value is the exp(s)-weighted average of the two
  values, the merged score is the log of exp(s_I) + exp(s_J);
* n-ary merge: the merged value is the softmax-over-scores weighted sum of
  the values, the merged score is the log-sum-exp of the scores;
* both pages note that the maximum score is subtracted in practice for
  numerical stability; that is done here.

The FlashInfer paper summary (A2, attention composition) states the same
binary operator on (O, LSE).  The identity element is (0, -inf): an empty
index set (reading R8).  Used only to pin the algebra and to check the GPU
merge kernel -- the oracle's attention results never go through it.
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf


def merge_pair(o_a, lse_a, o_b, lse_b):
    """Binary merge of two states of the same query rows.

    o_*: [..., D]; lse_*: [...].  Returns (o, lse) in float64.
    """
    o_a = np.asarray(o_a, np.float64)
    o_b = np.asarray(o_b, np.float64)
    la = np.asarray(lse_a, np.float64)
    lb = np.asarray(lse_b, np.float64)
    m = np.maximum(la, lb)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    ea = np.exp(la - m_safe)          # exp(s_I) / exp(m)
    eb = np.exp(lb - m_safe)          # exp(s_J) / exp(m)
    den = ea + eb
    den_safe = np.where(empty, 1.0, den)
    o = (o_a * ea[..., None] + o_b * eb[..., None]) / den_safe[..., None]
    o = np.where(empty[..., None], 0.0, o)
    lse = np.where(empty, NEG_INF, m_safe + np.log(den_safe))
    return o, lse


def merge_many(os, lses):
    """n-ary merge of n states of the same query rows.

    os: [n, ..., D]; lses: [n, ...].  Returns (o [..., D], lse [...]).
    With n = 0 or every score -inf the result is the identity (0, -inf).
    """
    os = np.asarray(os, np.float64)
    lses = np.asarray(lses, np.float64)
    if os.shape[0] == 0:
        return np.zeros(os.shape[1:]), np.full(lses.shape[1:], NEG_INF)
    m = lses.max(axis=0)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lses - m_safe)                       # exp(s(I_i) - max)
    wsum = w.sum(axis=0)
    wsum_safe = np.where(empty, 1.0, wsum)
    o = (w[..., None] * os).sum(axis=0) / wsum_safe[..., None]   # softmax(s(I_i)) weights
    o = np.where(empty[..., None], 0.0, o)
    lse = np.where(empty, NEG_INF, m_safe + np.log(wsum_safe))
    return o, lse
