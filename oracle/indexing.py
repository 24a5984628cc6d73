"""Integer indexing of the paged KV cache (oracle; test infrastructure only).

Follows the "Paged attention" page of the Hugging Face Transformers docs:

* Decode path, cache behaviour + indexing example: each batch row owns a row
  of ``block_table`` of shape (batch, max_blocks_per_seq) listing the
  physical cache block of each of its logical blocks; -1 marks a block that
  is not allocated; ``cache_seqlens[b]`` is the number of cached tokens.
  Token t of a sequence therefore lives in block ``block_table[b][t // P]``
  at slot ``t % P`` (P = cache block size).  Only the blocks that hold one of
  the first ``cache_seqlens[b]`` tokens are read; a block pre-allocated for
  the next token is not (reading adopted for the example's sequence 1).
* Varlen path, indexing example: cumulative lengths ``cu_seq_lens`` and the
  per-token request index.

The same arrays are the block-sparse (BSR) view of the KV cache in the
FlashInfer paper summary (section A3, "unified block-sparse format"): row
pointer = cumulative page counts, column indices = physical pages, block
column size B_c = page size.  Cascade levels reuse exactly that form.
"""

from __future__ import annotations

import numpy as np


def cu_seq_lens(lengths):
    """Cumulative sequence lengths [0, l0, l0+l1, ...] (varlen indexing)."""
    out = [0]
    for n in lengths:
        n = int(n)
        if n < 0:
            raise ValueError("negative length")
        out.append(out[-1] + n)
    return out


def max_length(lengths):
    """Largest per-sequence length (max_length_q / max_length_k)."""
    return max((int(n) for n in lengths), default=0)


def request_index(cu):
    """Owner request of every packed token: token i belongs to request r when
    cu[r] <= i < cu[r+1].  Requests with zero tokens own nothing."""
    owner = []
    for r in range(len(cu) - 1):
        owner.extend([r] * (cu[r + 1] - cu[r]))
    return owner


def token_pages(page_list, kv_begin, kv_end, page_size):
    """Physical (page, slot) of every token t in [kv_begin, kv_end) of one
    sequence whose logical blocks are ``page_list``.

    Raises on a block index outside the table or an unallocated (negative)
    entry inside the range: a caller error, never silently read.
    Returns two int64 arrays (pages, slots) of length kv_end - kv_begin.
    """
    if page_size <= 0:
        raise ValueError("page_size must be positive")
    if kv_begin < 0 or kv_end < kv_begin:
        raise ValueError("bad token range")
    t = np.arange(kv_begin, kv_end, dtype=np.int64)
    blk = t // page_size
    if t.size and int(blk[-1]) >= len(page_list):
        raise IndexError("token beyond the sequence's block table row")
    pages = np.asarray(page_list, dtype=np.int64)[blk] if t.size else blk
    if np.any(pages < 0):
        raise ValueError("unallocated block (-1) inside the sequence")
    return pages, t % page_size


def next_token_slot(page_list, cached_len, page_size):
    """Where the next token of a sequence goes: (logical block, physical page
    or -1 if that block is not allocated, slot).  Used only to pin the
    worked example's narrative; the hot path does not append."""
    j = cached_len // page_size
    page = int(page_list[j]) if j < len(page_list) else -1
    return j, page, cached_len % page_size


def referenced_pages(block_table, cache_seqlens, page_size, kv_start=None):
    """Set of physical pages that the decode of every row reads."""
    used = set()
    for b, row in enumerate(block_table):
        start = 0 if kv_start is None else int(kv_start[b])
        pages, _ = token_pages(row, start, int(cache_seqlens[b]), page_size)
        used.update(int(p) for p in pages)
    return used


def append_targets(block_table, cache_seqlens, page_size):
    """Physical (page, slot) where each sequence's next token is written, or None when the
    logical block cache_seqlens[b] // P is outside the row or not allocated ("Paged attention"
    page, decode path: the cache is updated in place; the worked example's next-token
    bullets)."""
    out = []
    for b, row in enumerate(block_table):
        j, page, slot = next_token_slot(row, int(cache_seqlens[b]), page_size)
        out.append((page, slot) if page >= 0 else None)
    return out


def append_kv(k_pool, v_pool, k_new, v_new, block_table, cache_seqlens, page_size):
    """Copies of the pools ([pages, P, Hkv, D]) with request b's new rows k_new[b], v_new[b]
    ([B, Hkv, D]) written at its next-token slot, and the new lengths (cache_seqlens[b] + 1,
    or unchanged when the target block is not allocated: nothing is written then)."""
    k = np.array(k_pool, copy=True)
    v = np.array(v_pool, copy=True)
    lens = [int(x) for x in cache_seqlens]
    for b, tgt in enumerate(append_targets(block_table, cache_seqlens, page_size)):
        if tgt is None or tgt[0] >= k.shape[0]:
            continue
        k[tgt[0], tgt[1]] = k_new[b]
        v[tgt[0], tgt[1]] = v_new[b]
        lens[b] += 1
    return k, v, lens


def append_kv_ragged(k_pool, v_pool, k_new, v_new, new_indptr, block_table, cache_seqlens,
                     page_size):
    """Multi-token append (prefill / append path over the paged cache): request b's new rows
    k_new[new_indptr[b] + i], v_new[...] (i < n_b = new_indptr[b+1] - new_indptr[b]) go to
    token positions cache_seqlens[b] + i, i.e. block (cache_seqlens[b] + i) // P of its
    block-table row at slot (cache_seqlens[b] + i) % P -- the rule of the "Paged attention"
    page's next-token bullets applied to every new token in order.  Reading adopted for
    failures: a request all of whose target blocks are allocated (inside the row, not -1, a
    page of the pool) writes every row and its length becomes cache_seqlens[b] + n_b; otherwise
    it writes nothing and keeps its length (with n_b = 1 this is the one-token append above).
    Returns copies of the pools and the new lengths."""
    k = np.array(k_pool, copy=True)
    v = np.array(v_pool, copy=True)
    num_pages = k.shape[0]
    lens = [int(x) for x in cache_seqlens]
    for b, row in enumerate(block_table):
        lo, hi = int(new_indptr[b]), int(new_indptr[b + 1])
        targets = []
        for i in range(hi - lo):
            t = lens[b] + i
            j = t // page_size
            page = int(row[j]) if j < len(row) else -1
            if page < 0 or page >= num_pages:
                targets = None
                break
            targets.append((page, t % page_size))
        if targets is None:
            continue
        for i, (page, slot) in enumerate(targets):
            k[page, slot] = k_new[lo + i]
            v[page, slot] = v_new[lo + i]
        lens[b] += hi - lo
    return k, v, lens
