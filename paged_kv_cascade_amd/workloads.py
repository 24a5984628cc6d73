"""Seeded synthetic workloads (inputs only; no attention arithmetic here).

Both the HIP path and the fp64 oracle consume these tensors; this module
computes nothing either of them computes.  Every workload has the shape of
the pages' own evaluation: LLaMA2-7B attention (32 heads x 128 dims), page
size 16, shared prefixes of up to 32768 tokens, batch >= 128, short unique
suffixes (Cascade Inference blog, evaluation section), plus the paged-decode
worked example of the Hugging Face "Paged attention" page.

Recipe: integer structure (lengths, page permutations, cut points) comes from
a CPU ``torch.Generator`` seeded with ``seed``; the float data come from a
generator on the target device seeded with ``seed + 1``, drawn in the order
q, k, v as float32 N(0, 1) * ``value_scale`` and cast round-to-nearest-even
to the workload dtype.  KV rows that no request reads are filled with NaN
("poison") so a wrongly gathered row shows up as a non-finite output.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

LLAMA2_7B_HEADS = 32
LLAMA2_7B_HEAD_DIM = 128


@dataclass
class Workload:
    name: str
    batch: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    dtype: torch.dtype
    sm_scale: float
    q: torch.Tensor                    # [B, Hq, D]
    k_pool: torch.Tensor               # [num_pages, P, Hkv, D]
    v_pool: torch.Tensor               # [num_pages, P, Hkv, D]
    block_table: torch.Tensor          # int32 [B, max_blocks] (suffix table in a cascade)
    cache_seqlens: torch.Tensor        # int32 [B]
    kv_start: Optional[torch.Tensor] = None   # int32 [B] or None
    levels: list = field(default_factory=list)   # cascade levels (host lists + int32 tensors)
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def esize(self) -> int:
        return torch.tensor([], dtype=self.dtype).element_size()

    def kv_tokens_per_request(self):
        """Tokens each request attends over (levels + own KV), host ints."""
        out = []
        lens = self.cache_seqlens.tolist()
        starts = self.kv_start.tolist() if self.kv_start is not None else [0] * self.batch
        for b in range(self.batch):
            n = lens[b] - starts[b]
            for lv in self.levels:
                qi = lv["qo_indptr"]
                for g in range(len(qi) - 1):
                    if qi[g] <= b < qi[g + 1]:
                        n += lv["kv_lens"][g]
            out.append(n)
        return out

    def algorithmic_kv_bytes(self) -> int:
        """K + V bytes one step must read when every shared run is read once:
        2 * D * esize per token per kv head."""
        per_tok = 2 * self.head_dim * self.esize * self.num_kv_heads
        lens = self.cache_seqlens.tolist()
        starts = self.kv_start.tolist() if self.kv_start is not None else [0] * self.batch
        n = sum(lens[b] - starts[b] for b in range(self.batch))
        for lv in self.levels:
            n += sum(lv["kv_lens"])
        return n * per_tok


def _cpu_gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def _values(shape, dtype, device, gen, scale):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(dtype)


def _pools(num_pages, P, hkv, D, dtype, device, gen, scale):
    k = _values((num_pages, P, hkv, D), dtype, device, gen, scale)
    v = _values((num_pages, P, hkv, D), dtype, device, gen, scale)
    return k, v


def _device_gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed + 1)
    return g


def _poison_rows(pool, used_mask):
    """NaN every (page, slot) row whose used_mask entry is False."""
    pool[~used_mask.to(pool.device)] = float("nan")


def _level(qo_indptr, groups_pages, kv_lens):
    """Cascade level descriptor: requests per group, each group's page run
    (BSR column indices) and KV length in tokens."""
    indptr = [0]
    flat = []
    for pages in groups_pages:
        flat.extend(int(p) for p in pages)
        indptr.append(len(flat))
    return {
        "qo_indptr": [int(x) for x in qo_indptr],
        "kv_page_indptr": indptr,
        "kv_page_indices": flat,
        "kv_lens": [int(x) for x in kv_lens],
    }


def tiny_paged(seed=1001, device="cpu", dtype=torch.float32, poison=True):
    """Hugging Face "Paged attention" decode example: 3 sequences with
    cache_seqlens [30, 32, 70], block size 32, 4 blocks per row, over an
    8-page pool; 2 heads of 64 dims; q/k/v ~ N(0, 1).  Also draws one cut
    point per sequence (uniform in 1 .. len-1) for the two-chunk split."""
    P, B, H, D = 32, 3, 2, 64
    bt = torch.tensor([[2, -1, -1, -1], [0, 1, -1, -1], [3, 5, 6, -1]], dtype=torch.int32)
    lens = torch.tensor([30, 32, 70], dtype=torch.int32)
    cg = _cpu_gen(seed)
    cuts = [int(torch.randint(1, int(n), (1,), generator=cg)) for n in lens.tolist()]
    dg = _device_gen(device, seed)
    q = _values((B, H, D), dtype, device, dg, 1.0)
    k, v = _pools(8, P, H, D, dtype, device, dg, 1.0)
    if poison:
        used = torch.zeros(8, P, dtype=torch.bool)
        used[2, :30] = True
        used[0, :32] = True
        used[3, :] = True
        used[5, :] = True
        used[6, :6] = True
        _poison_rows(k, used)
        _poison_rows(v, used)
    return Workload("tiny_paged_decode_b3_h2_d64_fp32_p32", B, H, H, D, P, dtype,
                    1.0 / math.sqrt(D), q, k, v, bt.to(device), lens.to(device),
                    None, [], seed, {"cuts": cuts})


def paged_decode(batch=64, heads=LLAMA2_7B_HEADS, kv_heads=None, head_dim=LLAMA2_7B_HEAD_DIM,
                 kv_len=4096, page_size=16, dtype=torch.float16, seed=1002, device="cpu",
                 value_scale=0.5):
    """Non-cascade batch decode: every request has kv_len tokens; the pool's
    pages are handed out by a seeded random permutation."""
    hkv = heads if kv_heads is None else kv_heads
    npg = -(-kv_len // page_size)
    num_pages = batch * npg
    cg = _cpu_gen(seed)
    perm = torch.randperm(num_pages, generator=cg).to(torch.int32)
    bt = perm.view(batch, npg).clone()
    lens = torch.full((batch,), kv_len, dtype=torch.int32)
    dg = _device_gen(device, seed)
    q = _values((batch, heads, head_dim), dtype, device, dg, value_scale)
    k, v = _pools(num_pages, page_size, hkv, head_dim, dtype, device, dg, value_scale)
    if kv_len % page_size:
        used = torch.ones(num_pages, page_size, dtype=torch.bool)
        used[bt[:, -1].long(), kv_len % page_size:] = False
        _poison_rows(k, used)
        _poison_rows(v, used)
    name = f"paged_decode_b{batch}_hq{heads}_hkv{hkv}_d{head_dim}_len{kv_len}_p{page_size}"
    return Workload(name, batch, heads, hkv, head_dim, page_size, dtype, 1.0 / math.sqrt(head_dim),
                    q, k, v, bt.to(device), lens.to(device), None, [], seed)


def loguniform_lengths(batch, lo, hi, gen):
    """l_b = floor(exp(U[ln lo, ln hi))) clamped to [lo, hi]."""
    u = torch.rand(batch, generator=gen, dtype=torch.float64)
    x = torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
    return [min(hi, max(lo, int(math.floor(float(t))))) for t in x]


def gqa_split(batch=256, heads=32, kv_heads=8, head_dim=128, lo=128, hi=32768,
              page_size=16, dtype=torch.bfloat16, seed=1004, device="cpu", value_scale=0.5):
    """GQA decode with log-uniform KV lengths (the variable-length mix the
    load-balancing plan is for).  Pool = exactly the pages the requests use,
    handed out by a seeded permutation; tail slots of last pages are NaN."""
    cg = _cpu_gen(seed)
    lens = loguniform_lengths(batch, lo, hi, cg)
    npgs = [-(-n // page_size) for n in lens]
    num_pages = sum(npgs)
    perm = torch.randperm(num_pages, generator=cg).to(torch.int32)
    maxb = max(npgs)
    bt = torch.full((batch, maxb), -1, dtype=torch.int32)
    used = torch.ones(num_pages, page_size, dtype=torch.bool)
    off = 0
    for b, n in enumerate(npgs):
        bt[b, :n] = perm[off:off + n]
        off += n
        if lens[b] % page_size:
            used[int(bt[b, n - 1]), lens[b] % page_size:] = False
    dg = _device_gen(device, seed)
    q = _values((batch, heads, head_dim), dtype, device, dg, value_scale)
    k, v = _pools(num_pages, page_size, kv_heads, head_dim, dtype, device, dg, value_scale)
    _poison_rows(k, used)
    _poison_rows(v, used)
    name = f"gqa_split_b{batch}_hq{heads}_hkv{kv_heads}_d{head_dim}_loguniform{lo}-{hi}_p{page_size}"
    return Workload(name, batch, heads, kv_heads, head_dim, page_size, dtype,
                    1.0 / math.sqrt(head_dim), q, k, v, bt.to(device),
                    torch.tensor(lens, dtype=torch.int32).to(device), None, [], seed)


def cascade_two_level(batch=128, heads=32, head_dim=128, prefix_len=32768, suffix_len=256,
                      page_size=16, dtype=torch.float16, seed=1003, device="cpu",
                      value_scale=0.5):
    """Shared-prefix batch decode: one prefix of prefix_len tokens stored as
    the contiguous page run 0 .. prefix_pages-1, plus suffix_len unique tokens
    per request in pages drawn from a permutation of the remaining pages."""
    ppg = -(-prefix_len // page_size)
    spg = -(-suffix_len // page_size)
    num_pages = ppg + batch * spg
    cg = _cpu_gen(seed)
    perm = (torch.randperm(batch * spg, generator=cg) + ppg).to(torch.int32)
    bt = perm.view(batch, spg).clone()
    lens = torch.full((batch,), suffix_len, dtype=torch.int32)
    used = torch.ones(num_pages, page_size, dtype=torch.bool)
    if prefix_len % page_size:
        used[ppg - 1, prefix_len % page_size:] = False
    if suffix_len % page_size:
        used[bt[:, -1].long(), suffix_len % page_size:] = False
    level0 = _level([0, batch], [list(range(ppg))], [prefix_len])
    dg = _device_gen(device, seed)
    q = _values((batch, heads, head_dim), dtype, device, dg, value_scale)
    k, v = _pools(num_pages, page_size, heads, head_dim, dtype, device, dg, value_scale)
    _poison_rows(k, used)
    _poison_rows(v, used)
    name = f"cascade_prefix{prefix_len}_suffix{suffix_len}_b{batch}_h{heads}_d{head_dim}_p{page_size}"
    return Workload(name, batch, heads, heads, head_dim, page_size, dtype, 1.0 / math.sqrt(head_dim),
                    q, k, v, bt.to(device), lens.to(device), None, [level0], seed)


def cascade_multi_level(batch=128, heads=32, head_dim=128, prefix_len=16384, groups=4,
                        group_prefix_len=4096, suffix_len=512, page_size=16,
                        dtype=torch.float16, seed=1005, device="cpu", value_scale=0.5):
    """Three-level cascade: a global prefix shared by all requests, one
    prefix per group of batch/groups consecutive requests, and a unique
    suffix per request; every page of the pool is placed by one seeded
    permutation."""
    assert batch % groups == 0
    P = page_size
    gpg = -(-prefix_len // P)
    lpg = -(-group_prefix_len // P)
    spg = -(-suffix_len // P)
    num_pages = gpg + groups * lpg + batch * spg
    cg = _cpu_gen(seed)
    perm = torch.randperm(num_pages, generator=cg).to(torch.int32).tolist()
    glob = perm[:gpg]
    grp = [perm[gpg + i * lpg: gpg + (i + 1) * lpg] for i in range(groups)]
    suf = perm[gpg + groups * lpg:]
    bt = torch.tensor(suf, dtype=torch.int32).view(batch, spg).clone()
    per = batch // groups
    level0 = _level([0, batch], [glob], [prefix_len])
    level1 = _level([i * per for i in range(groups + 1)], grp, [group_prefix_len] * groups)
    used = torch.ones(num_pages, P, dtype=torch.bool)
    if prefix_len % P:
        used[glob[-1], prefix_len % P:] = False
    if group_prefix_len % P:
        for pages in grp:
            used[pages[-1], group_prefix_len % P:] = False
    if suffix_len % P:
        used[bt[:, -1].long(), suffix_len % P:] = False
    lens = torch.full((batch,), suffix_len, dtype=torch.int32)
    dg = _device_gen(device, seed)
    q = _values((batch, heads, head_dim), dtype, device, dg, value_scale)
    k, v = _pools(num_pages, P, heads, head_dim, dtype, device, dg, value_scale)
    _poison_rows(k, used)
    _poison_rows(v, used)
    name = (f"cascade3_prefix{prefix_len}_groups{groups}x{group_prefix_len}_suffix{suffix_len}"
            f"_b{batch}_h{heads}_d{head_dim}_p{P}")
    return Workload(name, batch, heads, heads, head_dim, P, dtype, 1.0 / math.sqrt(head_dim),
                    q, k, v, bt.to(device), lens.to(device), None, [level0, level1], seed)


def by_number(n, device="cpu", **kw):
    """The five standard workloads by number (1 tiny paged decode, 2 paged
    decode, 3 two-level cascade, 4 GQA split decode, 5 multi-level cascade)."""
    return {1: tiny_paged, 2: paged_decode, 3: cascade_two_level, 4: gqa_split,
            5: cascade_multi_level}[n](device=device, **kw)


def fp8_e4m3_pool(pool, scale=1.0):
    """FP8 E4M3 code pool of a float pool: torch's round-to-nearest-even cast of pool / scale
    to float8_e4m3fn (poisoned NaN rows stay NaN codes).  Inputs only: the pool scale is the
    number the decode is then given."""
    x = pool.float()
    if scale != 1.0:
        x = x / scale
    return x.to(torch.float8_e4m3fn)
