"""GPU parity of the in-place KV append (the step before decode): the new rows land exactly
where the oracle (pinned to the worked example's next-token slots) puts them, nothing else
in the pools changes, and decoding over the new lengths matches the oracle's decode of the
appended pools."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import indexing as oidx
from tests.gpu_helpers import PoolView, check_state, gpu, host, needs_gpu, say

pytestmark = [gpu, needs_gpu]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def api():
    from paged_kv_cascade_amd import api as _api
    return _api


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


def _append_and_check(api, k_pool, v_pool, k_new, v_new, bt, lens, P, in_place=False):
    k_ref, v_ref, lens_ref = oidx.append_kv(_bits(k_pool), _bits(v_pool), _bits(k_new), _bits(v_new),
                                            bt.cpu().numpy().tolist(), lens.cpu().numpy().tolist(), P)
    out = lens if in_place else None
    new = api.append_kv(k_new, v_new, k_pool, v_pool, bt, lens, new_seqlens=out)
    torch.cuda.synchronize()
    assert new.cpu().tolist() == lens_ref
    assert np.array_equal(_bits(k_pool), k_ref), "K pool differs from the oracle's append (bitwise)"
    assert np.array_equal(_bits(v_pool), v_ref), "V pool differs from the oracle's append (bitwise)"
    return new


def test_append_on_worked_example_then_decode(api):
    say("case: append on the 'Paged attention' example (P=32, lens 30/32/70), fp32, then decode")
    g = json.load(open(os.path.join(GOLDEN, "hf_paged_decode_example.json")))
    P, B, H, D = g["page_size"], 3, 2, 64
    gen = torch.Generator(device="cuda").manual_seed(5)
    k_pool = torch.randn(8, P, H, D, generator=gen, device="cuda")
    v_pool = torch.randn(8, P, H, D, generator=gen, device="cuda")
    k_new = torch.randn(B, H, D, generator=gen, device="cuda")
    v_new = torch.randn(B, H, D, generator=gen, device="cuda")
    q = torch.randn(B, H, D, generator=gen, device="cuda")
    bt = torch.tensor(g["block_table"], dtype=torch.int32, device="cuda")
    lens = torch.tensor(g["cache_seqlens"], dtype=torch.int32, device="cuda")
    new = _append_and_check(api, k_pool, v_pool, k_new, v_new, bt, lens, P)
    for b, e in enumerate(g["next_token"]):
        assert torch.equal(k_pool[e["page"], e["slot"]], k_new[b]) and torch.equal(v_pool[e["page"], e["slot"]], v_new[b])
    o, lse = api.batch_decode_paged(q, k_pool, v_pool, bt, new, sm_scale=0.125)
    torch.cuda.synchronize()
    O, L = oatt.batch_decode(host(q), PoolView(k_pool), PoolView(v_pool), g["block_table"], new.cpu().numpy(), P, 0.125)
    check_state(o, lse, O, L, torch.float32, "decode after append")


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_append_twice_in_place_then_decode(api, dtype):
    """Two decode steps' appends (lengths updated in place), page boundaries crossed, GQA."""
    say(f"case: two in-place appends then decode, B=40 Hkv=4 g=4 D=128 P=16 {dtype}")
    B, Hkv, g, D, P = 40, 4, 4, 128, 16
    rng = np.random.default_rng(7)
    lens0 = rng.integers(0, 200, size=B)
    lens0[:4] = [0, 15, 16, 31]                       # empty, block end, block start, block end
    need = [(int(n) + 2 + P - 1) // P for n in lens0]  # room for two more tokens
    perm = rng.permutation(sum(need) + 3).tolist()
    bt = torch.full((B, max(need) + 1), -1, dtype=torch.int32)
    pos = 0
    for b, k in enumerate(need):
        bt[b, :k] = torch.tensor(perm[pos:pos + k])
        pos += k
    N = sum(need) + 3
    gen = torch.Generator(device="cuda").manual_seed(8)
    k_pool = (torch.randn(N, P, Hkv, D, generator=gen, device="cuda") * 0.5).to(dtype)
    v_pool = (torch.randn(N, P, Hkv, D, generator=gen, device="cuda") * 0.5).to(dtype)
    q = (torch.randn(B, Hkv * g, D, generator=gen, device="cuda") * 0.5).to(dtype)
    bt = bt.cuda()
    lens = torch.tensor(lens0, dtype=torch.int32, device="cuda")
    for step in range(2):
        k_new = (torch.randn(B, Hkv, D, generator=gen, device="cuda") * 0.5).to(dtype)
        v_new = (torch.randn(B, Hkv, D, generator=gen, device="cuda") * 0.5).to(dtype)
        _append_and_check(api, k_pool, v_pool, k_new, v_new, bt, lens, P, in_place=True)
    assert lens.cpu().tolist() == [int(n) + 2 for n in lens0]
    o, lse = api.batch_decode_paged(q, k_pool, v_pool, bt, lens)
    torch.cuda.synchronize()
    O, L = oatt.batch_decode(host(q), PoolView(k_pool), PoolView(v_pool), bt.cpu().numpy(), lens.cpu().numpy(), P,
                             1.0 / np.sqrt(D))
    # requests of 0..2 cached tokens give |O| near 1: bf16 output rounding alone exceeds 2e-3
    check_state(o, lse, O, L, dtype, "decode after two appends", rounding_allowance=dtype == torch.bfloat16)


def test_append_to_unallocated_block_is_skipped(api):
    say("case: append whose target block is unallocated or outside the row")
    P, H, D = 4, 1, 64
    bt = torch.tensor([[3, -1], [1, 2], [0, 9]], dtype=torch.int32, device="cuda")
    lens = torch.tensor([4, 8, 4], dtype=torch.int32, device="cuda")   # block 1 = -1; block 2 past the row; page 9 >= 4
    k_pool = torch.zeros(4, P, H, D, device="cuda")
    v_pool = torch.zeros(4, P, H, D, device="cuda")
    ones = torch.ones(3, H, D, device="cuda")
    new = _append_and_check(api, k_pool, v_pool, ones, ones, bt, lens, P)
    assert new.cpu().tolist() == [4, 8, 4] and not k_pool.any() and not v_pool.any()


# --- multi-token (ragged) append ----------------------------------------------------------------

def _ragged_case(seed, dtype, B, P, hkv=4, D=64):
    """Random ragged append: per request an old length, a number of new rows (some 0), a table
    row with room for them except for one request whose next block is -1 (all-or-nothing)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 3 * P, size=B)
    new = rng.choice([0, 1, 3, P, 2 * P + 1, 5 * P], size=B)
    nblk = [-(-(int(lens[b]) + int(new[b])) // P) for b in range(B)]
    width = max(nblk + [1]) + 1
    num_pages = sum(nblk) + 4
    perm = rng.permutation(num_pages)
    bt = np.full((B, width), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
    holes = [b for b in range(B) if new[b] > 0 and (int(lens[b]) + int(new[b]) - 1) // P > int(lens[b]) // P]
    if holes:   # one request loses its last target block: it must write nothing
        b = holes[0]
        bt[b, (int(lens[b]) + int(new[b]) - 1) // P] = -1
    indptr = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    g = torch.Generator(device="cuda").manual_seed(seed)
    k_pool = torch.randn(num_pages, P, hkv, D, generator=g, device="cuda").to(dtype)
    v_pool = torch.randn(num_pages, P, hkv, D, generator=g, device="cuda").to(dtype)
    k_new = torch.randn(int(indptr[-1]), hkv, D, generator=g, device="cuda").to(dtype)
    v_new = torch.randn(int(indptr[-1]), hkv, D, generator=g, device="cuda").to(dtype)
    return k_pool, v_pool, k_new, v_new, bt, lens.astype(np.int32), indptr, holes[:1]


@pytest.mark.parametrize("seed", range(6))
def test_ragged_append_matches_oracle_bitwise(api, seed):
    dtype = [torch.float16, torch.bfloat16, torch.float32][seed % 3]
    P = [16, 4, 1][seed % 3] if seed < 3 else [32, 8, 2][seed % 3]
    B = 7
    say(f"case: ragged append seed={seed} {dtype} P={P} B={B}")
    k_pool, v_pool, k_new, v_new, bt, lens, indptr, holes = _ragged_case(1500 + seed, dtype, B, P)
    k_ref, v_ref, lens_ref = oidx.append_kv_ragged(_bits(k_pool), _bits(v_pool), _bits(k_new), _bits(v_new),
                                                   indptr.tolist(), bt.tolist(), lens.tolist(), P)
    for b in holes:
        assert lens_ref[b] == lens[b]
    new = api.append_kv_ragged(k_new, v_new, torch.tensor(indptr, device="cuda"), k_pool, v_pool,
                               torch.tensor(bt, device="cuda"), torch.tensor(lens, device="cuda"))
    torch.cuda.synchronize()
    assert new.cpu().tolist() == lens_ref
    assert np.array_equal(_bits(k_pool), k_ref), "K pool differs from the oracle's append (bitwise)"
    assert np.array_equal(_bits(v_pool), v_ref), "V pool differs from the oracle's append (bitwise)"


def test_ragged_append_then_causal_prefill(api):
    """Append each request's new tokens, then run the causal prefill of those tokens over the
    new lengths: equal to the oracle's prefill over the oracle-appended pools."""
    import math
    B, P, hkv, g, D = 4, 16, 2, 2, 128
    lens = [0, 37, 100, 5]
    new = [40, 1, 77, 16]
    say(f"case: ragged append then causal prefill, lens={lens} new={new} fp16 P={P}")
    nblk = [-(-(lens[b] + new[b]) // P) for b in range(B)]
    perm = torch.randperm(sum(nblk) + 2, generator=torch.Generator().manual_seed(3)).tolist()
    bt = torch.full((B, max(nblk) + 1), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        bt[b, :nblk[b]] = torch.tensor(perm[off:off + nblk[b]], dtype=torch.int32)
        off += nblk[b]
    gen = torch.Generator(device="cuda").manual_seed(4)
    num_pages = sum(nblk) + 2
    k_pool = (torch.randn(num_pages, P, hkv, D, generator=gen, device="cuda") * 0.5).half()
    v_pool = (torch.randn(num_pages, P, hkv, D, generator=gen, device="cuda") * 0.5).half()
    T = sum(new)
    k_new = (torch.randn(T, hkv, D, generator=gen, device="cuda") * 0.5).half()
    v_new = (torch.randn(T, hkv, D, generator=gen, device="cuda") * 0.5).half()
    q = (torch.randn(T, hkv * g, D, generator=gen, device="cuda") * 0.5).half()
    indptr = [0]
    for n in new:
        indptr.append(indptr[-1] + n)
    k_ref, v_ref, lens_ref = oidx.append_kv_ragged(host(k_pool), host(v_pool), host(k_new), host(v_new), indptr,
                                                   bt.numpy(), lens, P)
    new_lens = api.append_kv_ragged(k_new, v_new, torch.tensor(indptr, dtype=torch.int32, device="cuda"),
                                    k_pool, v_pool, bt.cuda(), torch.tensor(lens, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert new_lens.cpu().tolist() == lens_ref == [lens[b] + new[b] for b in range(B)]
    info, ws, qi = api.prefill_plan(new, lens_ref, hkv * g, hkv, D, P, causal=True)
    o, lse = api.batch_prefill_paged(info, q, k_pool, v_pool, bt.cuda(), torch.tensor(qi, dtype=torch.int32, device="cuda"),
                                     new_lens, causal=True, sm_scale=1.0 / math.sqrt(D))
    torch.cuda.synchronize()
    O, L = oatt.batch_prefill(host(q), qi, k_ref, v_ref, bt.numpy(), lens_ref, P, 1.0 / math.sqrt(D), True)
    check_state(o, lse, O, L, torch.float16, "prefill after ragged append")


def test_ragged_append_rejects_aliased_lengths(api):
    say("case: ragged append with new_seqlens aliasing cache_seqlens is rejected before any launch")
    k_pool = torch.zeros(4, 16, 2, 64, dtype=torch.float16, device="cuda")
    k_new = torch.zeros(3, 2, 64, dtype=torch.float16, device="cuda")
    lens = torch.zeros(2, dtype=torch.int32, device="cuda")
    bt = torch.zeros(2, 1, dtype=torch.int32, device="cuda")
    with pytest.raises(api.PkcError):
        api.append_kv_ragged(k_new, k_new, torch.tensor([0, 1, 3], dtype=torch.int32, device="cuda"), k_pool,
                             k_pool, bt, lens, new_seqlens=lens)
