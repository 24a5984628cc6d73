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
    check_state(o, lse, O, L, dtype, "decode after two appends")


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
