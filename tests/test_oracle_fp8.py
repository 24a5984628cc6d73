"""Pins of the oracle's FP8 E4M3 decoding and of the decode over FP8 pools (CPU only).

The E4M3 table is checked against values the OCP 8-bit floating point
specification fixes (largest finite 448, smallest subnormal 2^-9, one, the two
NaN bytes, signed zeros), against torch's own float8_e4m3fn conversion for all
256 bytes, and against properties of any sign-magnitude float format
(monotone in the magnitude bits, sign symmetry).  The decode over FP8 pools is
checked against the decode over float pools holding the same values (decoded
by torch, not by the oracle), and the pool scales against their closed-form
effect on the scores and the output.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention, fp8


def test_e4m3_values_fixed_by_the_format():
    v = fp8.E4M3_TABLE
    assert v[0x00] == 0.0 and not math.copysign(1.0, v[0x00]) < 0
    assert v[0x80] == 0.0 and math.copysign(1.0, v[0x80]) < 0      # negative zero
    assert v[0x01] == 2.0 ** -9                                     # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9                                 # largest subnormal
    assert v[0x08] == 2.0 ** -6                                     # smallest normal
    assert v[0x38] == 1.0
    assert v[0x3C] == 1.5
    assert v[0x40] == 2.0
    assert v[0x78] == 256.0
    assert v[0x7E] == 448.0                                         # largest finite
    assert v[0xFE] == -448.0
    assert v[0xB8] == -1.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert int(np.isnan(v).sum()) == 2                              # no other NaN, no infinity
    assert np.all(np.isfinite(v[~np.isnan(v)]))


def test_e4m3_matches_torch_float8_e4m3fn_for_every_byte():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = fp8.E4M3_TABLE
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(mine[ok]))


def test_e4m3_monotone_and_sign_symmetric():
    v = fp8.E4M3_TABLE
    pos = v[0x00:0x7F]
    assert np.all(np.diff(pos) > 0), "magnitudes must increase with the code"
    assert np.array_equal(v[0x80:0xFF], -pos)
    # Each binade above the subnormals holds 8 equally spaced values.
    for e in range(1, 15):
        b = v[e * 8:(e + 1) * 8]
        assert np.allclose(np.diff(b), 2.0 ** (e - 7) / 8, rtol=0, atol=0)


def test_e4m3_round_trip_through_torch_cast():
    finite = [c for c in range(256) if not np.isnan(fp8.E4M3_TABLE[c])]
    vals = torch.tensor([fp8.E4M3_TABLE[c] for c in finite], dtype=torch.float64)
    back = vals.to(torch.float8_e4m3fn).view(torch.uint8).to(torch.int32).tolist()
    assert back == finite


def test_dequantize_scales_and_rejects_non_bytes():
    codes = np.array([[0x38, 0x40], [0xB8, 0x01]], dtype=np.uint8)
    assert np.array_equal(fp8.dequantize(codes, 0.5), [[0.5, 1.0], [-0.5, 2.0 ** -10]])
    with pytest.raises(ValueError):
        fp8.e4m3_value(256)


def _fp8_case(seed, B=4, hkv=2, g=2, D=16, P=4):
    """Small paged FP8 case: codes are torch's RNE cast of N(0, 1) * 0.7 values."""
    gen = torch.Generator().manual_seed(seed)
    lens = [0, 1, 7, 13][:B]
    npg = [-(-n // P) for n in lens]
    num_pages = sum(npg) + 2
    perm = torch.randperm(num_pages, generator=gen).tolist()
    bt = np.full((B, max(npg) + 1), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(npg):
        bt[b, :n] = perm[off:off + n]
        off += n
    q = torch.randn(B, hkv * g, D, generator=gen, dtype=torch.float64).numpy()
    kf = (torch.randn(num_pages, P, hkv, D, generator=gen) * 0.7).to(torch.float8_e4m3fn)
    vf = (torch.randn(num_pages, P, hkv, D, generator=gen) * 0.7).to(torch.float8_e4m3fn)
    return q, kf, vf, bt, np.array(lens), P


def test_fp8_decode_equals_decode_over_torch_decoded_pools():
    q, kf, vf, bt, lens, P = _fp8_case(5)
    kc, vc = kf.view(torch.uint8).numpy(), vf.view(torch.uint8).numpy()
    O8, L8 = fp8.batch_decode_fp8(q, kc, vc, 1.0, 1.0, bt, lens, P, 0.25)
    O, L = attention.batch_decode(q, kf.to(torch.float64).numpy(), vf.to(torch.float64).numpy(),
                                  bt, lens, P, 0.25)
    assert np.array_equal(np.isneginf(L8), np.isneginf(L))
    assert np.array_equal(O8, O) and np.array_equal(L8[~np.isneginf(L)], L[~np.isneginf(L)])


def test_fp8_scales_act_on_scores_and_output():
    """k_scale multiplies every score (same as multiplying sm_scale); v_scale multiplies O and
    leaves LSE alone."""
    q, kf, vf, bt, lens, P = _fp8_case(6)
    kc, vc = kf.view(torch.uint8).numpy(), vf.view(torch.uint8).numpy()
    O1, L1 = fp8.batch_decode_fp8(q, kc, vc, 1.0, 1.0, bt, lens, P, 0.25 * 3.0)
    O2, L2 = fp8.batch_decode_fp8(q, kc, vc, 3.0, 1.0, bt, lens, P, 0.25)
    fin = ~np.isneginf(L1)
    assert np.allclose(O1, O2, rtol=1e-13, atol=1e-15) and np.allclose(L1[fin], L2[fin], rtol=1e-13)
    O3, L3 = fp8.batch_decode_fp8(q, kc, vc, 1.0, 0.375, bt, lens, P, 0.25)
    O4, L4 = fp8.batch_decode_fp8(q, kc, vc, 1.0, 1.0, bt, lens, P, 0.25)
    assert np.allclose(O3, 0.375 * O4, rtol=1e-13, atol=1e-15)
    assert np.array_equal(L3[fin], L4[fin])


def test_fp8_single_token_returns_the_decoded_value_row():
    """Over one token the softmax weight is 1: O is that row's decoded values times v_scale,
    and LSE is the scaled score sm_scale * k_scale * (q . e4m3(k))."""
    q, kf, vf, bt, lens, P = _fp8_case(7)
    kc, vc = kf.view(torch.uint8).numpy(), vf.view(torch.uint8).numpy()
    O, L = fp8.batch_decode_fp8(q, kc, vc, 0.5, 2.0, bt, lens, P, 0.25)
    b = 1                                    # the request with one token
    page = bt[b, 0]
    for h in range(q.shape[1]):
        kh = h // 2
        vrow = vf[page, 0, kh].to(torch.float64).numpy()
        krow = kf[page, 0, kh].to(torch.float64).numpy()
        assert np.array_equal(O[b, h], 2.0 * vrow)
        assert math.isclose(L[b, h], 0.25 * 0.5 * float(q[b, h] @ krow), rel_tol=1e-14, abs_tol=1e-15)


def test_fp8_cascade_and_level_states_equal_torch_decoded_pools():
    """The cascade and per-level oracles over code pools equal the same oracles over float
    pools holding torch's decoding of the codes (two levels, one of them partial)."""
    gen = torch.Generator().manual_seed(11)
    P, hkv, g, D, B = 4, 1, 2, 8, 5
    kf = (torch.randn(12, P, hkv, D, generator=gen) * 0.7).to(torch.float8_e4m3fn)
    vf = (torch.randn(12, P, hkv, D, generator=gen) * 0.7).to(torch.float8_e4m3fn)
    q = torch.randn(B, hkv * g, D, generator=gen, dtype=torch.float64).numpy()
    levels = [{"qo_indptr": [0, 5], "kv_page_indptr": [0, 2], "kv_page_indices": [3, 7], "kv_lens": [6]},
              {"qo_indptr": [0, 2, 4], "kv_page_indptr": [0, 1, 3], "kv_page_indices": [0, 9, 4],
               "kv_lens": [3, 8]}]
    bt = np.array([[1, -1], [2, 5], [6, -1], [8, -1], [10, 11]], dtype=np.int32)
    lens = np.array([2, 7, 0, 4, 5])
    kc, vc = kf.view(torch.uint8).numpy(), vf.view(torch.uint8).numpy()
    kd, vd = kf.to(torch.float64).numpy(), vf.to(torch.float64).numpy()
    O8, L8 = fp8.cascade_decode_fp8(q, kc, vc, 1.0, 1.0, P, 0.5, levels, bt, lens)
    O, L = attention.cascade_decode(q, kd, vd, P, 0.5, levels, bt, lens)
    assert np.array_equal(O8, O) and np.array_equal(L8, L)
    for lv in levels:
        O8, L8 = fp8.level_prefix_states_fp8(q, kc, vc, 2.0, 0.5, P, 0.5, lv, B)
        O, L = attention.level_prefix_states(q, 2.0 * kd, 0.5 * vd, P, 0.5, lv, B)
        assert np.array_equal(np.isnan(L8), np.isnan(L))
        m = ~np.isnan(L)
        assert np.allclose(L8[m], L[m], rtol=1e-14, atol=1e-14)
        assert np.allclose(O8[m], O[m], rtol=1e-13, atol=1e-15)


def test_fp8_prefill_equals_prefill_over_torch_decoded_pools():
    q, kf, vf, bt, lens, P = _fp8_case(8)
    qo = [0, 2, 3, 8, 9]          # 4 requests with 2, 1, 5, 1 queries
    kc, vc = kf.view(torch.uint8).numpy(), vf.view(torch.uint8).numpy()
    qq = np.concatenate([q, q[:1], q, q[:1]])[:9]
    for causal in (False, True):
        O8, L8 = fp8.batch_prefill_fp8(qq, qo, kc, vc, 0.5, 2.0, bt, lens, P, 0.25, causal)
        O, L = attention.batch_prefill(qq, qo, 0.5 * kf.to(torch.float64).numpy(), 2.0 * vf.to(torch.float64).numpy(),
                                       bt, lens, P, 0.25, causal)
        fin = ~np.isneginf(L)
        assert np.array_equal(np.isneginf(L8), ~fin)
        assert np.allclose(O8, O, rtol=1e-13, atol=1e-15) and np.allclose(L8[fin], L[fin], rtol=1e-13)
