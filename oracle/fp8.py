"""FP8 KV storage for the oracle (test infrastructure only).

FlashInfer paper summary, appendix F "FP8-FP16 mixed-precision attention":
queries and outputs stay in fp16 while the KV cache is stored in fp8; the
kernels dequantise KV on the fly.  The page names neither the fp8 encoding
nor a scaling rule.  Reading taken here: the OCP 8-bit floating point
specification's E4M3 encoding (the "fn" variant: no infinities), with one
scale per pool, so that the stored key is k = k_scale * e4m3(code) and the
stored value v = v_scale * e4m3(code).  The attention result over FP8 pools
is then, by definition, the attention over those dequantised pools.

E4M3 as the OCP specification defines it, for a byte s.eeee.mmm:

* exponent bias 7;
* e = 0 encodes the subnormals (-1)^s * (m / 8) * 2^(1 - 7), including +0
  and -0;
* 1 <= e <= 15 encodes the normals (-1)^s * (1 + m / 8) * 2^(e - 7), except
  that e = 15 with m = 7 (bytes 0x7F and 0xFF) is NaN;
* there are no infinities, so the largest finite magnitude is
  (1 + 6/8) * 2^8 = 448.
"""

from __future__ import annotations

import math

import numpy as np

from .attention import batch_decode, batch_prefill, cascade_decode, level_prefix_states

BIAS = 7


def e4m3_value(code: int) -> float:
    """The real number (or NaN) that byte `code` encodes in OCP E4M3."""
    code = int(code)
    if not 0 <= code <= 255:
        raise ValueError("an E4M3 code is one byte")
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - BIAS)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - BIAS)


# float64 value of every byte, indexed by the byte.
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def dequantize(codes, scale=1.0):
    """scale * e4m3(codes) in float64, elementwise over an array of bytes."""
    return float(scale) * E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


class DequantizedPool:
    """A code pool seen as its dequantised values: ``view[pages, slots, head]`` gathers the
    bytes from ``codes`` (anything indexable that way, returning uint8) and decodes them."""

    def __init__(self, codes, scale):
        self.codes = codes
        self.scale = float(scale)
        self.shape = tuple(codes.shape)

    def __getitem__(self, idx):
        return dequantize(self.codes[idx], self.scale)


def batch_decode_fp8(q, k_codes, v_codes, k_scale, v_scale, block_table, cache_seqlens,
                     page_size, sm_scale, kv_start=None, requests=None, heads=None):
    """Paged batch decode over FP8 E4M3 pools: the decode of ``attention.batch_decode`` over
    the pools k_scale * e4m3(k_codes) and v_scale * e4m3(v_codes) (reading above)."""
    return batch_decode(q, DequantizedPool(k_codes, k_scale), DequantizedPool(v_codes, v_scale),
                        block_table, cache_seqlens, page_size, sm_scale, kv_start=kv_start,
                        requests=requests, heads=heads)


def cascade_decode_fp8(q, k_codes, v_codes, k_scale, v_scale, page_size, sm_scale, levels,
                       suffix_block_table, suffix_seqlens, requests=None, heads=None):
    """Cascade decode over FP8 E4M3 pools: ``attention.cascade_decode`` (one softmax over each
    request's level token sets and suffix) over the dequantised pools."""
    return cascade_decode(q, DequantizedPool(k_codes, k_scale), DequantizedPool(v_codes, v_scale),
                          page_size, sm_scale, levels, suffix_block_table, suffix_seqlens,
                          requests=requests, heads=heads)


def level_prefix_states_fp8(q, k_codes, v_codes, k_scale, v_scale, page_size, sm_scale, level,
                            num_requests):
    """``attention.level_prefix_states`` over the dequantised FP8 E4M3 pools."""
    return level_prefix_states(q, DequantizedPool(k_codes, k_scale), DequantizedPool(v_codes, v_scale),
                               page_size, sm_scale, level, num_requests)


def batch_prefill_fp8(q, qo_indptr, k_codes, v_codes, k_scale, v_scale, block_table, kv_lens,
                      page_size, sm_scale, causal, rows=None, heads=None):
    """``attention.batch_prefill`` (ragged multi-token queries) over the dequantised FP8 E4M3
    pools."""
    return batch_prefill(q, qo_indptr, DequantizedPool(k_codes, k_scale), DequantizedPool(v_codes, v_scale),
                         block_table, kv_lens, page_size, sm_scale, causal, rows=rows, heads=heads)
