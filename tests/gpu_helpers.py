"""Shared helpers of the GPU parity tests (no attention arithmetic here)."""

import math
import sys

import numpy as np
import pytest
import torch

# Tolerances against the fp64 oracle (elementwise absolute): 16-bit inputs with fp32
# accumulation, and fp32 inputs.
TOL = {torch.float16: (2e-3, 1e-3), torch.bfloat16: (2e-3, 1e-3), torch.float32: (1e-5, 1e-5)}

gpu = pytest.mark.gpu
needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def say(*args):
    """Print a progress line and flush it (names the case before each GPU step)."""
    print(*args, flush=True)
    sys.stdout.flush()


class PoolView:
    """Lets the oracle gather rows of a device pool: pool[pages, slots] returns only the
    requested rows, upcast exactly to float32 and copied to the host."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        pages, slots, head = idx
        dev = self.t.device
        p = torch.as_tensor(np.asarray(pages), dtype=torch.long, device=dev)
        s = torch.as_tensor(np.asarray(slots), dtype=torch.long, device=dev)
        return self.t[p, s, int(head)].float().cpu().numpy()


class HostPool:
    """Like PoolView, over a host copy of the pool taken once (the full-size tests gather every
    request's rows for several heads; one device-to-host copy is much cheaper than a copy per
    request).  Rows come back upcast exactly to float32."""

    def __init__(self, t):
        self.t = t.detach().cpu()
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        pages, slots, head = idx
        p = torch.as_tensor(np.asarray(pages), dtype=torch.long)
        s = torch.as_tensor(np.asarray(slots), dtype=torch.long)
        return self.t[p, s, int(head)].float().numpy()


# Query heads compared at full size: every request (so every row of the 128-row MFMA tile and
# every decode workgroup's item) on three heads spread over the head range.
FULL_SIZE_HEADS = [0, 13, 31]


def host(t):
    """Exact float64 host copy of a small device tensor."""
    return t.detach().float().cpu().double().numpy()


# Bits of precision of the output formats: rounding the fp32 result once to the output dtype
# (round to nearest even) moves it by at most |O| * 2^-p.
OUT_PRECISION = {torch.float16: 11, torch.bfloat16: 8, torch.float32: 24}


def check_state(o, lse, o_ref, lse_ref, dtype, label="", rows=None, rounding_allowance=False):
    """Max |dO| and |dLSE| against the oracle over the computed (non-NaN) reference entries.

    `dtype` is the input dtype and sets the bound: |dO| <= 2e-3 and |dLSE| <= 1e-3 for 16-bit
    inputs with fp32 accumulation, 1e-5 for fp32 inputs (elementwise, absolute).

    ``rounding_allowance`` is for the stress cases with N(0, 1) inputs only: there a few
    tokens can give |O| near 1 or above, and the one final rounding of O to a bf16 output
    alone moves it by up to |O| * 2^-8 (3.9e-3 at |O| = 1), more than the absolute budget.
    With it, O may also differ by |O_ref| * 2^-p (p = 11 for fp16, 8 for bf16).  The standard
    workloads (values N(0, 1) * 0.5, |O| well below 0.5) are checked without it.

    -inf LSE must match exactly, and the output must be finite there."""
    tol_o, tol_l = TOL[dtype]
    rnd = 2.0 ** -OUT_PRECISION[o.dtype] if rounding_allowance else 0.0
    o = host(o)
    lse = lse.detach().cpu().double().numpy()
    mask = ~np.isnan(lse_ref)
    if rows is not None:
        m2 = np.zeros_like(mask)
        m2[rows] = mask[rows]
        mask = m2
    assert mask.any(), "nothing to compare"
    lr, lg = lse_ref[mask], lse[mask]
    inf_ref = np.isneginf(lr)
    assert np.array_equal(np.isneginf(lg), inf_ref), f"{label}: -inf LSE pattern differs"
    assert np.all(np.isfinite(o[mask])), f"{label}: non-finite output"
    d_l = float(np.max(np.abs(lg[~inf_ref] - lr[~inf_ref]))) if (~inf_ref).any() else 0.0
    err = np.abs(o[mask] - o_ref[mask])
    allowed = tol_o + np.abs(o_ref[mask]) * rnd
    d_o = float(np.max(err))
    worst = float(np.max(err - allowed))
    bound = f"tol {tol_o:g} + |O|*2^-{-int(np.log2(rnd))}" if rnd else f"tol {tol_o:g}"
    say(f"  {label}: max|dO| = {d_o:.3e} ({bound}), max|dLSE| = {d_l:.3e} (tol {tol_l:g}), "
        f"{int(mask.sum())} (row, head) states compared")
    assert worst <= 0.0, f"{label}: |dO| exceeds its bound by {worst} (max|dO| {d_o})"
    assert d_l <= tol_l, f"{label}: max|dLSE| {d_l} > {tol_l}"
    return d_o, d_l


def scale_of(D):
    return 1.0 / math.sqrt(D)


class CodeView:
    """Lets the oracle gather rows of a device FP8 pool as raw bytes: pool[pages, slots, head]
    returns the uint8 codes of only the requested rows (decoding is the oracle's job)."""

    def __init__(self, t):
        self.t = t.view(torch.uint8)
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        pages, slots, head = idx
        dev = self.t.device
        p = torch.as_tensor(np.asarray(pages), dtype=torch.long, device=dev)
        s = torch.as_tensor(np.asarray(slots), dtype=torch.long, device=dev)
        return self.t[p, s, int(head)].cpu().numpy()


class HostCodeView:
    """Like CodeView, over a host copy of the FP8 pool's bytes taken once."""

    def __init__(self, t):
        self.t = t.detach().view(torch.uint8).cpu()
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        pages, slots, head = idx
        p = torch.as_tensor(np.asarray(pages), dtype=torch.long)
        s = torch.as_tensor(np.asarray(slots), dtype=torch.long)
        return self.t[p, s, int(head)].numpy()
