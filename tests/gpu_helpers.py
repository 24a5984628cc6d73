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


def host(t):
    """Exact float64 host copy of a small device tensor."""
    return t.detach().float().cpu().double().numpy()


# Bits of precision of the output formats: rounding the fp32 result once to the output dtype
# (round to nearest even) moves it by at most |O| * 2^-p.
OUT_PRECISION = {torch.float16: 11, torch.bfloat16: 8, torch.float32: 24}


def check_state(o, lse, o_ref, lse_ref, dtype, label="", rows=None):
    """Max |dO| and |dLSE| against the oracle over the computed (non-NaN) reference entries.

    `dtype` is the input dtype: it sets the accumulation budget (2e-3 / 1e-3 for 16-bit
    inputs, 1e-5 for fp32).  On top of it, O may differ by the one final rounding to its own
    storage dtype, |O_ref| * 2^-p (p = 11 for fp16, 8 for bf16).  LSE is always fp32.
    -inf LSE must match exactly, and the output must be finite there."""
    tol_o, tol_l = TOL[dtype]
    rnd = 2.0 ** -OUT_PRECISION[o.dtype]
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
    say(f"  {label}: max|dO| = {d_o:.3e} (tol {tol_o:g} + |O|*2^-{-int(np.log2(rnd))}), "
        f"max|dLSE| = {d_l:.3e} (tol {tol_l:g})")
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
