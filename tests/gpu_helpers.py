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


def check_state(o, lse, o_ref, lse_ref, dtype, label="", rows=None):
    """Max |dO| and |dLSE| against the oracle over the computed (non-NaN) reference entries.
    -inf LSE must match exactly, and the output must be finite there."""
    tol_o, tol_l = TOL[dtype]
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
    d_o = float(np.max(np.abs(o[mask] - o_ref[mask])))
    say(f"  {label}: max|dO| = {d_o:.3e} (tol {tol_o:g}), max|dLSE| = {d_l:.3e} (tol {tol_l:g})")
    assert d_o <= tol_o, f"{label}: max|dO| {d_o} > {tol_o}"
    assert d_l <= tol_l, f"{label}: max|dLSE| {d_l} > {tol_l}"
    return d_o, d_l


def scale_of(D):
    return 1.0 / math.sqrt(D)
