"""Shared helpers of the GPU parity tests (the GPU side is always the HIP library)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

# Tolerances of the parity bar: fp32 inputs 1e-5 max-abs; bf16 inputs (fp32
# accumulation) 2e-2 max-abs and 1e-2 mean relative error sum|a-b| / sum|b|.
TOL = {torch.float32: {"max_abs": 1e-5, "mean_rel": None},
       torch.bfloat16: {"max_abs": 2e-2, "mean_rel": 1e-2}}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from shared_prefix_block_amd import psa
    psa.load()  # raises if libpsa.so is missing: GPU tests never run without it


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def compare(name, got, want, dtype, mask=None, out_round=0.0):
    """Element-wise parity of a GPU tensor with the oracle's float64 array.

    ``out_round`` (relative) widens the max-abs bound by the rounding of an output
    stored in a narrower type than the fp32 it was accumulated in: a bf16 output is
    off its fp32 value by up to 2^-9 of its magnitude, whatever the kernel does."""
    g = got.detach().float().cpu().numpy().astype(np.float64) if hasattr(got, "detach") else \
        np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    assert g.shape == w.shape, (name, g.shape, w.shape)
    if mask is not None:
        g, w = g[mask], w[mask]
    fin_w = np.isfinite(w)
    # non-finite entries (LSE = -inf on rows with no key) must match exactly
    bad = ~fin_w & (g != w)
    assert not bad.any(), f"{name}: {int(bad.sum())} non-finite mismatches"
    assert np.isfinite(g[fin_w]).all(), f"{name}: non-finite values where the oracle is finite"
    if not fin_w.any():
        return 0.0, 0.0
    diff = np.abs(g[fin_w] - w[fin_w])
    denom = float(np.abs(w[fin_w]).sum())
    mean_rel = float(diff.sum() / denom) if denom > 0 else 0.0
    if out_round:  # max-abs is judged after the allowance for the output's own rounding
        diff = np.maximum(diff - out_round * (np.abs(w[fin_w]) + TOL[dtype]["max_abs"]), 0.0)
    max_abs = float(diff.max())
    tol = TOL[dtype]
    if max_abs > tol["max_abs"]:
        at = int(np.argmax(diff))
        where = np.unravel_index(np.flatnonzero(fin_w)[at], w.shape) if mask is None else at
        raise AssertionError(f"{name}: max-abs {max_abs:.3e} > {tol['max_abs']} at {where}: "
                             f"got {g[fin_w][at]:.9g}, want {w[fin_w][at]:.9g}")
    if tol["mean_rel"] is not None:
        assert mean_rel <= tol["mean_rel"], f"{name}: mean-rel {mean_rel:.3e} > {tol['mean_rel']}"
    return max_abs, mean_rel
