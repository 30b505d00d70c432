"""Helpers shared by the GPU parity tests: seeded inputs, oracle calls and the
pass criteria (max |dO| and max |dLSE| over rows with finite LSE; empty rows
exactly O = 0 and LSE = -inf; no NaN anywhere)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads

TOL = {"bf16": (1e-2, 1e-3), "f32": (1e-5, 1e-5)}


def inputs(B, H, N, d, dtype, seed):
    q, k, v = workloads.make_qkv(B, H, N, d, dtype, seed)
    return q, k, v


def compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype, label=""):
    """o_gpu/lse_gpu: numpy float64 of the GPU outputs (rows already selected)."""
    tol_o, tol_l = TOL[dtype]
    assert not np.isnan(o_gpu).any(), f"{label}: NaN in O"
    assert not np.isnan(lse_gpu).any(), f"{label}: NaN in LSE"
    empty = ~np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_gpu), ~empty), f"{label}: empty-row pattern differs"
    if empty.any():
        assert np.all(o_gpu[empty] == 0.0), f"{label}: empty rows must give O == 0"
        assert np.all(lse_gpu[empty] == -np.inf), f"{label}: empty rows must give LSE == -inf"
    live = ~empty
    do = float(np.max(np.abs(o_gpu[live] - o_ref[live]))) if live.any() else 0.0
    dl = float(np.max(np.abs(lse_gpu[live] - lse_ref[live]))) if live.any() else 0.0
    assert do <= tol_o, f"{label}: max|dO| = {do:.3e} > {tol_o}"
    assert dl <= tol_l, f"{label}: max|dLSE| = {dl:.3e} > {tol_l}"
    return do, dl


def to64(t):
    return t.detach().to("cpu", torch.float64).numpy()
