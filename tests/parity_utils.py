"""Helpers shared by the GPU parity tests: seeded inputs, oracle calls and the
pass criteria.

Forward: max |dO| and max |dLSE| over rows with finite LSE; empty rows exactly
O = 0 and LSE = -inf; no NaN anywhere.

Backward: the reference is the oracle's gradient computed from the same O
(bf16) and LSE (fp32) the kernel receives.  The kernel rounds P and dS to bf16
(relative error at most u = 2^-8 each; dS also inherits P's) before the
products, accumulates in fp32 and stores dQ, dK, dV in bf16.  Each output
element is a sum of n terms t (dV: P_ij dO_ic; dK: scale dS_ij Q_ic; dQ:
scale dS_ij K_jc) whose rounding errors are independent with relative size
at most e (u for dV, 2u for dK and dQ), so their sum has standard deviation
at most e/sqrt(3) * sqrt(sum t^2).  Allowed per element: six such standard
deviations, plus u |x| for the output rounding, plus 2^-20 sum |t| for fp32
accumulation and for the cancellation in dP - D.
"""
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


def per_head(fn, q, k, v, workers=8):
    """Full-row oracle results of every (b, h), one head per task on a thread
    pool (numpy's exponentials and BLAS release the GIL).  fn(q, k, v, b, h)
    gets [1, 1, N, d] slices and returns the oracle's (O, LSE) for them."""
    from concurrent.futures import ThreadPoolExecutor
    B, H, N, d = q.shape
    jobs = [(b, h) for b in range(B) for h in range(H)]

    def run(bh):
        b, h = bh
        sl = (slice(b, b + 1), slice(h, h + 1))
        return fn(q[sl], k[sl], v[sl], b, h)

    with ThreadPoolExecutor(workers) as ex:
        res = list(ex.map(run, jobs))
    o = np.concatenate([r[0].reshape(1, N, d) for r in res]).reshape(B, H, N, d)
    lse = np.concatenate([r[1].reshape(1, N) for r in res]).reshape(B, H, N)
    return o, lse


def to64(t):
    return t.detach().to("cpu", torch.float64).numpy()


U_BF16 = 2.0 ** -8
F_ACC = 2.0 ** -20


def bwd_bounds_head(q, k, v, do, scale, allowed_fn, o_in, lse_in, row_chunk=512):
    """Per-element allowed error of (dQ, dK, dV) for one head, excluding the
    output rounding u|x|.  Inputs float64 [N, d] (lse_in [N]); allowed_fn(rows)
    gives the boolean mask rows x N."""
    from oracle import attention as A
    from oracle import backward as BW
    N, d = q.shape
    aq, ak, av, ado, ao = (np.abs(x) for x in (q, k, v, do, o_in))
    rss_v = np.zeros((N, d)); lin_v = np.zeros((N, d))
    rss_k = np.zeros((N, d)); lin_k = np.zeros((N, d))
    rss_q = np.zeros((N, d)); lin_q = np.zeros((N, d))
    for c0 in range(0, N, row_chunk):
        rows = np.arange(c0, min(N, c0 + row_chunk))
        s = A.scores_stage(q[rows], k, scale, allowed_fn(rows))
        p = BW.probabilities_from_lse(s, lse_in[rows])
        dp = do[rows] @ v.T
        ds = BW.score_gradient(p, dp, BW.row_scalar_d(do[rows], o_in[rows]))
        # fp32 cancellation in dP - D, as an absolute error on dS
        ds_floor = p * ((ado[rows] @ av.T) + (ado[rows] * ao[rows]).sum(axis=1)[:, None])
        ads = np.abs(ds) + ds_floor
        rss_v += (p * p).T @ (do[rows] ** 2)
        lin_v += p.T @ ado[rows]
        rss_k += (ds * ds).T @ (q[rows] ** 2)
        lin_k += ads.T @ aq[rows]
        rss_q[rows] = (ds * ds) @ (k ** 2)
        lin_q[rows] = ads @ ak
    six = 6.0 / np.sqrt(3.0)
    b_v = six * U_BF16 * np.sqrt(rss_v) + F_ACC * lin_v
    b_k = scale * (six * 2 * U_BF16 * np.sqrt(rss_k) + F_ACC * lin_k)
    b_q = scale * (six * 2 * U_BF16 * np.sqrt(rss_q) + F_ACC * lin_q)
    return b_q, b_k, b_v


def compare_grad(got, ref, bound, label):
    """|got - ref| <= bound + u |ref| element by element; no NaN."""
    assert not np.isnan(got).any(), f"{label}: NaN"
    err = np.abs(got - ref)
    allowed = bound + U_BF16 * np.abs(ref) + 1e-30
    ratio = err / allowed
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio[worst] <= 1.0, (f"{label}: error {err[worst]:.3e} > allowed {allowed[worst]:.3e} at {worst} "
                                 f"(ref {ref[worst]:.3e}); max |err| {err.max():.3e}")
    return float(err.max()), float(ratio.max())
