"""Plain float64 gradient of softmax attention: the oracle the GPU backward is checked against.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module; only the tests, the smoke check and the bench's CPU-baseline leg do.

The forward is O = softmax(scale * Q K^T + M) V row by row, with M = 0 on the
allowed pairs and -inf elsewhere (the same allowed set as the forward oracle:
causal keeps j <= i; the block-sparse pattern keeps j when its key block is
listed for the query block of i; duplicates count once).  Given the upstream
gradient dO (PyTorch's grad_output), the chain rule through the three stages
gives, per (batch, head) ("Exact Blocks, Rings, and Sparsity", section 3,
"FlashAttention Backward: recomputing P"):

* value mixture:   dV = P^T dO  and  dP = dO V^T;
* row softmax:     dS_ij = P_ij (dP_ij - D_i), with the one row scalar
                   D_i = sum_j P_ij dP_ij, which equals dO_i . O_i because
                   O_i = sum_j P_ij V_j (the preprocessing step of that
                   section computes it this way, from O and dO alone);
* scores:          S = scale Q K^T, so dQ = scale dS K and dK = scale dS^T Q;
                   the mask does not depend on Q or K.

The FlashAttention notes, section 5.3 (backward recomputation), give the same
chain: P rebuilt from the saved row statistics, D_i = dO_i . O_i in place of
the row reduction P_i . dP_i, dS_ij = P_ij (dP_ij - D_i).

P is rebuilt from the saved log-normaliser, P_ij = exp(S_ij - LSE_i) on
allowed pairs and 0 elsewhere (same section, "Reconstructing a probability
tile without saving P").  A query row with no allowed key has P = 0, hence
dS = 0: it contributes nothing to dK or dV and gets dQ = 0.

Everything is float64, computed from whole score rows (S and P of a chunk of
query rows are materialised in host memory); O and LSE come from the forward
oracle unless the caller passes its own.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .attention import (_as64, meta_index, output_stage, scores_stage, softmax_stage, token_mask_block_sparse,
                        token_mask_dense)


def probabilities_from_lse(s: np.ndarray, lse: np.ndarray) -> np.ndarray:
    """P_ij = exp(S_ij - LSE_i) on allowed pairs (S_ij finite), 0 elsewhere and
    on rows with LSE = -inf."""
    finite = np.isfinite(lse)
    lse_safe = np.where(finite, lse, 0.0)
    p = np.exp(s - lse_safe[:, None])      # exp(-inf) = 0 on masked pairs
    p[~finite] = 0.0
    return p


def row_scalar_d(do_rows: np.ndarray, o_rows: np.ndarray) -> np.ndarray:
    """D_i = dO_i . O_i (the preprocessing step)."""
    return np.sum(do_rows * o_rows, axis=1)


def score_gradient(p: np.ndarray, dp: np.ndarray, d_rows: np.ndarray) -> np.ndarray:
    """dS = P * (dP - D[:, None]) (row-softmax gradient)."""
    return p * (dp - d_rows[:, None])


def attention_head_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
                       mask_fn, o: Optional[np.ndarray] = None, lse: Optional[np.ndarray] = None,
                       row_chunk: int = 1024) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """dQ, dK, dV of one head ([N, d] float64 each).

    ``mask_fn(rows)`` returns the allowed[rows, :] boolean mask.  Query rows are
    processed in chunks of ``row_chunk``: dQ of a chunk needs only its rows,
    dK and dV sum the chunk's contributions.
    """
    N, d = q.shape
    dq = np.zeros((N, d))
    dk = np.zeros((N, d))
    dv = np.zeros((N, d))
    for c0 in range(0, N, row_chunk):
        rows = np.arange(c0, min(N, c0 + row_chunk))
        s = scores_stage(q[rows], k, scale, mask_fn(rows))
        if o is None or lse is None:
            p_fwd, lse_c = softmax_stage(s)
            o_c = output_stage(p_fwd, v)
        else:
            o_c, lse_c = o[rows], lse[rows]
        p = probabilities_from_lse(s, lse_c)
        dv += p.T @ do[rows]
        dp = do[rows] @ v.T
        ds = score_gradient(p, dp, row_scalar_d(do[rows], o_c))
        dq[rows] = scale * (ds @ k)
        dk += scale * (ds.T @ q[rows])
    return dq, dk, dv


def _run_bwd(q, k, v, do, scale, mask_for_head, o, lse, row_chunk):
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    if o is not None:
        o, lse = _as64(o), _as64(lse)
    B, H, N, d = q.shape
    for t in (k, v, do):
        if t.shape != q.shape:
            raise ValueError("Q, K, V, dO must share the shape [B, H, N, d]")
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = attention_head_bwd(
                q[b, h], k[b, h], v[b, h], do[b, h], scale, mask_for_head(b, h),
                None if o is None else o[b, h], None if lse is None else lse[b, h], row_chunk)
    return dq, dk, dv


def attn_bwd(q, k, v, do, scale: float, causal: bool, o=None, lse=None, row_chunk: int = 1024):
    """Gradients (dQ, dK, dV) of dense, optionally causal, attention for
    [B,H,N,d] inputs and upstream gradient dO.  ``o``/``lse``: the forward's
    outputs to rebuild P and D from (default: the forward oracle's, exact)."""
    N = q.shape[2]
    mask_for_head = lambda b, h: (lambda rows: token_mask_dense(N, causal, rows))
    return _run_bwd(q, k, v, do, scale, mask_for_head, o, lse, row_chunk)


def attn_bwd_blocksparse(q, k, v, do, scale: float, causal: bool, block: int, raw_row_ptr, raw_col,
                         meta_heads: int, o=None, lse=None, row_chunk: int = 1024):
    """Gradients of block-sparse attention renormalised over the allowed pairs
    (raw, uncanonicalised lists; meta_heads 1 or H, as the forward oracle)."""
    B, H, N, d = q.shape
    if meta_heads not in (1, H, B * H):
        raise ValueError("meta_heads must be 1, H or B*H")
    mask_for_head = lambda b, h: (lambda rows: token_mask_block_sparse(
        N, causal, block, raw_row_ptr, raw_col, meta_index(b, h, H, meta_heads), rows))
    return _run_bwd(q, k, v, do, scale, mask_for_head, o, lse, row_chunk)
