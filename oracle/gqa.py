"""Grouped-query attention in the oracle (test infrastructure only).

TEST INFRASTRUCTURE ONLY: nothing on the product path imports this module.

Definition ("Exact Blocks, Rings, and Sparsity", section 5, the GQA remarks in
"The selector must cost less than the tiles it skips" and under NSA): H query
heads share Hkv key/value heads; query head h reads key/value head
h // (H / Hkv).  Under block sparsity the query heads of a group share one
key-block list (meta_heads == Hkv), so the group loads one set of K/V blocks
instead of the union of unrelated sets.  The forward is the dense/sparse
oracle with each key/value head repeated for its query heads; the gradient of
a shared K/V head is the sum of the gradients its query heads send it.
"""
from __future__ import annotations

import numpy as np

from .attention import _as64, attn_fwd, attn_fwd_blocksparse
from .backward import attn_bwd, attn_bwd_blocksparse


def expand_kv(x, H: int) -> np.ndarray:
    """[B, Hkv, N, d] -> [B, H, N, d]: query head h gets key/value head h // (H / Hkv)."""
    x = _as64(x)
    Hkv = x.shape[1]
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    return np.repeat(x, H // Hkv, axis=1)


def expand_lists(raw_row_ptr, raw_col, meta_heads: int, H: int, Hkv: int, nqb: int):
    """Raw per-query-block lists for meta_heads in {1, Hkv, H}, rewritten as
    one list set per query head (meta head of query head h: 0, h // (H/Hkv) or h)."""
    raw_row_ptr = np.asarray(raw_row_ptr, dtype=np.int64)
    raw_col = np.asarray(raw_col, dtype=np.int64)
    if meta_heads == 1:
        src = [0] * H
    elif meta_heads == H:
        src = list(range(H))
    elif meta_heads == Hkv:
        src = [h // (H // Hkv) for h in range(H)]
    else:
        raise ValueError("meta_heads must be 1, Hkv or H")
    rows = []
    for h in range(H):
        for qb in range(nqb):
            r = src[h] * nqb + qb
            rows.append(raw_col[raw_row_ptr[r]:raw_row_ptr[r + 1]])
    row_ptr = np.zeros(len(rows) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    col = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)
    return row_ptr, col


def attn_fwd_gqa(q, k, v, scale: float, causal: bool, block=None, raw_row_ptr=None, raw_col=None,
                 meta_heads: int = 1, rows=None):
    """O, LSE of query heads [B, H, N, d] against key/value heads [B, Hkv, N, d]."""
    q = _as64(q)
    B, H, N, d = q.shape
    Hkv = np.shape(k)[1]
    ke, ve = expand_kv(k, H), expand_kv(v, H)
    if block is None:
        return attn_fwd(q, ke, ve, scale, causal, rows=rows)
    rp, col = expand_lists(raw_row_ptr, raw_col, meta_heads, H, Hkv, -(-N // block))
    return attn_fwd_blocksparse(q, ke, ve, scale, causal, block, rp, col, H, rows=rows)


def attn_bwd_gqa(q, k, v, do, scale: float, causal: bool, block=None, raw_row_ptr=None, raw_col=None,
                 meta_heads: int = 1, o=None, lse=None):
    """dQ [B, H, N, d] and dK, dV [B, Hkv, N, d]: each shared head's gradient is
    the sum over the query heads of its group."""
    q = _as64(q)
    B, H, N, d = q.shape
    Hkv = np.shape(k)[1]
    ke, ve = expand_kv(k, H), expand_kv(v, H)
    if block is None:
        dq, dk, dv = attn_bwd(q, ke, ve, do, scale, causal, o=o, lse=lse)
    else:
        rp, col = expand_lists(raw_row_ptr, raw_col, meta_heads, H, Hkv, -(-N // block))
        dq, dk, dv = attn_bwd_blocksparse(q, ke, ve, do, scale, causal, block, rp, col, H, o=o, lse=lse)
    g = H // Hkv
    return dq, dk.reshape(B, Hkv, g, N, d).sum(axis=2), dv.reshape(B, Hkv, g, N, d).sum(axis=2)
