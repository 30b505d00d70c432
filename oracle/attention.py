"""Plain float64 three-stage softmax attention: the oracle the GPU path is checked against.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module; only the tests, the smoke check and the bench's CPU-baseline leg do.

What it computes, stage by stage, for one (batch, head) and every query row i:

1. scores:  S = scale * Q K^T, with S_ij = -inf where the pair (i, j) is not
   allowed.  The logit scale is an explicit argument ("Exact Blocks, Rings,
   and Sparsity", section 5, defines s_ij = q_i.k_j / sqrt(d); the
   FlashAttention notes, section 1, write S = QK^T with no scale).
2. softmax: m_i = max_j S_ij, e_ij = exp(S_ij - m_i), l_i = sum_j e_ij,
   P = e / l and LSE_i = m_i + ln l_i (FlashAttention notes, section 5.1, for
   m, f, l; "Exact Blocks, Rings, and Sparsity", section 3, for the saved
   log-normaliser).  A row with no allowed key has P = 0 and LSE = -inf.
3. output:  O = P V.

This is the conventional three-kernel pipeline of "Exact Blocks, Rings, and
Sparsity", section 1 (S and P are materialised, here in host memory), in
float64.  The allowed set is built from logical token pairs, never from
compressed block metadata ("block-sparse attention patterns", final
section): causal keeps j <= i; the block-sparse pattern keeps j when its key
block floor(j/b) is in the set of key blocks listed for the query block
floor(i/b), so a repeated entry counts once and list order does not matter.
Pairs with i >= N or j >= N do not exist.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# masks from logical token pairs
# ---------------------------------------------------------------------------

def token_mask_dense(N: int, causal: bool, rows: np.ndarray) -> np.ndarray:
    """allowed[r, j] for query rows ``rows`` and keys j in [0, N)."""
    j = np.arange(N)
    allowed = np.ones((len(rows), N), dtype=bool)
    if causal:
        allowed &= j[None, :] <= np.asarray(rows)[:, None]
    return allowed


def _row_block_sets(raw_row_ptr: np.ndarray, raw_col: np.ndarray, meta_head: int, nqb: int,
                    nkb: int) -> list:
    raw_row_ptr = np.asarray(raw_row_ptr, dtype=np.int64)
    raw_col = np.asarray(raw_col, dtype=np.int64)
    sets = []
    for qb in range(nqb):
        r = meta_head * nqb + qb
        entries = raw_col[raw_row_ptr[r]:raw_row_ptr[r + 1]]
        if entries.size and (entries.min() < 0 or entries.max() >= nkb):
            raise ValueError(f"block index out of range [0, {nkb}) in query block {qb}")
        sets.append(set(int(e) for e in entries))
    return sets


def token_mask_block_sparse(N: int, causal: bool, block: int, raw_row_ptr: np.ndarray,
                            raw_col: np.ndarray, meta_head: int, rows: np.ndarray) -> np.ndarray:
    """allowed[r, j]: causal condition AND key block of j listed for the query
    block of row r (set semantics over the raw, uncanonicalised list)."""
    nqb = -(-N // block)
    sets = _row_block_sets(raw_row_ptr, raw_col, meta_head, nqb, nqb)
    rows = np.asarray(rows, dtype=np.int64)
    allowed = token_mask_dense(N, causal, rows)
    listed = np.zeros((nqb, nqb), dtype=bool)      # listed[query block, key block]
    for qb, s in enumerate(sets):
        if s:
            listed[qb, list(s)] = True
    key_block = np.arange(N) // block
    allowed &= listed[rows // block][:, key_block]
    return allowed


# ---------------------------------------------------------------------------
# the three stages
# ---------------------------------------------------------------------------

def scores_stage(q_rows: np.ndarray, k: np.ndarray, scale: float, allowed: np.ndarray) -> np.ndarray:
    """Stage 1: S = scale * Q K^T (float64), -inf where not allowed."""
    s = float(scale) * (q_rows.astype(np.float64) @ k.astype(np.float64).T)
    s[~allowed] = -np.inf
    return s


def softmax_stage(s: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Stage 2: row softmax of S with its log-sum-exp.  Rows whose entries are
    all -inf give P = 0 and LSE = -inf."""
    m = np.max(s, axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 on masked pairs
    ell = e.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(empty[:, None], 0.0, e / np.where(empty, 1.0, ell)[:, None])
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, ell)))
    return p, lse


def output_stage(p: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Stage 3: O = P V (float64)."""
    return p @ v.astype(np.float64)


def attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   allowed: np.ndarray, rows: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """O and LSE of one head for query rows ``rows`` (default: all)."""
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    s = scores_stage(q[rows], k, scale, allowed)
    p, lse = softmax_stage(s)
    return output_stage(p, v), lse


def _as64(t) -> np.ndarray:
    if hasattr(t, "detach"):          # torch tensor: widen its exact values
        import torch
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def _run(q, k, v, scale, rows_per_head, mask_fn, row_chunk):
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, d = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("Q, K, V must share the shape [B, H, N, d]")
    outs, lses = [], []
    for b in range(B):
        for h in range(H):
            rows = rows_per_head(b, h)
            o_h = np.empty((len(rows), d))
            l_h = np.empty(len(rows))
            for c0 in range(0, len(rows), row_chunk):
                r = rows[c0:c0 + row_chunk]
                o_h[c0:c0 + len(r)], l_h[c0:c0 + len(r)] = attention_head(
                    q[b, h], k[b, h], v[b, h], scale, mask_fn(b, h, r), r)
            outs.append(o_h)
            lses.append(l_h)
    return outs, lses


def attn_fwd(q, k, v, scale: float, causal: bool, rows: Optional[Sequence] = None,
             row_chunk: int = 1024):
    """Dense (optionally causal) attention of [B,H,N,d] inputs.

    ``rows``: None for every query row, else a callable (b, h) -> row indices
    or one array used for every head.  Returns (O, LSE): arrays [B,H,N,d] and
    [B,H,N] when every row is computed, else lists (one per (b,h), in b-major
    order) of [len(rows), d] and [len(rows)] arrays.
    """
    B, H, N, d = q.shape
    rows_fn = _rows_fn(rows, N)
    outs, lses = _run(q, k, v, scale, rows_fn, lambda b, h, r: token_mask_dense(N, causal, r), row_chunk)
    return _pack(outs, lses, B, H, N, d, rows)


def attn_fwd_blocksparse(q, k, v, scale: float, causal: bool, block: int, raw_row_ptr, raw_col,
                         meta_heads: int, rows: Optional[Sequence] = None, row_chunk: int = 1024):
    """Block-sparse attention renormalised over the allowed pairs.

    The raw lists hold ``meta_heads * ceil(N/block)`` rows: one list per query
    block, shared by every (b,h) when meta_heads == 1, else one set per head h.
    """
    B, H, N, d = q.shape
    if meta_heads not in (1, H, B * H):
        raise ValueError("meta_heads must be 1, H or B*H")
    rows_fn = _rows_fn(rows, N)
    mask_fn = lambda b, h, r: token_mask_block_sparse(N, causal, block, raw_row_ptr, raw_col,
                                                      meta_index(b, h, H, meta_heads), r)
    outs, lses = _run(q, k, v, scale, rows_fn, mask_fn, row_chunk)
    return _pack(outs, lses, B, H, N, d, rows)


def meta_index(b: int, h: int, H: int, meta_heads: int) -> int:
    """Which pattern (b, h) uses: one for every head (meta_heads 1), one per
    head (H), or one per (batch, head) (B*H, b-major)."""
    if meta_heads == 1:
        return 0
    if meta_heads == H:
        return h
    return b * H + h


def _rows_fn(rows, N):
    if rows is None:
        all_rows = np.arange(N)
        return lambda b, h: all_rows
    if callable(rows):
        return lambda b, h: np.asarray(rows(b, h))
    fixed = np.asarray(rows)
    return lambda b, h: fixed


def _pack(outs, lses, B, H, N, d, rows):
    if rows is not None:
        return outs, lses
    return np.stack(outs).reshape(B, H, N, d), np.stack(lses).reshape(B, H, N)


# ---------------------------------------------------------------------------
# online-softmax state merge (used to check the oracle, not by it)
# ---------------------------------------------------------------------------

def merge_states(m_a, l_a, a_a, m_b, l_b, a_b):
    """Merge two partial softmax states (m, l, A) over disjoint key sets:
    m = max(m_a, m_b), l = e^(m_a-m) l_a + e^(m_b-m) l_b, and A likewise
    (FlashAttention notes, section 5.1; "Exact Blocks, Rings, and Sparsity",
    section 2 merge invariant and section 4 associative merge).  A state with
    m = -inf (no keys) contributes nothing."""
    m_a, l_a, a_a = np.asarray(m_a, float), np.asarray(l_a, float), np.asarray(a_a, float)
    m_b, l_b, a_b = np.asarray(m_b, float), np.asarray(l_b, float), np.asarray(a_b, float)
    m = np.maximum(m_a, m_b)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    wa = np.where(np.isfinite(m_a), np.exp(m_a - m_safe), 0.0)
    wb = np.where(np.isfinite(m_b), np.exp(m_b - m_safe), 0.0)
    l = wa * l_a + wb * l_b
    a = wa[..., None] * a_a + wb[..., None] * a_b
    return m, l, a


# ---------------------------------------------------------------------------
# one ring step: a query block against a key/value block at global positions
# ---------------------------------------------------------------------------

def token_mask_offsets(n_q: int, n_k: int, causal: bool, q_offset: int, k_offset: int) -> np.ndarray:
    """allowed[i, j] for query i at global position q_offset + i and key j at
    global position k_offset + j: every pair, or, when causal, the pairs with
    k_offset + j <= q_offset + i."""
    allowed = np.ones((n_q, n_k), dtype=bool)
    if causal:
        qpos = q_offset + np.arange(n_q)
        kpos = k_offset + np.arange(n_k)
        allowed &= kpos[None, :] <= qpos[:, None]
    return allowed


def attn_fwd_block(q, k, v, scale: float, causal: bool, q_offset: int = 0, k_offset: int = 0):
    """Partial attention of query rows [B,H,Nq,d] against one key/value block
    [B,H,Nk,d] whose tokens sit at global positions k_offset + j ("Exact Blocks,
    Rings, and Sparsity", section 4: device g keeps Q_g and meets one KV block
    per ring step; a causal step masks the pairs in the future).  Returns the
    block's normalised output O_b [B,H,Nq,d] and LSE_b [B,H,Nq] (natural log;
    -inf and O_b = 0 for rows that see no key of the block), the state that
    ``merge_lse`` combines."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    if k.shape != (B, H, n_k, d) or v.shape != k.shape:
        raise ValueError("K and V must be [B, H, Nk, d] with Q's B, H and d")
    allowed = token_mask_offsets(n_q, n_k, causal, q_offset, k_offset)
    o = np.empty((B, H, n_q, d))
    lse = np.empty((B, H, n_q))
    for b in range(B):
        for h in range(H):
            s = scores_stage(q[b, h], k[b, h], scale, allowed)
            p, lse[b, h] = softmax_stage(s)
            o[b, h] = output_stage(p, v[b, h])
    return o, lse


def merge_lse(o_parts, lse_parts):
    """Merge normalised partial outputs over disjoint key sets, given in the
    (O, LSE) form: LSE = log sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s.
    This is the (m, l, A) merge of ``merge_states`` with A_s = l_s O_s and
    LSE_s = m_s + ln l_s ("Exact Blocks, Rings, and Sparsity", sections 2 and
    4).  Parts with LSE = -inf contribute nothing; if every part is empty the
    result is O = 0 and LSE = -inf.  o_parts [S, ..., d], lse_parts [S, ...]."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = np.max(lse_parts, axis=0)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lse_parts - m_safe[None])              # exp(-inf) = 0 for empty parts
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, tot)))
        o = np.where(empty[..., None], 0.0,
                     np.einsum("s...,s...d->...d", w, o_parts) / np.where(empty, 1.0, tot)[..., None])
    return o, lse
