"""Mean-pooled block selector in the oracle (test infrastructure only).

TEST INFRASTRUCTURE ONLY: nothing on the product path imports this module.

Source: "Exact Blocks, Rings, and Sparsity", section 5, "Fixed pooling: a cheap
proxy, not the true block mass".  A key block b is summarised by the mean of
its keys; the mean logit of query i over block b is then
    s_bar(i, b) = (1 / |B_b|) sum_{j in B_b} scale q_i . k_j = scale q_i . k_bar_b,
and ranking blocks by s_bar approximates ranking by the exact block mass
log sum_{j in B_b} exp(s_ij) = s_bar + log|B_b| + (a term that vanishes when
the logits inside the block are equal).  The kernel's unit is a query tile, so
the score of (query block a, key block b) is the mean of s_bar over the rows
of a, which by linearity is scale q_bar_a . k_bar_b: the mean logit of the
whole tile.  Readings (the pages' formulas were lost in extraction):
* means run over the tokens a block actually holds (the last block of a
  sequence whose length is not a multiple of b holds fewer);
* candidates of query block a: every key block, or, when causal, the blocks
  kb <= a (a later block holds no allowed pair);
* C_a = the topk candidates with the largest score, ties to the lower block
  index; fewer candidates than topk keep them all; the list is sorted
  ascending (the canonical order);
* with grouped-query attention and shared selection, the scores of the query
  heads of a group are averaged and every head of the group gets the same
  list, so the group loads one set of K/V blocks (section 5, GQA remark).
"""
from __future__ import annotations

import numpy as np

from .attention import _as64


def block_means(x, block: int) -> np.ndarray:
    """[..., N, d] -> [..., ceil(N/block), d]: the mean of each block's rows."""
    x = _as64(x)
    N = x.shape[-2]
    nb = -(-N // block)
    out = np.empty(x.shape[:-2] + (nb, x.shape[-1]))
    for b in range(nb):
        out[..., b, :] = x[..., b * block:min(N, (b + 1) * block), :].mean(axis=-2)
    return out


def meanpool_scores(q, k, scale: float, block: int, causal: bool, share_groups: bool = False) -> np.ndarray:
    """Scores [B, H, nb, nb] (query block, key block): scale * q_bar . k_bar,
    -inf for non-candidates (kb > qb when causal).  k may have fewer heads than
    q (grouped-query attention); with share_groups the scores are averaged over
    each group's query heads."""
    qm = block_means(q, block)                      # [B, H, nb, d]
    km = block_means(k, block)                      # [B, Hkv, nb, d]
    B, H, nb, _ = qm.shape
    Hkv = km.shape[1]
    g = H // Hkv
    s = float(scale) * np.einsum("bhad,bhcd->bhac", qm, np.repeat(km, g, axis=1))
    if share_groups:
        s = np.repeat(s.reshape(B, Hkv, g, nb, nb).mean(axis=2), g, axis=1)
    if causal:
        s = np.where(np.tril(np.ones((nb, nb), dtype=bool))[None, None], s, -np.inf)
    return s


def select_topk(scores: np.ndarray, topk: int):
    """Per row of scores [..., nb]: the indices of the topk largest finite
    entries, ties to the lower index, sorted ascending."""
    flat = scores.reshape(-1, scores.shape[-1])
    out = []
    for row in flat:
        cand = [j for j in range(row.size) if np.isfinite(row[j])]
        cand.sort(key=lambda j: (-row[j], j))
        out.append(sorted(cand[:topk]))
    return out


def meanpool_select(q, k, scale: float, block: int, causal: bool, topk: int, share_groups: bool = False):
    """Raw lists (one per (b, h, query block), b-major, as CSR) of the
    mean-pooled top-k selector: (row_ptr, col) with meta_heads = B * H."""
    s = meanpool_scores(q, k, scale, block, causal, share_groups)
    lists = select_topk(s, topk)
    row_ptr = np.zeros(len(lists) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum([len(x) for x in lists])
    col = np.array([j for x in lists for j in x], dtype=np.int64)
    return row_ptr, col
