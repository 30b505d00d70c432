"""Canonical form of block-sparse metadata, and its pair counts (test infrastructure only).

TEST INFRASTRUCTURE ONLY: the product's metadata builder is checked against
this, bit for bit; nothing on the product path imports it.

Definition ("Exact Blocks, Rings, and Sparsity", section 5, "Why the sparse
unit is usually a block": the active key-block set C_a per query tile a;
"block-sparse attention patterns", "Count active blocks and acknowledge the
changed operator"):

* raw input: one list of key-block indices per query block (per meta head),
  possibly unordered, with repeats, empty, and, under causal, naming future
  blocks.  An index outside [0, ceil(N/b)) is an error.
* canonical row qb: sorted(set(raw[qb])), dropping blocks kb > qb when
  causal (no pair of such a tile satisfies j <= i, so it contributes
  nothing); a repeated entry is kept once.
* flags per canonical entry: bit 0 when the tile needs the triangular
  element mask: causal and the b x b tile, padded positions included, holds
  a pair with j > i, which is the diagonal tile kb == qb when b > 1 (a
  lower-triangular block pattern still holds future pairs inside its
  diagonal blocks); bit 1 when the key block is partial (the last block when N % b != 0;
  boundary padding changes the valid pair count).
* allowed_pairs[h]: the number of logical (i, j) pairs, i, j in [0, N),
  allowed by the pattern of meta head h, counted from the token-pair mask.
* executed_tile_pairs[h]: the number of b x b tiles the kernel executes for
  one (batch, head) of meta head h, i.e. canonical entries.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from .attention import token_mask_block_sparse

FLAG_DIAGONAL = 1
FLAG_PARTIAL = 2


def canonical_blockmask(raw_row_ptr, raw_col, meta_heads: int, N: int, block: int, causal: bool,
                        count_chunk: int = 2048) -> Dict[str, np.ndarray]:
    raw_row_ptr = np.asarray(raw_row_ptr, dtype=np.int64)
    raw_col = np.asarray(raw_col, dtype=np.int64)
    nqb = -(-N // block)
    nkb = nqb
    if raw_row_ptr.shape != (meta_heads * nqb + 1,):
        raise ValueError("raw_row_ptr must have meta_heads * ceil(N/b) + 1 entries")
    if raw_row_ptr[0] != 0 or raw_row_ptr[-1] != raw_col.size or np.any(np.diff(raw_row_ptr) < 0):
        raise ValueError("raw_row_ptr must start at 0, be non-decreasing and end at len(raw_col)")
    if raw_col.size and (raw_col.min() < 0 or raw_col.max() >= nkb):
        raise ValueError("block index out of range")
    partial = (N % block) != 0
    row_ptr = [0]
    col, flags = [], []
    executed = np.zeros(meta_heads, dtype=np.int64)
    for h in range(meta_heads):
        for qb in range(nqb):
            r = h * nqb + qb
            entries = sorted({int(c) for c in raw_col[raw_row_ptr[r]:raw_row_ptr[r + 1]]
                              if (not causal) or c <= qb})
            for kb in entries:
                col.append(kb)
                f = 0
                if causal and kb == qb and block > 1:
                    f |= FLAG_DIAGONAL
                if partial and kb == nkb - 1:
                    f |= FLAG_PARTIAL
                flags.append(f)
            executed[h] += len(entries)
            row_ptr.append(len(col))
    allowed = np.zeros(meta_heads, dtype=np.int64)
    for h in range(meta_heads):
        for r0 in range(0, N, count_chunk):
            rows = np.arange(r0, min(N, r0 + count_chunk))
            allowed[h] += np.count_nonzero(
                token_mask_block_sparse(N, causal, block, raw_row_ptr, raw_col, h, rows))
    return {
        "row_ptr": np.asarray(row_ptr, dtype=np.int32),
        "col": np.asarray(col, dtype=np.int32),
        "flags": np.asarray(flags, dtype=np.uint8),
        "nnz": np.int64(len(col)),
        "allowed_pairs": allowed,
        "executed_tile_pairs": executed,
    }
