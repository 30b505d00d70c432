"""Seeded synthetic workloads shared by the tests, the oracle checks and the bench.

This module only *generates inputs*: tensor shapes, seeded N(0,1) draws, the
block lists of the local/global/random sparse pattern and the sampled query
rows of the long-context case.  It holds none of the attention arithmetic, so
that the CPU oracle and the HIP path can both consume its output without
sharing any code that computes the method.

Random integers come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014), written out here from its
published definition so that the block lists do not depend on a numpy or
torch version.  Gaussian tensors come from a seeded CPU ``torch.Generator``
(or a seeded device generator in the bench) and are rounded to bf16 with
round-to-nearest-even by ``Tensor.to``.

Block-pattern vocabulary follows "block-sparse attention patterns"
(study.greatitself.com, "Count active blocks and acknowledge the changed
operator"): patterns combine local, global and random block connections, may
hold duplicate entries, unordered entries and empty rows, and the realised
pattern is kept so a numerical test can be reproduced.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

MASK64 = (1 << 64) - 1


class SplitMix64:
    """SplitMix64 generator: a Weyl sequence with step 0x9E3779B97F4A7C15 and
    the 'variant 13' 64-bit finaliser (shifts 30/27/31)."""

    def __init__(self, seed: int):
        self.state = seed & MASK64

    def next_u64(self) -> int:
        self.state = (self.state + 0x9E3779B97F4A7C15) & MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        return z ^ (z >> 31)

    def below(self, n: int) -> int:
        """Integer in [0, n) as next_u64() mod n (n >= 1)."""
        if n <= 0:
            raise ValueError("below(n) needs n >= 1")
        return self.next_u64() % n


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f32" or "bf16"
    causal: bool
    sparse: bool
    block: int          # block size b of the sparse pattern (0 when dense)
    seed: int
    sample_rows: int    # 0: every query row is checked; else rows sampled per head
    description: str

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))


CONFIGS: Dict[str, Config] = {
    "dense-f32-h1-n256-d64": Config("dense-f32-h1-n256-d64", 1, 1, 256, 64, "f32", False, False, 0, 1, 0,
                 "dense non-causal, B=1 H=1 N=256 d=64, fp32"),
    "causal-b4-h16-n2048-d64": Config("causal-b4-h16-n2048-d64", 4, 16, 2048, 64, "bf16", True, False, 0, 2, 0,
                 "causal, B=4 H=16 N=2048 d=64, bf16"),
    "dense-h32-n8192-d128": Config("dense-h32-n8192-d128", 1, 32, 8192, 128, "bf16", False, False, 0, 3, 0,
                 "dense non-causal, B=1 H=32 N=8192 d=128, bf16"),
    "sparse-causal-h16-n16300-d128": Config("sparse-causal-h16-n16300-d128", 1, 16, 16300, 128, "bf16", True, True, 128, 4, 0,
                 "block-sparse causal, B=1 H=16 N=16300 d=128, b=128, bf16, "
                 "local band 4 + 2 global + 2 random earlier blocks, duplicates, empty rows"),
    "causal-h8-n131072-d128": Config("causal-h8-n131072-d128", 1, 8, 131072, 128, "bf16", True, False, 0, 5, 1024,
                 "causal long context, B=1 H=8 N=131072 d=128, bf16, 1024 sampled rows per head"),
}


def make_qkv(B: int, H: int, N: int, d: int, dtype: str, seed: int, device: str = "cpu"):
    """Q, K, V as torch tensors [B,H,N,d]: fp32 N(0,1) drawn in Q, K, V order
    from a generator seeded with ``seed``, then rounded to bf16 when asked."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = []
    for _ in range(3):
        t = torch.randn((B, H, N, d), generator=gen, dtype=torch.float32, device=device)
        if dtype == "bf16":
            t = t.to(torch.bfloat16)
        elif dtype != "f32":
            raise ValueError(f"unknown dtype {dtype}")
        out.append(t.contiguous())
    return tuple(out)


def make_grad(B: int, H: int, N: int, d: int, seed: int, device: str = "cpu"):
    """Upstream gradient dO [B,H,N,d] bf16: fp32 N(0,1) from a generator seeded
    with ``seed + 7919`` (independent of the Q, K, V draw), rounded to bf16."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 7919)
    return torch.randn((B, H, N, d), generator=gen, dtype=torch.float32, device=device).to(torch.bfloat16).contiguous()


def local_global_random_lists(N: int, block: int, seed: int, band: int = 4, n_global: int = 2,
                              n_random: int = 2, n_empty: int = 4) -> List[List[int]]:
    """Raw per-query-block key-block lists of the local/global/random pattern.

    For query block qb, in this order: the band qb, qb-1, ..., qb-band+1 (kept
    when >= 0, so the list is not sorted); the global blocks 0..n_global-1;
    n_random draws with replacement from [0, qb) (none when qb == 0); then one
    duplicate of the diagonal entry qb.  Finally ``n_empty`` distinct query
    blocks, never the last one (which holds the partial block), get an empty
    list.  Entries may name future blocks (the global ones for qb < n_global);
    a causal consumer must drop them.
    """
    nqb = -(-N // block)
    rng = SplitMix64(seed)
    rows: List[List[int]] = []
    for qb in range(nqb):
        r = [qb - t for t in range(band) if qb - t >= 0]
        r += [g for g in range(n_global) if g < nqb]
        if qb > 0:
            r += [rng.below(qb) for _ in range(n_random)]
        r.append(qb)
        rows.append(r)
    if nqb > 1:
        empties = set()
        while len(empties) < min(n_empty, nqb - 1):
            empties.add(rng.below(nqb - 1))
        for e in sorted(empties):
            rows[e] = []
    return rows


def lists_to_csr(rows: List[List[int]]) -> Tuple[np.ndarray, np.ndarray]:
    """Concatenate per-row lists into (row_ptr int32 [len+1], col int32)."""
    row_ptr = np.zeros(len(rows) + 1, dtype=np.int32)
    for i, r in enumerate(rows):
        row_ptr[i + 1] = row_ptr[i] + len(r)
    col = np.array([c for r in rows for c in r], dtype=np.int32)
    return row_ptr, col


def random_lists(nqb: int, nkb: int, rng: SplitMix64, max_len: int, empty_prob_per_mille: int = 100
                 ) -> List[List[int]]:
    """Arbitrary raw lists for property tests: random length in [0, max_len],
    entries uniform in [0, nkb) with repeats, some rows forced empty."""
    rows = []
    for _ in range(nqb):
        if rng.below(1000) < empty_prob_per_mille:
            rows.append([])
            continue
        n = rng.below(max_len + 1)
        rows.append([rng.below(nkb) for _ in range(n)])
    return rows


def sample_rows(N: int, n: int, seed: int) -> np.ndarray:
    """Sorted sample of query rows: {0, 127, 128, N-1} (those < N) plus
    distinct rows drawn uniformly without replacement from the rest, up to n."""
    fixed = sorted({r for r in (0, 127, 128, N - 1) if 0 <= r < N})
    chosen = set(fixed)
    target = min(n, N)
    rng = SplitMix64(seed)
    while len(chosen) < target:
        chosen.add(rng.below(N))
    return np.array(sorted(chosen), dtype=np.int64)


def config_rows(cfg: Config, h: int) -> Optional[np.ndarray]:
    """Query rows checked for head h of a sampled config (None: every row)."""
    if cfg.sample_rows == 0:
        return None
    return sample_rows(cfg.N, cfg.sample_rows, cfg.seed * 1000 + h)


def config_block_lists(cfg: Config) -> Tuple[np.ndarray, np.ndarray]:
    """Raw CSR (shared by every (b,h), i.e. meta_heads == 1) of a sparse config."""
    if not cfg.sparse:
        raise ValueError(f"{cfg.name} is not block-sparse")
    return lists_to_csr(local_global_random_lists(cfg.N, cfg.block, cfg.seed))
