"""GPU parity of key splits, ring steps and the partial-state merge, through
the C ABI, against the float64 oracle.

* attn_fwd_splitkv equals the full attention (oracle.attn_fwd) within the bf16
  forward tolerance, for every split count, dense and causal;
* attn_fwd_block (one ring step at global offsets) equals oracle.attn_fwd_block,
  including rows that see no key of the block;
* a whole ring emulated on one GPU (each shard meets every key/value block in
  ring order, merging in place) equals the full attention of its rows;
* attn_merge equals oracle.merge_lse on random fp32 states with empty parts.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_utils import compare, inputs, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    import block_sparse_softmax_attn_amd as m
    return m


SHAPES = [(1, 1, 1, 64), (1, 2, 100, 128), (2, 2, 300, 64), (1, 3, 1000, 128), (1, 1, 4100, 128)]


@pytest.mark.parametrize("splits", [1, 2, 3, 8])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}H{}N{}d{}".format(*s))
def test_splitkv_matches_oracle(lib, shape, causal, splits):
    B, H, N, d = shape
    print(f"case splitkv {shape} causal={causal} splits={splits}", flush=True)
    q, k, v = inputs(B, H, N, d, "bf16", 6000 + N + d)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = lib.attn_fwd_splitkv(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=causal, num_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, scale, causal)
    compare(to64(o), to64(lse), o_ref, lse_ref, "bf16", f"splitkv {shape} causal={causal} splits={splits}")


@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_few_heads_long_sequence(lib, causal):
    # B*H*ceil(N/256) = 128 query tiles: half the GPU without splits
    B, H, N, d = 1, 4, 8192, 128
    print(f"case splitkv B1 H4 N8192 causal={causal}", flush=True)
    q, k, v = inputs(B, H, N, d, "bf16", 6100 + causal)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = lib.attn_fwd_splitkv(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=causal, num_splits=4)
    torch.cuda.synchronize()
    rows = workloads.sample_rows(N, 256, 6100)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, scale, causal, rows=rows)
    o64, l64 = to64(o), to64(lse)
    for h in range(H):
        compare(o64[0, h][rows], l64[0, h][rows], o_ref[h], lse_ref[h], "bf16", f"splitkv long h{h}")


BLOCKS = [  # (Nq, Nk, q_offset, k_offset)
    (64, 64, 0, 0), (100, 300, 500, 0), (257, 130, 0, 200), (300, 300, 300, 0), (33, 500, 1000, 700),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("blk", BLOCKS, ids=lambda b: "q{}k{}qo{}ko{}".format(*b))
@pytest.mark.parametrize("d", [64, 128])
def test_ring_step_matches_oracle(lib, blk, causal, d):
    nq, nk, qo, ko = blk
    B, H = 1, 2
    print(f"case ring step {blk} causal={causal} d={d}", flush=True)
    g = torch.Generator().manual_seed(6200 + nq + nk + d)
    q = torch.randn((B, H, nq, d), generator=g).to(torch.bfloat16)
    k = torch.randn((B, H, nk, d), generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, nk, d), generator=g).to(torch.bfloat16)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = lib.attn_fwd_block(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=causal, q_offset=qo, k_offset=ko)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd_block(q, k, v, scale, causal, qo, ko)
    compare(to64(o).reshape(-1, d), to64(lse).reshape(-1), o_ref.reshape(-1, d), lse_ref.reshape(-1), "bf16",
            f"ring step {blk} causal={causal} d={d}")


@pytest.mark.parametrize("causal", [False, True])
def test_ring_emulated_on_one_gpu(lib, causal):
    # G shards of the sequence; shard g keeps its queries and meets the G
    # key/value blocks in ring order g, g-1, ..., merging each into its state
    B, H, N, d, G = 1, 2, 1024, 128, 4
    print(f"case ring emulation causal={causal}", flush=True)
    q, k, v = inputs(B, H, N, d, "bf16", 6300 + causal)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    scale = float(np.float32(1.0 / math.sqrt(d)))
    n = N // G
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, scale, causal)
    for gdev in range(G):
        rows = slice(gdev * n, (gdev + 1) * n)
        state_o = torch.empty((2, B, H, n, d), dtype=torch.float32, device="cuda")
        state_l = torch.empty((2, B, H, n), dtype=torch.float32, device="cuda")
        for step in range(G):
            j = (gdev - step) % G
            slot = 0 if step == 0 else 1
            lib.attn_fwd_block(qd[:, :, rows].contiguous(), kd[:, :, j * n:(j + 1) * n].contiguous(),
                               vd[:, :, j * n:(j + 1) * n].contiguous(), scale=scale, causal=causal,
                               q_offset=gdev * n, k_offset=j * n, o_part=state_o[slot], lse_part=state_l[slot])
            if step > 0:
                lib.attn_merge(state_o, state_l, out=state_o[0], lse=state_l[0])
        torch.cuda.synchronize()
        compare(to64(state_o[0]).reshape(-1, d), to64(state_l[0]).reshape(-1),
                o_ref[:, :, rows].reshape(-1, d), lse_ref[:, :, rows].reshape(-1), "bf16",
                f"ring shard {gdev} causal={causal}")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("S,d", [(1, 64), (2, 128), (5, 64), (9, 128)])
def test_merge_matches_oracle(lib, S, d, out_dtype):
    B, H, N = 2, 3, 77
    rng = np.random.default_rng(6400 + S + d)
    o_parts = rng.standard_normal((S, B, H, N, d)).astype(np.float32)
    lse_parts = (rng.standard_normal((S, B, H, N)) * 5).astype(np.float32)
    lse_parts[rng.random((S, B, H, N)) < 0.3] = -np.inf       # empty parts
    lse_parts[:, 0, 0, :5] = -np.inf                           # rows with no keys at all
    o_parts[np.isneginf(lse_parts)] = 0.0
    o, lse = lib.attn_merge(torch.from_numpy(o_parts).cuda(), torch.from_numpy(lse_parts).cuda(), out_dtype=out_dtype)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.merge_lse(o_parts.astype(np.float64), lse_parts.astype(np.float64))
    tol_o = 1e-5 if out_dtype == torch.float32 else 1e-2
    compare(to64(o).reshape(-1, d), to64(lse).reshape(-1), o_ref.reshape(-1, d), lse_ref.reshape(-1),
            "f32" if out_dtype == torch.float32 else "bf16", f"merge S={S} d={d}")
    assert np.max(np.abs(to64(o) - o_ref)) <= tol_o
