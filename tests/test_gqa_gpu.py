"""GPU parity of grouped-query attention (H query heads sharing Hkv key/value
heads), through the C ABI, against the float64 oracle (oracle.attn_fwd_gqa,
oracle.attn_bwd_gqa).

Forward: the bf16 / fp32 forward tolerances.  Backward: the bound of
``parity_utils.bwd_bounds_head`` per query head; a shared dK or dV head sums
its group's contributions in fp32 before one bf16 rounding, so its allowed
error is the sum of the group's per-head bounds plus u|x|.  Bitwise checks:
the grouped forward equals the plain forward on K and V repeated per query
head (same arithmetic), and Hkv == H equals the plain entry points.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_utils import bwd_bounds_head, compare, compare_grad, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    import block_sparse_softmax_attn_amd as m
    return m


def _inputs(B, H, Hkv, N, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, H, N, d), generator=g)
    k = torch.randn((B, Hkv, N, d), generator=g)
    v = torch.randn((B, Hkv, N, d), generator=g)
    if dtype == "bf16":
        q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    return q.contiguous(), k.contiguous(), v.contiguous()


FWD = [(1, 4, 2, 300, 128), (2, 6, 1, 129, 64), (1, 8, 4, 1000, 128), (1, 4, 1, 64, 64)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", FWD, ids=lambda s: "B{}H{}Hkv{}N{}d{}".format(*s))
def test_gqa_forward(lib, shape, causal, dtype):
    B, H, Hkv, N, d = shape
    print(f"case gqa fwd {shape} causal={causal} {dtype}", flush=True)
    q, k, v = _inputs(B, H, Hkv, N, d, dtype, 7000 + N + H)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = lib.attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd_gqa(q, k, v, scale, causal)
    compare(to64(o).reshape(-1, d), to64(lse).reshape(-1), o_ref.reshape(-1, d), lse_ref.reshape(-1), dtype,
            f"gqa fwd {shape} causal={causal}")


@pytest.mark.parametrize("meta", ["1", "Hkv", "H"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [64, 128])
def test_gqa_sparse_forward(lib, block, causal, meta):
    B, H, Hkv, N, d = 1, 6, 2, 700, 128
    print(f"case gqa sparse b={block} causal={causal} meta={meta}", flush=True)
    nb = -(-N // block)
    mh = {"1": 1, "Hkv": Hkv, "H": H}[meta]
    rng = workloads.SplitMix64(7100 + block + causal)
    rp, col = workloads.lists_to_csr(workloads.random_lists(mh * nb, nb, rng, max_len=2 * nb,
                                                            empty_prob_per_mille=150))
    q, k, v = _inputs(B, H, Hkv, N, d, "bf16", 7100)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    mask = lib.blockmask_build(rp, col, mh, N, block, causal)
    o, lse = lib.attn_fwd_blocksparse(q.cuda(), k.cuda(), v.cuda(), mask, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd_gqa(q, k, v, scale, causal, block, rp, col, mh)
    compare(to64(o).reshape(-1, d), to64(lse).reshape(-1), o_ref.reshape(-1, d), lse_ref.reshape(-1), "bf16",
            f"gqa sparse b={block} causal={causal} meta={meta}")


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_forward_equals_repeated_kv_bitwise(lib, causal):
    B, H, Hkv, N, d = 1, 8, 2, 777, 128
    q, k, v = (t.cuda() for t in _inputs(B, H, Hkv, N, d, "bf16", 7200))
    o, lse = lib.attn_fwd(q, k, v, causal=causal)
    ke = k.repeat_interleave(H // Hkv, dim=1).contiguous()
    ve = v.repeat_interleave(H // Hkv, dim=1).contiguous()
    o2, lse2 = lib.attn_fwd(q, ke, ve, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def _bwd_check(lib, B, H, Hkv, N, d, causal, seed, sparse=None):
    scale = float(np.float32(1.0 / math.sqrt(d)))
    q, k, v = _inputs(B, H, Hkv, N, d, "bf16", seed)
    do = workloads.make_grad(B, H, N, d, seed)
    if sparse is None:
        o_ex, lse_ex = oracle.attn_fwd_gqa(q, k, v, scale, causal)
    else:
        block, rp, col, mh = sparse
        o_ex, lse_ex = oracle.attn_fwd_gqa(q, k, v, scale, causal, block, rp, col, mh)
    o_in = torch.from_numpy(o_ex).to(torch.bfloat16)
    lse_in = torch.from_numpy(lse_ex).to(torch.float32)
    args = [t.cuda() for t in (q, k, v, o_in, lse_in, do)]
    if sparse is None:
        grads = lib.attn_bwd(*args, scale=scale, causal=causal)
        ref = oracle.attn_bwd_gqa(q, k, v, do, scale, causal, o=o_in, lse=lse_in)
    else:
        mask = lib.blockmask_build(rp, col, mh, N, block, causal)
        grads = lib.attn_bwd_blocksparse(*args, mask, scale=scale)
        ref = oracle.attn_bwd_gqa(q, k, v, do, scale, causal, block, rp, col, mh, o=o_in, lse=lse_in)
    torch.cuda.synchronize()
    gq, gk, gv = (to64(g) for g in grads)
    q64, k64, v64, do64, o64, l64 = (to64(t) for t in (q, k, v, do, o_in, lse_in))
    group = H // Hkv
    from oracle import attention as A
    bk = np.zeros_like(k64)
    bv = np.zeros_like(v64)
    for b in range(B):
        for h in range(H):
            j = h // group
            if sparse is None:
                allowed = lambda rows: A.token_mask_dense(N, causal, rows)
            else:
                erp, ecol = oracle.expand_lists(rp, col, mh, H, Hkv, -(-N // block))
                allowed = (lambda hh: (lambda rows: A.token_mask_block_sparse(N, causal, block, erp, ecol, hh,
                                                                               rows)))(h)
            b_q, b_k, b_v = bwd_bounds_head(q64[b, h], k64[b, j], v64[b, j], do64[b, h], scale, allowed,
                                            o64[b, h], l64[b, h])
            compare_grad(gq[b, h], ref[0][b, h], b_q, f"gqa dQ ({b},{h})")
            bk[b, j] += b_k
            bv[b, j] += b_v
    for b in range(B):
        for j in range(Hkv):
            compare_grad(gk[b, j], ref[1][b, j], bk[b, j], f"gqa dK ({b},{j})")
            compare_grad(gv[b, j], ref[2][b, j], bv[b, j], f"gqa dV ({b},{j})")


BWD = [(1, 4, 2, 300, 128), (2, 6, 1, 200, 64), (1, 8, 4, 577, 128)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", BWD, ids=lambda s: "B{}H{}Hkv{}N{}d{}".format(*s))
def test_gqa_backward(lib, shape, causal):
    B, H, Hkv, N, d = shape
    print(f"case gqa bwd {shape} causal={causal}", flush=True)
    _bwd_check(lib, B, H, Hkv, N, d, causal, 7300 + N + H)


@pytest.mark.parametrize("meta", ["Hkv", "H"])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_sparse_backward(lib, causal, meta):
    B, H, Hkv, N, d, block = 1, 4, 2, 640, 128, 128
    print(f"case gqa sparse bwd causal={causal} meta={meta}", flush=True)
    nb = -(-N // block)
    mh = {"Hkv": Hkv, "H": H}[meta]
    rng = workloads.SplitMix64(7400 + causal)
    rp, col = workloads.lists_to_csr(workloads.random_lists(mh * nb, nb, rng, max_len=2 * nb,
                                                            empty_prob_per_mille=150))
    _bwd_check(lib, B, H, Hkv, N, d, causal, 7400, sparse=(block, rp, col, mh))


def test_gqa_sparse_backward_long_key_lists_are_split(lib):
    # key block 0 of 64-key blocks is listed by all 36 query blocks of both query heads of each
    # key/value head: 72 query tiles > 32, so its dK/dV are summed from 3 pieces
    B, H, Hkv, N, d, block = 1, 4, 2, 2304, 64, 64
    print("case gqa sparse bwd split", flush=True)
    nb = N // block
    rp, col = workloads.lists_to_csr([[0, qb] if qb else [0] for qb in range(nb)])
    mask = lib.blockmask_build(rp, col, 1, N, block, True)
    least = int(lib._get_lib().attn_bwd_blocksparse_workspace_bytes(B, H, Hkv, N, d, 1, block, None, 1))
    assert lib.bwd_blocksparse_workspace_bytes(B, H, N, d, mask, Hkv=Hkv) > least
    _bwd_check(lib, B, H, Hkv, N, d, True, 7500, sparse=(block, rp, col, 1))


def test_hkv_equal_h_matches_plain_bitwise(lib):
    B, H, N, d = 1, 4, 300, 128
    q, k, v = (t.cuda() for t in _inputs(B, H, H, N, d, "bf16", 7500))
    do = workloads.make_grad(B, H, N, d, 7500).cuda()
    o, lse = lib.attn_fwd(q, k, v, causal=True)
    ws = torch.empty(lib.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    plain = [torch.empty_like(q) for _ in range(3)]
    st = lib._get_lib().attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                                 plain[0].data_ptr(), plain[1].data_ptr(), plain[2].data_ptr(), B, H, N, d, 1,
                                 ctypes.c_float(1 / math.sqrt(d)), 1, ws.data_ptr(), ws.numel(),
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    grouped = [torch.empty_like(q) for _ in range(3)]
    st = lib._get_lib().attn_bwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                     do.data_ptr(), grouped[0].data_ptr(), grouped[1].data_ptr(), grouped[2].data_ptr(),
                                     B, H, H, N, d, 1, ctypes.c_float(1 / math.sqrt(d)), 1,
                                     ws.data_ptr(), ws.numel(),
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    for a, b in zip(plain, grouped):
        assert torch.equal(a, b)
