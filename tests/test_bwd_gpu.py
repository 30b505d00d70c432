"""GPU parity of the backward: the HIP kernels, called through the C ABI,
against the float64 oracle's gradient on the same seeded inputs.

On every head that is compared, the kernel receives O rounded to bf16 and LSE
rounded to fp32 from the forward ORACLE; the reference is the oracle's
gradient rebuilt from those same O and LSE, and the allowed error per element
is the bound of ``parity_utils.bwd_bounds_head`` (bf16 rounding of P and dS,
fp32 accumulation, bf16 outputs).  Small shapes are compared on every head.
The full-size workloads are compared on every head (c2, c3) or on 8 of the
16 heads (c4); heads are independent, so the other heads take their O and LSE
from the GPU forward (their gradients are not compared).  The per-head oracle work runs on a thread pool (numpy's
BLAS and elementwise loops release the GIL).
"""
from concurrent.futures import ThreadPoolExecutor
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import attention as A
from parity_utils import bwd_bounds_head, compare_grad, inputs, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    import block_sparse_softmax_attn_amd as m
    return m


def _setup(B, H, N, d, seed, fwd, heads=None, gpu_fwd=None, workers=8):
    """Seeded bf16 Q, K, V, dO and the backward's O (bf16) and LSE (fp32) inputs:
    the forward oracle's on every head in ``heads`` (all heads when None),
    the GPU forward's (``gpu_fwd``) on the others."""
    q, k, v = inputs(B, H, N, d, "bf16", seed)
    do = workloads.make_grad(B, H, N, d, seed)
    if heads is None:
        o_ex, lse_ex = fwd(q, k, v)
        return q, k, v, do, torch.from_numpy(o_ex).to(torch.bfloat16), torch.from_numpy(lse_ex).to(torch.float32)
    o_g, lse_g = gpu_fwd(q.cuda(), k.cuda(), v.cuda())
    o_in, lse_in = o_g.cpu(), lse_g.cpu()
    sls = [(slice(b, b + 1), slice(h, h + 1)) for b, h in heads]
    with ThreadPoolExecutor(workers) as ex:
        outs = list(ex.map(lambda sl: fwd(q[sl], k[sl], v[sl]), sls))
    for sl, (o_ex, lse_ex) in zip(sls, outs):
        o_in[sl] = torch.from_numpy(o_ex).to(torch.bfloat16)
        lse_in[sl] = torch.from_numpy(lse_ex).to(torch.float32)
    return q, k, v, do, o_in, lse_in


def _check_heads(grads, q, k, v, do, o_in, lse_in, scale, heads, allowed_for_head, ref_bwd, label, workers=8):
    """Compare GPU (dQ, dK, dV) with the oracle on the listed (b, h) heads."""
    gq, gk, gv = (to64(g) for g in grads)
    q64, k64, v64, do64, o64, l64 = (to64(t) for t in (q, k, v, do, o_in, lse_in))

    def one(bh):
        b, h = bh
        rq, rk, rv = ref_bwd(b, h, q64[b, h], k64[b, h], v64[b, h], do64[b, h], o64[b, h], l64[b, h])
        bq, bk, bv = bwd_bounds_head(q64[b, h], k64[b, h], v64[b, h], do64[b, h], scale, allowed_for_head(b, h),
                                     o64[b, h], l64[b, h])
        worst = 0.0
        for name, got, ref, bd in (("dQ", gq, rq, bq), ("dK", gk, rk, bk), ("dV", gv, rv, bv)):
            _, r = compare_grad(got[b, h], ref, bd, f"{label} ({b},{h}) {name}")
            worst = max(worst, r)
        return worst

    with ThreadPoolExecutor(workers) as ex:
        return max(ex.map(one, heads))


def _dense_ref(N, causal, scale):
    def ref(b, h, q, k, v, do, o, lse):
        return oracle.attention_head_bwd(q, k, v, do, scale, lambda rows: A.token_mask_dense(N, causal, rows),
                                         o=o, lse=lse)
    return ref


def _dense_case(lib, B, H, N, d, causal, seed, heads=None, workers=8):
    scale = float(np.float32(1.0 / math.sqrt(d)))
    fwd = lambda q, k, v: oracle.attn_fwd(q, k, v, scale, causal)
    gpu_fwd = lambda q, k, v: lib.attn_fwd(q, k, v, scale=scale, causal=causal)
    q, k, v, do, o_in, lse_in = _setup(B, H, N, d, seed, fwd, heads, gpu_fwd, workers)
    grads = lib.attn_bwd(*(t.cuda() for t in (q, k, v, o_in, lse_in, do)), scale=scale, causal=causal)
    torch.cuda.synchronize()
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    allowed = lambda b, h: (lambda rows: A.token_mask_dense(N, causal, rows))
    return _check_heads(grads, q, k, v, do, o_in, lse_in, scale, heads, allowed, _dense_ref(N, causal, scale),
                        f"bwd dense B{B} H{H} N{N} d{d} causal={causal}", workers)


SMALL = [(1, 1, 1, 64), (1, 2, 33, 128), (2, 1, 64, 64), (1, 2, 200, 128), (1, 1, 256, 64),
         (2, 2, 300, 128), (1, 1, 577, 128), (1, 2, 1000, 64)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}H{}N{}d{}".format(*s))
def test_bwd_dense_small(lib, shape, causal):
    B, H, N, d = shape
    print(f"case bwd dense {shape} causal={causal}", flush=True)
    _dense_case(lib, B, H, N, d, causal, seed=2000 + N + d + causal)


def _sparse_case(lib, B, H, N, d, block, causal, lists, meta_heads, seed, heads=None, workers=8):
    scale = float(np.float32(1.0 / math.sqrt(d)))
    rp, col = workloads.lists_to_csr(lists)
    fwd = lambda q, k, v: oracle.attn_fwd_blocksparse(q, k, v, scale, causal, block, rp, col, meta_heads)
    mask = lib.blockmask_build(rp, col, meta_heads, N, block, causal)
    gpu_fwd = lambda q, k, v: lib.attn_fwd_blocksparse(q, k, v, mask, scale=scale)
    if heads is not None:
        assert meta_heads == 1, "per-head patterns are compared on every head"
    q, k, v, do, o_in, lse_in = _setup(B, H, N, d, seed, fwd, heads, gpu_fwd, workers)
    grads = lib.attn_bwd_blocksparse(*(t.cuda() for t in (q, k, v, o_in, lse_in, do)), mask, scale=scale)
    torch.cuda.synchronize()
    heads = heads or [(b, h) for b in range(B) for h in range(H)]

    def allowed(b, h):
        mh = 0 if meta_heads == 1 else h
        return lambda rows: A.token_mask_block_sparse(N, causal, block, rp, col, mh, rows)

    def ref(b, h, q_, k_, v_, do_, o_, l_):
        return oracle.attention_head_bwd(q_, k_, v_, do_, scale, allowed(b, h), o=o_, lse=l_)

    worst = _check_heads(grads, q, k, v, do, o_in, lse_in, scale, heads, allowed, ref,
                         f"bwd sparse N{N} d{d} b{block} causal={causal} mh={meta_heads}", workers)
    return grads, worst


SPARSE = [(1, 2, 640, 64, 128), (2, 2, 300, 128, 64), (1, 3, 1000, 128, 128), (1, 1, 129, 64, 64)]


@pytest.mark.parametrize("meta_per_head", [False, True])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SPARSE, ids=lambda s: "B{}H{}N{}d{}b{}".format(*s))
def test_bwd_sparse_random(lib, shape, causal, meta_per_head):
    B, H, N, d, block = shape
    nb = -(-N // block)
    mh = H if meta_per_head else 1
    rng = workloads.SplitMix64(4000 + N + block + 2 * causal + meta_per_head)
    lists = workloads.random_lists(mh * nb, nb, rng, max_len=2 * nb, empty_prob_per_mille=200)
    print(f"case bwd sparse {shape} causal={causal} meta_heads={mh}", flush=True)
    _sparse_case(lib, B, H, N, d, block, causal, lists, mh, seed=4100 + N + d)


def test_bwd_sparse_empty_rows_and_unseen_keys_are_exact_zeros(lib):
    B, H, N, d, block = 1, 2, 512, 128, 128
    # query block 1 empty; key block 2 listed by nobody
    lists = [[0], [], [0, 1], [1, 3, 3]]
    grads, _ = _sparse_case(lib, B, H, N, d, block, True, lists, 1, seed=4200)
    dq, dk, dv = (to64(g) for g in grads)
    assert np.all(dq[:, :, 128:256] == 0)
    assert np.all(dk[:, :, 256:384] == 0) and np.all(dv[:, :, 256:384] == 0)


def test_bwd_identical_value_rows(lib):
    # every dP_ij of a row is the same constant, so the exact dS is zero
    B, H, N, d = 1, 2, 300, 64
    scale = float(np.float32(1.0 / math.sqrt(d)))
    q, k, _ = inputs(B, H, N, d, "bf16", 4300)
    v = q[:, :, :1, :].expand(B, H, N, d).contiguous()
    do = workloads.make_grad(B, H, N, d, 4300)
    o_ex, lse_ex = oracle.attn_fwd(q, k, v, scale, True)
    o_in = torch.from_numpy(o_ex).to(torch.bfloat16)
    lse_in = torch.from_numpy(lse_ex).to(torch.float32)
    grads = lib.attn_bwd(*(t.cuda() for t in (q, k, v, o_in, lse_in, do)), scale=scale, causal=True)
    torch.cuda.synchronize()
    allowed = lambda b, h: (lambda rows: A.token_mask_dense(N, True, rows))
    _check_heads(grads, q, k, v, do, o_in, lse_in, scale, [(0, 0), (0, 1)], allowed, _dense_ref(N, True, scale),
                 "bwd identical V rows")
    assert float(grads[0].abs().max()) < 1e-2 and float(grads[1].abs().max()) < 1e-2


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_all_active_equals_dense_bitwise(lib, causal):
    B, H, N, d = 1, 2, 700, 128
    q, k, v = (t.cuda() for t in inputs(B, H, N, d, "bf16", 4400 + causal))
    do = workloads.make_grad(B, H, N, d, 4400).cuda()
    o, lse = lib.attn_fwd(q, k, v, causal=causal)
    dense = lib.attn_bwd(q, k, v, o, lse, do, causal=causal)
    nb = -(-N // 128)
    rp, col = workloads.lists_to_csr([list(range(nb))] * nb)
    mask = lib.blockmask_build(rp, col, 1, N, 128, causal)
    sparse = lib.attn_bwd_blocksparse(q, k, v, o, lse, do, mask)
    torch.cuda.synchronize()
    for a, b in zip(dense, sparse):
        assert torch.equal(a, b)


def test_bwd_deterministic(lib):
    B, H, N, d = 1, 4, 1100, 128
    q, k, v = (t.cuda() for t in inputs(B, H, N, d, "bf16", 4500))
    do = workloads.make_grad(B, H, N, d, 4500).cuda()
    o, lse = lib.attn_fwd(q, k, v, causal=True)
    a = lib.attn_bwd(q, k, v, o, lse, do, causal=True)
    b = lib.attn_bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_workspace_too_small_is_rejected(lib):
    q, k, v = (t.cuda() for t in inputs(1, 1, 64, 64, "bf16", 4600))
    o, lse = lib.attn_fwd(q, k, v)
    with pytest.raises(ValueError):
        lib.attn_bwd(q, k, v, o, lse, q, workspace=torch.empty(64, dtype=torch.uint8, device="cuda"))


# ---- full-size workloads ----

def test_bwd_causal_b4_h16_n2048_d64(lib):
    # every head
    cfg = workloads.CONFIGS["causal-b4-h16-n2048-d64"]
    print("case bwd causal-b4-h16-n2048-d64 (all heads)", flush=True)
    _dense_case(lib, cfg.B, cfg.H, cfg.N, cfg.d, True, cfg.seed,
                heads=[(b, h) for b in range(cfg.B) for h in range(cfg.H)])


def test_bwd_dense_b1_h32_n8192_d128(lib):
    # every head
    cfg = workloads.CONFIGS["dense-h32-n8192-d128"]
    print("case bwd dense-h32-n8192-d128 (all heads)", flush=True)
    _dense_case(lib, cfg.B, cfg.H, cfg.N, cfg.d, False, cfg.seed, heads=[(0, h) for h in range(cfg.H)])


def _global_column_lists(nb):
    """Every query block lists key block 0 (a globally attended block) and its own block."""
    return [[0, qb] if qb else [0] for qb in range(nb)]


@pytest.mark.parametrize("split", [True, False])
def test_bwd_sparse_long_key_lists_split_or_not(lib, split):
    # key block 0 of 64-key blocks is listed by all 70 query blocks (70 tiles > 32): with the full
    # workspace its dK/dV are summed from 3 pieces, with the minimum workspace in one workgroup
    B, H, N, d, block = 1, 2, 4480, 64, 64
    print(f"case bwd sparse split={split}", flush=True)
    lists = _global_column_lists(N // block)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    rp, col = workloads.lists_to_csr(lists)
    mask = lib.blockmask_build(rp, col, 1, N, block, True)
    fwd = lambda q, k, v: oracle.attn_fwd_blocksparse(q, k, v, scale, True, block, rp, col, 1)
    q, k, v, do, o_in, lse_in = _setup(B, H, N, d, 4800, fwd, [(0, 1)],
                                       lambda q, k, v: lib.attn_fwd_blocksparse(q, k, v, mask, scale=scale))
    full = lib.bwd_blocksparse_workspace_bytes(B, H, N, d, mask)
    least = int(lib._get_lib().attn_bwd_blocksparse_workspace_bytes(B, H, H, N, d, 1, block, None, 1))
    assert full > least
    ws = torch.empty(full if split else least, dtype=torch.uint8, device="cuda")
    grads = lib.attn_bwd_blocksparse(*(t.cuda() for t in (q, k, v, o_in, lse_in, do)), mask, scale=scale,
                                     workspace=ws)
    again = lib.attn_bwd_blocksparse(*(t.cuda() for t in (q, k, v, o_in, lse_in, do)), mask, scale=scale,
                                     workspace=ws)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(grads, again))   # deterministic, split or not
    allowed = lambda b, h: (lambda rows: A.token_mask_block_sparse(N, True, block, rp, col, 0, rows))
    ref = lambda b, h, q_, k_, v_, do_, o_, l_: oracle.attention_head_bwd(q_, k_, v_, do_, scale, allowed(b, h),
                                                                        o=o_, lse=l_)
    _check_heads(grads, q, k, v, do, o_in, lse_in, scale, [(0, 1)], allowed, ref, f"bwd sparse split={split}")


def test_bwd_block_sparse_b1_h16_n16300_d128(lib):
    cfg = workloads.CONFIGS["sparse-causal-h16-n16300-d128"]
    print("case bwd sparse-causal-h16-n16300-d128", flush=True)
    lists = workloads.local_global_random_lists(cfg.N, cfg.block, cfg.seed)
    # 8 of the 16 heads, the first and the last included (~28 s of host work per head)
    _sparse_case(lib, cfg.B, cfg.H, cfg.N, cfg.d, cfg.block, True, lists, 1, cfg.seed,
                 heads=[(0, h) for h in (0, 2, 5, 7, 9, 11, 13, 15)])
