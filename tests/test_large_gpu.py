"""Tensors past 2^32 bytes: B*H = 8320 heads of N = 2048, d = 128 in bf16, so
each [B, H, N, d] tensor spans 4.36e9 bytes and the last heads start past byte
offset 2^32 (head 4100 past 2^31).  A 32-bit product anywhere in a head, row or
metadata offset would move those heads' reads or writes; the compute is small
(milliseconds).  Inputs are drawn on the GPU; the compared heads are copied to
the host and checked against the float64 oracle: the causal forward, the
block-sparse forward with one shared pattern, and the causal backward (on the
compared heads the backward receives the oracle's O and LSE, as in the other
backward tests)."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A
from parity_utils import bwd_bounds_head, compare, compare_grad, to64

pytestmark = pytest.mark.gpu

B, H, N, D = 1, 8320, 2048, 128
HEADS = [0, 4100, H - 1]


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    import block_sparse_softmax_attn_amd as m
    return m


@pytest.fixture(scope="module")
def big():
    per = B * H * N * D * 2
    assert per > (1 << 32)
    free, _ = torch.cuda.mem_get_info()
    if free < 10 * per:
        pytest.skip(f"needs {10 * per / 1e9:.0f} GB of free GPU memory")
    g = torch.Generator(device="cuda")
    g.manual_seed(9100)
    t = {n: torch.randn((B, H, N, D), generator=g, device="cuda", dtype=torch.bfloat16) for n in ("q", "k", "v", "do")}
    yield t
    t.clear()
    torch.cuda.empty_cache()


def _head(x, h):
    return x[:, h:h + 1].cpu()


def test_causal_forward_past_4_gib(lib, big):
    print(f"case large causal forward B{B} H{H} N{N} d{D}", flush=True)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    o, lse = lib.attn_fwd(big["q"], big["k"], big["v"], scale=scale, causal=True)
    torch.cuda.synchronize()
    for h in HEADS:
        o_ref, lse_ref = oracle.attn_fwd(_head(big["q"], h), _head(big["k"], h), _head(big["v"], h), scale, True)
        compare(to64(_head(o, h)).reshape(-1, D), to64(_head(lse, h)).reshape(-1), o_ref.reshape(-1, D),
                lse_ref.reshape(-1), "bf16", f"large causal forward head {h}")


def test_blocksparse_forward_past_4_gib(lib, big):
    print(f"case large block-sparse forward B{B} H{H} N{N} d{D}", flush=True)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    block, nb = 128, N // 128
    rng = np.random.default_rng(9101)
    lists = [sorted({0, qb, int(rng.integers(0, nb))}) for qb in range(nb)]   # one pattern for every head
    rp = np.concatenate([[0], np.cumsum([len(x) for x in lists])])
    col = np.array([c for x in lists for c in x])
    mask = lib.blockmask_build(rp, col, 1, N, block, True)
    o, lse = lib.attn_fwd_blocksparse(big["q"], big["k"], big["v"], mask, scale=scale)
    torch.cuda.synchronize()
    for h in HEADS:
        o_ref, lse_ref = oracle.attn_fwd_blocksparse(_head(big["q"], h), _head(big["k"], h), _head(big["v"], h),
                                                     scale, True, block, rp, col, 1)
        compare(to64(_head(o, h)).reshape(-1, D), to64(_head(lse, h)).reshape(-1), o_ref.reshape(-1, D),
                lse_ref.reshape(-1), "bf16", f"large block-sparse forward head {h}")


def test_causal_backward_past_4_gib(lib, big):
    print(f"case large causal backward B{B} H{H} N{N} d{D}", flush=True)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    o, lse = lib.attn_fwd(big["q"], big["k"], big["v"], scale=scale, causal=True)
    ref_in = {}
    for h in HEADS:   # the compared heads take the oracle's O (bf16) and LSE (fp32)
        o_ex, lse_ex = oracle.attn_fwd(_head(big["q"], h), _head(big["k"], h), _head(big["v"], h), scale, True)
        o[:, h:h + 1] = torch.from_numpy(o_ex).to(torch.bfloat16).cuda()
        lse[:, h:h + 1] = torch.from_numpy(lse_ex).to(torch.float32).cuda()
        ref_in[h] = (o_ex, lse_ex)
    dq, dk, dv = lib.attn_bwd(big["q"], big["k"], big["v"], o, lse, big["do"], scale=scale, causal=True)
    torch.cuda.synchronize()
    allowed = lambda rows: A.token_mask_dense(N, True, rows)
    for h in HEADS:
        q64, k64, v64, do64 = (to64(_head(big[n], h))[0, 0] for n in ("q", "k", "v", "do"))
        o64 = to64(_head(o, h))[0, 0]
        l64 = to64(_head(lse, h))[0, 0]
        refs = oracle.attention_head_bwd(q64, k64, v64, do64, scale, allowed, o=o64, lse=l64)
        bounds = bwd_bounds_head(q64, k64, v64, do64, scale, allowed, o64, l64)
        for name, got, ref, bd in zip(("dQ", "dK", "dV"), (dq, dk, dv), refs, bounds):
            compare_grad(to64(_head(got, h))[0, 0], ref, bd, f"large causal backward head {h} {name}")
    del o, lse, dq, dk, dv


def test_backward_with_more_heads_than_grid_rows(lib):
    # 70 000 heads: the statistics launch caps its grid rows at 65535 and
    # strides over the heads, so the last heads take the second pass
    Bs, Hs, Ns, Ds = 2, 35000, 64, 64
    print(f"case backward B{Bs} H{Hs} N{Ns} d{Ds}", flush=True)
    scale = float(np.float32(1.0 / math.sqrt(Ds)))
    g = torch.Generator(device="cuda")
    g.manual_seed(9102)
    q, k, v, do = (torch.randn((Bs, Hs, Ns, Ds), generator=g, device="cuda", dtype=torch.bfloat16) for _ in range(4))
    o, lse = lib.attn_fwd(q, k, v, scale=scale, causal=False)
    heads = [(0, 0), (1, 30534), (1, Hs - 1)]   # flat heads 0, 65534, 69999
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        o_ex, lse_ex = oracle.attn_fwd(q[sl].cpu(), k[sl].cpu(), v[sl].cpu(), scale, False)
        o[sl] = torch.from_numpy(o_ex).to(torch.bfloat16).cuda()
        lse[sl] = torch.from_numpy(lse_ex).to(torch.float32).cuda()
    dq, dk, dv = lib.attn_bwd(q, k, v, o, lse, do, scale=scale, causal=False)
    torch.cuda.synchronize()
    allowed = lambda rows: A.token_mask_dense(Ns, False, rows)
    for b, h in heads:
        q64, k64, v64, do64, o64 = (to64(t[b, h]) for t in (q, k, v, do, o))
        l64 = to64(lse[b, h])
        refs = oracle.attention_head_bwd(q64, k64, v64, do64, scale, allowed, o=o64, lse=l64)
        bounds = bwd_bounds_head(q64, k64, v64, do64, scale, allowed, o64, l64)
        for name, got, ref, bd in zip(("dQ", "dK", "dV"), (dq, dk, dv), refs, bounds):
            compare_grad(to64(got[b, h]), ref, bd, f"backward 70000 heads ({b},{h}) {name}")


def test_prepared_v_long_head_past_int32_dimension_offsets(lib):
    """One head of N = 20 971 520 keys, d = 128: in the V^T buffer, dimension
    row c starts at c * npad elements, past 2^31 for c >= 103, so the tile
    loads of the prepared-V forward need 64-bit offsets.  The pattern keeps
    only each query block's own (diagonal) block, so every query block reads
    all 128 V^T rows of its block and its result is the dense causal
    attention of that 128-row slice (checked against the oracle on three
    blocks)."""
    n_big, d, block = 20 * (1 << 20), 128, 128
    assert 103 * n_big > (1 << 31)
    per = n_big * d * 2
    free, _ = torch.cuda.mem_get_info()
    if free < 6 * per + (8 << 30):
        pytest.skip(f"needs {(6 * per + (8 << 30)) / 1e9:.0f} GB of free GPU memory")
    print(f"case prepared V long head N{n_big} d{d}", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(9200)
    q, k, v = (torch.randn((1, 1, n_big, d), generator=g, device="cuda", dtype=torch.bfloat16) for _ in range(3))
    scale = float(np.float32(1.0 / math.sqrt(d)))
    nb = n_big // block
    rp = np.arange(nb + 1, dtype=np.int32)
    col = np.arange(nb, dtype=np.int32)
    mask = lib.blockmask_build(rp, col, 1, n_big, block, True)
    vt = torch.empty(lib.prepared_v_bytes(1, 1, n_big, d), dtype=torch.uint8, device="cuda")
    lib.prepare_v(v, vt)
    o, lse = lib.attn_fwd_blocksparse_prepared(q, k, vt, mask, scale=scale, causal=True)
    torch.cuda.synchronize()
    for b in (0, nb // 2, nb - 1):
        sl = slice(b * block, (b + 1) * block)
        o_ref, lse_ref = oracle.attn_fwd(q[:, :, sl].cpu(), k[:, :, sl].cpu(), v[:, :, sl].cpu(), scale, True)
        compare(to64(o[:, :, sl].cpu()).reshape(-1, d), to64(lse[:, :, sl].cpu()).reshape(-1),
                o_ref.reshape(-1, d), lse_ref.reshape(-1), "bf16", f"prepared V long head, block {b}")
    del q, k, v, vt, o, lse
    torch.cuda.empty_cache()
