"""GPU checks of the mean-pooled block selector against the float64 oracle.

Several selections can be correct where two blocks' scores are closer than
the fp32 scoring error, so the test checks what is unique and that the rest is
valid: every row holds min(topk, candidates) ascending entries of causal
candidates, and no chosen block scores (in float64) below an unchosen one by
more than the allowed fp32 error.  The allowed error of a tile score is
2^-14 * scale * sum_c mean|q_c| mean|k_c| (block means summed in fp32 over at
most 128 rows, a d-term fp32 dot product).  row_ptr follows the closed form,
flags equal the host builder's for the same lists, bit for bit.  End to end:
on inputs whose oracle ranking has a clear gap at the top-k boundary the GPU
selection equals the oracle's exactly, and the block-sparse forward on the
GPU's metadata matches the oracle's attention on the oracle's own lists.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_utils import compare, to64

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
    if dtype == "bf16":
        q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    return q.contiguous(), k.contiguous()


def _eps(q64, k64, scale, block, group):
    """Allowed fp32 error of every tile score [B, H, nb, nb]."""
    aq = oracle.block_means(np.abs(q64), block)
    ak = np.repeat(oracle.block_means(np.abs(k64), block), group, axis=1)
    return 2.0 ** -14 * scale * np.einsum("bhad,bhcd->bhac", aq, ak) + 1e-7


def _check_selection(mask, q64, k64, scale, block, causal, topk, share, heads=None):
    B, H, N, _ = q64.shape
    Hkv = k64.shape[1]
    nb = -(-N // block)
    scores = oracle.meanpool_scores(q64, k64, scale, block, causal, share)
    eps = _eps(q64, k64, scale, block, H // Hkv)
    rp = mask._dev[0].cpu().numpy().astype(np.int64)
    col = mask._dev[1].cpu().numpy().astype(np.int64)
    fl = mask._dev[2].cpu().numpy()
    # row_ptr: closed form
    lens = [min(topk, (qb + 1) if causal else nb) for qb in range(nb)]
    expect = np.concatenate([[0], np.cumsum(np.tile(lens, B * H))])
    assert np.array_equal(rp, expect)
    # flags: bit for bit the host builder's
    host = mask.host()
    assert np.array_equal(host.col, col) and np.array_equal(host.flags, fl)
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in heads:
        for qb in range(nb):
            r = (b * H + h) * nb + qb
            chosen = list(col[rp[r]:rp[r + 1]])
            cand = list(range(qb + 1)) if causal else list(range(nb))
            assert chosen == sorted(set(chosen)) and set(chosen) <= set(cand)
            assert len(chosen) == min(topk, len(cand))
            rest = [c for c in cand if c not in chosen]
            if rest:
                s = scores[b, h, qb]
                e = 2 * eps[b, h, qb].max()
                worst_in = min(s[c] for c in chosen)
                best_out = max(s[c] for c in rest)
                assert worst_in >= best_out - e, (b, h, qb, worst_in, best_out, e)
    if share:
        g = H // Hkv
        lists = [list(col[rp[r]:rp[r + 1]]) for r in range(B * H * nb)]
        for b in range(B):
            for h in range(H):
                base = (b * H + (h // g) * g) * nb
                assert lists[(b * H + h) * nb:(b * H + h + 1) * nb] == lists[base:base + nb]


CASES = [(2, 4, 2, 1000, 64, 64, 4), (1, 4, 4, 3000, 128, 128, 8), (1, 2, 1, 777, 128, 64, 1)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("share", [False, True])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}Hkv{}N{}d{}b{}k{}".format(*c))
def test_selection_is_valid(lib, case, causal, share, dtype):
    B, H, Hkv, N, d, block, topk = case
    print(f"case select {case} causal={causal} share={share} {dtype}", flush=True)
    q, k = _inputs(B, H, Hkv, N, d, dtype, 8000 + N + d)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    mask = lib.select_meanpool(q.cuda(), k.cuda(), block, topk, causal=causal, scale=scale, share_groups=share)
    torch.cuda.synchronize()
    _check_selection(mask, to64(q), to64(k), scale, block, causal, topk, share)


def test_selection_long_context(lib):
    # B1 H8 N131072 d128 causal, 1024 key blocks of 128, 16 kept per query block
    B, H, N, d, block, topk = 1, 8, 131072, 128, 128, 16
    print("case select long context", flush=True)
    q, k = _inputs(B, H, H, N, d, "bf16", 8100)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    mask = lib.select_meanpool(q.cuda(), k.cuda(), block, topk, causal=True, scale=scale)
    torch.cuda.synchronize()
    _check_selection(mask, to64(q), to64(k), scale, block, True, topk, False, heads=[(0, 0), (0, 7)])


def test_selection_then_sparse_attention_end_to_end(lib):
    B, H, N, d, block, topk = 1, 2, 2048, 128, 128, 4
    q, k = _inputs(B, H, H, N, d, "bf16", 8200)
    g = torch.Generator().manual_seed(8201)
    v = torch.randn((B, H, N, d), generator=g).to(torch.bfloat16)
    # give every key block a distinct offset so the ranking has clear gaps
    off = torch.linspace(-2, 2, N // block).repeat_interleave(block)[None, None, :, None]
    k = (k.float() + off * torch.ones(d) / math.sqrt(d)).to(torch.bfloat16).contiguous()
    q = (q.float() + 1.0).to(torch.bfloat16).contiguous()
    scale = float(np.float32(1.0 / math.sqrt(d)))
    q64, k64 = to64(q), to64(k)
    scores = oracle.meanpool_scores(q64, k64, scale, block, True)
    eps = _eps(q64, k64, scale, block, 1)
    nb = N // block
    for h in range(H):
        for qb in range(nb):
            s = np.sort(scores[0, h, qb][np.isfinite(scores[0, h, qb])])[::-1]
            if len(s) > topk:
                assert s[topk - 1] - s[topk] > 4 * eps[0, h, qb].max()   # no near tie at the boundary
    rp, col = oracle.meanpool_select(q64, k64, scale, block, True, topk)
    mask = lib.select_meanpool(q.cuda(), k.cuda(), block, topk, causal=True, scale=scale)
    o, lse = lib.attn_fwd_blocksparse(q.cuda(), k.cuda(), v.cuda(), mask, scale=scale)
    torch.cuda.synchronize()
    assert np.array_equal(mask._dev[1].cpu().numpy(), col)
    assert np.array_equal(mask._dev[0].cpu().numpy(), rp)
    o_ref, lse_ref = oracle.attn_fwd_blocksparse(q, k, v, scale, True, block, rp, col, B * H)
    compare(to64(o).reshape(-1, d), to64(lse).reshape(-1), o_ref.reshape(-1, d), lse_ref.reshape(-1), "bf16",
            "selector + sparse forward")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nb,topk,share", [(40, 15, False), (40, 15, True), (1100, 64, False)],
                         ids=["nb40-k15", "nb40-k15-shared", "nb1100-k64"])
def test_exact_ties_go_to_the_lower_index(lib, nb, topk, share, causal):
    # Every key block is a bitwise copy of one of four patterns whose mean
    # logits sit far apart, so scores tie exactly inside a pattern's class and
    # the top-k boundary falls inside a class: the selection is then fixed by
    # the tie rule alone (lower block index first) and must equal the oracle's.
    block, d = 64, 64
    H, Hkv = (2, 1) if share else (1, 1)
    N = nb * block
    print(f"case select ties nb={nb} topk={topk} share={share} causal={causal}", flush=True)
    g = torch.Generator().manual_seed(8300 + nb)
    alpha = torch.tensor([2.0, 1.0, 0.0, -1.0])
    pat = 0.5 * torch.randn((4, block, d), generator=g) + alpha[:, None, None]
    cls = (torch.arange(nb) * 7) % 4          # classes interleaved over the 64-block slices
    k = pat[cls].reshape(1, 1, N, d).repeat(1, Hkv, 1, 1).to(torch.bfloat16).contiguous()
    q = (torch.randn((1, H, N, d), generator=g) + 1.0).to(torch.bfloat16).contiguous()
    scale = float(np.float32(1.0 / math.sqrt(d)))
    rp, col = oracle.meanpool_select(to64(q), to64(k), scale, block, causal, topk, share)
    mask = lib.select_meanpool(q.cuda(), k.cuda(), block, topk, causal=causal, scale=scale, share_groups=share)
    torch.cuda.synchronize()
    assert np.array_equal(mask._dev[0].cpu().numpy(), rp)
    assert np.array_equal(mask._dev[1].cpu().numpy(), col)
