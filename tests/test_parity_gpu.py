"""GPU parity: the HIP kernels, called through the C ABI, against the float64
oracle on the same seeded inputs, element by element.

Small shapes are compared in full (several tiles, ragged tails, edge cases);
the five named workloads run at full size in the bench's launch configuration.
All but the 131072-token causal one are compared on every row of every head;
that one on 1024 seeded rows per head (the oracle's cost grows as N^2).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_utils import compare, inputs, per_head, to64

pytestmark = pytest.mark.gpu



@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    import block_sparse_softmax_attn_amd as m
    return m


def _dense_case(lib, B, H, N, d, dtype, causal, seed, scale=None):
    q, k, v = inputs(B, H, N, d, dtype, seed)
    scale = float(np.float32(1.0 / math.sqrt(d))) if scale is None else scale
    o, lse = lib.attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, scale, causal)
    return compare(to64(o), to64(lse), o_ref, lse_ref, dtype, f"dense B{B} H{H} N{N} d{d} {dtype} causal={causal}")


SMALL = [
    (1, 1, 1, 64), (1, 2, 17, 64), (2, 1, 64, 128), (1, 3, 100, 128), (1, 2, 129, 64),
    (2, 2, 300, 128), (1, 1, 1000, 64), (1, 2, 513, 128),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}H{}N{}d{}".format(*s))
def test_dense_small(lib, shape, causal, dtype):
    B, H, N, d = shape
    print(f"case dense {shape} causal={causal} {dtype}", flush=True)
    _dense_case(lib, B, H, N, d, dtype, causal, seed=1000 + N + d + causal)


def test_dense_f32_h1_n256_d64_full(lib):
    cfg = workloads.CONFIGS["dense-f32-h1-n256-d64"]
    print("case dense-f32-h1-n256-d64", flush=True)
    _dense_case(lib, cfg.B, cfg.H, cfg.N, cfg.d, cfg.dtype, cfg.causal, cfg.seed, cfg.scale)


def test_causal_b4_h16_n2048_d64_full(lib):
    cfg = workloads.CONFIGS["causal-b4-h16-n2048-d64"]
    print("case causal-b4-h16-n2048-d64", flush=True)
    _dense_case(lib, cfg.B, cfg.H, cfg.N, cfg.d, cfg.dtype, cfg.causal, cfg.seed, cfg.scale)


@pytest.mark.parametrize("B,H,N", [(1, 8, 12400), (2, 8, 6400)])
def test_causal_folded_schedule_every_row(lib, B, H, N):
    # d = 64 causal launches of 4-wave workgroups with between one and two
    # resident rounds of query tiles (776 and 800 tiles against 768 slots on a
    # 256-CU part) run two query tiles in some workgroups; per XCD the single
    # tiles number 95 (odd) and 92 (even), and N = 12400 leaves a ragged last tile
    d = 64
    print(f"case causal folded B{B} H{H} N{N} d{d}", flush=True)
    q, k, v = inputs(B, H, N, d, "bf16", 4242 + N)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = lib.attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = per_head(lambda q1, k1, v1, b, h: oracle.attn_fwd(q1, k1, v1, scale, True), q, k, v)
    do, dl = compare(to64(o), to64(lse), o_ref, lse_ref, "bf16", f"causal folded B{B} H{H} N{N}")
    print(f"max|dO| {do:.3e} max|dLSE| {dl:.3e}", flush=True)


def _sampled_dense(lib, cfg, rows_per_head=None):
    q, k, v = workloads.make_qkv(cfg.B, cfg.H, cfg.N, cfg.d, cfg.dtype, cfg.seed)
    o, lse = lib.attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=cfg.scale, causal=cfg.causal)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    n = rows_per_head or cfg.sample_rows
    rows_fn = lambda b, h: workloads.sample_rows(cfg.N, n, cfg.seed * 1000 + h)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, cfg.scale, cfg.causal, rows=rows_fn)
    worst = (0.0, 0.0)
    i = 0
    for b in range(cfg.B):
        for h in range(cfg.H):
            r = rows_fn(b, h)
            do, dl = compare(to64(o[b, h, r]), to64(lse[b, h, r]), o_ref[i], lse_ref[i], cfg.dtype,
                             f"{cfg.name} b{b} h{h}")
            worst = (max(worst[0], do), max(worst[1], dl))
            i += 1
    print(f"{cfg.name}: max|dO| {worst[0]:.3e} max|dLSE| {worst[1]:.3e}", flush=True)


def test_dense_h32_n8192_d128_full(lib):
    # every row of every head
    cfg = workloads.CONFIGS["dense-h32-n8192-d128"]
    print("case dense-h32-n8192-d128 (all rows)", flush=True)
    q, k, v = workloads.make_qkv(cfg.B, cfg.H, cfg.N, cfg.d, cfg.dtype, cfg.seed)
    o, lse = lib.attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=cfg.scale, causal=cfg.causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = per_head(lambda q1, k1, v1, b, h: oracle.attn_fwd(q1, k1, v1, cfg.scale, cfg.causal),
                              q, k, v)
    do, dl = compare(to64(o), to64(lse), o_ref, lse_ref, cfg.dtype, cfg.name)
    print(f"{cfg.name}: max|dO| {do:.3e} max|dLSE| {dl:.3e} over {cfg.B * cfg.H * cfg.N} rows", flush=True)


def test_causal_h8_n131072_d128_sampled(lib):
    print("case causal-h8-n131072-d128", flush=True)
    _sampled_dense(lib, workloads.CONFIGS["causal-h8-n131072-d128"])


# ---------------------------------------------------------------------------
# block-sparse
# ---------------------------------------------------------------------------

def _sparse_case(lib, B, H, N, d, dtype, causal, block, rows, meta_heads, seed, sample=None):
    q, k, v = inputs(B, H, N, d, dtype, seed)
    rp, col = workloads.lists_to_csr(rows)
    mask = lib.blockmask_build(rp, col, meta_heads, N, block, causal)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = lib.attn_fwd_blocksparse(q.cuda(), k.cuda(), v.cuda(), mask, scale=scale, causal=causal)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    label = f"sparse B{B} H{H} N{N} d{d} {dtype} causal={causal} b={block} mh={meta_heads}"
    if sample is None:
        o_ref, lse_ref = oracle.attn_fwd_blocksparse(q, k, v, scale, causal, block, rp, col, meta_heads)
        return compare(to64(o), to64(lse), o_ref, lse_ref, dtype, label)
    rows_fn = lambda b, h: sample(h)
    o_ref, lse_ref = oracle.attn_fwd_blocksparse(q, k, v, scale, causal, block, rp, col, meta_heads, rows=rows_fn)
    i = 0
    for b in range(B):
        for h in range(H):
            r = sample(h)
            compare(to64(o[b, h, r]), to64(lse[b, h, r]), o_ref[i], lse_ref[i], dtype, f"{label} b{b} h{h}")
            i += 1


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [64, 128])
@pytest.mark.parametrize("N,d,meta", [(300, 64, 1), (517, 128, 2), (1024, 128, 1), (64, 64, 2)])
def test_sparse_random_lists(lib, N, d, meta, block, causal, dtype):
    B, H = 1, 2
    nqb = -(-N // block)
    rng = workloads.SplitMix64(7 * N + block + causal)
    mh = 1 if meta == 1 else H
    rows = workloads.random_lists(mh * nqb, nqb, rng, max_len=2 * nqb + 1, empty_prob_per_mille=150)
    print(f"case sparse N{N} d{d} b{block} causal={causal} {dtype} mh={mh}", flush=True)
    _sparse_case(lib, B, H, N, d, dtype, causal, block, rows, mh, seed=N + d)


def test_sparse_causal_h16_n16300_d128_full(lib):
    # every row of every head: empty query blocks, the partial last block and
    # every local/global/random block of the pattern
    cfg = workloads.CONFIGS["sparse-causal-h16-n16300-d128"]
    rows = workloads.local_global_random_lists(cfg.N, cfg.block, cfg.seed)
    rp, col = workloads.lists_to_csr(rows)
    print("case sparse-causal-h16-n16300-d128 (all rows)", flush=True)
    q, k, v = workloads.make_qkv(cfg.B, cfg.H, cfg.N, cfg.d, cfg.dtype, cfg.seed)
    mask = lib.blockmask_build(rp, col, 1, cfg.N, cfg.block, cfg.causal)
    o, lse = lib.attn_fwd_blocksparse(q.cuda(), k.cuda(), v.cuda(), mask, scale=cfg.scale, causal=cfg.causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = per_head(
        lambda q1, k1, v1, b, h: oracle.attn_fwd_blocksparse(q1, k1, v1, cfg.scale, cfg.causal, cfg.block,
                                                             rp, col, 1), q, k, v)
    assert any(not r for r in rows) and cfg.N % cfg.block
    do, dl = compare(to64(o), to64(lse), o_ref, lse_ref, cfg.dtype, cfg.name)
    print(f"{cfg.name}: max|dO| {do:.3e} max|dLSE| {dl:.3e} over {cfg.B * cfg.H * cfg.N} rows", flush=True)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_sparse_many_blocks_every_row(lib, d, causal):
    # 2 x 8 heads x 41 query blocks of 128 = 656 > 512 workgroup slots: each
    # workgroup runs a sequence of query blocks (persistent form), the next
    # block's first tile and query rows loaded during the current block's last
    # tile.  One pattern per head, empty blocks, a ragged last block.
    B, H, N, block = 2, 8, 5200, 128
    nqb = -(-N // block)
    rng = workloads.SplitMix64(4000 + d + causal)
    rows = workloads.random_lists(H * nqb, nqb, rng, max_len=6, empty_prob_per_mille=120)
    print(f"case sparse persistent d={d} causal={causal}", flush=True)
    q, k, v = inputs(B, H, N, d, "bf16", 4100 + d)
    rp, col = workloads.lists_to_csr(rows)
    mask = lib.blockmask_build(rp, col, H, N, block, causal)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = lib.attn_fwd_blocksparse(q.cuda(), k.cuda(), v.cuda(), mask, scale=scale, causal=causal)
    torch.cuda.synchronize()
    assert B * H * nqb > 512 and any(not r for r in rows)
    o_ref, lse_ref = per_head(
        lambda q1, k1, v1, b, h: oracle.attn_fwd_blocksparse(q1, k1, v1, scale, causal, block, rp[h * nqb:(h + 1) * nqb + 1] - rp[h * nqb],
                                                             col[rp[h * nqb]:rp[(h + 1) * nqb]], 1), q, k, v)
    compare(to64(o), to64(lse), o_ref, lse_ref, "bf16", f"sparse persistent d={d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block,d", [(128, 128), (64, 64), (64, 128)])
def test_all_active_mask_equals_dense(lib, causal, block, d):
    # Where the block-sparse kernel steps through keys in the dense kernel's 64-key
    # tiles, an all-active mask gives the dense result bit for bit.  64-key blocks
    # at d = 128 step 32 keys at a time (LDS budget), so the running max and the
    # denominator's partial sums are taken over other key sets: the two results
    # then agree up to rounding, and both are checked against the oracle.
    B, H, N = 1, 3, 700
    q, k, v = inputs(B, H, N, d, "bf16", 77)
    nqb = -(-N // block)
    rp, col = workloads.lists_to_csr([list(range(nqb))[::-1] + [0] for _ in range(nqb)])
    mask = lib.blockmask_build(rp, col, 1, N, block, causal)
    o_s, l_s = lib.attn_fwd_blocksparse(q.cuda(), k.cuda(), v.cuda(), mask, causal=causal)
    o_d, l_d = lib.attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal)
    torch.cuda.synchronize()
    if not (block == 64 and d == 128):
        assert torch.equal(o_s, o_d) and torch.equal(l_s, l_d)
        return
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, scale, causal)
    compare(to64(o_s), to64(l_s), o_ref, lse_ref, "bf16", f"all-active b{block} d{d} causal={causal}")
    compare(to64(o_d), to64(l_d), o_ref, lse_ref, "bf16", f"dense d{d} causal={causal}")


def test_shuffled_duplicated_lists_give_identical_output(lib):
    B, H, N, d, block = 1, 2, 640, 128, 128
    nqb = N // block
    q, k, v = (t.cuda() for t in inputs(B, H, N, d, "bf16", 78))
    rng = workloads.SplitMix64(79)
    base = [sorted({rng.below(nqb) for _ in range(3)}) for _ in range(nqb)]
    shuffled = []
    for r in base:
        r2 = r + r[:1]
        r2 = [r2[(i * 7 + 3) % len(r2)] for i in range(len(r2))] if r2 else []
        shuffled.append(r2 + r2[:2])
    outs = []
    for rows in (base, shuffled):
        rp, col = workloads.lists_to_csr(rows)
        mask = lib.blockmask_build(rp, col, 1, N, block, True)
        outs.append(lib.attn_fwd_blocksparse(q, k, v, mask, causal=True))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_run_to_run_bitwise_determinism(lib):
    q, k, v = (t.cuda() for t in inputs(2, 4, 1111, 128, "bf16", 80))
    a = lib.attn_fwd(q, k, v, causal=True)
    b = lib.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_outputs_not_written_past_n(lib):
    """Guard band: O and LSE views inside larger buffers; the canaries after
    the last row must survive."""
    B, H, N, d = 1, 2, 200, 64
    q, k, v = (t.cuda() for t in inputs(B, H, N, d, "bf16", 81))
    big_o = torch.full((B * H * N * d + 4096,), 7.0, device="cuda", dtype=torch.bfloat16)
    big_l = torch.full((B * H * N + 1024,), 7.0, device="cuda", dtype=torch.float32)
    o = big_o[:B * H * N * d].view(B, H, N, d)
    lse = big_l[:B * H * N].view(B, H, N)
    lib.attn_fwd(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(big_o[B * H * N * d:] == 7.0) and torch.all(big_l[B * H * N:] == 7.0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_growing_logits_rescale_every_tile(lib, d, causal):
    # key j = (j + 1) * k0: for queries with q . k0 > 0 the logits grow along the keys, so on
    # most tiles some exponential against the row's current reference value passes 2^64, the
    # tile's sum check fails, and the kernel raises the reference to the tile's max, rescales
    # and recomputes the tile; queries with q . k0 < 0 keep their first tile's reference
    B, H, N = 1, 2, 777
    print(f"case growing logits d={d} causal={causal}", flush=True)
    q, k, v = inputs(B, H, N, d, "bf16", 91 + d)
    growth = torch.arange(1, N + 1, dtype=torch.float32).view(1, 1, N, 1)
    k = (k[:, :, :1, :].float() * growth).to(torch.bfloat16).contiguous()
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = lib.attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, scale, causal)
    # Attention here sits on a few keys of |V| up to ~4, where the fixed 1e-2 bound of the N(0,1)
    # workloads is below bf16 resolution.  Bound per element from the arithmetic: P rounded to
    # bf16 (relative 2^-8 per weight) gives at most 2^-8 sum_j P_ij |V_jc|; O stored in bf16
    # adds half an ulp of |O|; 1e-4 covers the fp32 scores, exponentials and sums.
    q64, k64, v64 = to64(q), to64(k), to64(v)
    logits = scale * np.einsum("bhid,bhjd->bhij", q64, k64)
    if causal:
        logits = np.where(np.tril(np.ones((N, N), dtype=bool)), logits, -np.inf)
    prob = np.exp(logits - lse_ref[..., None])
    half_ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(o_ref), 2.0 ** -126))) - 8)
    bound = 2.0 ** -8 * np.einsum("bhij,bhjc->bhic", prob, np.abs(v64)) + half_ulp + 1e-4
    err = np.abs(to64(o) - o_ref)
    assert np.all(err <= bound), f"max excess {np.max(err - bound):.3e}, max|dO| {err.max():.3e}"
    assert np.max(np.abs(to64(lse) - lse_ref)) <= 1e-3
    # The same rescaling schedule with |V| <= ~1 stays inside the fixed bounds of the N(0,1)
    # workloads (P rounding at most 2^-8 max|V|, half an ulp of |O| <= 2^-9).
    v_small = (v.float() * 0.25).to(torch.bfloat16)
    o2, lse2 = lib.attn_fwd(q.cuda(), k.cuda(), v_small.cuda(), scale=scale, causal=causal)
    torch.cuda.synchronize()
    o2_ref, lse2_ref = oracle.attn_fwd(q, k, v_small, scale, causal)
    assert np.max(np.abs(to64(v_small))) <= 1.5
    assert np.max(np.abs(to64(o2) - o2_ref)) <= 1e-2
    assert np.max(np.abs(to64(lse2) - lse2_ref)) <= 1e-3


def test_single_key_gives_its_value_on_gpu(lib):
    q, k, v = (t.cuda() for t in inputs(2, 3, 1, 128, "bf16", 82))
    o, lse = lib.attn_fwd(q, k, v, causal=False)
    torch.cuda.synchronize()
    assert torch.equal(o, v)
    ref = (q.float() * k.float()).sum(-1) * float(np.float32(1 / math.sqrt(128)))
    assert torch.allclose(lse, ref, atol=1e-3, rtol=0)


def test_causal_row_zero_equals_v0(lib):
    q, k, v = (t.cuda() for t in inputs(1, 4, 333, 64, "bf16", 83))
    o, _ = lib.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :, 0], v[:, :, 0])


def test_prepared_v_path_is_bitwise_equal(lib):
    B, H, N, d = 1, 3, 517, 128
    q, k, v = (t.cuda() for t in inputs(B, H, N, d, "bf16", 84))
    for causal in (False, True):
        ref = lib.attn_fwd(q, k, v, causal=causal)
        ws = lib.prepare_v(v)
        got = lib.attn_fwd_prepared(q, k, ws, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
    # 128-key blocks (64-key tile steps) and 64-key blocks (32-key steps at d = 128)
    for block in (128, 64):
        nqb = -(-N // block)
        rng = workloads.SplitMix64(85 + block)
        rp, col = workloads.lists_to_csr(workloads.random_lists(nqb, nqb, rng, max_len=nqb,
                                                                empty_prob_per_mille=200))
        mask = lib.blockmask_build(rp, col, 1, N, block, True)
        ref = lib.attn_fwd_blocksparse(q, k, v, mask)
        got = lib.attn_fwd_blocksparse_prepared(q, k, lib.prepare_v(v), mask)
        torch.cuda.synchronize()
        assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1]), f"block {block}"


def test_prepared_v_buffer_too_small_is_rejected(lib):
    q, k, v = (t.cuda() for t in inputs(1, 1, 64, 64, "bf16", 86))
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        lib.attn_fwd_prepared(q, k, small)
    with pytest.raises(ValueError):
        lib.prepare_v(v, small)
