"""CPU checks of the C-ABI library: it loads, exports every function the
header declares, validates arguments before any launch, and its host-side
metadata builder matches the oracle's canonicaliser bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsattn.h")


@pytest.fixture(scope="module")
def m():
    import block_sparse_softmax_attn_amd as m
    m._get_lib()      # loads now: a missing library fails here, loudly
    return m


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(m):
    from block_sparse_softmax_attn_amd import _lib
    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTED)
    raw = ctypes.CDLL(m.LIB_PATH)
    for name in declared:
        assert hasattr(raw, name), f"{name} not exported"


def test_status_strings(m):
    from block_sparse_softmax_attn_amd import _lib
    for code in (0, -1, -2, -3, -4):
        assert m.status_string(code) and m.status_string(code) != "unknown status"
    assert m.status_string(12345) == "unknown status"


FAKE = 1 << 20   # 16-aligned, never dereferenced: every call below fails validation first


@pytest.mark.parametrize("args,expect", [
    (dict(q=0), -1),
    (dict(B=0), -1), (dict(H=-1), -1), (dict(N=0), -1),
    (dict(d=96), -2), (dict(d=256), -2), (dict(dtype=7), -2),
    (dict(scale=0.0), -1), (dict(scale=-1.0), -1), (dict(scale=float("nan")), -1), (dict(scale=float("inf")), -1),
    (dict(causal=2), -1),
    (dict(q=FAKE + 2), -1),
    (dict(N=1 << 31), -1),
    (dict(v=0), -1), (dict(v=FAKE + 8), -1),
])
def test_attn_fwd_rejects_bad_arguments(m, args, expect):
    from block_sparse_softmax_attn_amd._lib import get
    lib = get()
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=16, d=64, dtype=1, scale=0.125, causal=0)
    a.update(args)
    st = lib.attn_fwd(a["q"] or None, a["k"], a["v"] or None, a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                      a["dtype"], ctypes.c_float(a["scale"]), a["causal"], None)
    assert st == expect


@pytest.mark.parametrize("args,expect", [
    (dict(block=32), -2), (dict(block=0), -2),
    (dict(meta_heads=3), -1), (dict(row_ptr=0), -1), (dict(nnz=-1), -1), (dict(nnz=4, col=0), -1),
    (dict(d=80), -2), (dict(v=0), -1), (dict(lse=FAKE + 4), -1),
])
def test_attn_fwd_blocksparse_rejects_bad_arguments(m, args, expect):
    from block_sparse_softmax_attn_amd._lib import get
    lib = get()
    a = dict(d=64, block=128, row_ptr=FAKE, col=FAKE, flags=FAKE, nnz=4, meta_heads=1, v=FAKE, lse=FAKE)
    a.update(args)
    st = lib.attn_fwd_blocksparse(FAKE, FAKE, a["v"] or None, FAKE, a["lse"], 1, 2, 256, a["d"], 1,
                                  ctypes.c_float(0.1), 1, a["block"], a["row_ptr"] or None, a["col"] or None,
                                  a["flags"], a["nnz"], a["meta_heads"], None)
    assert st == expect


def test_prepared_entry_points_reject_bad_arguments(m):
    from block_sparse_softmax_attn_amd._lib import get
    lib = get()
    f = ctypes.c_float(0.125)
    # prepare: fp32 has no V^T form, null v, bad d, small or misaligned V^T buffer
    assert lib.attn_prepare_v(FAKE, 1, 2, 100, 64, 0, FAKE, 1 << 20, None) == -2
    assert lib.attn_prepare_v(None, 1, 2, 100, 64, 1, FAKE, 1 << 20, None) == -1
    assert lib.attn_prepare_v(FAKE, 1, 2, 100, 96, 1, FAKE, 1 << 20, None) == -2
    assert lib.attn_prepare_v(FAKE, 1, 2, 100, 64, 1, FAKE, 100, None) == -3
    assert lib.attn_prepare_v(FAKE, 1, 2, 100, 64, 1, FAKE + 4, 1 << 20, None) == -1
    assert lib.attn_prepare_v(FAKE, 0, 2, 100, 64, 1, FAKE, 1 << 20, None) == -1
    # one transpose grid row per head: B*H above 65535 is refused before the buffer check
    assert lib.attn_prepare_v(FAKE, 2, 32768, 100, 64, 1, FAKE, 100, None) == -2
    assert lib.attn_prepare_v(FAKE, 3, 21845, 100, 64, 1, FAKE, 100, None) == -3
    # prepared forwards: bf16 only, V^T buffer required
    assert lib.attn_fwd_prepared(FAKE, FAKE, FAKE, FAKE, 1, 2, 100, 64, 0, f, 0, FAKE, 1 << 20, None) == -2
    assert lib.attn_fwd_prepared(FAKE, FAKE, FAKE, FAKE, 1, 2, 100, 64, 1, f, 0, None, 1 << 20, None) == -1
    assert lib.attn_fwd_prepared(FAKE, FAKE, FAKE, FAKE, 1, 2, 100, 64, 1, f, 0, FAKE, 64, None) == -3
    assert lib.attn_fwd_prepared(None, FAKE, FAKE, FAKE, 1, 2, 100, 64, 1, f, 0, FAKE, 1 << 20, None) == -1
    assert lib.attn_fwd_blocksparse_prepared(FAKE, FAKE, FAKE, FAKE, 1, 2, 100, 64, 1, f, 1, 32, FAKE, FAKE, FAKE,
                                             4, 1, FAKE, 1 << 20, None) == -2
    assert lib.attn_fwd_blocksparse_prepared(FAKE, FAKE, FAKE, FAKE, 1, 2, 100, 64, 1, f, 1, 64, None, FAKE, FAKE,
                                             4, 1, FAKE, 1 << 20, None) == -1


def test_prepared_v_bytes(m):
    from block_sparse_softmax_attn_amd._lib import get
    lib = get()
    assert lib.attn_prepared_v_bytes(1, 32, 8192, 128, 1) == 32 * 128 * 8192 * 2
    assert lib.attn_prepared_v_bytes(1, 16, 16300, 128, 1) == 16 * 128 * 16384 * 2
    assert lib.attn_prepared_v_bytes(2, 3, 1, 64, 1) == 6 * 64 * 128 * 2
    # one long head: dimension rows of V^T start past 2^31 elements (the kernel's offsets are 64-bit)
    assert lib.attn_prepared_v_bytes(1, 1, 20 * 2 ** 20, 128, 1) == 128 * 20 * 2 ** 20 * 2
    assert lib.attn_prepared_v_bytes(1, 1, 256, 64, 0) == -1     # bf16 only
    assert lib.attn_prepared_v_bytes(1, 1, 256, 96, 1) == -1
    assert lib.attn_prepared_v_bytes(0, 1, 256, 64, 1) == -1
    assert m.prepared_v_bytes(1, 2, 300, 128) == 2 * 128 * 384 * 2


def _check_builder(m, rows, meta_heads, N, block, causal):
    rp, col = workloads.lists_to_csr(rows)
    got = m.blockmask_build(rp, col, meta_heads, N, block, causal)
    ref = oracle.canonical_blockmask(rp, col, meta_heads, N, block, causal)
    assert np.array_equal(got.row_ptr, ref["row_ptr"]) and got.row_ptr.dtype == np.int32
    assert np.array_equal(got.col, ref["col"]) and got.col.dtype == np.int32
    assert np.array_equal(got.flags, ref["flags"]) and got.flags.dtype == np.uint8
    assert got.nnz == int(ref["nnz"])
    assert np.array_equal(got.allowed_pairs, ref["allowed_pairs"])
    assert np.array_equal(got.executed_tile_pairs, ref["executed_tile_pairs"])


@pytest.mark.parametrize("causal", [False, True])
def test_builder_matches_oracle_random(m, causal):
    rng = workloads.SplitMix64(101 + causal)
    for _ in range(60):
        block = [1, 3, 8, 64, 128][rng.below(5)]
        N = 1 + rng.below(1500)
        nqb = -(-N // block)
        if nqb > 200:
            continue
        mh = 1 + rng.below(3)
        rows = workloads.random_lists(mh * nqb, nqb, rng, max_len=min(3 * nqb, 40), empty_prob_per_mille=120)
        _check_builder(m, rows, mh, N, block, causal)


def test_builder_matches_oracle_on_sparse_workload(m):
    cfg = workloads.CONFIGS["sparse-causal-h16-n16300-d128"]
    rows = workloads.local_global_random_lists(cfg.N, cfg.block, cfg.seed)
    _check_builder(m, rows, 1, cfg.N, cfg.block, True)
    _check_builder(m, rows, 1, cfg.N, cfg.block, False)


def test_builder_errors(m):
    from block_sparse_softmax_attn_amd import AttnError
    rp, col = workloads.lists_to_csr([[0], [3]])
    with pytest.raises(AttnError) as e:
        m.blockmask_build(rp, col, 1, 16, 8, False)          # block 3 out of range for 2 blocks
    assert e.value.status == -1
    rp, col = workloads.lists_to_csr([[0], [-1]])
    with pytest.raises(AttnError):
        m.blockmask_build(rp, col, 1, 16, 8, False)
    bad_rp = np.array([0, 2, 1], dtype=np.int32)              # decreasing offsets
    with pytest.raises(AttnError):
        m.blockmask_build(bad_rp, np.array([0, 1], np.int32), 1, 16, 8, False)


def test_builder_capacity_error(m):
    from block_sparse_softmax_attn_amd._lib import ATTN_ECAPACITY, get
    lib = get()
    rp, col = workloads.lists_to_csr([[1, 0], [1, 1, 0]])
    out_rp = np.zeros(3, np.int32)
    out_col = np.zeros(2, np.int32)
    out_fl = np.zeros(2, np.uint8)
    nnz = np.zeros(1, np.int64)
    al = np.zeros(1, np.int64)
    ex = np.zeros(1, np.int64)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    st = lib.attn_blockmask_build(p(rp), p(col), 1, 16, 8, 0, p(out_rp), p(out_col), p(out_fl), 2, p(nnz), p(al), p(ex))
    assert st == ATTN_ECAPACITY and nnz[0] == 4 and list(out_rp) == [0, 2, 4] and al[0] == 256 and ex[0] == 4


def test_builder_and_transpose_capacity_sweep(m):
    # every capacity from 0 to nnz + 1 with output arrays of exactly that size:
    # short capacities report ECAPACITY with the full nnz and offsets and write
    # nothing past the arrays (the sanitized build checks the bounds); enough
    # capacity gives the canonical result
    from block_sparse_softmax_attn_amd._lib import ATTN_ECAPACITY, ATTN_OK, get
    lib = get()
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p) if a.size else None
    rng = workloads.SplitMix64(303)
    for trial in range(12):
        block = [1, 8, 64][trial % 3]
        N = 1 + rng.below(400)
        nqb = -(-N // block)
        if nqb > 120:
            continue
        mh = 1 + rng.below(2)
        causal = trial % 2
        rows = workloads.random_lists(mh * nqb, nqb, rng, max_len=min(2 * nqb, 12), empty_prob_per_mille=200)
        rp, col = workloads.lists_to_csr(rows)
        full = m.blockmask_build(rp, col, mh, N, block, bool(causal))
        for cap in range(full.nnz + 2):
            out_rp = np.zeros(mh * nqb + 1, np.int32)
            out_col = np.full(cap, -7, np.int32)
            out_fl = np.full(cap, 0xEE, np.uint8)
            nnz, al, ex = np.zeros(1, np.int64), np.zeros(mh, np.int64), np.zeros(mh, np.int64)
            st = lib.attn_blockmask_build(p(rp), p(col), mh, N, block, causal, p(out_rp), p(out_col), p(out_fl),
                                          cap, p(nnz), p(al), p(ex))
            assert nnz[0] == full.nnz and np.array_equal(out_rp, full.row_ptr)
            if cap < full.nnz:
                assert st == ATTN_ECAPACITY
                assert np.array_equal(out_col, full.col[:cap]) and np.array_equal(out_fl, full.flags[:cap])
            else:
                assert st == ATTN_OK
                assert np.array_equal(out_col[:full.nnz], full.col) and np.all(out_col[full.nnz:] == -7)
            t_rp = np.zeros(mh * nqb + 1, np.int32)
            t_col = np.full(cap, -7, np.int32)
            fr, fc = full.row_ptr.astype(np.int32), full.col.astype(np.int32)
            st = lib.attn_blockmask_transpose(p(fr), p(fc), mh, N, block, p(t_rp), p(t_col), cap)
            assert st == (ATTN_ECAPACITY if cap < full.nnz else ATTN_OK)
            assert t_rp[-1] == full.nnz
            if st == ATTN_OK:
                assert np.all(t_col[full.nnz:] == -7)
            else:
                assert np.all(t_col == -7)


# ---------------------------------------------------------------------------
# backward entry points (argument checks only; no launch without a GPU)
# ---------------------------------------------------------------------------

def test_bwd_workspace_bytes(m):
    from block_sparse_softmax_attn_amd._lib import get
    lib = get()
    # three transposed tensors [BH][d][npad] bf16 + row statistics [BH][npad/64 + 1][128] fp32
    # row statistics only: per head, ceil(N/128)*2 + 1 blocks of 64 rows x (LSE, D) fp32
    assert lib.attn_bwd_workspace_bytes(1, 32, 8192, 128, 1) == 32 * 129 * 512
    assert lib.attn_bwd_workspace_bytes(1, 16, 16300, 128, 1) == 16 * 257 * 512
    assert lib.attn_bwd_workspace_bytes(2, 3, 1, 64, 1) == 6 * 3 * 512
    assert lib.attn_bwd_workspace_bytes(1, 1, 256, 64, 0) == -1          # fp32 backward not provided
    assert lib.attn_bwd_workspace_bytes(1, 1, 256, 96, 1) == -1
    assert lib.attn_bwd_workspace_bytes(1, 0, 256, 64, 1) == -1
    assert m.bwd_workspace_bytes(1, 2, 300, 128) == 2 * 7 * 512


def test_bwd_blocksparse_workspace_bytes_counts_split_slots(m):
    from block_sparse_softmax_attn_amd._lib import get
    lib = get()
    a256 = lambda x: (x + 255) // 256 * 256
    B, H, Hkv, N, d, block = 1, 4, 2, 8192, 128, 128
    nb = N // block
    # key block 0 is listed by every query block (64 entries = 128 tiles of 64
    # queries per query head), the others by one query block each
    lists = [[0, qb] if qb else [0] for qb in range(nb)]
    rp, col = workloads.lists_to_csr(lists)
    mask = m.blockmask_build(rp, col, 1, N, block, False)
    t_rp = np.ascontiguousarray(mask.transposed()[0], dtype=np.int32)
    ptr = t_rp.ctypes.data_as(ctypes.c_void_p)
    base = a256(B * H * (nb * 2 + 1) * 512) + a256(B * Hkv * nb * 8)
    assert lib.attn_bwd_blocksparse_workspace_bytes(B, H, Hkv, N, d, 1, block, None, 1) == base
    # group of 2 query heads: 256 tiles on key block 0 -> min(8, ceil(256 / 32)) = 8 pieces per key/value
    # head; each slot holds fp32 partial dK, dV and one 8-byte entry of the extra-piece list
    slot = 2 * block * d * 4 + 8
    assert lib.attn_bwd_blocksparse_workspace_bytes(B, H, Hkv, N, d, 1, block, ptr, 1) == base + 256 + 2 * 8 * slot
    assert m.bwd_blocksparse_workspace_bytes(B, H, N, d, mask, Hkv=Hkv) == base + 256 + 2 * 8 * slot
    # one query head per key/value head: 128 tiles -> 4 pieces
    assert lib.attn_bwd_blocksparse_workspace_bytes(B, H, H, N, d, 1, block, ptr, 1) == (
        a256(B * H * (nb * 2 + 1) * 512) + a256(B * H * nb * 8) + 256 + 4 * 4 * slot)
    # lists of at most 32 tiles are not split
    short = [[qb] for qb in range(nb)]
    rp2, col2 = workloads.lists_to_csr(short)
    t2 = np.ascontiguousarray(m.blockmask_build(rp2, col2, 1, N, block, False).transposed()[0], dtype=np.int32)
    assert lib.attn_bwd_blocksparse_workspace_bytes(B, H, Hkv, N, d, 1, block, t2.ctypes.data_as(ctypes.c_void_p),
                                                    1) == base
    # a call uses at most 2^18 slots: 64-key blocks that each see 33 query tiles split in 2 pieces;
    # 2^17 of them fill the cap exactly, one more block of them needs more and gets no split at all
    for nkt, slots in ((1 << 17, 1 << 18), ((1 << 17) + 1, 0)):
        t_big = np.arange(0, 33 * nkt + 1, 33, dtype=np.int32)
        n_big = 64 * nkt
        least = lib.attn_bwd_blocksparse_workspace_bytes(1, 1, 1, n_big, 64, 1, 64, None, 1)
        full = lib.attn_bwd_blocksparse_workspace_bytes(1, 1, 1, n_big, 64, 1, 64,
                                                        t_big.ctypes.data_as(ctypes.c_void_p), 1)
        assert full == (least + 256 + slots * (2 * 64 * 64 * 4 + 8) if slots else least)
    # rejected: fp32, block size, meta_heads
    assert lib.attn_bwd_blocksparse_workspace_bytes(B, H, Hkv, N, d, 0, block, None, 1) == -1
    assert lib.attn_bwd_blocksparse_workspace_bytes(B, H, Hkv, N, d, 1, 32, None, 1) == -1
    assert lib.attn_bwd_blocksparse_workspace_bytes(B, H, Hkv, N, d, 1, block, None, 3) == -1


@pytest.mark.parametrize("args,expect", [
    (dict(q=0), -1), (dict(dout=0), -1), (dict(dq=0), -1), (dict(dv=FAKE + 4), -1), (dict(lse=FAKE + 8), -1),
    (dict(B=0), -1), (dict(N=0), -1), (dict(d=96), -2), (dict(dtype=0), -2), (dict(dtype=5), -2),
    (dict(scale=0.0), -1), (dict(scale=float("nan")), -1), (dict(causal=3), -1),
    (dict(ws_bytes=1000), -3), (dict(ws=0), -1), (dict(ws=FAKE + 16), -1),
])
def test_attn_bwd_rejects_bad_arguments(m, args, expect):
    from block_sparse_softmax_attn_amd._lib import get
    lib = get()
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, H=2, N=100, d=64,
             dtype=1, scale=0.125, causal=0, ws=FAKE, ws_bytes=1 << 24)
    a.update(args)
    st = lib.attn_bwd(a["q"] or None, a["k"], a["v"], a["o"], a["lse"], a["dout"] or None, a["dq"] or None,
                      a["dk"], a["dv"], a["B"], a["H"], a["N"], a["d"], a["dtype"], ctypes.c_float(a["scale"]),
                      a["causal"], a["ws"] or None, a["ws_bytes"], None)
    assert st == expect


@pytest.mark.parametrize("args,expect", [
    (dict(block=32), -2), (dict(meta_heads=3), -1), (dict(row_ptr=0), -1), (dict(t_row_ptr=0), -1),
    (dict(t_col=0), -1), (dict(nnz=-2), -1), (dict(ws_bytes=10), -3),
])
def test_attn_bwd_blocksparse_rejects_bad_arguments(m, args, expect):
    from block_sparse_softmax_attn_amd._lib import get
    lib = get()
    a = dict(block=128, row_ptr=FAKE, t_row_ptr=FAKE, t_col=FAKE, nnz=4, meta_heads=1, ws_bytes=1 << 24)
    a.update(args)
    st = lib.attn_bwd_blocksparse(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 256, 64, 1,
                                  ctypes.c_float(0.1), 1, a["block"], a["row_ptr"] or None, FAKE, FAKE, a["nnz"],
                                  a["t_row_ptr"] or None, a["t_col"] or None, a["meta_heads"], FAKE, a["ws_bytes"],
                                  None)
    assert st == expect


def _transpose_brute(row_ptr, col, meta_heads, nb):
    lists = [[] for _ in range(meta_heads * nb)]
    for h in range(meta_heads):
        for qb in range(nb):
            for e in range(row_ptr[h * nb + qb], row_ptr[h * nb + qb + 1]):
                lists[h * nb + int(col[e])].append(qb)
    return workloads.lists_to_csr(lists)


@pytest.mark.parametrize("causal", [False, True])
def test_blockmask_transpose_matches_brute_force(m, causal):
    rng = workloads.SplitMix64(303 + causal)
    for _ in range(40):
        block = [1, 8, 64, 128][rng.below(4)]
        N = 1 + rng.below(3000)
        nb = -(-N // block)
        if nb > 150:
            continue
        mh = 1 + rng.below(3)
        rows = workloads.random_lists(mh * nb, nb, rng, max_len=min(2 * nb, 30), empty_prob_per_mille=150)
        rp, col = workloads.lists_to_csr(rows)
        mask = m.blockmask_build(rp, col, mh, N, block, causal)
        t_rp, t_col = mask.transposed()
        ref_rp, ref_col = _transpose_brute(mask.row_ptr, mask.col, mh, nb)
        assert np.array_equal(t_rp, ref_rp)
        assert np.array_equal(t_col[:mask.nnz], ref_col)
        # every transposed row is strictly increasing (canonical rows are unique)
        for r in range(mh * nb):
            seg = t_col[t_rp[r]:t_rp[r + 1]]
            assert np.all(np.diff(seg) > 0)


def test_blockmask_transpose_errors(m):
    from block_sparse_softmax_attn_amd._lib import ATTN_ECAPACITY, get
    lib = get()
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    rp = np.array([0, 1, 3], np.int32)
    col = np.array([0, 0, 1], np.int32)
    t_rp = np.zeros(3, np.int32)
    t_col = np.zeros(3, np.int32)
    assert lib.attn_blockmask_transpose(p(rp), p(col), 1, 16, 8, p(t_rp), p(t_col), 3) == 0
    assert list(t_rp) == [0, 2, 3] and list(t_col) == [0, 1, 1]
    assert lib.attn_blockmask_transpose(p(rp), p(col), 1, 16, 8, p(t_rp), p(t_col), 2) == ATTN_ECAPACITY
    bad = np.array([0, 1, 3], np.int32), np.array([0, 0, 2], np.int32)   # block 2 of 2 blocks
    assert lib.attn_blockmask_transpose(p(bad[0]), p(bad[1]), 1, 16, 8, p(t_rp), p(t_col), 3) == -1
    assert lib.attn_blockmask_transpose(None, p(col), 1, 16, 8, p(t_rp), p(t_col), 3) == -1


# ---------------------------------------------------------------------------
# key splits, ring steps, merge (argument checks only)
# ---------------------------------------------------------------------------

def test_splitkv_workspace_bytes(m):
    from block_sparse_softmax_attn_amd._lib import get
    lib = get()
    a256 = lambda x: (x + 255) // 256 * 256
    # B1 H4 N8192 d128, 4 splits of 2048 keys: the fp32 partial states
    assert lib.attn_fwd_splitkv_workspace_bytes(1, 4, 8192, 128, 1, 4) == a256(4 * 4 * 8192 * 128 * 4) + a256(4 * 4 * 8192 * 4)
    # N = 100 holds two 64-key tiles: at most two ranges
    assert lib.attn_fwd_splitkv_workspace_bytes(1, 1, 100, 64, 1, 8) == a256(2 * 100 * 64 * 4) + a256(2 * 100 * 4)
    assert lib.attn_fwd_splitkv_workspace_bytes(1, 1, 100, 64, 0, 2) == -1     # bf16 only
    assert lib.attn_fwd_splitkv_workspace_bytes(1, 1, 100, 64, 1, 0) == -1
    assert lib.attn_fwd_splitkv_workspace_bytes(1, 1, 100, 64, 1, 65) == -1
    assert lib.attn_fwd_splitkv_workspace_bytes(1, 1, 100, 96, 1, 2) == -1


def test_split_and_ring_entry_points_reject_bad_arguments(m):
    from block_sparse_softmax_attn_amd._lib import get
    lib = get()
    f = ctypes.c_float(0.1)
    # split-KV: bad splits, fp32, small workspace, misaligned workspace
    assert lib.attn_fwd_splitkv(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 256, 64, 1, f, 0, 0, FAKE, 1 << 24, None) == -1
    assert lib.attn_fwd_splitkv(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 256, 64, 0, f, 0, 2, FAKE, 1 << 24, None) == -2
    assert lib.attn_fwd_splitkv(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 256, 64, 1, f, 0, 2, FAKE, 100, None) == -3
    assert lib.attn_fwd_splitkv(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 256, 64, 1, f, 0, 2, FAKE + 16, 1 << 24, None) == -1
    assert lib.attn_fwd_splitkv(None, FAKE, FAKE, FAKE, FAKE, 1, 2, 256, 64, 1, f, 0, 2, FAKE, 1 << 24, None) == -1
    # ring step: negative offsets, zero keys, fp32, null or misaligned V
    blk = lambda **kw: lib.attn_fwd_block(FAKE, FAKE, kw.get("v", FAKE), FAKE, FAKE, 1, 2, kw.get("nq", 64),
                                          kw.get("nk", 128), 64, kw.get("dt", 1), f, 1, kw.get("qo", 0),
                                          kw.get("ko", 0), None)
    assert blk(qo=-1) == -1 and blk(ko=-5) == -1 and blk(nk=0) == -1 and blk(nq=0) == -1
    assert blk(dt=0) == -2 and blk(v=None) == -1 and blk(v=FAKE + 4) == -1
    # merge: parts, d, dtype, alignment
    mg = lambda **kw: lib.attn_merge(kw.get("op", FAKE), FAKE, kw.get("s", 2), 1, 2, 64, kw.get("d", 64), FAKE, FAKE,
                                     kw.get("dt", 0), None)
    assert mg(s=0) == -1 and mg(s=2000) == -1 and mg(d=96) == -2 and mg(dt=5) == -2
    assert mg(op=None) == -1 and mg(op=FAKE + 4) == -1


# ---------------------------------------------------------------------------
# grouped-query attention (argument checks only)
# ---------------------------------------------------------------------------

def test_gqa_workspace_and_bad_groups(m):
    from block_sparse_softmax_attn_amd._lib import get
    lib = get()
    # statistics per query head
    assert lib.attn_bwd_gqa_workspace_bytes(1, 8, 2, 1024, 128, 1) == 8 * 17 * 512
    assert lib.attn_bwd_gqa_workspace_bytes(1, 8, 8, 1024, 128, 1) == lib.attn_bwd_workspace_bytes(1, 8, 1024, 128, 1)
    assert lib.attn_bwd_gqa_workspace_bytes(1, 8, 3, 1024, 128, 1) == -1
    assert lib.attn_bwd_gqa_workspace_bytes(1, 8, 0, 1024, 128, 1) == -1
    assert lib.attn_bwd_gqa_workspace_bytes(1, 8, 16, 1024, 128, 1) == -1
    f = ctypes.c_float(0.1)
    for hkv in (0, 3, 16):
        assert lib.attn_fwd_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, hkv, 256, 64, 1, f, 0, None) == -1
        assert lib.attn_fwd_blocksparse_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, hkv, 256, 64, 1, f, 0, 128, FAKE,
                                            FAKE, FAKE, 4, 1, None) == -1
        assert lib.attn_bwd_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, hkv, 256, 64, 1, f, 0,
                                FAKE, 1 << 26, None) == -1
    # meta_heads must be 1, Hkv or H
    assert lib.attn_fwd_blocksparse_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 256, 64, 1, f, 0, 128, FAKE, FAKE,
                                        FAKE, 4, 4, None) == -1
    # null V
    assert lib.attn_fwd_gqa(FAKE, FAKE, None, FAKE, FAKE, 1, 8, 2, 256, 64, 1, f, 0, None) == -1


# ---------------------------------------------------------------------------
# mean-pooled selector (argument checks and closed forms only)
# ---------------------------------------------------------------------------

def test_select_nnz_and_workspace(m):
    from block_sparse_softmax_attn_amd._lib import get
    lib = get()
    # non-causal: every row keeps min(topk, nb); causal: row qb keeps min(topk, qb + 1)
    assert lib.attn_select_meanpool_nnz(2, 3, 1000, 64, 0, 4) == 6 * 16 * 4
    assert lib.attn_select_meanpool_nnz(1, 1, 1000, 64, 1, 4) == sum(min(4, qb + 1) for qb in range(16))
    assert lib.attn_select_meanpool_nnz(1, 1, 100, 128, 0, 8) == 1
    assert lib.attn_select_meanpool_nnz(1, 8, 131072, 128, 1, 16) == 8 * sum(min(16, qb + 1) for qb in range(1024))
    assert lib.attn_select_meanpool_nnz(1, 1, 1000, 32, 0, 4) == -1        # block
    assert lib.attn_select_meanpool_nnz(1, 1, 1000, 64, 0, 0) == -1        # topk
    assert lib.attn_select_meanpool_nnz(1, 1, 1000, 64, 0, 65) == -1
    assert lib.attn_select_meanpool_nnz(1, 1, 2049 * 128, 128, 0, 4) == -1  # too many blocks
    assert lib.attn_select_meanpool_workspace_bytes(1, 8, 2, 1000, 128, 64) == (8 + 2) * 16 * 128 * 4
    assert lib.attn_select_meanpool_workspace_bytes(1, 8, 3, 1000, 128, 64) == -1


def test_select_rejects_bad_arguments(m):
    from block_sparse_softmax_attn_amd._lib import get
    lib = get()
    f = ctypes.c_float(0.1)
    call = lambda **kw: lib.attn_select_meanpool(kw.get("q", FAKE), FAKE, 1, 4, kw.get("hkv", 2), 1000, kw.get("d", 64),
                                                 kw.get("dt", 1), ctypes.c_float(kw.get("sc", 0.1)), 1,
                                                 kw.get("blk", 64), kw.get("topk", 4), kw.get("share", 0), FAKE, FAKE,
                                                 FAKE, kw.get("cap", 1 << 20), FAKE, kw.get("ws", 1 << 24), None)
    assert call(q=None) == -1 and call(sc=0.0) == -1 and call(share=2) == -1 and call(hkv=3) == -1
    assert call(d=96) == -2 and call(dt=7) == -2 and call(blk=32) == -2 and call(topk=65) == -2
    assert call(topk=0) == -1
    assert call(cap=10) == -3 and call(ws=100) == -3


def test_select_rejects_an_oversized_pooling_grid(m):
    # one pooling workgroup per (head of Q or K, block): 16 blocks * 6 heads * B >= 2^24
    from block_sparse_softmax_attn_amd._lib import get
    lib = get()
    B = -(-(1 << 24) // 96)
    st = lib.attn_select_meanpool(FAKE, FAKE, B, 4, 2, 1000, 64, 1, ctypes.c_float(0.1), 1, 64, 4, 0, FAKE, FAKE,
                                  FAKE, 1 << 40, FAKE, 1 << 40, None)
    assert st == -2
    st = lib.attn_select_meanpool(FAKE, FAKE, B - 1, 4, 2, 1000, 64, 1, ctypes.c_float(0.1), 1, 64, 4, 0, FAKE, FAKE,
                                  FAKE, 10, FAKE, 1 << 40, None)
    assert st == -3     # just under the limit: only the capacity is short
