"""Pins for the float64 CPU oracle of the attention gradient.

What fixes the gradient independently of the oracle's own formulas:
* central finite differences of the forward oracle (itself pinned in
  test_oracle.py) on tiny inputs, for dense, causal and block-sparse masks
  with empty rows and a partial block;
* PyTorch's float64 autograd through scaled_dot_product_attention with the
  same boolean mask (a library special case, rows with at least one key);
* closed forms: identical value rows give dQ = dK = 0 (every dP_ij of a row is
  the same constant, the example of "Exact Blocks, Rings, and Sparsity",
  section 3); identical keys give dQ = 0 and dV_j = sum over the rows that see
  j of dO_i / n_i; a single key gives dV = dO and dQ = dK = 0;
* invariants: sum_j dK_j = 0, sum_j dV_j = sum of dO over non-empty rows,
  empty rows get dQ = 0, keys no row sees get dK = dV = 0, and
  D_i = dO_i . O_i = sum_j P_ij dP_ij.
``test_planted_mistakes_are_caught`` checks that plausible mistakes (the D
term dropped, a wrong D, P not normalised, a missing scale, dQ and dK swapped,
P used untransposed) fail the finite-difference pin.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import attention as A
from oracle import backward as BW


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _loss(fwd, q, k, v, do):
    o, _ = fwd(q, k, v)
    return float(np.sum(o * do))


def _finite_diff(fwd, q, k, v, do, h=1e-5):
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(args[which])
        it = np.nditer(args[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            orig = args[which][idx]
            args[which][idx] = orig + h
            lp = _loss(fwd, *args, do)
            args[which][idx] = orig - h
            lm = _loss(fwd, *args, do)
            args[which][idx] = orig
            g[idx] = (lp - lm) / (2 * h)
        grads.append(g)
    return grads


def _tiny_sparse():
    # N = 7, block 2: four query blocks, the last one partial; two meta heads;
    # query block 1 of head 0 is empty, repeats and a future block under causal
    raw = [[0, 0, 2], [], [2, 1], [3, 0, 3],     # head 0
           [1], [0, 1], [0, 2, 2], [1, 3]]       # head 1
    rp, col = workloads.lists_to_csr(raw)
    return rp, col


CASES = ["dense", "causal", "sparse", "sparse_causal"]


def _fwd_bwd(case, scale):
    if case in ("dense", "causal"):
        causal = case == "causal"
        fwd = lambda q, k, v: oracle.attn_fwd(q, k, v, scale, causal)
        bwd = lambda q, k, v, do, **kw: oracle.attn_bwd(q, k, v, do, scale, causal, **kw)
    else:
        causal = case == "sparse_causal"
        rp, col = _tiny_sparse()
        fwd = lambda q, k, v: oracle.attn_fwd_blocksparse(q, k, v, scale, causal, 2, rp, col, 2)
        bwd = lambda q, k, v, do, **kw: oracle.attn_bwd_blocksparse(q, k, v, do, scale, causal, 2, rp, col, 2,
                                                                   **kw)
    return fwd, bwd


@pytest.mark.parametrize("case", CASES)
def test_finite_differences(case):
    shape = (1, 2, 7, 3)
    q, k, v, do = (_rand(shape, s) for s in (1, 2, 3, 4))
    scale = 0.7
    fwd, bwd = _fwd_bwd(case, scale)
    dq, dk, dv = bwd(q, k, v, do)
    for got, ref in zip((dq, dk, dv), _finite_diff(fwd, q, k, v, do)):
        np.testing.assert_allclose(got, ref, rtol=1e-7, atol=1e-8)


def _sdpa_grads(q, k, v, do, scale, allowed):
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
    o = torch.nn.functional.scaled_dot_product_attention(t[0], t[1], t[2], attn_mask=torch.tensor(allowed),
                                                         scale=scale)
    o.backward(torch.tensor(do, dtype=torch.float64))
    return [x.grad.numpy() for x in t]


@pytest.mark.parametrize("causal", [False, True])
def test_sdpa_autograd_dense(causal):
    B, H, N, d = 2, 2, 40, 8
    q, k, v, do = (_rand((B, H, N, d), s) for s in (11, 12, 13, 14))
    scale = 1 / np.sqrt(d)
    allowed = A.token_mask_dense(N, causal, np.arange(N))
    ref = _sdpa_grads(q, k, v, do, scale, allowed)
    got = oracle.attn_bwd(q, k, v, do, scale, causal)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_sdpa_autograd_block_sparse(causal):
    # every query block lists its own diagonal block, so no row is empty
    B, H, N, d, b = 1, 2, 45, 8, 8
    nqb = -(-N // b)
    rng = workloads.SplitMix64(21)
    lists = [[qb] + [rng.below(nqb) for _ in range(3)] for qb in range(nqb)]
    rp, col = workloads.lists_to_csr(lists)
    q, k, v, do = (_rand((B, H, N, d), s) for s in (15, 16, 17, 18))
    scale = 0.3
    allowed = A.token_mask_block_sparse(N, causal, b, rp, col, 0, np.arange(N))
    ref = _sdpa_grads(q, k, v, do, scale, allowed)
    got = oracle.attn_bwd_blocksparse(q, k, v, do, scale, causal, b, rp, col, 1)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_value_rows_give_zero_score_gradients(causal):
    # dP_ij = dO_i . v is the same for every key of row i, so dS = 0
    B, H, N, d = 1, 1, 33, 5
    q, k, do = (_rand((B, H, N, d), s) for s in (21, 22, 23))
    v = np.broadcast_to(_rand((d,), 24), (B, H, N, d)).copy()
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 0.5, causal)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    assert np.abs(dv).max() > 0.1


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_closed_form(causal):
    B, H, N, d = 1, 1, 29, 4
    q, v, do = (_rand((B, H, N, d), s) for s in (31, 32, 33))
    k = np.broadcast_to(_rand((d,), 34), (B, H, N, d)).copy()
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 0.9, causal)
    assert np.abs(dq).max() < 1e-12
    allowed = A.token_mask_dense(N, causal, np.arange(N))
    n = allowed.sum(axis=1)
    dv_ref = (allowed / n[:, None]).T @ do[0, 0]
    np.testing.assert_allclose(dv[0, 0], dv_ref, rtol=1e-12, atol=1e-13)


def test_single_key():
    q, k, v, do = (_rand((2, 3, 1, 6), s) for s in (41, 42, 43, 44))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 0.4, True)
    np.testing.assert_array_equal(dv, do)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14


@pytest.mark.parametrize("case", ["dense", "causal", "sparse_causal_empty"])
def test_invariants(case):
    B, H, N, d, b = 1, 2, 70, 6, 16
    q, k, v, do = (_rand((B, H, N, d), s) for s in (51, 52, 53, 54))
    scale = 0.6
    if case == "sparse_causal_empty":
        # query block 1 empty; key block 2 listed by no query block
        lists = [[0], [], [0, 1], [1, 3, 3], [0, 4]]
        rp, col = workloads.lists_to_csr(lists)
        allowed = A.token_mask_block_sparse(N, True, b, rp, col, 0, np.arange(N))
        dq, dk, dv = oracle.attn_bwd_blocksparse(q, k, v, do, scale, True, b, rp, col, 1)
        o, lse = oracle.attn_fwd_blocksparse(q, k, v, scale, True, b, rp, col, 1)
    else:
        causal = case == "causal"
        allowed = A.token_mask_dense(N, causal, np.arange(N))
        dq, dk, dv = oracle.attn_bwd(q, k, v, do, scale, causal)
        o, lse = oracle.attn_fwd(q, k, v, scale, causal)
    nonempty = allowed.any(axis=1)
    seen = allowed.any(axis=0)
    for h in range(H):
        np.testing.assert_allclose(dk[0, h].sum(axis=0), 0.0, atol=1e-12)
        np.testing.assert_allclose(dv[0, h].sum(axis=0), do[0, h][nonempty].sum(axis=0), rtol=1e-12, atol=1e-12)
        assert np.all(dq[0, h][~nonempty] == 0)
        assert np.all(dk[0, h][~seen] == 0) and np.all(dv[0, h][~seen] == 0)
        # D_i = dO_i . O_i equals sum_j P_ij dP_ij
        s = A.scores_stage(q[0, h], k[0, h], scale, allowed)
        p = BW.probabilities_from_lse(s, lse[0, h])
        dp = do[0, h] @ v[0, h].T
        np.testing.assert_allclose(BW.row_scalar_d(do[0, h], o[0, h]), np.sum(p * dp, axis=1),
                                   rtol=1e-12, atol=1e-12)
    if case == "sparse_causal_empty":
        assert (~nonempty).sum() == b and (~seen).sum() == b


def test_all_active_block_mask_equals_dense():
    B, H, N, d, b = 1, 1, 50, 4, 16
    q, k, v, do = (_rand((B, H, N, d), s) for s in (61, 62, 63, 64))
    nqb = -(-N // b)
    rp, col = workloads.lists_to_csr([list(range(nqb))] * nqb)
    for causal in (False, True):
        ref = oracle.attn_bwd(q, k, v, do, 0.5, causal)
        got = oracle.attn_bwd_blocksparse(q, k, v, do, 0.5, causal, b, rp, col, 1)
        for g, r in zip(got, ref):
            np.testing.assert_allclose(g, r, rtol=1e-13, atol=1e-14)


def test_explicit_forward_outputs_and_row_chunks():
    B, H, N, d = 1, 2, 37, 5
    q, k, v, do = (_rand((B, H, N, d), s) for s in (71, 72, 73, 74))
    o, lse = oracle.attn_fwd(q, k, v, 0.5, True)
    ref = oracle.attn_bwd(q, k, v, do, 0.5, True)
    got = oracle.attn_bwd(q, k, v, do, 0.5, True, o=o, lse=lse, row_chunk=8)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=1e-12, atol=1e-13)


def test_planted_mistakes_are_caught(monkeypatch):
    shape = (1, 1, 6, 3)
    q, k, v, do = (_rand(shape, s) for s in (81, 82, 83, 84))
    scale = 0.8
    fwd, bwd = _fwd_bwd("causal", scale)
    fd = _finite_diff(fwd, q, k, v, do)

    def matches(grads):
        return all(np.allclose(g, r, rtol=1e-6, atol=1e-7) for g, r in zip(grads, fd))

    assert matches(bwd(q, k, v, do))
    mistakes = {
        "D dropped": ("score_gradient", lambda p, dp, d_rows: p * dp),
        "D from dO alone": ("row_scalar_d", lambda do_r, o_r: np.sum(do_r, axis=1)),
        "D sign": ("score_gradient", lambda p, dp, d_rows: p * (dp + d_rows[:, None])),
        "P unnormalised": ("probabilities_from_lse", lambda s, lse: np.where(np.isfinite(s), np.exp(s), 0.0)),
    }
    for name, (fn, bad) in mistakes.items():
        with monkeypatch.context() as mp:
            mp.setattr(BW, fn, bad)
            assert not matches(bwd(q, k, v, do)), name
    dq, dk, dv = bwd(q, k, v, do)
    allowed = A.token_mask_dense(6, True, np.arange(6))
    p, _ = A.softmax_stage(A.scores_stage(q[0, 0], k[0, 0], scale, allowed))
    assert not matches((dq / scale, dk, dv)), "scale missing in dQ"
    assert not matches((dq, dk / scale, dv)), "scale missing in dK"
    assert not matches((dk, dq, dv)), "dQ and dK swapped"
    assert not matches((dq, dk, (p @ do[0, 0])[None, None])), "P untransposed in dV"
