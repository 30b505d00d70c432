"""Pins for the oracle's grouped-query attention.

* Hkv == H reduces to the plain forward and gradient oracles;
* torch float64 scaled_dot_product_attention with enable_gqa (forward and
  autograd), dense, causal and with a block-sparse boolean mask (a library
  special case);
* central finite differences of the GQA forward for the shared K/V gradient
  (the sum over a group's query heads);
* a group's shared key-block list (meta_heads == Hkv) gives every query head of
  the group the same allowed set;
* planted mistakes (head h reading key/value head h % Hkv instead of
  h // (H/Hkv); the shared gradient averaged instead of summed) fail.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import attention as A


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_hkv_equal_h_reduces_to_plain_oracles():
    q, k, v, do = (_rand((1, 3, 40, 8), s) for s in (1, 2, 3, 4))
    for causal in (False, True):
        o, lse = oracle.attn_fwd_gqa(q, k, v, 0.4, causal)
        o2, lse2 = oracle.attn_fwd(q, k, v, 0.4, causal)
        np.testing.assert_array_equal(o, o2)
        np.testing.assert_array_equal(lse, lse2)
        g = oracle.attn_bwd_gqa(q, k, v, do, 0.4, causal)
        g2 = oracle.attn_bwd(q, k, v, do, 0.4, causal)
        for a, b in zip(g, g2):
            np.testing.assert_allclose(a, b, rtol=1e-14, atol=1e-15)


def _sdpa(q, k, v, do, scale, mask):
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
    o = torch.nn.functional.scaled_dot_product_attention(t[0], t[1], t[2], attn_mask=torch.tensor(mask),
                                                         scale=scale, enable_gqa=True)
    o.backward(torch.tensor(do))
    return o.detach().numpy(), [x.grad.numpy() for x in t]


@pytest.mark.parametrize("H,Hkv", [(4, 2), (6, 1), (8, 4)])
@pytest.mark.parametrize("causal", [False, True])
def test_sdpa_enable_gqa(H, Hkv, causal):
    B, N, d = 2, 33, 8
    q, do = _rand((B, H, N, d), 5), _rand((B, H, N, d), 6)
    k, v = _rand((B, Hkv, N, d), 7), _rand((B, Hkv, N, d), 8)
    mask = A.token_mask_dense(N, causal, np.arange(N))
    o_ref, g_ref = _sdpa(q, k, v, do, 0.35, mask)
    o, _ = oracle.attn_fwd_gqa(q, k, v, 0.35, causal)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    for a, b in zip(oracle.attn_bwd_gqa(q, k, v, do, 0.35, causal), g_ref):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


def test_sdpa_enable_gqa_block_sparse_shared_lists():
    B, H, Hkv, N, d, b = 1, 4, 2, 40, 8, 8
    nb = -(-N // b)
    rng = workloads.SplitMix64(9)
    # one list set per key/value head; every query block lists its diagonal
    lists = [[qb] + [rng.below(nb) for _ in range(2)] for _ in range(Hkv) for qb in range(nb)]
    rp, col = workloads.lists_to_csr(lists)
    q, do = _rand((B, H, N, d), 10), _rand((B, H, N, d), 11)
    k, v = _rand((B, Hkv, N, d), 12), _rand((B, Hkv, N, d), 13)
    mask = np.stack([A.token_mask_block_sparse(N, True, b, rp, col, h // (H // Hkv), np.arange(N)) for h in range(H)])
    o_ref, g_ref = _sdpa(q, k, v, do, 0.3, mask[None])
    o, _ = oracle.attn_fwd_gqa(q, k, v, 0.3, True, b, rp, col, Hkv)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    for a, r in zip(oracle.attn_bwd_gqa(q, k, v, do, 0.3, True, b, rp, col, Hkv), g_ref):
        np.testing.assert_allclose(a, r, rtol=1e-11, atol=1e-12)


def test_finite_differences_of_shared_heads():
    B, H, Hkv, N, d = 1, 4, 2, 6, 3
    q, do = _rand((B, H, N, d), 14), _rand((B, H, N, d), 15)
    k, v = _rand((B, Hkv, N, d), 16), _rand((B, Hkv, N, d), 17)
    loss = lambda kk, vv: float(np.sum(oracle.attn_fwd_gqa(q, kk, vv, 0.8, True)[0] * do))
    _, dk, dv = oracle.attn_bwd_gqa(q, k, v, do, 0.8, True)
    h = 1e-5
    for which, grad in ((0, dk), (1, dv)):
        for idx in np.ndindex(k.shape):
            kp, vp, km, vm = k.copy(), v.copy(), k.copy(), v.copy()
            (kp if which == 0 else vp)[idx] += h
            (km if which == 0 else vm)[idx] -= h
            fd = (loss(kp, vp) - loss(km, vm)) / (2 * h)
            assert fd == pytest.approx(grad[idx], rel=1e-6, abs=1e-8)


def test_shared_lists_give_the_group_one_allowed_set():
    H, Hkv, N, b = 6, 2, 30, 8
    nb = -(-N // b)
    rng = workloads.SplitMix64(18)
    rp, col = workloads.lists_to_csr(workloads.random_lists(Hkv * nb, nb, rng, max_len=6))
    erp, ecol = oracle.expand_lists(rp, col, Hkv, H, Hkv, nb)
    masks = [A.token_mask_block_sparse(N, False, b, erp, ecol, h, np.arange(N)) for h in range(H)]
    for h in range(H):
        assert np.array_equal(masks[h], masks[(h // 3) * 3])
    assert not np.array_equal(masks[0], masks[3])      # the two groups' lists differ for this seed


def test_planted_mistakes_are_caught():
    B, H, Hkv, N, d = 1, 4, 2, 20, 4
    q, k, v, do = _rand((B, H, N, d), 19), _rand((B, Hkv, N, d), 20), _rand((B, Hkv, N, d), 21), _rand((B, H, N, d), 22)
    mask = A.token_mask_dense(N, True, np.arange(N))
    o_ref, g_ref = _sdpa(q, k, v, do, 0.5, mask)
    wrong_map = np.stack([k[:, h % Hkv] for h in range(H)], axis=1)
    wrong_v = np.stack([v[:, h % Hkv] for h in range(H)], axis=1)
    o_bad, _ = oracle.attn_fwd(q, wrong_map, wrong_v, 0.5, True)
    assert not np.allclose(o_bad, o_ref)
    _, dk, _ = oracle.attn_bwd_gqa(q, k, v, do, 0.5, True)
    assert not np.allclose(dk / (H // Hkv), g_ref[1])
