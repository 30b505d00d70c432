"""Pins for the oracle's ring-step attention (a query block against one
key/value block at global positions) and its (O, LSE) merge.

* zero offsets and Nq == Nk reduce to the forward oracle;
* a scalar brute force on tiny rectangular blocks with offsets;
* splitting the keys into blocks (any number, any order), attending each block
  at its offset and merging gives the full attention, dense and causal, which
  is the ring's exactness claim ("Exact Blocks, Rings, and Sparsity",
  section 4: blocks may arrive in any order);
* the LSE-form merge equals the (m, l, A) merge with A = l O;
* empty parts: causal blocks wholly in the future give LSE = -inf, O = 0 and
  leave the merge unchanged; all-empty gives O = 0, LSE = -inf.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import attention as A


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_zero_offsets_reduce_to_forward():
    q, k, v = (_rand((2, 2, 37, 8), s) for s in (1, 2, 3))
    for causal in (False, True):
        o, lse = oracle.attn_fwd_block(q, k, v, 0.4, causal)
        o_ref, lse_ref = oracle.attn_fwd(q, k, v, 0.4, causal)
        np.testing.assert_allclose(o, o_ref, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse, lse_ref, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("q_off,k_off", [(0, 0), (5, 2), (3, 7), (20, 0)])
def test_scalar_brute_force(q_off, k_off):
    nq, nk, d = 5, 6, 3
    q, k, v = _rand((1, 1, nq, d), 4), _rand((1, 1, nk, d), 5), _rand((1, 1, nk, d), 6)
    scale = 0.9
    o, lse = oracle.attn_fwd_block(q, k, v, scale, True, q_off, k_off)
    for i in range(nq):
        keys = [j for j in range(nk) if k_off + j <= q_off + i]
        if not keys:
            assert lse[0, 0, i] == -np.inf and np.all(o[0, 0, i] == 0)
            continue
        logits = [scale * sum(q[0, 0, i, c] * k[0, 0, j, c] for c in range(d)) for j in keys]
        mx = max(logits)
        w = [math.exp(x - mx) for x in logits]
        z = sum(w)
        assert lse[0, 0, i] == pytest.approx(mx + math.log(z), rel=1e-13)
        for c in range(d):
            ref = sum(wi * v[0, 0, j, c] for wi, j in zip(w, keys)) / z
            assert o[0, 0, i, c] == pytest.approx(ref, rel=1e-12, abs=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cuts", [[0, 64], [0, 20, 64], [0, 7, 8, 31, 50, 64]])
def test_blocks_merged_in_any_order_equal_full_attention(causal, cuts):
    N, d = 64, 8
    q, k, v = (_rand((1, 2, N, d), s) for s in (7, 8, 9))
    # the query rows of one "device": global positions 16..47
    q_lo, q_hi = 16, 48
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, 0.5, causal)
    parts = [oracle.attn_fwd_block(q[:, :, q_lo:q_hi], k[:, :, a:b], v[:, :, a:b], 0.5, causal, q_lo, a)
             for a, b in zip(cuts[:-1], cuts[1:])]
    order = list(range(len(parts)))[::-1]          # ring order differs from memory order
    o, lse = oracle.merge_lse([parts[i][0] for i in order], [parts[i][1] for i in order])
    np.testing.assert_allclose(o, o_ref[:, :, q_lo:q_hi], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref[:, :, q_lo:q_hi], rtol=1e-13, atol=1e-13)


def test_lse_merge_equals_state_merge():
    rng = np.random.default_rng(10)
    o_a, o_b = rng.standard_normal((2, 5, 3))
    l_a, l_b = rng.uniform(0.5, 3.0, (2, 5))
    m_a, m_b = rng.standard_normal((2, 5)) * 4
    m, l, acc = oracle.merge_states(m_a, l_a, l_a[:, None] * o_a, m_b, l_b, l_b[:, None] * o_b)
    o, lse = oracle.merge_lse([o_a, o_b], [m_a + np.log(l_a), m_b + np.log(l_b)])
    np.testing.assert_allclose(lse, m + np.log(l), rtol=1e-14)
    np.testing.assert_allclose(o, acc / l[:, None], rtol=1e-13, atol=1e-14)


def test_empty_parts():
    q, k, v = (_rand((1, 1, 8, 4), s) for s in (11, 12, 13))
    # keys at positions 100.. are in the future of queries 0..7
    o_f, lse_f = oracle.attn_fwd_block(q, k, v, 0.5, True, 0, 100)
    assert np.all(lse_f == -np.inf) and np.all(o_f == 0)
    o_p, lse_p = oracle.attn_fwd_block(q, k, v, 0.5, True, 0, 0)
    o, lse = oracle.merge_lse([o_p, o_f], [lse_p, lse_f])
    np.testing.assert_array_equal(o, o_p)
    np.testing.assert_array_equal(lse, lse_p)
    o, lse = oracle.merge_lse([o_f, o_f], [lse_f, lse_f])
    assert np.all(o == 0) and np.all(lse == -np.inf)


def test_planted_offset_mistake_is_caught():
    # swapping the roles of the offsets must break the merge-equals-full pin
    N, d = 40, 4
    q, k, v = (_rand((1, 1, N, d), s) for s in (14, 15, 16))
    o_ref, _ = oracle.attn_fwd(q, k, v, 0.5, True)
    parts = [oracle.attn_fwd_block(q[:, :, 10:30], k[:, :, a:b], v[:, :, a:b], 0.5, True, a, 10)
             for a, b in ((0, 20), (20, 40))]
    o, _ = oracle.merge_lse([p[0] for p in parts], [p[1] for p in parts])
    assert not np.allclose(o, o_ref[:, :, 10:30])
