"""Pins for the oracle's mean-pooled block selector.

* the pooled score of a (query block, key block) tile equals the mean of the
  tile's logits computed pair by pair (linearity; partial last blocks average
  their real tokens only; grouped-query heads read their key/value head);
* the selection is a valid top-k: size min(topk, candidates), every chosen
  score >= every unchosen candidate's, ties to the lower index, ascending,
  causal candidates only;
* the pages' claim for homogeneous blocks: when the keys inside each key
  block and the queries inside each query block are equal, the exact block
  mass log sum_j exp(s_ij) is s_bar + log|B_b|, so with equal-sized blocks the
  pooled ranking equals the ranking by exact mass;
* shared selection under grouped-query attention gives a group's heads one
  list; with Hkv == H it changes nothing;
* per-(batch, head) patterns feed the attention oracle (meta_heads = B*H);
* planted mistakes (dividing a partial block by the block size; ties to the
  higher index) fail.
"""
import numpy as np
import pytest

import oracle
import workloads
from oracle import attention as A
from oracle import selector as SEL


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("N,block", [(64, 16), (70, 16), (33, 8)])
def test_score_is_the_mean_tile_logit(N, block):
    B, H, Hkv, d = 2, 4, 2, 5
    q, k = _rand((B, H, N, d), 1), _rand((B, Hkv, N, d), 2)
    scale = 0.7
    s = oracle.meanpool_scores(q, k, scale, block, False)
    nb = -(-N // block)
    for b in range(B):
        for h in range(H):
            full = scale * q[b, h] @ k[b, h // (H // Hkv)].T
            for a in range(nb):
                for c in range(nb):
                    tile = full[a * block:min(N, (a + 1) * block), c * block:min(N, (c + 1) * block)]
                    assert s[b, h, a, c] == pytest.approx(tile.mean(), rel=1e-12, abs=1e-12)


def _check_valid_topk(scores, lists, topk):
    for row, chosen in zip(scores.reshape(-1, scores.shape[-1]), lists):
        cand = [j for j in range(row.size) if np.isfinite(row[j])]
        assert len(chosen) == min(topk, len(cand))
        assert chosen == sorted(chosen) and set(chosen) <= set(cand)
        rest = [j for j in cand if j not in chosen]
        if chosen and rest:
            assert min(row[j] for j in chosen) >= max(row[j] for j in rest)
            # ties at the boundary go to the lower index
            lo = min(row[j] for j in chosen)
            tied_out = [j for j in rest if row[j] == lo]
            tied_in = [j for j in chosen if row[j] == lo]
            assert all(i < o for i in tied_in for o in tied_out)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("topk", [1, 3, 8, 20])
def test_selection_is_a_valid_topk(causal, topk):
    q, k = _rand((1, 2, 200, 6), 3), _rand((1, 2, 200, 6), 4)
    s = oracle.meanpool_scores(q, k, 0.5, 16, causal)
    lists = oracle.select_topk(s, topk)
    _check_valid_topk(s, lists, topk)
    if causal:
        nb = s.shape[-1]
        for r, chosen in enumerate(lists):
            assert all(c <= r % nb for c in chosen)


def test_ties_go_to_the_lower_index():
    s = np.array([[1.0, 2.0, 2.0, 2.0, 0.5]])
    assert oracle.select_topk(s, 2) == [[1, 2]]
    assert oracle.select_topk(s, 4) == [[0, 1, 2, 3]]


def test_homogeneous_blocks_rank_like_exact_mass():
    B, H, N, d, block = 1, 1, 128, 4, 16
    nb = N // block
    rng = np.random.default_rng(5)
    # equal keys inside each key block, equal queries inside each query block
    k = np.repeat(rng.standard_normal((nb, d)), block, axis=0)[None, None]
    q = np.repeat(rng.standard_normal((nb, d)), block, axis=0)[None, None]
    scale = 0.9
    s = oracle.meanpool_scores(q, k, scale, block, False)
    full = scale * q[0, 0] @ k[0, 0].T
    for a in range(nb):
        i = a * block
        mass = [np.log(np.exp(full[i, c * block:(c + 1) * block]).sum()) for c in range(nb)]
        np.testing.assert_allclose(np.array(mass), s[0, 0, a] + np.log(block), rtol=1e-12)
        for topk in (1, 3, 5):
            by_mass = sorted(sorted(range(nb), key=lambda c: (-mass[c], c))[:topk])
            assert oracle.select_topk(s[0, 0, a:a + 1], topk) == [by_mass]


def test_shared_group_selection():
    B, H, Hkv, N, d = 1, 6, 2, 160, 8
    q, k = _rand((B, H, N, d), 6), _rand((B, Hkv, N, d), 7)
    rp, col = oracle.meanpool_select(q, k, 0.4, 32, True, 3, share_groups=True)
    nb = 5
    lists = [list(col[rp[r]:rp[r + 1]]) for r in range(B * H * nb)]
    for h in range(H):
        assert lists[h * nb:(h + 1) * nb] == lists[(h // 3) * 3 * nb:((h // 3) * 3 + 1) * nb]
    q2, k2 = _rand((B, 3, N, d), 8), _rand((B, 3, N, d), 9)
    a = oracle.meanpool_select(q2, k2, 0.4, 32, False, 2, share_groups=True)
    b = oracle.meanpool_select(q2, k2, 0.4, 32, False, 2, share_groups=False)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_per_batch_head_patterns_feed_the_attention_oracle():
    B, H, N, d, block = 2, 2, 96, 4, 16
    q, k, v = (_rand((B, H, N, d), s) for s in (10, 11, 12))
    rp, col = oracle.meanpool_select(q, k, 0.5, block, True, 2)
    o, lse = oracle.attn_fwd_blocksparse(q, k, v, 0.5, True, block, rp, col, B * H)
    nb = N // block
    for b in range(B):
        for h in range(H):
            r0 = (b * H + h) * nb
            sub_rp = rp[r0:r0 + nb + 1] - rp[r0]
            sub_col = col[rp[r0]:rp[r0 + nb]]
            o1, l1 = oracle.attn_fwd_blocksparse(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                                                 0.5, True, block, sub_rp, sub_col, 1)
            np.testing.assert_array_equal(o[b, h], o1[0, 0])
            np.testing.assert_array_equal(lse[b, h], l1[0, 0])


def test_planted_mistakes_are_caught(monkeypatch):
    N, block, d = 70, 16, 3
    q, k = _rand((1, 1, N, d), 13), _rand((1, 1, N, d), 14)
    full = q[0, 0] @ k[0, 0].T
    last = full[:16, 64:70].mean()

    def bad_means(x, blk):
        x = np.asarray(x, dtype=np.float64)
        nb = -(-x.shape[-2] // blk)
        pad = np.zeros(x.shape[:-2] + (nb * blk - x.shape[-2], x.shape[-1]))
        return np.concatenate([x, pad], axis=-2).reshape(x.shape[:-2] + (nb, blk, x.shape[-1])).mean(axis=-2)

    with monkeypatch.context() as mp:
        mp.setattr(SEL, "block_means", bad_means)
        s_bad = SEL.meanpool_scores(q, k, 1.0, block, False)
    assert s_bad[0, 0, 0, 4] != pytest.approx(last, rel=1e-9)
    s = np.array([[1.0, 2.0, 2.0, 0.0]])
    higher = [sorted(sorted(range(4), key=lambda j: (-s[0, j], -j))[:1])]
    with pytest.raises(AssertionError):
        _check_valid_topk(s, higher, 1)
