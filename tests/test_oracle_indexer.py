"""Pins for the indexer score, flat top-k and HISA oracles (CPU)."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(99)


def test_score_worked_example():
    e = json.load(open(os.path.join(GOLD, "worked_examples.json")))["index_score"]
    S = oracle.index_scores(np.array(e["q_i"]), np.array(e["keys"]), np.array(e["w_i"]))
    np.testing.assert_array_equal(S, np.array(e["S"]))


def test_score_special_cases():
    H, d, n = 3, 5, 40
    keys = rng.integers(-8, 9, (n, d)).astype(float)
    # one head, unit weight, keys and query non-negative: a plain dot product
    qp = np.abs(rng.integers(-8, 9, (1, d))).astype(float)
    np.testing.assert_array_equal(oracle.index_scores(qp, np.abs(keys), np.ones(1)), np.abs(keys) @ qp[0])
    # the ReLU: an all-negative pairing scores exactly 0
    np.testing.assert_array_equal(oracle.index_scores(-qp, np.abs(keys), np.ones(1)), np.zeros(n))
    # every head the same with weights 1/H reduces to one head
    q1 = rng.integers(-8, 9, (1, d)).astype(float)
    S1 = oracle.index_scores(q1, keys, np.ones(1))
    np.testing.assert_allclose(oracle.index_scores(np.repeat(q1, H, 0), keys, np.full(H, 1.0 / H)), S1, rtol=1e-14)
    # heads add: the score of a 2-head query is the sum of its two 1-head scores
    q2 = rng.integers(-8, 9, (2, d)).astype(float)
    w2 = np.array([0.25, 3.0])
    np.testing.assert_array_equal(
        oracle.index_scores(q2, keys, w2),
        0.25 * oracle.index_scores(q2[:1], keys, np.ones(1)) + 3.0 * oracle.index_scores(q2[1:], keys, np.ones(1)))
    # the score is the query's, not the key's: swapping roles changes it
    assert not np.array_equal(oracle.index_scores(keys[:2], q2, np.ones(2)), oracle.index_scores(q2, keys[:2], np.ones(2)))


def brute_topk(scores, n, k):
    order = sorted(range(n), key=lambda i: (-scores[i], i))[: min(k, n)]
    return sorted(order) + [-1] * (k - min(k, n))


@pytest.mark.parametrize("trial", range(30))
def test_topk_select_brute_force(trial):
    n = int(rng.integers(0, 60))
    k = int(rng.integers(1, 70))
    s = rng.integers(-3, 4, 80).astype(float)  # many ties
    s[s == 0] = rng.choice([0.0, -0.0], size=int((s == 0).sum()))
    n_valid = min(n, 80)
    assert list(oracle.topk_select(s, n_valid, k)) == brute_topk(list(s), n_valid, k)


def test_topk_ties_lower_index_and_all_when_k_large():
    s = np.array([1.0, 5.0, 5.0, 5.0, 2.0, 5.0])
    assert list(oracle.topk_select(s, 6, 2)) == [1, 2]
    assert list(oracle.topk_select(s, 6, 4)) == [1, 2, 3, 5]
    assert list(oracle.topk_select(s, 6, 8)) == [0, 1, 2, 3, 4, 5, -1, -1]
    assert list(oracle.topk_select(s, 3, 8)) == [0, 1, 2, -1, -1, -1, -1, -1]
    assert list(oracle.topk_select(s, 0, 2)) == [-1, -1]
    # -0.0 and +0.0 are the same score: the lower index wins
    assert list(oracle.topk_select(np.array([-0.0, 0.0, -1.0]), 3, 1)) == [0]


def test_flat_topk_respects_visibility():
    N, H, d = 50, 2, 4
    k_i = rng.integers(-8, 9, (N, d)).astype(float)
    q_i = rng.integers(-8, 9, (3, H, d)).astype(float)
    w_i = np.floor(rng.random((3, H)) * 256) / 256
    n_vis = np.array([0, 7, 50])
    idx = oracle.flat_topk(q_i, k_i, w_i, n_vis, 10)
    assert list(idx[0]) == [-1] * 10
    assert list(idx[1][:7]) == list(range(7)) and list(idx[1][7:]) == [-1] * 3
    S = oracle.index_scores(q_i[2], k_i, w_i[2])
    assert list(idx[2]) == brute_topk(list(S), 50, 10)


def _tiny_indexer(N, H=2, d=4, nq=6, lo=-4, hi=4):
    k_i = rng.integers(lo, hi + 1, (N, d)).astype(float)
    q_i = rng.integers(lo, hi + 1, (nq, H, d)).astype(float)
    w_i = np.floor(rng.random((nq, H)) * 256) / 256
    return q_i, k_i, w_i


def test_pool_is_block_mean_with_zero_padded_tail():
    k_i = rng.standard_normal((10, 3))
    reps = oracle.hisa_pool(k_i, 4)
    np.testing.assert_allclose(reps[0], k_i[0:4].mean(0), rtol=1e-14)
    np.testing.assert_allclose(reps[1], k_i[4:8].mean(0), rtol=1e-14)
    np.testing.assert_allclose(reps[2], k_i[8:10].sum(0) / 4, rtol=1e-14)


@pytest.mark.parametrize("N,B,m", [(37, 8, 5), (64, 16, 4), (64, 4, 16), (13, 16, 1)])
def test_hisa_equals_flat_when_all_blocks_kept(N, B, m):
    q_i, k_i, w_i = _tiny_indexer(N)
    n_vis = rng.integers(0, N + 1, q_i.shape[0])
    k = 9
    idx_h, blk = oracle.hisa_topk(q_i, k_i, w_i, n_vis, B, m, k)
    np.testing.assert_array_equal(idx_h, oracle.flat_topk(q_i, k_i, w_i, n_vis, k))


def test_hisa_block_size_one_and_m_at_least_k_equals_flat():
    N = 60
    q_i, k_i, w_i = _tiny_indexer(N)
    n_vis = np.array([60, 59, 31, 5, 1, 0])
    for m in (8, 12):
        idx_h, _ = oracle.hisa_topk(q_i, k_i, w_i, n_vis, 1, m, 8)
        np.testing.assert_array_equal(idx_h, oracle.flat_topk(q_i, k_i, w_i, n_vis, 8))


def test_hisa_single_planted_block():
    N, B, d = 64, 8, 4
    k_i = rng.integers(-1, 2, (N, d)).astype(float)
    k_i[24:32] = 6.0  # block 3 dominates for a positive query
    q_i = np.ones((1, 1, d))
    w_i = np.ones((1, 1))
    idx, blk = oracle.hisa_topk(q_i, k_i, w_i, np.array([N]), B, 1, 5)
    assert list(blk[0]) == [3]
    assert list(idx[0]) == [24, 25, 26, 27, 28]
    # a query that cannot see block 3's first entry never picks it
    idx, blk = oracle.hisa_topk(q_i, k_i, w_i, np.array([24]), B, 1, 5)
    assert blk[0][0] != 3 and all(i < 24 for i in idx[0] if i >= 0)


def test_hisa_brute_force_enumeration():
    # Enumerate every choice of m blocks; the chosen set must be the one whose
    # (score desc, id asc) ordering is lexicographically best, then the token
    # top-k is brute-forced inside it with pure-Python loops.
    N, B, m, k = 30, 4, 3, 5
    q_i, k_i, w_i = _tiny_indexer(N, H=2, d=3)
    n_vis = np.array([30, 29, 17, 9, 4, 1])
    idx, blk = oracle.hisa_topk(q_i, k_i, w_i, n_vis, B, m, k)
    for q in range(q_i.shape[0]):
        n = int(n_vis[q])
        nbq = (n + B - 1) // B

        def score(vec):
            tot = 0.0
            for h in range(q_i.shape[1]):
                dot = sum(q_i[q, h, c] * vec[c] for c in range(k_i.shape[1]))
                tot += w_i[q, h] * max(0.0, dot)
            return tot

        reps = []
        for b in range(nbq):
            acc = [0.0] * k_i.shape[1]
            for i in range(b * B, min(N, b * B + B)):
                for c in range(k_i.shape[1]):
                    acc[c] += k_i[i, c]
            reps.append([a / B for a in acc])
        rs = [score(r) for r in reps]
        best = None
        for combo in itertools.combinations(range(nbq), min(m, nbq)):
            keyseq = sorted(((-rs[b], b) for b in combo))
            if best is None or keyseq < best[0]:
                best = (keyseq, combo)
        chosen = sorted(best[1]) if best else []
        assert list(blk[q]) == chosen + [-1] * (m - len(chosen))
        cand = [i for b in chosen for i in range(b * B, min(n, b * B + B))]
        ts = sorted(cand, key=lambda i: (-score(k_i[i]), i))[:k]
        assert list(idx[q]) == sorted(ts) + [-1] * (k - len(ts))


# ---- block-sparse (MoBA/NSA-style) baseline --------------------------------

def _brute_block_sparse(q, k_i, w, n, B, m):
    """Loops only: block sums, the block score with explicit head and channel
    loops, blocks ranked with Python sorted, chosen blocks expanded."""
    N, d = k_i.shape
    nb = (N + B - 1) // B
    cand = (n + B - 1) // B
    score = []
    for b in range(cand):
        rep = [sum(k_i[i][c] for i in range(b * B, min(N, b * B + B))) / B for c in range(d)]
        s = 0.0
        for h in range(q.shape[0]):
            dot = sum(q[h][c] * rep[c] for c in range(d))
            s += w[h] * max(0.0, dot)
        score.append(s)
    chosen = sorted(sorted(range(cand), key=lambda b: (-score[b], b))[:m])
    ent = [e for b in chosen for e in range(b * B, min(n, b * B + B))]
    return ent + [-1] * (m * B - len(ent)), chosen + [-1] * (m - len(chosen))


@pytest.mark.parametrize("trial", range(12))
def test_block_sparse_brute_force(trial):
    N = int(rng.integers(1, 70))
    B = int(rng.choice([1, 2, 4, 8]))
    m = int(rng.integers(1, 6))
    nq, H, d = 3, 2, 3
    q = rng.integers(-2, 3, (nq, H, d)).astype(float)
    k_i = rng.integers(-2, 3, (N, d)).astype(float)  # ties among block scores
    w = rng.integers(0, 4, (nq, H)).astype(float) / 4
    n_vis = rng.integers(0, N + 1, nq)
    idx, blk = oracle.block_sparse_topk(q, k_i, w, n_vis, B, m)
    for j in range(nq):
        r_idx, r_blk = _brute_block_sparse(q[j], k_i, w[j], int(n_vis[j]), B, m)
        assert list(idx[j]) == r_idx, (trial, j)
        assert list(blk[j]) == r_blk, (trial, j)


def test_block_sparse_every_block_and_unit_blocks():
    N, nq, H, d = 50, 4, 3, 5
    q = rng.standard_normal((nq, H, d))
    k_i = rng.standard_normal((N, d))
    w = rng.uniform(0, 1, (nq, H))
    n_vis = np.array([50, 37, 8, 1])
    # m * B >= N: every visible entry, in order, whatever the scores
    idx, _ = oracle.block_sparse_topk(q, k_i, w, n_vis, 8, 7)
    for j, n in enumerate(n_vis):
        assert list(idx[j][:n]) == list(range(n)) and (idx[j][n:] == -1).all()
    # B = 1: each block is one entry, so the selection is the flat top-m
    idx1, _ = oracle.block_sparse_topk(q, k_i, w, n_vis, 1, 9)
    np.testing.assert_array_equal(idx1, oracle.flat_topk(q, k_i, w, n_vis, 9))


def test_block_sparse_planted_block_and_whole_blocks():
    # one block of large keys aligned with the query: chosen, and taken whole
    N, B, d = 64, 8, 4
    k_i = rng.standard_normal((N, d)) * 0.1
    k_i[24:32] = 5.0
    q = np.ones((1, 1, d))
    idx, blk = oracle.block_sparse_topk(q, k_i, np.ones((1, 1)), np.array([N]), B, 1)
    assert list(blk[0]) == [3]
    assert list(idx[0]) == list(range(24, 32))
    # unlike the token-level top-k, a chosen block keeps its weak entries
    k_i[28] = -5.0
    idx, _ = oracle.block_sparse_topk(q, k_i, np.ones((1, 1)), np.array([N]), B, 1)
    assert 28 in idx[0]
    assert 28 not in oracle.flat_topk(q, k_i, np.ones((1, 1)), np.array([N]), 8)[0]
