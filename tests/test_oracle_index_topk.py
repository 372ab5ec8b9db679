"""Pins of the oracle's lightning-indexer scores, visibility rule and top-k selection.

Sources: yudonglee.me "DeepSeek-V4 详解" 2.2 Steps 2-3 and 2.3 Step 1; hongke120.com/20112.html
2.2-2.3; deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一. Count pins come from
tests/golden/page_counts.json.
"""
import json
import os

import numpy as np
import pytest

from oracle import csa_oracle as o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_counts.json")


def test_index_worked_example():
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    w = np.array([2.0, -1.0])
    k = np.array([[1.0, 1.0], [-1.0, 2.0], [3.0, -1.0], [5.0, 5.0]])
    # head 0 dots: 1, -1, 3 -> ReLU 1, 0, 3; head 1 dots: 1, 2, -1 -> ReLU 1, 2, 0.
    s = o.index_scores(q, w, k, n_vis=3)
    assert s[:3].tolist() == [1.0, -2.0, 6.0] and s[3] == -np.inf


def test_index_single_head_unit_weight_is_relu_dot():
    rng = np.random.default_rng(0)
    q, k = rng.standard_normal((1, 16)), rng.standard_normal((30, 16))
    s = o.index_scores(q, np.array([1.0]), k, 30)
    np.testing.assert_allclose(s, np.maximum(k @ q[0], 0.0), rtol=0, atol=1e-14)
    s_neg = o.index_scores(q, np.array([-1.0]), k, 30)
    np.testing.assert_allclose(s_neg, -np.maximum(k @ q[0], 0.0), rtol=0, atol=1e-14)


def test_index_brute_force_loops():
    rng = np.random.default_rng(1)
    H, d, N, nv = 3, 5, 11, 8
    q, k, w = rng.standard_normal((H, d)), rng.standard_normal((N, d)), rng.standard_normal(H)
    s = o.index_scores(q, w, k, nv)
    for j in range(N):
        if j >= nv:
            assert s[j] == -np.inf
            continue
        want = 0.0
        for h in range(H):
            dot = sum(q[h, t] * k[j, t] for t in range(d))
            want += w[h] * (dot if dot > 0 else 0.0)
        assert abs(s[j] - want) < 1e-13


def test_positive_query_scaling_keeps_topk():
    rng = np.random.default_rng(2)
    q, k, w = rng.standard_normal((4, 8)), rng.standard_normal((50, 8)), rng.standard_normal(4)
    a, _ = o.topk(o.index_scores(q, w, k, 50), 50, 7)
    b, _ = o.topk(o.index_scores(3.5 * q, w, k, 50), 50, 7)
    assert (a == b).all()


def test_visibility_counts():
    assert o.n_visible(0, 4, 100) == 0 and o.n_visible(2, 4, 100) == 0
    assert o.n_visible(3, 4, 100) == 1 and o.n_visible(7, 4, 100) == 2
    assert o.n_visible(10_000, 4, 100) == 100


def _rank_topk(s, nv, k):
    """Rank formulation: entry j is selected iff fewer than k visible entries precede it in the
    order (score descending, index ascending)."""
    sel = []
    for j in range(nv):
        beat = sum(1 for i in range(nv) if s[i] > s[j] or (s[i] == s[j] and i < j))
        if beat < k:
            sel.append(j)
    return sel


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_rank_brute_force(seed):
    rng = np.random.default_rng(seed)
    N = 23
    s = np.round(rng.standard_normal(N), 1)       # coarse values force ties
    for nv in (0, 1, 5, 23):
        for k in (1, 3, 8, 23, 30):
            idx, _ = o.topk(s, nv, k)
            want = _rank_topk(s, nv, k)
            assert idx[:len(want)].tolist() == want
            assert (idx[len(want):] == -1).all()


def test_topk_special_cases():
    s = np.array([0.5, 2.0, -1.0, 2.0, 0.1])
    idx, gap = o.topk(s, 5, 1)
    assert idx.tolist() == [1] and gap == 0.0              # tie at the top goes to index 1
    idx, gap = o.topk(s, 5, 9)
    assert idx.tolist() == [0, 1, 2, 3, 4, -1, -1, -1, -1] and gap == np.inf
    idx, _ = o.topk(np.zeros(10), 10, 4)
    assert idx.tolist() == [0, 1, 2, 3]
    idx, gap = o.topk(s, 5, 2)
    assert idx.tolist() == [1, 3] and gap == pytest.approx((2.0 - 0.5) / 2.0)


def test_topk_permutation_equivariance():
    rng = np.random.default_rng(3)
    s = rng.standard_normal(40)
    perm = rng.permutation(40)
    a, _ = o.topk(s, 40, 9)
    b, _ = o.topk(s[perm], 40, 9)
    assert sorted(perm[b].tolist()) == a.tolist()


def test_page_counts():
    with open(GOLDEN) as f:
        g = json.load(f)
    ctx = g["context_tokens"]
    # CSA: 4-fold compression of a 1M context, and top-1024 blocks covering 4096 tokens.
    assert o.n_visible(ctx - 1, g["csa_m"], 1 << 40) == g["csa_entries_at_1m"]
    assert g["csa_topk"] * g["csa_m"] == g["csa_topk_tokens"]
    # HCA: 128-fold compression into 8192 summaries; dense attention cost ratio (L/N)^2.
    n_hca = o.n_visible(ctx - 1, g["hca_m"], 1 << 40)
    assert n_hca == g["hca_entries_at_1m"]
    assert (ctx // n_hca) ** 2 == g["hca_dense_cost_ratio"]
    # The page's rounded statements agree with the exact counts.
    assert abs(g["csa_entries_at_1m"] - g["csa_entries_stated_approx"]) / 262144 < 0.05
    assert abs(n_hca - g["hca_entries_stated_approx"]) / n_hca < 0.05


# ---- low-precision indexer: MXFP4 vectors, bf16 scores ---------------------------------------
# deepseek.csdn.net "一文搞懂 DeepSeek", V4 的其他升级 (FP4 paragraph).

def test_bf16_score_storage():
    s = np.array([1.0 + 2.0 ** -9, 1.0 + 3 * 2.0 ** -9, -np.inf, 3.0])
    out = o.store_scores_bf16(s)
    # 1 + 2^-9 is halfway between 1 and 1 + 2^-7: ties to even -> 1; 1 + 3 * 2^-9 -> 1 + 2^-7.
    assert out[0] == 1.0 and out[1] == 1.0 + 2.0 ** -7
    assert out[2] == -np.inf and out[3] == 3.0


def test_mxfp4_index_worked_example():
    # One head, w = 1: query block 0 = [1, 1, 0, ...] (scale 2^0), keys: [2, 0.5, ...] -> 2.5,
    # [-1, 0, ...] -> ReLU 0, [6, 6, ...] with scale 2^-2 -> 3. bf16 keeps all three exactly.
    from oracle.numerics import mxfp4_decode
    q = np.zeros((1, 32), np.uint8)
    q[0, 0] = 0x22                                   # codes 2, 2: 1.0, 1.0
    qs = np.array([[127, 127]], np.uint8)
    k = np.zeros((3, 32), np.uint8)
    k[0, 0] = 0x14                                   # 2.0, 0.5
    k[1, 0] = 0x0A                                   # -1.0, 0
    k[2, 0] = 0x77                                   # 6, 6
    ks = np.array([[127, 127], [127, 127], [125, 127]], np.uint8)
    s = o.store_scores_bf16(o.index_scores(mxfp4_decode(q, qs), np.array([1.0]),
                                           mxfp4_decode(k, ks), 3))
    assert s.tolist() == [2.5, 0.0, 3.0]


def test_recall():
    assert o.recall(np.array([3, 5, 9, -1]), np.array([3, 5, 7, -1])) == 2 / 3
    assert o.recall(np.array([1, 2]), np.array([-1, -1])) == 1.0
    sel, _ = o.topk(np.arange(10.0), 10, 4)
    assert o.recall(sel, sel) == 1.0
