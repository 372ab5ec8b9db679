"""Pins of the oracle's CSA and HCA attention against textbook attention and closed forms.

Textbook attention here is PyTorch's scaled_dot_product_attention in float64 on the CPU, a library
routine independent of the oracle. Sources: deepseek.csdn.net "一文搞懂 DeepSeek" (MLA section;
V4 改进一), yudonglee.me "DeepSeek-V4 详解" 2.2 Step 4 and 2.3 Step 2.
"""
import math

import numpy as np
import pytest
import torch

from oracle import csa_oracle as o


def textbook(q, keys, vals, scale, mask=None):
    """q [H, dk]; keys [n, dk]; vals [n, dv]; mask [n] bool (True = attend) -> o [H, dv], lse [H]."""
    H = q.shape[0]
    qt = torch.from_numpy(q)[None, :, None, :]                  # [1, H, 1, dk]
    kt = torch.from_numpy(keys)[None, None].expand(1, H, -1, -1)
    vt = torch.from_numpy(vals)[None, None].expand(1, H, -1, -1)
    m = None if mask is None else torch.from_numpy(mask)[None, None, None, :]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    logits = scale * (torch.from_numpy(q) @ torch.from_numpy(keys).T)
    if mask is not None:
        logits = logits.masked_fill(~torch.from_numpy(mask)[None, :], -math.inf)
    lse = torch.logsumexp(logits, dim=1)
    return out[0, :, 0, :].numpy(), lse.numpy()


def _r(shape, seed, s=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * s


def _store(c, r=None, scale=None, pos0=0):
    return (c, r, scale, pos0)


def test_closed_form_two_keys():
    q = np.array([[1.0, 0.0]])
    keys = np.array([[0.0, 0.0], [math.log(3.0), 5.0]])
    vals = np.array([[4.0], [8.0]])
    out, lse = o.softmax_attention(q, keys, vals, 1.0)
    np.testing.assert_allclose(out, [[0.25 * 4 + 0.75 * 8]], atol=1e-14)
    np.testing.assert_allclose(lse, [math.log(4.0)], atol=1e-14)


def test_single_key_and_zero_query():
    keys, vals = _r((1, 6), 0), _r((1, 4), 1)
    out, lse = o.softmax_attention(_r((3, 6), 2), keys, vals, 0.3)
    np.testing.assert_allclose(out, np.repeat(vals, 3, axis=0), atol=1e-15)
    keys, vals = _r((9, 6), 3), _r((9, 4), 4)
    out, lse = o.softmax_attention(np.zeros((2, 6)), keys, vals, 1.0)
    np.testing.assert_allclose(out, np.repeat(vals.mean(0, keepdims=True), 2, axis=0), atol=1e-15)
    np.testing.assert_allclose(lse, math.log(9.0), atol=1e-15)


def test_empty_key_set():
    out, lse = o.softmax_attention(_r((2, 4), 5), np.zeros((0, 4)), np.zeros((0, 3)), 1.0)
    assert (out == 0).all() and (lse == -np.inf).all()


def test_matches_textbook_and_permutation_invariance():
    q, keys, vals = _r((5, 12), 6), _r((17, 12), 7), _r((17, 8), 8)
    out, lse = o.softmax_attention(q, keys, vals, 0.4)
    t_out, t_lse = textbook(q, keys, vals, 0.4)
    np.testing.assert_allclose(out, t_out, atol=1e-13)
    np.testing.assert_allclose(lse, t_lse, atol=1e-13)
    p = np.random.default_rng(9).permutation(17)
    out2, lse2 = o.softmax_attention(q, keys[p], vals[p], 0.4)
    np.testing.assert_allclose(out2, out, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, atol=1e-13)


def test_lse_merge_is_identity():
    q, keys, vals = _r((4, 10), 10, 2), _r((30, 10), 11), _r((30, 7), 12)
    full = o.softmax_attention(q, keys, vals, 0.9)
    parts = [o.softmax_attention(q, keys[a:b], vals[a:b], 0.9) for a, b in
             [(0, 7), (7, 7), (7, 19), (19, 30)]]                     # includes an empty part
    out, lse = o.lse_merge(parts)
    np.testing.assert_allclose(out, full[0], atol=1e-13)
    np.testing.assert_allclose(lse, full[1], atol=1e-13)


def test_row_scale_multiplies_latent_only():
    c, r = _r((5, 4), 13), _r((5, 2), 14)
    sc = np.array([2.0, 0.5, 1.0, 3.0, 1.0])
    keys, vals = o.kv_rows(c, r, sc, np.array([3, 0]))
    np.testing.assert_array_equal(keys, [[*(3 * c[3]), *r[3]], [*(2 * c[0]), *r[0]]])
    np.testing.assert_array_equal(vals, [3 * c[3], 2 * c[0]])


def test_window_only_is_sliding_window_attention():
    T, d, H, w, pos = 40, 6, 3, 7, 29
    x, q = _r((T, d), 15), _r((H, d), 16)
    entries = _store(_r((10, d), 17))
    out, lse = o.csa_attend_one(q, entries, np.full(4, -1), _store(x), pos, w, 0.5)
    mask = np.zeros(T, bool)
    mask[pos - w + 1:pos + 1] = True
    t_out, t_lse = textbook(q, x, x, 0.5, mask)
    np.testing.assert_allclose(out, t_out, atol=1e-13)
    np.testing.assert_allclose(lse, t_lse, atol=1e-13)
    # Near the sequence start the window is clipped at position 0.
    out, _ = o.csa_attend_one(q, entries, np.full(4, -1), _store(x), 3, w, 0.5)
    t_out, _ = textbook(q, x[:4], x[:4], 0.5)
    np.testing.assert_allclose(out, t_out, atol=1e-13)


def test_topk_only_is_attention_over_gathered_rows():
    d_c, d_r, H = 8, 4, 5
    c, r, sc = _r((20, d_c), 18), _r((20, d_r), 19), np.abs(_r(20, 20)) + 0.5
    q = _r((H, d_c + d_r), 21)
    idx = np.array([2, 5, 11, 17, -1, -1])
    raw = _store(_r((50, d_c), 22), _r((50, d_r), 23), np.ones(50))
    out, lse = o.csa_attend_one(q, _store(c, r, sc), idx, raw, 49, 0, 0.7)
    sel = [2, 5, 11, 17]
    keys = np.concatenate([c[sel] * sc[sel, None], r[sel]], axis=1)
    t_out, t_lse = textbook(q, keys, c[sel] * sc[sel, None], 0.7)
    np.testing.assert_allclose(out, t_out, atol=1e-13)
    np.testing.assert_allclose(lse, t_lse, atol=1e-13)


def _dense_causal(q, x, pos, scale):
    mask = np.arange(x.shape[0]) <= pos
    return textbook(q, x, x, scale, mask)


def test_m1_full_topk_no_window_is_dense_causal_attention():
    T, d, H, pos = 24, 5, 2, 17
    x, g = _r((T, d), 24), _r((T, d), 25)
    entries = o.compress(x, g, np.array([0.3]), 1)                # identity pooling
    q = _r((H, d), 26)
    nv = o.n_visible(pos, 1, T)
    idx, _ = o.topk(o.index_scores(_r((2, 3), 27), _r(2, 28), _r((T, 3), 29), nv), nv, T)
    out, lse = o.csa_attend_one(q, _store(entries), idx, _store(x), pos, 0, 0.6)
    t_out, t_lse = _dense_causal(q, x, pos, 0.6)
    np.testing.assert_allclose(out, t_out, atol=1e-13)
    np.testing.assert_allclose(lse, t_lse, atol=1e-13)
    # With a window the window rows enter a second time (no de-duplication).
    w = 5
    out, _ = o.csa_attend_one(q, _store(entries), idx, _store(x), pos, w, 0.6)
    multiset = np.concatenate([x[:pos + 1], x[pos - w + 1:pos + 1]], axis=0)
    t_out, _ = textbook(q, multiset, multiset, 0.6)
    np.testing.assert_allclose(out, t_out, atol=1e-13)


def test_hca_m1_is_dense_causal_and_matches_csa_full_selection():
    T, d_c, d_r, H = 30, 6, 2, 3
    x = _r((T, d_c + d_r), 30)
    q = _r((H, d_c + d_r), 31)
    ent = _store(x[:, :d_c], x[:, d_c:])
    for pos in (0, 13, 29):
        out, lse = o.hca_attend_one(q, ent, pos, 1, 0.8)
        t_out, t_lse = textbook(q, x, x[:, :d_c], 0.8, np.arange(T) <= pos)
        np.testing.assert_allclose(out, t_out, atol=1e-13)
        np.testing.assert_allclose(lse, t_lse, atol=1e-13)
    # HCA with m' equals CSA with k >= N and no window over the same entries.
    xr, gr = _r((8 * 9 + 3, d_c + d_r), 32), _r((8 * 9 + 3, d_c + d_r), 33)
    e = o.compress(xr, gr, _r(8, 34), 8)
    ent = _store(e[:, :d_c], e[:, d_c:])
    raw = _store(xr[:, :d_c], xr[:, d_c:])
    for pos in (6, 7, 40, 74):
        nv = o.n_visible(pos, 8, e.shape[0])
        a = o.hca_attend_one(q, ent, pos, 8, 0.8)
        b = o.csa_attend_one(q, ent, np.concatenate([np.arange(nv), -np.ones(20, int)]), raw,
                             pos, 0, 0.8)
        np.testing.assert_allclose(a[0], b[0], atol=1e-13)
        np.testing.assert_array_equal(a[1], b[1]) if nv == 0 else \
            np.testing.assert_allclose(a[1], b[1], atol=1e-13)


def test_hca_query_before_first_block_sees_nothing():
    ent = _store(_r((4, 3), 35))
    out, lse = o.hca_attend_one(_r((2, 3), 36), ent, 126, 128, 1.0)
    assert (out == 0).all() and (lse == -np.inf).all()


def test_window_longer_than_ring_raises():
    with pytest.raises(ValueError):
        o.window_rows(pos=100, window=11, pos0=0, n_rows=10)


def test_window_ring_rows_worked_example():
    # Ring of 5 rows, offset 2: position p in row (p - 2) mod 5. Window of 4 at position 9:
    # positions 6, 7, 8, 9 -> rows 4, 0, 1, 2.
    assert o.window_rows(pos=9, window=4, pos0=2, n_rows=5).tolist() == [4, 0, 1, 2]
    # A store holding every position from pos0 on: no wrap.
    assert o.window_rows(pos=9, window=4, pos0=3, n_rows=100).tolist() == [3, 4, 5, 6]


def test_ring_store_equals_linear_store():
    # A ring of R >= window rows, written token by token (row p mod R), holds the same window as
    # the store of every position: CSA attention over either is the same.
    T, d, H, R, w = 41, 6, 3, 7, 5
    x = _r((T, d), 40)
    ring = np.zeros((R, d))
    for p in range(T):
        ring[p % R] = x[p]
    q = _r((H, d), 41)
    e = _r((6, d), 42)
    ent = _store(e[:, :4], e[:, 4:])
    idx = np.array([0, 3, 5])
    a = o.csa_attend_one(q, ent, idx, _store(x[:, :4], x[:, 4:]), T - 1, w, 0.7)
    b = o.csa_attend_one(q, ent, idx, _store(ring[:, :4], ring[:, 4:]), T - 1, w, 0.7)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# ---- token selection: the original tokens of the selected blocks ---------------------------
# hongke120.com 2.2 item 3; yudonglee.me "DeepSeek-V4 详解" 2.2 Steps 3-4.

def test_tokens_m1_equals_entry_attention():
    # With m = 1 every block is one token and pooling is the identity (compress pin), so token
    # selection over the raw rows equals entry selection over the m = 1 entries.
    T, d, H = 30, 5, 3
    x, g = _r((T, d), 60), _r((T, d), 61)
    e = o.compress(x, g, np.array([0.3]), 1)
    q = _r((H, d), 62)
    idx = np.array([1, 4, -1, 9, 17])
    raw = _store(x[:, :3], x[:, 3:])
    a = o.csa_attend_tokens_one(q, raw, idx, 1, 25, 4, 0.6)
    b = o.csa_attend_one(q, _store(e[:, :3], e[:, 3:]), idx, raw, 25, 4, 0.6)
    np.testing.assert_allclose(a[0], b[0], atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], atol=1e-14)


def test_tokens_brute_force_against_textbook():
    # m = 4: blocks 2 and 5 give positions 8..11 and 20..23, then the window 26..29 (position 29
    # is the query); textbook attention over exactly that multiset of rows.
    T, d, H, m = 30, 6, 4, 4
    x = _r((T, d), 63)
    q = _r((H, d), 64)
    out, lse = o.csa_attend_tokens_one(q, _store(x[:, :4], x[:, 4:]), np.array([5, -1, 2]), m,
                                       29, 4, 0.45)
    rows = [20, 21, 22, 23, 8, 9, 10, 11, 26, 27, 28, 29]
    want_o, want_l = textbook(q, x[rows], x[rows][:, :4], 0.45)
    np.testing.assert_allclose(out, want_o, atol=1e-13)
    np.testing.assert_allclose(lse, want_l, atol=1e-13)


def test_tokens_store_offset_and_missing_rows():
    T, d, m = 24, 4, 4
    x = _r((T, d), 65)
    q = _r((2, d), 66)
    full = o.csa_attend_tokens_one(q, _store(x[:, :2], x[:, 2:]), np.array([3, 4]), m, 23, 3, 1.0)
    part = o.csa_attend_tokens_one(q, _store(x[8:, :2], x[8:, 2:], None, 8), np.array([3, 4]), m,
                                   23, 3, 1.0)
    np.testing.assert_array_equal(full[0], part[0])
    with pytest.raises(ValueError):
        o.csa_attend_tokens_one(q, _store(x[8:, :2], x[8:, 2:], None, 8), np.array([1]), m, 23, 3,
                                1.0)
