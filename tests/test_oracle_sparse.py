"""Pins of the block-sparse oracle: against the dense oracle, key subsets, empty rows and a
hand-derived case."""
import math

import numpy as np

import oracle


def _rand(B, N, H, D, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, N, H, D)) for _ in range(3)]


def test_all_ones_mask_equals_dense():
    q, k, v = _rand(2, 300, 2, 16, 1)
    mask = np.ones((2, 2) + oracle.mask_shape(300), np.uint8)
    sel = oracle.all_rows(2, 300, 2)
    o, l = oracle.sparse_attention_rows(q, k, v, 0.25, mask, sel)
    od, ld = oracle.attention_rows(q, k, v, 0.25, sel)
    np.testing.assert_allclose(o, od, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l, ld, rtol=1e-12)


def test_one_block_equals_dense_on_that_key_subset():
    # query block 1 may only see key block 2 (keys 256 .. 299): dense attention over the
    # sliced keys; query block 0 sees blocks 0 and 2
    B, N, H, D = 1, 300, 1, 8
    q, k, v = _rand(B, N, H, D, 2)
    mask = np.zeros((1, 1) + oracle.mask_shape(N), np.uint8)
    mask[0, 0, 1, 2] = 1
    mask[0, 0, 0, [0, 2]] = 1
    rows = np.arange(128, 256)
    sel = np.stack([np.zeros_like(rows), np.zeros_like(rows), rows], 1)
    o, l = oracle.sparse_attention_rows(q, k, v, 0.3, mask, sel)
    keys = np.arange(256, 300)
    od, ld = oracle.attention_rows(q[:, 128:256], k[:, keys], v[:, keys], 0.3,
                                   np.stack([np.zeros(128, int), np.zeros(128, int),
                                             np.arange(128)], 1))
    np.testing.assert_allclose(o, od, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l, ld, rtol=1e-12)
    rows0 = np.arange(0, 128)
    keys0 = np.concatenate([np.arange(0, 128), np.arange(256, 300)])
    o0, _ = oracle.sparse_attention_rows(q, k, v, 0.3, mask,
                                         np.stack([0 * rows0, 0 * rows0, rows0], 1))
    od0, _ = oracle.attention_rows(q[:, :128], k[:, keys0], v[:, keys0], 0.3,
                                   np.stack([0 * rows0, 0 * rows0, rows0], 1))
    np.testing.assert_allclose(o0, od0, rtol=1e-12, atol=1e-12)


def test_empty_row_gives_zero_and_minus_inf():
    q, k, v = _rand(1, 200, 1, 4, 3)
    mask = np.ones((1, 1) + oracle.mask_shape(200), np.uint8)
    mask[0, 0, 1, :] = 0                      # rows 128 .. 199 see nothing
    o, l = oracle.sparse_attention_rows(q, k, v, 1.0, mask, [[0, 0, 150], [0, 0, 5]])
    assert np.all(o[0] == 0) and l[0] == -np.inf
    assert np.isfinite(l[1]) and np.any(o[1] != 0)


def test_hand_case_two_allowed_keys():
    # bq = bk = 1 so the mask is per key: row 0 sees keys 1 and 2 only, scale 1:
    # s = [1, 0], weights e/(e+1), 1/(e+1), O = (e*v1 + v2)/(e+1), lse = ln(e + 1)
    q = np.zeros((1, 3, 1, 2)); k = np.zeros((1, 3, 1, 2)); v = np.zeros((1, 3, 1, 2))
    q[0, 0, 0] = [1, 0]
    k[0, 0, 0] = [5, 5]; k[0, 1, 0] = [1, 3]; k[0, 2, 0] = [0, 7]
    v[0, 0, 0] = [100, 100]; v[0, 1, 0] = [2, 0]; v[0, 2, 0] = [0, 4]
    mask = np.array([[[[0, 1, 1], [1, 1, 1], [1, 1, 1]]]], np.uint8)
    o, l = oracle.sparse_attention_rows(q, k, v, 1.0, mask, [[0, 0, 0]], bq=1, bk=1)
    e = math.e
    np.testing.assert_allclose(o[0], [2 * e / (e + 1), 4 / (e + 1)], rtol=1e-14)
    np.testing.assert_allclose(l[0], math.log(e + 1), rtol=1e-14)
