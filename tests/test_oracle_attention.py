"""Pins for the fp64 attention oracle (CPU only).

Each pin is independent of the oracle's own code: hand-derived closed forms
(tests/golden/attention_closed_forms.json), torch's fp64 scaled_dot_product_attention
(a library routine), and invariants that softmax attention satisfies exactly.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "attention_closed_forms.json")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _sdpa(q, k, v, scale):
    """torch fp64 SDPA on token-major [B, N, H, D] -> token-major output."""
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    logits = torch.einsum("bhid,bhjd->bhij", tq, tk) * scale
    lse = torch.logsumexp(logits, dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy()


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_closed_forms(case):
    q, k, v = (np.array(case[x], dtype=np.float64) for x in ("q", "k", "v"))
    o, lse = oracle.attention_rows(q, k, v, case["scale"], case["q_rows"])
    np.testing.assert_allclose(o, np.array(case["O"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, np.array(case["lse"]), rtol=0, atol=1e-13)


@pytest.mark.parametrize("B,N,H,D", [(2, 37, 3, 16), (1, 1, 1, 8), (1, 130, 2, 64), (2, 65, 1, 128)])
def test_matches_torch_sdpa_fp64(B, N, H, D):
    q, k, v = _rand((B, N, H, D), 1), _rand((B, N, H, D), 2), _rand((B, N, H, D), 3)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attention(q, k, v, scale)
    o_ref, lse_ref = _sdpa(q, k, v, scale)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_bf16_inputs_match_torch_on_widened_values():
    rng = np.random.default_rng(5)
    shape = (1, 50, 2, 64)
    bits = [torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)
            .view(torch.int16).numpy().view(np.uint16) for _ in range(3)]
    scale = 0.125
    o, lse = oracle.attention(*bits, scale)
    wide = [oracle.widen_bf16(b) for b in bits]
    o_ref, lse_ref = _sdpa(*wide, scale)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_widen_bf16_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.widen_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    finite = np.isfinite(ref)
    assert np.array_equal(mine[finite], ref[finite])
    assert np.array_equal(np.isnan(mine), np.isnan(ref))


def test_large_logits_do_not_overflow():
    q = _rand((1, 20, 1, 32), 7, 30.0)
    k = _rand((1, 20, 1, 32), 8, 30.0)
    v = _rand((1, 20, 1, 32), 9)
    o, lse = oracle.attention(q, k, v, 1.0)
    o_ref, lse_ref = _sdpa(q, k, v, 1.0)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-11)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-14)


def test_rows_are_probability_vectors():
    # V = identity (D = N) makes each output row the softmax row itself.
    N = 24
    q, k = _rand((1, N, 1, N), 11), _rand((1, N, 1, N), 12)
    v = np.eye(N).reshape(1, N, 1, N)
    o, _ = oracle.attention(q, k, v, 0.4)
    assert (o >= 0).all()
    np.testing.assert_allclose(o.sum(axis=-1), 1.0, rtol=0, atol=1e-14)


def test_zero_query_gives_mean_of_values():
    q = np.zeros((2, 33, 2, 16))
    k, v = _rand(q.shape, 13), _rand(q.shape, 14)
    o, lse = oracle.attention(q, k, v, 0.25)
    mean = v.mean(axis=1, keepdims=True)
    np.testing.assert_allclose(o, np.broadcast_to(mean, o.shape), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse, math.log(33), rtol=1e-15)


def test_key_value_permutation_invariance():
    q, k, v = _rand((1, 40, 2, 16), 15), _rand((1, 40, 2, 16), 16), _rand((1, 40, 2, 16), 17)
    perm = np.random.default_rng(18).permutation(40)
    o1, l1 = oracle.attention(q, k, v, 0.3)
    o2, l2 = oracle.attention(q, k[:, perm], v[:, perm], 0.3)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-14)
    # permuting only the values must change the result (guards against a swapped operand)
    o3, _ = oracle.attention(q, k, v[:, perm], 0.3)
    assert np.abs(o3 - o1).max() > 1e-3


def test_common_key_shift_is_invisible():
    q, k, v = _rand((1, 30, 1, 8), 19), _rand((1, 30, 1, 8), 20), _rand((1, 30, 1, 8), 21)
    u = _rand((8,), 22)
    o1, l1 = oracle.attention(q, k, v, 0.5)
    o2, l2 = oracle.attention(q, k + u, v, 0.5)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    shift = 0.5 * np.einsum("bnhd,d->bhn", q, u)
    np.testing.assert_allclose(l2 - l1, shift, rtol=0, atol=1e-12)


def test_constant_and_linear_in_values():
    q, k = _rand((1, 25, 2, 8), 23), _rand((1, 25, 2, 8), 24)
    o, _ = oracle.attention(q, k, np.full(q.shape, 2.5), 0.6)
    np.testing.assert_allclose(o, 2.5, rtol=1e-14)
    v1, v2 = _rand(q.shape, 25), _rand(q.shape, 26)
    o1, _ = oracle.attention(q, k, v1, 0.6)
    o2, _ = oracle.attention(q, k, v2, 0.6)
    o12, _ = oracle.attention(q, k, 3.0 * v1 - 2.0 * v2, 0.6)
    np.testing.assert_allclose(o12, 3.0 * o1 - 2.0 * o2, rtol=0, atol=1e-13)


def test_split_keys_merge_by_lse():
    # attention over keys A u B equals the lse-weighted merge of attention over A and B
    q, k, v = _rand((1, 20, 1, 16), 27), _rand((1, 50, 1, 16), 28), _rand((1, 50, 1, 16), 29)
    scale = 0.25
    sel = np.array([[0, 0, i] for i in range(20)])
    o_all, l_all = oracle.attention_rows(q, k, v, scale, sel)
    oa, la = oracle.attention_rows(q, k[:, :30], v[:, :30], scale, sel)
    ob, lb = oracle.attention_rows(q, k[:, 30:], v[:, 30:], scale, sel)
    lm = np.logaddexp(la, lb)
    merged = (np.exp(la - lm)[:, None] * oa + np.exp(lb - lm)[:, None] * ob)
    np.testing.assert_allclose(merged, o_all, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lm, l_all, rtol=1e-14)


def test_sharp_query_selects_argmax_value():
    q, k, v = _rand((1, 16, 1, 8), 30), _rand((1, 16, 1, 8), 31), _rand((1, 16, 1, 8), 32)
    o, _ = oracle.attention(q, k, v, 1e4)
    logits = np.einsum("id,jd->ij", q[0, :, 0], k[0, :, 0])
    np.testing.assert_allclose(o[0, :, 0], v[0, logits.argmax(axis=1), 0], rtol=0, atol=1e-9)


def test_batch_head_slices_are_independent():
    q, k, v = _rand((2, 12, 3, 8), 33), _rand((2, 12, 3, 8), 34), _rand((2, 12, 3, 8), 35)
    o1, l1 = oracle.attention(q, k, v, 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[1, :, 2] += 5.0
    v2[1, :, 2] *= -3.0
    o2, l2 = oracle.attention(q, k2, v2, 0.5)
    mask = np.ones((2, 3), bool)
    mask[1, 2] = False
    for b in range(2):
        for h in range(3):
            same = np.array_equal(o1[b, :, h], o2[b, :, h])
            assert same == mask[b, h]


def test_rejects_bad_rows():
    q = np.zeros((1, 4, 1, 2))
    with pytest.raises(RuntimeError):
        oracle.attention_rows(q, q, q, 1.0, [[0, 0, 4]])
