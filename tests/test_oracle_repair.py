"""Pins for the token-repair oracle (CPU only).

Pins: the repair budget on the pages' rho = 0.005 at the workload sizes; the error
measure on a hand-worked block (a normal and a subnormal-range tie); the selection
against its rank-counting definition on random inputs with planted ties; fp8 attention
with repaired tokens on a two-key case worked by hand; no repaired token gives the plain
fp8 oracle bit for bit; every token repaired gives exact logits, hence the lse of the
fp64 C oracle.
"""
import math

import numpy as np
import pytest

import oracle


def _bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_repair_count():
    assert oracle.repair_count(16896, 0.005) == 85      # ceil(84.48), 2048^2 T2I
    assert oracle.repair_count(4608, 0.005) == 24       # ceil(23.04), 1024^2 T2I
    assert oracle.repair_count(33280, 0.005) == 167     # ceil(166.4), 2048^2 I2I
    assert oracle.repair_count(200, 0.005) == 1         # rho * N rounds to exactly 1.0
    assert oracle.repair_count(77, 0.0) == 0 and oracle.repair_count(77, 1.0) == 77
    assert oracle.repair_count(0, 0.5) == 0
    with pytest.raises(ValueError):
        oracle.repair_count(10, 1.5)


def test_residual_linf_hand_block():
    # one block, amax 3.5 -> scale 2**-7 (3.5 * 128 = 448); codes = e4m3(x * 128)
    x = np.zeros((1, 4, 1, 2), np.float32)
    x[0, :, 0, :] = [[3.5, 1 + 2 ** -7],     # 129 -> 128 (step 16): residual 2**-7
                     [-3.5, 0.75],           # 96 on the grid: 0
                     [2 ** -7, -1.5],        # 1 and -192 on the grid: 0
                     [2 ** -14 + 2 ** -17, 0.0]]   # 4.5 * 2**-9 (subnormal step 2**-9):
                                                    # tie to even -> 4 * 2**-9, residual 2**-17
    codes, scales = oracle.quantise_qk(_bits(x))
    assert scales[0, 0, 0] == np.float32(2.0 ** -7)
    err = oracle.residual_linf(_bits(x), codes, scales)
    assert err.shape == (1, 1, 4)
    assert err[0, 0].tolist() == [2.0 ** -7, 0.0, 0.0, 2.0 ** -17]


@pytest.mark.parametrize("B,H,N,n,levels", [(1, 1, 10, 3, 3), (2, 3, 57, 5, 4),
                                             (1, 2, 300, 0, 5), (1, 2, 40, 40, 2),
                                             (2, 1, 129, 128, 1000)])
def test_selection_is_rank_definition(B, H, N, n, levels):
    # token i is chosen iff fewer than n tokens rank before it: larger error, or equal
    # error and a lower index (few levels -> many ties)
    rng = np.random.default_rng(N + n)
    err = rng.integers(0, levels, size=(B, H, N)).astype(np.float64) * 0.25
    sel = oracle.select_repair_tokens(err, n)
    for b in range(B):
        for h in range(H):
            want = [i for i in range(N)
                    if sum(1 for j in range(N)
                           if err[b, h, j] > err[b, h, i]
                           or (err[b, h, j] == err[b, h, i] and j < i)) < n]
            assert sel[b, h].tolist() == want


def _two_key_case():
    # K block: k0 = [3.5, 2], k1 = [1 + 2**-7, 0]   -> scale 2**-7, k1 rounds to [1, 0]
    # Q block: q0 = [1, 0],   q1 = [0.5, 17 * 2**-12] -> scale 2**-8, 17/16 -> 1 (tie to
    #          even), so q1 rounds to [0.5, 2**-8]
    # V: v0 = [1, 0], v1 = [0, 1] -> channel scales 2**-8, exact
    q = np.zeros((1, 2, 1, 2), np.float32)
    k = np.zeros((1, 2, 1, 2), np.float32)
    v = np.zeros((1, 2, 1, 2), np.float32)
    q[0, :, 0] = [[1.0, 0.0], [0.5, 17 * 2 ** -12]]
    k[0, :, 0] = [[3.5, 2.0], [1 + 2 ** -7, 0.0]]
    v[0, :, 0] = [[1.0, 0.0], [0.0, 1.0]]
    return _bits(q), _bits(k), _bits(v)


def test_two_key_case_by_hand():
    q, k, v = _two_key_case()
    q8, qs, qerr, qsel = oracle.quantise_qk_repair(q, 1)
    k8, ks, kerr, ksel = oracle.quantise_qk_repair(k, 1)
    v8, vs = oracle.quantise_v(v)
    assert qerr[0, 0].tolist() == [0.0, 2.0 ** -12] and qsel[0, 0].tolist() == [1]
    assert kerr[0, 0].tolist() == [0.0, 2.0 ** -7] and ksel[0, 0].tolist() == [1]
    # softmax_scale = ln 2 makes the base-2 logit t the plain dot product
    sel = np.array([[0, 0, 0], [0, 0, 1]])
    o, lse = oracle.fp8_attention_rows(q8, k8, v8, qs, ks, vs, math.log(2.0), sel,
                                       q_exact=q, k_exact=k, q_rep=qsel, k_rep=ksel)
    # row 0 (q0 not repaired, exact anyway): t = [3.5, 1 + 2**-7], M = 4,
    #   256 p = [181.02, 32.17] -> e4m3 [176, 32]
    # row 1 (q1 repaired): t = [1.75 + 17 * 2**-11, 0.5 + 2**-8], M = 2,
    #   256 p = [216.51, 90.76] -> e4m3 [224, 88]
    for r, (t, M, P) in enumerate([([3.5, 1 + 2 ** -7], 4, [176.0, 32.0]),
                                   ([1.75 + 17 * 2 ** -11, 0.5 + 2 ** -8], 2, [224.0, 88.0])]):
        l = math.fsum(2.0 ** (x - M) for x in t)
        assert np.allclose(o[r], np.array(P) / (256.0 * l), rtol=1e-14, atol=0)
        assert abs(lse[r] - (M + math.log2(l)) * math.log(2.0)) < 1e-13
    # without repair both rows differ (k1 -> 1.0, q1 -> [0.5, 2**-8])
    o0, _ = oracle.fp8_attention_rows(q8, k8, v8, qs, ks, vs, math.log(2.0), sel)
    assert np.abs(o0 - o).max() > 1e-4


def _workload(seed=3, N=300, D=64):
    from joint_attention_amd import synth
    w = synth.custom("rep", B=1, H=2, D=D, stream_lens=(40, N - 40), outliers=4, seed=seed)
    st = synth.make_streams(w)
    q, _ = oracle.pack_tokens(st.q)
    k, _ = oracle.pack_tokens(st.k)
    v, _ = oracle.pack_tokens(st.v)
    return w, q, k, v


def test_no_repair_is_plain_bitwise():
    w, q, k, v = _workload()
    q8, qs, _, qsel = oracle.quantise_qk_repair(q, 0)
    k8, ks, _, ksel = oracle.quantise_qk_repair(k, 0)
    v8, vs = oracle.quantise_v(v)
    sel = oracle.all_rows(w.B, w.N, w.H)
    a = oracle.fp8_attention_rows(q8, k8, v8, qs, ks, vs, 0.125, sel)
    b = oracle.fp8_attention_rows(q8, k8, v8, qs, ks, vs, 0.125, sel, q_exact=q, k_exact=k,
                                  q_rep=qsel, k_rep=ksel)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_all_repaired_gives_exact_lse():
    # every token repaired: the logits are the exact bf16 dot products, and the lse does
    # not depend on the e4m3 rounding of P or V -> equals the fp64 C oracle's
    w, q, k, v = _workload(seed=5)
    q8, qs, _, qsel = oracle.quantise_qk_repair(q, w.N)
    k8, ks, _, ksel = oracle.quantise_qk_repair(k, w.N)
    v8, vs = oracle.quantise_v(v)
    sel = oracle.all_rows(w.B, w.N, w.H)
    scale = 1.0 / math.sqrt(w.D)
    o, lse = oracle.fp8_attention_rows(q8, k8, v8, qs, ks, vs, scale, sel, q_exact=q,
                                       k_exact=k, q_rep=qsel, k_rep=ksel)
    ref, ref_lse = oracle.attention_rows(q, k, v, scale, sel)
    assert np.abs(lse - ref_lse).max() <= 1e-12 * np.abs(ref_lse).max()
    # O keeps only the e4m3 roundings of P and V (3 mantissa bits each)
    assert np.linalg.norm(o - ref) / np.linalg.norm(ref) < 0.06


def test_repair_moves_towards_exact():
    # repairing the worst tokens lowers the error against the exact result
    w, q, k, v = _workload(seed=7, N=512)
    sel = oracle.all_rows(w.B, w.N, w.H)
    scale = 1.0 / math.sqrt(w.D)
    ref, _ = oracle.attention_rows(q, k, v, scale, sel)
    v8, vs = oracle.quantise_v(v)
    errs = []
    for n in (0, 26, 128):
        q8, qs, _, qsel = oracle.quantise_qk_repair(q, n)
        k8, ks, _, ksel = oracle.quantise_qk_repair(k, n)
        o, _ = oracle.fp8_attention_rows(q8, k8, v8, qs, ks, vs, scale, sel, q_exact=q,
                                         k_exact=k, q_rep=qsel, k_rep=ksel)
        errs.append(np.linalg.norm(o - ref) / np.linalg.norm(ref))
    assert errs[0] > errs[1] > errs[2], errs
