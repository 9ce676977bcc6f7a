"""Pins for the reference e4m3 codec, quantiser and fp8 attention (CPU only).

Pins: hand-derived e4m3 codes from the OCP FP8 definition (tests/golden/e4m3_codes.json),
torch's float8_e4m3fn casts (a library routine) over every code and over all rounding
boundaries, hand-derived quantiser cases, an fp8-attention case worked by hand, and a
case where every fp8 rounding is exact so the fp8 attention must equal the fp64 oracle.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_codes.json")


def _torch_e4m3(x32: np.ndarray) -> np.ndarray:
    """torch's cast (ties-to-even); callers clamp first because torch gives NaN past 464."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_hand_codes():
    for value, code, why in json.load(open(GOLDEN))["values"]:
        got = int(oracle.e4m3_encode(np.array([value]))[0])
        assert got == code, (value, why)
        if value not in (464.0, 1.0e6) and abs(value) <= 448 and why.find("tie") < 0 \
                and why.find("nearer") < 0:
            assert oracle.e4m3_decode(np.array([code], np.uint8))[0] == value


def test_decode_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.isnan(mine).sum() == 2                      # 0x7F and 0xFF


def test_encode_rounding_boundaries_match_torch():
    # every representable value, every midpoint between neighbours, and 1 ulp (binary32)
    # either side of each: these are all the places where rounding can go wrong
    vals = oracle.e4m3_decode(np.arange(0, 127, dtype=np.uint8))      # 0 .. 448
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids]).astype(np.float32)
    around = np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)),
                             np.nextafter(pts, np.float32(-np.inf))])
    around = around[np.abs(around) <= 448]
    x = np.concatenate([around, -around]).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(x), _torch_e4m3(x))


def test_encode_random_and_clamp_match_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000) * 50,
        np.exp2(rng.uniform(-20, 9, 200000)) * rng.choice([-1, 1], 200000),
        rng.uniform(-600, 600, 50000),
    ]).astype(np.float32)
    clamped = np.clip(x, -448, 448)
    assert np.array_equal(oracle.e4m3_encode(x), _torch_e4m3(clamped))


def _bits(x):
    """float values that are exact in bf16 -> bf16 bit patterns."""
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_quantise_qk_hand_case():
    # one (b, h), block amax 7 -> scale = 7/448 = 2**-6 exactly, inverse 64
    x = np.zeros((1, 3, 1, 2), np.float32)
    x[0, :, 0, :] = [[7.0, 1.0], [-3.5, 0.0], [0.5, -7.0]]
    codes, scales = oracle.quantise_qk(_bits(x))
    assert scales.shape == (1, 1, 1) and scales[0, 0, 0] == np.float32(2.0 ** -6)
    # 7*64 = 448 -> 0x7E; 1*64 = 64 -> exponent 13 -> 0x68; -3.5*64 = -224 -> 0xF6;
    # 0.5*64 = 32 -> exponent 12 -> 0x60; -7*64 -> 0xFE
    assert codes[0, :, 0, :].tolist() == [[0x7E, 0x68], [0xF6, 0x00], [0x60, 0xFE]]


def test_quantise_qk_blocks_follow_packed_tokens():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 130, 3, 8)).astype(np.float32)
    x[1, 128:, 2, :] *= 1e-3                               # a short, quiet last block
    codes, scales = oracle.quantise_qk(_bits(x))
    assert scales.shape == (2, 3, 2)
    xw = oracle.widen_bf16(_bits(x))
    for b in range(2):
        for h in range(3):
            for blk, (lo, hi) in enumerate([(0, 128), (128, 130)]):
                amax = np.abs(xw[b, lo:hi, h]).max()
                sc = float(scales[b, h, blk])
                assert sc == 2.0 ** round(math.log2(sc))          # a power of two
                assert amax <= 448 * sc and amax > 224 * sc       # the smallest that fits
    # the block's largest element lands in (224, 448]
    top = np.abs(xw[1, 128:, 2]).argmax()
    assert (codes[1, 128:, 2].ravel()[top] & 0x7F) >= 0x76            # 224 = 0x76
    deq = oracle.e4m3_decode(codes) * np.repeat(scales, [128, 2], axis=2).transpose(0, 2, 1)[..., None]
    rel = np.abs(deq - xw) / np.maximum(np.abs(xw), 1e-30)
    assert rel[np.abs(xw) > np.repeat(scales, [128, 2], axis=2).transpose(0, 2, 1)[..., None] * 2 ** -6].max() <= 2 ** -4


def test_pow2_scale_hand_values():
    # smallest power of two s with amax <= 448 s: 448 -> 1, 449 -> 2, 7 = 448/64 -> 2^-6,
    # 7.01 -> 2^-5, 1 -> 2^-8 (448/256 = 1.75 >= 1 > 448/512), 0.875 = 448/512 -> 2^-9,
    # 0 -> 1, a denormal -> 2^-126 (the floor)
    amax = [448.0, 449.0, 7.0, 7.01, 1.0, 0.875, 0.0, 1e-45]
    want = [1.0, 2.0, 2.0 ** -6, 2.0 ** -5, 2.0 ** -8, 2.0 ** -9, 1.0, 2.0 ** -126]
    assert oracle.pow2_scale(np.array(amax)).tolist() == [np.float32(w) for w in want]


def test_quantise_zero_block_and_channel():
    x = np.zeros((1, 4, 1, 3), np.float32)
    x[0, :, 0, 1] = [1.0, -2.0, 0.5, 0.25]
    codes, scales = oracle.quantise_qk(_bits(x))
    assert scales[0, 0, 0] == np.float32(2.0 ** -7)           # 2 <= 448 * 2^-7 = 3.5
    vcodes, vscales = oracle.quantise_v(_bits(x))
    assert vscales[0, 0].tolist() == [1.0, 2.0 ** -7, 1.0]    # amax 0 -> 1
    assert (vcodes[0, :, 0, 0] == 0).all() and (vcodes[0, :, 0, 2] == 0).all()
    # channel 1: -2 / 2^-7 = -256 -> 0xF8; 1 -> 128 -> 0x70; 0.5 -> 64 -> 0x68
    assert vcodes[0, 1, 0, 1] == 0xF8 and vcodes[0, 0, 0, 1] == 0x70
    assert vcodes[0, 2, 0, 1] == 0x68


def test_fp8_attention_hand_case():
    # one query (code 1.0), keys 0 and 0.5, values 1 and 2, all scales 1, scale = ln 2 so
    # logits in base 2 are t = [0, 0.5]; M = ceil(0.5) = 1; p = [2^-1, 2^-0.5];
    # 2^8 p = [128, 181.02] -> e4m3 [128, 176];
    # O = (128*1 + 176*2) / (256 * (0.5 + 2^-0.5)); lse = ln(1 + sqrt 2)
    q8 = np.array([0x38, 0x00], np.uint8).reshape(1, 2, 1, 1)
    k8 = np.array([0x00, 0x30], np.uint8).reshape(1, 2, 1, 1)
    v8 = np.array([0x38, 0x40], np.uint8).reshape(1, 2, 1, 1)
    one = np.ones((1, 1, 1), np.float32)
    o, lse = oracle.fp8_attention_rows(q8, k8, v8, one, one, one, math.log(2.0), [[0, 0, 0]])
    assert o[0, 0] == pytest.approx(480.0 / (256.0 * (0.5 + 2 ** -0.5)), rel=1e-15)
    assert lse[0] == pytest.approx(math.log(1 + math.sqrt(2.0)), rel=1e-15)


def test_fp8_attention_equals_fp64_when_every_rounding_is_exact():
    # integer base-2 logits in [-6, 2] make every 2^8 * 2^(t - M) a power of two >= 4, which
    # e4m3 holds exactly; then the fp8 attention must equal plain attention on the
    # dequantised inputs.  Scales are powers of two (q) and arbitrary (v).
    rng = np.random.default_rng(3)
    N, D = 40, 4
    ints = rng.integers(-6, 3, size=N).astype(np.float64)
    q = np.zeros((1, N, 1, D)); q[0, :, 0, 0] = 1.0
    k = np.zeros((1, N, 1, D)); k[0, :, 0, 0] = ints
    q8 = oracle.e4m3_encode(q * 2.0)                         # q_scale 0.5 undoes the 2
    k8 = oracle.e4m3_encode(k)
    v8 = rng.integers(0, 126, size=(1, N, 1, D)).astype(np.uint8) | (rng.integers(0, 2, size=(1, N, 1, D)) << 7).astype(np.uint8)
    qs = np.full((1, 1, 1), 0.5, np.float32)
    ks = np.ones((1, 1, 1), np.float32)
    vs = np.array([[[0.37, 1.5, 2.0 ** -5, 3.0]]], np.float32)
    sel = [[0, 0, i] for i in range(N)]
    o8, l8 = oracle.fp8_attention_rows(q8, k8, v8, qs, ks, vs, math.log(2.0), sel)
    qd = oracle.e4m3_decode(q8) * 0.5
    kd = oracle.e4m3_decode(k8)
    vd = oracle.e4m3_decode(v8) * vs.astype(np.float64)[:, None, :, :]
    o64, l64 = oracle.attention_rows(qd, kd, vd, math.log(2.0), sel)
    np.testing.assert_allclose(o8, o64, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(l8, l64, rtol=1e-14)


def test_fp8_attention_rounding_of_p_is_visible():
    # with non-integer logits the e4m3 rounding of P must move the result a little,
    # by less than e4m3's relative step, and the lse must not move at all
    rng = np.random.default_rng(4)
    N, D = 64, 8
    x = rng.standard_normal((1, N, 1, D)).astype(np.float32)
    bits = _bits(x)
    q8, qs = oracle.quantise_qk(bits)
    k8, ks = oracle.quantise_qk(_bits(rng.standard_normal((1, N, 1, D)).astype(np.float32)))
    v8, vs = oracle.quantise_v(_bits(rng.standard_normal((1, N, 1, D)).astype(np.float32)))
    sel = [[0, 0, i] for i in range(N)]
    scale = 1 / math.sqrt(D)
    o8, l8 = oracle.fp8_attention_rows(q8, k8, v8, qs, ks, vs, scale, sel)
    qd = oracle.e4m3_decode(q8) * qs[0, 0, 0]
    kd = oracle.e4m3_decode(k8) * ks[0, 0, 0]
    vd = oracle.e4m3_decode(v8) * vs[:, None, :, :].astype(np.float64)
    o64, l64 = oracle.attention_rows(qd, kd, vd, scale, sel)
    np.testing.assert_allclose(l8, l64, rtol=1e-13)
    err = np.abs(o8 - o64).max()
    assert 1e-6 < err < 2 ** -4 * np.abs(vd).max()


def test_fp8_attention_integer_max_is_the_ceiling():
    # one key with base-2 logit t = 0.875 (exact in e4m3: q = 1, k = 0.875):
    # M = ceil(0.875) = 1, p = 2^-0.125 = 0.917, 2^8 p = 234.8 -> e4m3 240 (spacing 16),
    # so O = v * 240 / (256 * 2^-0.125).  (With the floor, 2^8 p = 469.7 would clamp to 448.)
    q8 = np.array([0x38], np.uint8).reshape(1, 1, 1, 1)
    k8 = oracle.e4m3_encode(np.array([0.875])).reshape(1, 1, 1, 1)
    v8 = np.array([0x38], np.uint8).reshape(1, 1, 1, 1)
    one = np.ones((1, 1, 1), np.float32)
    o, lse = oracle.fp8_attention_rows(q8, k8, v8, one, one, one, math.log(2.0), [[0, 0, 0]])
    assert o[0, 0] == pytest.approx(240.0 / (256.0 * 2 ** -0.125), rel=1e-15)
    assert lse[0] == pytest.approx(0.875 * math.log(2.0), rel=1e-15)


def test_fp8_attention_uses_each_rows_block_scales():
    # 200 tokens = two Q/K scale blocks (128 + 72) with different power-of-two scales;
    # integer base-2 logits keep every rounding exact, so the result must equal fp64
    # attention on the dequantised operands -- only if each token takes its own block's scale
    rng = np.random.default_rng(6)
    N, D = 200, 4
    ints = rng.integers(-5, 3, size=N).astype(np.float64)
    qs = np.array([[[0.5, 0.25]]], np.float32)
    ks = np.array([[[2.0, 4.0]]], np.float32)
    blk = np.arange(N) // 128
    qv = np.zeros((1, N, 1, D)); qv[0, :, 0, 1] = 1.0
    kv = np.zeros((1, N, 1, D)); kv[0, :, 0, 1] = ints
    q8 = oracle.e4m3_encode(qv / qs[0, 0, blk][None, :, None, None])
    k8 = oracle.e4m3_encode(kv / ks[0, 0, blk][None, :, None, None])
    v8 = rng.integers(0, 126, size=(1, N, 1, D)).astype(np.uint8)
    vs = np.array([[[1.0, 0.5, 3.0, 0.1]]], np.float32)
    sel = [[0, 0, i] for i in (0, 127, 128, 199)]
    o8, l8 = oracle.fp8_attention_rows(q8, k8, v8, qs, ks, vs, math.log(2.0), sel)
    vd = oracle.e4m3_decode(v8) * vs.astype(np.float64)[:, None, :, :]
    o64, l64 = oracle.attention_rows(qv, kv, vd, math.log(2.0), sel)
    np.testing.assert_allclose(o8, o64, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(l8, l64, rtol=1e-14)


def test_select_hi_channels_hand_case():
    # channel scores amax|q| * amax|k|: c0 = 1*1, c1 = 8*8 (outlier), c2 = 2*3, c3 = 3*2 (tie
    # with c2: lower index wins); r = 2 keeps {1, 2}
    q = np.zeros((1, 3, 1, 4), np.float32)
    k = np.zeros((1, 3, 1, 4), np.float32)
    q[0, :, 0, :] = [[1, -8, 2, 3], [0.5, 4, -1, 1], [0, 1, 1, -2]]
    k[0, :, 0, :] = [[1, 1, 3, -2], [-0.5, 8, 1, 1], [0, 1, 1, 1]]
    assert oracle.select_hi_channels(_bits(q), _bits(k), r=2).tolist() == [[[1, 2]]]


def test_quantise_split_zeroes_codes_and_keeps_exact_values():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, 130, 2, 8)).astype(np.float32)
    sel = np.array([[[1, 5], [0, 7]]], np.int32)
    bits = _bits(x)
    codes, scales, hi = oracle.quantise_qk_split(bits, sel)
    c0, s0 = oracle.quantise_qk(bits)
    assert np.array_equal(scales, s0)
    xw = oracle.widen_bf16(bits)
    for h in range(2):
        others = [c for c in range(8) if c not in sel[0, h]]
        assert (codes[0, :, h, sel[0, h]] == 0).all()
        assert np.array_equal(codes[0, :, h, others], c0[0, :, h, others])
        blk = np.arange(130) // 128
        back = hi[0, :, h, :] * scales[0, h, blk][:, None]
        assert np.array_equal(back, xw[0][:, h, sel[0, h]])      # exact


def test_fp8_split_mode_exact_case_equals_fp64():
    # 32 channels, 16 kept in the split; integer base-2 logits (scale ln 2) and values that
    # e4m3 holds exactly make every rounding exact, so the split-mode fp8 attention must
    # equal fp64 attention on the original values.  A missing block scale on the kept part,
    # or a kept channel also counted in the e4m3 part, breaks the equality.
    rng = np.random.default_rng(8)
    N, D = 150, 32
    q = np.zeros((1, N, 1, D)); k = np.zeros((1, N, 1, D))
    q[0, :, 0, 3] = 1.0; k[0, :, 0, 3] = rng.integers(-4, 2, N)        # kept channel
    q[0, :, 0, 20] = 2.0; k[0, :, 0, 20] = rng.integers(-2, 1, N) * 0.5  # e4m3 channel
    v = oracle.e4m3_decode(rng.integers(0, 120, (1, N, 1, D)).astype(np.uint8))
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    sel = np.array([[list(range(0, 16))]], np.int32)
    q8, qs, qh = oracle.quantise_qk_split(qb, sel)
    k8, ks, kh = oracle.quantise_qk_split(kb, sel)
    v8, vs = oracle.quantise_v(vb)
    rows = [[0, 0, i] for i in range(0, N, 7)]
    o8, l8 = oracle.fp8_attention_rows(q8, k8, v8, qs, ks, vs, math.log(2.0), rows,
                                       q_hi=qh, k_hi=kh)
    o64, l64 = oracle.attention_rows(q, k, v, math.log(2.0), rows)
    np.testing.assert_allclose(o8, o64, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l8, l64, rtol=1e-13)


def test_e4m3_midpoint_distance_hand_values():
    # grid steps: 2**-9 below 2**-6, 0.125 on [1, 2), 16 on [128, 256), 32 on [256, 448]
    d, st = oracle.e4m3_midpoint_distance(np.array([1.0625, 1.0, 2.0 ** -7, 448.0, 136.0, 130.0]))
    np.testing.assert_array_equal(st, [0.125, 0.125, 2.0 ** -9, 32.0, 16.0, 16.0])
    np.testing.assert_array_equal(d, [0.0, 0.0625, 2.0 ** -10, 16.0, 0.0, 6.0])
    # the midpoints are exactly where the encoder switches
    for x, step in ((1.0625, 0.125), (136.0, 16.0), (2.0 ** -7 + 2.0 ** -10, 2.0 ** -9)):
        lo = oracle.e4m3_decode(oracle.e4m3_encode(x - 1e-9))
        hi = oracle.e4m3_decode(oracle.e4m3_encode(x + 1e-9))
        assert hi - lo == step


def test_fp8_attention_flip_bound_hand_case():
    # Two keys through one kept channel (exact float64 values), scale ln 2 so t = q_hi.k_hi:
    # t = [0, log2(136/256)] -> M = 0, 2**8 p = [256, 136]; 136 is the midpoint between the
    # e4m3 values 128 and 144, so key 1 may round either way.  Bound for every channel:
    # 16 * |v_1| / (2**8 * (1 + 136/256)) = 2/49 with v_1 = 1.  Key 0 (256, mid-step) adds 0.
    D = 16
    q8 = np.zeros((1, 2, 1, D), np.uint8)
    k8 = np.zeros((1, 2, 1, D), np.uint8)
    v8 = np.zeros((1, 2, 1, D), np.uint8)
    v8[0, 1, 0, :] = oracle.e4m3_encode(1.0)
    v8[0, 0, 0, :] = oracle.e4m3_encode(-2.0)
    one = np.ones((1, 1, 1), np.float32)
    vs = np.ones((1, 1, D), np.float32)
    q_hi = np.zeros((1, 2, 1, 1)); q_hi[0, 0, 0, 0] = 1.0
    outs = []
    for nudge in (-1e-9, 0.0, 1e-9):
        k_hi = np.zeros((1, 2, 1, 1)); k_hi[0, 1, 0, 0] = math.log2(136 / 256) + nudge
        outs.append(oracle.fp8_attention_rows(q8, k8, v8, one, one, vs, math.log(2.0),
                                              [[0, 0, 0]], q_hi=q_hi, k_hi=k_hi,
                                              rel_window=1e-6))
    np.testing.assert_allclose(outs[1][2], np.full((1, D), 2.0 / 49.0), rtol=1e-12)
    # the bound is what the flip does: nudging the logit across the midpoint moves O by it
    jump = outs[2][0] - outs[0][0]
    np.testing.assert_allclose(jump, np.full((1, D), 2.0 / 49.0), rtol=1e-6)
    # far from any midpoint the bound vanishes
    k_hi = np.zeros((1, 2, 1, 1)); k_hi[0, 1, 0, 0] = math.log2(130 / 256)
    far = oracle.fp8_attention_rows(q8, k8, v8, one, one, vs, math.log(2.0), [[0, 0, 0]],
                                    q_hi=q_hi, k_hi=k_hi, rel_window=1e-6)
    assert np.all(far[2] == 0.0)
