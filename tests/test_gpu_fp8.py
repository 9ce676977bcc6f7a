"""GPU: fp8 quantiser (bit-exact) and fp8 forward (against the fp8 reference) through
the C ABI.

The quantiser's codes and scales must equal the oracle's bit for bit.  The fp8 forward
is compared with the oracle's fp8 attention (same quantised operands, same P rounding
rule) at the bf16-output bar, rel_F <= 5e-3 and max |err| <= 2e-2; its distance to the
fp64 attention on the unquantised inputs is printed and bounded by what the fp8 recipe
itself loses (the reference's own distance, plus the output rounding).
"""
import math

import numpy as np
import pytest

import oracle
from joint_attention_amd import synth

from _common import (FP8_MAX_ABS, FP8_REL_F, device_packed, from_device_bf16, gather_rows,
                     host_streams, max_abs, packed_host, rel_frobenius, widen_bf16)

pytestmark = pytest.mark.gpu


def _quant_both(w, bh_slices=None):
    import joint_attention_amd as ja
    import torch
    st = host_streams(w)
    q, k, vt, offs = device_packed(st)
    q8, k8, v8t, qs, ks, vs = ja.joint_attn_quant_fp8(q, k, vt)
    torch.cuda.synchronize()
    qh, kh, vh, _ = packed_host(st)
    if bh_slices is not None:                           # compare a few (b, h) slices only
        b, h = bh_slices
        qh, kh, vh = qh[b:b + 1, :, h:h + 1], kh[b:b + 1, :, h:h + 1], vh[b:b + 1, :, h:h + 1]
        pick = lambda t: t[b:b + 1, h:h + 1].cpu().numpy()
    else:
        pick = lambda t: t.cpu().numpy()
    return dict(dev=(q, k, vt, q8, k8, v8t, qs, ks, vs), st=st,
                got=tuple(pick(t) for t in (q8, k8, v8t, qs, ks, vs)),
                host=(qh, kh, vh))


def _assert_quant_equal(res, N):
    q8g, k8g, v8tg, qsg, ksg, vsg = res["got"]
    qh, kh, vh = res["host"]
    q8r, qsr = oracle.quantise_qk(qh)
    k8r, ksr = oracle.quantise_qk(kh)
    v8r, vsr = oracle.quantise_v(vh)
    assert np.array_equal(q8g, oracle.to_bhnd(q8r))
    assert np.array_equal(k8g, oracle.to_bhnd(k8r))
    assert np.array_equal(v8tg, oracle.to_bhdn(v8r, v8tg.shape[3]))
    for g, r in ((qsg, qsr), (ksg, ksr), (vsg, vsr)):
        assert np.array_equal(g.view(np.uint32), r.view(np.uint32))


@pytest.mark.parametrize("lens,D", [((32, 256), 64), ((1,), 128), ((100, 29), 128),
                                    ((127, 2, 0, 1), 64), ((129, 64, 66), 128), ((512, 1000), 128)])
def test_quant_bit_exact_small(lens, D):
    w = synth.custom("q", B=2, H=3, D=D, stream_lens=lens, outliers=4 if D == 128 else 0,
                     seed=sum(lens))
    print("quant", lens, D, flush=True)
    _assert_quant_equal(_quant_both(w), w.N)


@pytest.mark.parametrize("b,h", [(0, 0), (1, 23)])
def test_quant_bit_exact_t2i_2048_slices(b, h):
    w = synth.WORKLOADS["t2i_2048_fp8"]
    print("quant t2i_2048 slice", b, h, flush=True)
    _assert_quant_equal(_quant_both(w, (b, h)), w.N)


def _fwd_fp8(w, sel=None):
    """GPU fp8 forward vs the oracle's fp8 attention and its fp64 attention.  The oracle
    side runs per (b, h) slice (the method is independent per slice), so full-size
    workloads only quantise the slices that the sampled rows touch."""
    import joint_attention_amd as ja
    import torch
    res = _quant_both(w)
    q, k, vt, q8, k8, v8t, qs, ks, vs = res["dev"]
    scale = 1.0 / math.sqrt(w.D)
    o, lse = ja.joint_attn_fwd_fp8(q8, k8, v8t, qs, ks, vs, scale, return_lse=True)
    torch.cuda.synchronize()
    qh, kh, vh = res["host"]
    if sel is None:
        sel = oracle.all_rows(w.B, w.N, w.H)
    ref8 = np.empty((len(sel), w.D))
    lse8 = np.empty(len(sel))
    ref64 = np.empty((len(sel), w.D))
    for b, h in sorted(set(map(tuple, sel[:, :2].tolist()))):
        m = (sel[:, 0] == b) & (sel[:, 1] == h)
        sl = lambda x: np.ascontiguousarray(x[b:b + 1, :, h:h + 1])
        qb, kb, vb = sl(qh), sl(kh), sl(vh)
        q8r, qsr = oracle.quantise_qk(qb)
        k8r, ksr = oracle.quantise_qk(kb)
        v8r, vsr = oracle.quantise_v(vb)
        loc = np.stack([np.zeros(m.sum(), np.int64), np.zeros(m.sum(), np.int64), sel[m, 2]], 1)
        ref8[m], lse8[m] = oracle.fp8_attention_rows(q8r, k8r, v8r, qsr, ksr, vsr, scale, loc)
        ref64[m], _ = oracle.attention_rows(qb, kb, vb, scale, loc)
    got = gather_rows(widen_bf16(from_device_bf16(o)), sel)
    got_lse = lse.cpu().numpy()[sel[:, 0], sel[:, 1], sel[:, 2]].astype(np.float64)
    return got, ref8, ref64, got_lse, lse8


def _assert_fp8(tag, got, ref8, ref64, got_lse, lse8):
    rf, ma = rel_frobenius(got, ref8), max_abs(got, ref8)
    recipe = rel_frobenius(ref8, ref64)
    vs64 = rel_frobenius(got, ref64)
    lse_err = float(np.abs(got_lse - lse8).max())
    print("%s: vs fp8 reference rel_F %.3e max %.3e lse %.2e | vs fp64 unquantised: "
          "kernel %.3e, reference itself %.3e" % (tag, rf, ma, lse_err, vs64, recipe), flush=True)
    assert rf <= FP8_REL_F, (tag, rf)
    assert ma <= FP8_MAX_ABS, (tag, ma)
    assert vs64 <= recipe + 5e-3, (tag, vs64, recipe)
    assert lse_err <= 1e-3 * max(1.0, float(np.abs(lse8).max())), (tag, lse_err)


def test_fp8_tiny_every_row():
    w = synth.custom("fp8tiny", B=1, H=2, D=64, stream_lens=(32, 256))
    _assert_fp8("fp8 tiny", *_fwd_fp8(w))


@pytest.mark.parametrize("lens,D", [((1,), 128), ((63,), 64), ((100, 29), 128),
                                    ((129, 64, 66), 128), ((127, 2, 0, 1), 64)])
def test_fp8_ragged_every_row(lens, D):
    w = synth.custom("fp8r", B=2, H=2, D=D, stream_lens=lens, outliers=4 if D == 128 else 0,
                     seed=3 + sum(lens))
    _assert_fp8("fp8 ragged %s D=%d" % (lens, D), *_fwd_fp8(w))


def test_fp8_t2i_2048_sampled_rows():
    w = synth.WORKLOADS["t2i_2048_fp8"]
    sel = synth.row_sample(w, 256, seed=12, n_pairs=3)
    _assert_fp8("fp8 t2i_2048", *_fwd_fp8(w, sel))
