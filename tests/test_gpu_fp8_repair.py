"""GPU: token repair of fp8 attention (joint_attn_quant_fp8_repair and
joint_attn_fwd_fp8_repair) through the C ABI.

Quantiser: codes and scales equal the plain mode's (the oracle's, bit for bit); each
token's residual equals the oracle's exactly (it is exact in binary32); the repaired
token lists equal the oracle's selection.

Forward: against the oracle's fp8 attention with the same repaired tokens (same P
rounding rule).  Rows of unrepaired queries come from the main kernel, whose fp8 matrix
cores add groups of 8 products at reduced precision: on inputs with x8 outlier channels
the plain mode's loose bar, otherwise the tight one (as for the plain forward).  Rows of
repaired queries are recomputed on bf16 matrix cores from exact products: the split
mode's bar (rel_F, and max |err| beyond what a near-midpoint P code may change).  With
no token repaired the result equals the plain forward bit for bit.
"""
import math

import numpy as np
import pytest

import oracle
from joint_attention_amd import synth

from _common import (FP8_MAX_ABS, FP8_PLAIN_MAX_ABS, FP8_PLAIN_REL_F, FP8_REL_F,
                     device_packed, from_device_bf16, gather_rows, host_streams, max_abs,
                     packed_host, rel_frobenius, widen_bf16)

pytestmark = pytest.mark.gpu

P_FLIP_WINDOW = 2.0 ** -12          # as for the other fp8 modes


def _run(w, rho, sel=None, fwd=True):
    import joint_attention_amd as ja
    import torch
    st = host_streams(w)
    q, k, vt, _ = device_packed(st)
    t = ja.joint_attn_quant_fp8_repair(q, k, vt, rho)
    o = lse = None
    if fwd:
        o, lse = ja.joint_attn_fwd_fp8(t, 1.0 / math.sqrt(w.D), return_lse=True)
    torch.cuda.synchronize()
    qh, kh, vh, _ = packed_host(st)
    return dict(t=t, o=o, lse=lse, host=(qh, kh, vh), dev=(q, k, vt))


def _ref_quant(qh, kh, vh, n):
    r = {}
    r["q8"], r["q_scale"], r["q_err"], r["q_sel"] = oracle.quantise_qk_repair(qh, n)
    r["k8"], r["k_scale"], r["k_err"], r["k_sel"] = oracle.quantise_qk_repair(kh, n)
    r["v8"], r["v_scale"] = oracle.quantise_v(vh)
    return r


def _assert_quant(res, n):
    t = res["t"]
    qh, kh, vh = res["host"]
    r = _ref_quant(qh, kh, vh, n)
    assert t.n_repair == n
    assert np.array_equal(t.q8.cpu().numpy(), oracle.to_bhnd(r["q8"]))
    assert np.array_equal(t.k8.cpu().numpy(), oracle.to_bhnd(r["k8"]))
    v8t = t.v8t.cpu().numpy()
    assert np.array_equal(v8t, oracle.to_bhdn(r["v8"], v8t.shape[3]))
    for nm in ("q_scale", "k_scale", "v_scale"):
        assert np.array_equal(getattr(t, nm).cpu().numpy().view(np.uint32),
                              r[nm].view(np.uint32)), nm
    for nm in ("q_err", "k_err"):
        assert np.array_equal(getattr(t, nm).cpu().numpy().astype(np.float64), r[nm]), nm
    for nm in ("q_sel", "k_sel"):
        assert np.array_equal(getattr(t, nm).cpu().numpy(), r[nm]), nm


@pytest.mark.parametrize("lens,D,rho", [((32, 256), 64, 0.05), ((1,), 128, 1.0),
                                        ((100, 29), 128, 0.3), ((127, 2, 0, 1), 64, 0.5),
                                        ((129, 64, 66), 128, 0.005), ((512, 1000), 128, 0.005),
                                        ((300,), 128, 0.0)])
def test_quant_repair_bit_exact(lens, D, rho):
    w = synth.custom("rq", B=2, H=3, D=D, stream_lens=lens, outliers=4 if D == 128 else 0,
                     seed=7 + sum(lens))
    n = oracle.repair_count(w.N, rho)
    print("quant repair", lens, D, rho, "n", n, flush=True)
    _assert_quant(_run(w, rho, fwd=False), n)


def _compare(w, rho, sel=None):
    res = _run(w, rho)
    qh, kh, vh = res["host"]
    n = oracle.repair_count(w.N, rho)
    scale = 1.0 / math.sqrt(w.D)
    if sel is None:
        sel = oracle.all_rows(w.B, w.N, w.H)
    ref = np.empty((len(sel), w.D))
    lse8 = np.empty(len(sel))
    flip = np.empty((len(sel), w.D))
    plain = np.empty((len(sel), w.D))
    ref64 = np.empty((len(sel), w.D))
    rep_row = np.zeros(len(sel), bool)
    for b, h in sorted(set(map(tuple, sel[:, :2].tolist()))):
        m = (sel[:, 0] == b) & (sel[:, 1] == h)
        sl = lambda x: np.ascontiguousarray(x[b:b + 1, :, h:h + 1])
        qb, kb, vb = sl(qh), sl(kh), sl(vh)
        r = _ref_quant(qb, kb, vb, n)
        loc = np.stack([np.zeros(m.sum(), np.int64), np.zeros(m.sum(), np.int64), sel[m, 2]], 1)
        ref[m], lse8[m], flip[m] = oracle.fp8_attention_rows(
            r["q8"], r["k8"], r["v8"], r["q_scale"], r["k_scale"], r["v_scale"], scale, loc,
            rel_window=P_FLIP_WINDOW, q_exact=qb, k_exact=kb, q_rep=r["q_sel"],
            k_rep=r["k_sel"])
        plain[m], _ = oracle.fp8_attention_rows(r["q8"], r["k8"], r["v8"], r["q_scale"],
                                                r["k_scale"], r["v_scale"], scale, loc)
        ref64[m], _ = oracle.attention_rows(qb, kb, vb, scale, loc)
        rep_row[m] = np.isin(sel[m, 2], r["q_sel"][0, 0])
    got = gather_rows(widen_bf16(from_device_bf16(res["o"])), sel)
    got_lse = res["lse"].cpu().numpy()[sel[:, 0], sel[:, 1], sel[:, 2]].astype(np.float64)
    return dict(got=got, ref=ref, lse=got_lse, lse8=lse8, flip=flip, plain=plain, ref64=ref64,
                rep_row=rep_row, n=n)


def _assert_repair(tag, c, *, outliers: bool):
    got, ref, flip, rep = c["got"], c["ref"], c["flip"], c["rep_row"]
    lse_err = float(np.abs(c["lse"] - c["lse8"]).max())
    msg = "%s n=%d: lse %.2e" % (tag, c["n"], lse_err)
    if (~rep).any():
        rf = rel_frobenius(got[~rep], ref[~rep])
        ma = max_abs(got[~rep], ref[~rep])
        beyond = float((np.abs(got[~rep] - ref[~rep]) - flip[~rep]).max())
        msg += " | unrepaired rows: rel_F %.3e max %.3e (beyond flip bound %.3e)" % (rf, ma,
                                                                                  beyond)
        if outliers:
            assert rf <= FP8_PLAIN_REL_F and ma <= FP8_PLAIN_MAX_ABS, (tag, rf, ma)
        else:
            assert rf <= FP8_REL_F and beyond <= FP8_MAX_ABS, (tag, rf, beyond)
    if rep.any():
        rf = rel_frobenius(got[rep], ref[rep])
        beyond = float((np.abs(got[rep] - ref[rep]) - flip[rep]).max())
        msg += " | repaired rows (%d): rel_F %.3e max beyond flip bound %.3e" % (rep.sum(), rf,
                                                                                   beyond)
        assert rf <= FP8_REL_F and beyond <= FP8_MAX_ABS, (tag, rf, beyond)
    vs64, plain64 = rel_frobenius(got, c["ref64"]), rel_frobenius(c["plain"], c["ref64"])
    msg += " | vs fp64: kernel %.3e, repaired reference %.3e, plain reference %.3e" % (
        vs64, rel_frobenius(ref, c["ref64"]), plain64)
    print(msg, flush=True)
    assert lse_err <= 1e-3 * max(1.0, float(np.abs(c["lse8"]).max())), (tag, lse_err)


@pytest.mark.parametrize("lens,D,rho", [((1,), 128, 0.5), ((63,), 64, 0.1),
                                        ((100, 29), 128, 0.05), ((129, 64, 66), 128, 0.1),
                                        ((127, 2, 0, 1), 64, 0.3), ((64, 700), 128, 0.005)])
def test_repair_every_row(lens, D, rho):
    w = synth.custom("rf", B=2, H=2, D=D, stream_lens=lens, outliers=4 if D == 128 else 0,
                     seed=11 + sum(lens))
    _assert_repair("repair %s D=%d rho=%g" % (lens, D, rho), _compare(w, rho),
                   outliers=w.outliers > 0)


@pytest.mark.parametrize("lens,rho", [((100, 29), 0.05), ((64, 700), 0.005)])
def test_repair_no_outliers_every_row(lens, rho):
    # head size 128 without outlier channels: unrepaired rows at the tight bar too
    w = synth.custom("rfn", B=2, H=2, D=128, stream_lens=lens, outliers=0, seed=12 + sum(lens))
    _assert_repair("repair no outliers %s rho=%g" % (lens, rho), _compare(w, rho),
                   outliers=False)


@pytest.mark.parametrize("D", [64, 128])
def test_repair_all_tokens(D):
    # every key through the extra tiles (its code term cancelled), every row recomputed
    w = synth.custom("rall", B=1, H=2, D=D, stream_lens=(40, 260), outliers=4 if D == 128 else 0,
                     seed=D)
    _assert_repair("repair all D=%d" % D, _compare(w, 1.0), outliers=w.outliers > 0)


@pytest.mark.parametrize("D", [64, 128])
def test_repair_none_is_plain_bitwise(D):
    import joint_attention_amd as ja
    import torch
    w = synth.custom("rnone", B=2, H=2, D=D, stream_lens=(77, 500), outliers=4 if D == 128 else 0,
                     seed=3)
    res = _run(w, 0.0)
    q, k, vt = res["dev"]
    plain = ja.joint_attn_fwd_fp8(ja.joint_attn_quant_fp8(q, k, vt, ja.JA_FP8_PLAIN),
                                  1.0 / math.sqrt(D))
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), res["o"].view(torch.int16))


def test_repair_t2i_2048_sampled_rows():
    w = synth.WORKLOADS["t2i_2048_fp8"]
    sel = synth.row_sample(w, 256, seed=12, n_pairs=3)
    res_sel = _run(w, 0.005, fwd=False)["t"]
    # the sampled rows plus every repaired row of the sampled (b, h) pairs
    qs = res_sel.q_sel.cpu().numpy()
    extra = [(b, h, int(i)) for b, h in sorted(set(map(tuple, sel[:, :2].tolist())))
             for i in qs[b, h]]
    sel = np.asarray(sorted(set(map(tuple, sel.tolist())) | set(extra)), dtype=np.int64)
    c = _compare(w, 0.005, sel)
    assert c["n"] == 85 and c["rep_row"].sum() == 3 * 85
    _assert_repair("repair t2i_2048 rho=0.005", c, outliers=True)


def test_repair_deterministic():
    import joint_attention_amd as ja
    import torch
    w = synth.custom("rdet", B=1, H=3, D=128, stream_lens=(64, 700), outliers=4, seed=9)
    q, k, vt, _ = device_packed(host_streams(w))
    t = ja.joint_attn_quant_fp8_repair(q, k, vt, 0.05)
    a = ja.joint_attn_fwd_fp8(t)
    b = ja.joint_attn_fwd_fp8(t)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
