"""GPU: joint_attn_fwd_bf16_streams reads Q, K, V in place from the streams.

Its results must equal, bit for bit, joint_attn_pack x3 + joint_attn_fwd_bf16 on the same
streams (the arithmetic is the same; only where the operands come from differs), and meet
the bf16 bar against the fp64 oracle.  Cases cover stream boundaries inside key tiles,
zero-length streams, N below one tile, both head sizes and the full-size workloads.
"""
import numpy as np
import pytest

import oracle
from joint_attention_amd import synth

from _common import (BF16_MAX_ABS, BF16_REL_F, device_packed, from_device_bf16, gather_rows,
                     host_streams, max_abs, packed_host, rel_frobenius, to_device, widen_bf16)

pytestmark = pytest.mark.gpu


def _both(w):
    import joint_attention_amd as ja
    import torch
    st = host_streams(w)
    qd = [to_device(x) for x in st.q]
    kd = [to_device(x) for x in st.k]
    vd = [to_device(x) for x in st.v]
    scale = 1.0 / np.sqrt(w.D)
    o_f, offs_f, lse_f = ja.joint_attn_fwd_bf16_streams(qd, kd, vd, scale, return_lse=True)
    q, k, vt, offs = device_packed(st)
    o_p, lse_p = ja.joint_attn_fwd_bf16(q, k, vt, scale, return_lse=True)
    torch.cuda.synchronize()
    return st, offs_f, offs, o_f, lse_f, o_p, lse_p


def _check(w, sel=None, tag=""):
    import torch
    st, offs_f, offs_p, o_f, lse_f, o_p, lse_p = _both(w)
    print("streams", tag, w.stream_lens, "D", w.D, flush=True)
    assert offs_f == offs_p == oracle.stream_offsets([x.shape[1] for x in st.q]).tolist()
    assert torch.equal(o_f.view(torch.int16), o_p.view(torch.int16)), "O differs from packed path"
    assert torch.equal(lse_f.view(torch.int32), lse_p.view(torch.int32)), "lse differs"
    qh, kh, vh, _ = packed_host(st)
    if sel is None:
        sel = oracle.all_rows(w.B, w.N, w.H)
    ref, _ = oracle.attention_rows(qh, kh, vh, 1.0 / np.sqrt(w.D), sel)
    got = gather_rows(widen_bf16(from_device_bf16(o_f)), sel)
    rf, ma = rel_frobenius(got, ref), max_abs(got, ref)
    print("  vs oracle rel_F %.3e max %.3e" % (rf, ma), flush=True)
    assert rf <= BF16_REL_F and ma <= BF16_MAX_ABS, (tag, rf, ma)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("lens", [(1,), (31,), (32, 256), (100, 29), (127, 2, 0, 1),
                                  (0, 45, 0, 300), (129, 64, 66), (5, 5, 5, 5, 5, 5, 5),
                                  (17, 300, 0)])
def test_streams_small_every_row(D, lens):
    w = synth.custom("fs", B=2, H=3, D=D, stream_lens=lens, n_reference=max(0, len(lens) - 2),
                     outliers=4 if D == 128 else 0, seed=7 + sum(lens))
    _check(w, tag="small")


@pytest.mark.parametrize("name", ["t2i_1024_bf16", "t2i_2048_bf16", "i2i_2048_bf16",
                                  "i2i_1024_r3_bf16"])
def test_streams_full_size(name):
    w = synth.WORKLOADS[name]
    _check(w, sel=synth.row_sample(w, 256, seed=21, n_pairs=4), tag=name)


def _quant_both(w, mode):
    import joint_attention_amd as ja
    import torch
    st = host_streams(w)
    qd = [to_device(x) for x in st.q]
    kd = [to_device(x) for x in st.k]
    vd = [to_device(x) for x in st.v]
    t_s, offs_s = ja.joint_attn_quant_fp8_streams(qd, kd, vd, mode)
    q, k, vt, offs = device_packed(st)
    t_p = ja.joint_attn_quant_fp8(q, k, vt, mode)
    torch.cuda.synchronize()
    return t_s, offs_s, t_p, offs


def _assert_same_fp8(t_s, t_p, mode, tag):
    import torch
    names = ["q8", "k8", "v8t", "q_scale", "k_scale", "v_scale"]
    if mode == 1:
        names += ["q_hi", "k_hi", "hi_idx", "ch_amax"]
    for n in names:
        a, b = getattr(t_s, n), getattr(t_p, n)
        assert a.shape == b.shape, (tag, n)
        va = a.view(torch.uint8) if a.dtype == torch.uint8 else a.contiguous().view(torch.int8)
        vb = b.view(torch.uint8) if b.dtype == torch.uint8 else b.contiguous().view(torch.int8)
        assert torch.equal(va, vb), (tag, n)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("lens", [(1,), (31,), (100, 29), (127, 2, 0, 1), (0, 45, 0, 300),
                                  (129, 64, 66), (300, 17, 0)])
def test_quant_streams_equals_packed(lens, D, mode):
    w = synth.custom("qs", B=2, H=3, D=D, stream_lens=lens, n_reference=max(0, len(lens) - 2),
                     outliers=4 if D == 128 else 0, seed=11 + sum(lens))
    print("quant streams", lens, D, mode, flush=True)
    t_s, offs_s, t_p, offs = _quant_both(w, mode)
    assert offs_s == offs
    _assert_same_fp8(t_s, t_p, mode, (lens, D, mode))


@pytest.mark.parametrize("mode", [0, 1])
def test_quant_streams_t2i_2048_equals_packed_and_forward(mode):
    import joint_attention_amd as ja
    import torch
    w = synth.WORKLOADS["t2i_2048_fp8"]
    t_s, offs_s, t_p, offs = _quant_both(w, mode)
    assert offs_s == offs
    _assert_same_fp8(t_s, t_p, mode, ("t2i_2048", mode))
    o_s = ja.joint_attn_fwd_fp8(t_s)
    o_p = ja.joint_attn_fwd_fp8(t_p)
    torch.cuda.synchronize()
    assert torch.equal(o_s.view(torch.int16), o_p.view(torch.int16))
