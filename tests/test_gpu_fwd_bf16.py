"""GPU parity of joint_attn_fwd_bf16 (through the C ABI) against the fp64 CPU oracle.

Bar: relative Frobenius error <= 5e-3 and max |err| <= 2e-2 over the compared rows.
Small and ragged shapes compare every output row; the full-size workloads compare a
row sample (every row within two tokens of each stream boundary plus random rows) of
the plain forward.  The split-KV forward that the benchmark's step times is compared at
full size, including rows of its split tiles, in test_gpu_splitkv.py.
"""
import math

import numpy as np
import pytest

import oracle
from joint_attention_amd import synth

from _common import (BF16_MAX_ABS, BF16_REL_F, device_packed, from_device_bf16, gather_rows,
                     host_streams, max_abs, packed_host, rel_frobenius, widen_bf16)

pytestmark = pytest.mark.gpu


def _run(w, seed=None, sel=None):
    import joint_attention_amd as ja
    import torch
    st = host_streams(w, seed)
    q, k, vt, offs = device_packed(st)
    scale = 1.0 / math.sqrt(w.D)
    o, lse = ja.joint_attn_fwd_bf16(q, k, vt, scale, return_lse=True)
    torch.cuda.synchronize()
    qh, kh, vh, ref_offs = packed_host(st)
    assert offs == ref_offs.tolist()
    if sel is None:
        sel = oracle.all_rows(w.B, w.N, w.H)
    ref, ref_lse = oracle.attention_rows(qh, kh, vh, scale, sel)
    got = gather_rows(widen_bf16(from_device_bf16(o)), sel)
    got_lse = lse.cpu().numpy()[sel[:, 0], sel[:, 1], sel[:, 2]].astype(np.float64)
    return got, ref, got_lse, ref_lse, o


def _assert_parity(tag, got, ref, got_lse, ref_lse):
    rf, ma = rel_frobenius(got, ref), max_abs(got, ref)
    lse_err = float(np.abs(got_lse - ref_lse).max())
    print("%s: rel_F %.3e  max_abs %.3e  lse_max %.3e" % (tag, rf, ma, lse_err), flush=True)
    assert rf <= BF16_REL_F, (tag, rf)
    assert ma <= BF16_MAX_ABS, (tag, ma)
    assert lse_err <= 1e-3 * max(1.0, float(np.abs(ref_lse).max())), (tag, lse_err)


def test_tiny_every_row():
    w = synth.WORKLOADS["tiny_bf16"]
    _assert_parity("tiny", *_run(w)[:4])


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("lens", [(1,), (2,), (63,), (1, 64), (64, 1), (100, 29), (127, 2, 0, 1),
                                  (129, 64, 66)])
def test_ragged_every_row(D, lens):
    w = synth.custom("ragged", B=2, H=3, D=D, stream_lens=lens, outliers=4 if D == 128 else 0,
                     seed=len(lens) * 7 + sum(lens))
    _assert_parity("ragged D=%d %s" % (D, lens), *_run(w)[:4])


def test_t2i_1024_every_row_of_two_heads():
    w = synth.WORKLOADS["t2i_1024_bf16"]
    sel = np.concatenate([oracle.all_rows(1, w.N, 1) + np.array([1, 5, 0]),
                          oracle.all_rows(1, w.N, 1) + np.array([0, 23, 0])])
    _assert_parity("t2i_1024 heads", *_run(w, sel=sel)[:4])


@pytest.mark.parametrize("name", ["t2i_1024_bf16", "t2i_2048_bf16", "i2i_2048_bf16",
                                  "i2i_1024_r1_bf16", "i2i_1024_r3_bf16", "i2i_2048_r3_bf16"])
def test_full_size_sampled_rows(name):
    w = synth.WORKLOADS[name]
    if name == "i2i_2048_r3_bf16":
        # N = 66048 with four image streams; the heads are independent, so 4 of the 24
        # keep the host-side generation small while the sequence keeps its full length
        w = synth.custom(name, B=w.B, H=4, D=w.D, stream_lens=w.stream_lens,
                         n_reference=w.n_reference, outliers=w.outliers)
    sel = synth.row_sample(w, 384, seed=11)
    got, ref, gl, rl, o = _run(w, sel=sel)
    _assert_parity(name, got, ref, gl, rl)
    # per-stream segments (text / target / reference rows) also meet the bar
    offs = np.concatenate([[0], np.cumsum(w.stream_lens)])
    for s in range(len(w.stream_lens)):
        m = (sel[:, 2] >= offs[s]) & (sel[:, 2] < offs[s + 1])
        if m.sum() >= 8:
            assert rel_frobenius(got[m], ref[m]) <= BF16_REL_F, (name, s)


def test_zero_query_gives_mean_of_values():
    import joint_attention_amd as ja
    import torch
    w = synth.custom("zq", B=1, H=2, D=128, stream_lens=(40, 150))
    st = host_streams(w)
    q, k, vt, _ = device_packed(st)
    o = ja.joint_attn_fwd_bf16(torch.zeros_like(q), k, vt)
    torch.cuda.synchronize()
    _, _, vh, _ = packed_host(st)
    mean = widen_bf16(vh).mean(axis=1)                 # [B, H, D]
    got = widen_bf16(from_device_bf16(o))
    err = np.abs(got - mean[:, None, :, :]).max()
    print("zero-q max err %.3e" % err, flush=True)
    assert err <= 1e-2


def test_deterministic_and_key_permutation():
    import joint_attention_amd as ja
    import torch
    w = synth.custom("perm", B=1, H=2, D=128, stream_lens=(64, 200), outliers=4, seed=3)
    st = host_streams(w)
    q, k, vt, _ = device_packed(st)
    o1 = ja.joint_attn_fwd_bf16(q, k, vt)
    o2 = ja.joint_attn_fwd_bf16(q, k, vt)
    perm = torch.from_numpy(np.random.default_rng(0).permutation(w.N)).cuda()
    kp = k[:, :, perm, :].contiguous()
    vtp = vt[:, :, :, :w.N][:, :, :, perm]
    vtp = torch.nn.functional.pad(vtp, (0, vt.shape[3] - w.N)).contiguous()
    o3 = ja.joint_attn_fwd_bf16(q, kp, vtp)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    a, b = widen_bf16(from_device_bf16(o1)), widen_bf16(from_device_bf16(o3))
    assert rel_frobenius(b, a) <= 5e-3
