"""GPU: the allocation-free split-KV forward (joint_attn_fwd_bf16_splitkv_noalloc, partial
results in the library's static scratch array) against the workspace variant
(joint_attn_fwd_bf16_splitkv) on the same inputs: equal bit for bit, on two calls in a row
whose second input is smaller than the first (the scratch keeps the first call's partials),
at the 2048^2 T2I step's configuration, plus the fp64 oracle's bar on sampled rows; and the
rejection of a call whose partials exceed the scratch."""
import ctypes

import numpy as np
import pytest

import oracle
from joint_attention_amd import synth

from _common import (BF16_MAX_ABS, BF16_REL_F, device_packed, from_device_bf16, gather_rows,
                     host_streams, max_abs, packed_host, rel_frobenius, widen_bf16,
                     with_split_tile_rows)

pytestmark = pytest.mark.gpu


def _both(w, n_split):
    import joint_attention_amd as ja
    import torch
    q, k, vt, _ = device_packed(host_streams(w))
    B, H, N, D = w.B, w.H, w.N, w.D
    o_ws = torch.empty((B, N, H, D), dtype=torch.bfloat16, device="cuda")
    l_ws = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    o_st = torch.full_like(o_ws, float("nan"))
    l_st = torch.full_like(l_ws, float("nan"))
    ja.joint_attn_fwd_bf16_splitkv(q, k, vt, n_split=n_split, out=o_ws)
    lib = ja.load()
    ws = torch.empty((int(lib.joint_attn_fwd_bf16_splitkv_workspace(B, H, N, D, n_split)),),
                     dtype=torch.uint8, device="cuda")
    st = lib.joint_attn_fwd_bf16_splitkv(q.data_ptr(), k.data_ptr(), vt.data_ptr(), B, H, N, D,
                                         int(vt.shape[3]), 1.0 / np.sqrt(D), n_split,
                                         ws.data_ptr(), ws.numel(), o_ws.data_ptr(),
                                         l_ws.data_ptr(), ctypes.c_void_p(0))
    assert st == 0
    torch.cuda.synchronize()
    st = lib.joint_attn_fwd_bf16_splitkv_noalloc(q.data_ptr(), k.data_ptr(), vt.data_ptr(), B, H,
                                                 N, D, int(vt.shape[3]), 1.0 / np.sqrt(D),
                                                 n_split, o_st.data_ptr(), l_st.data_ptr(),
                                                 ctypes.c_void_p(0))
    assert st == 0, lib.joint_attn_strerror(st)
    torch.cuda.synchronize()
    return o_ws, l_ws, o_st, l_st


def _check(w, n_split, n_oracle_rows):
    import torch
    o_ws, l_ws, o_st, l_st = _both(w, n_split)
    same = torch.equal(o_ws.view(torch.int16), o_st.view(torch.int16)) and torch.equal(
        l_ws.view(torch.int32), l_st.view(torch.int32))
    print("%s n_split %d: equal to the workspace variant: %s" % (w.name, n_split, same),
          flush=True)
    assert same
    # and the oracle's bar on sampled rows, split tiles included
    sel = synth.row_sample(w, n_oracle_rows, seed=3, n_pairs=min(2, w.B * w.H))
    sel, n_in = with_split_tile_rows(w, sel, "bf16", n_rows=n_oracle_rows, seed=3)
    qh, kh, vh, _ = packed_host(host_streams(w))
    ref, _ = oracle.attention_rows(qh, kh, vh, 1.0 / np.sqrt(w.D), sel)
    got = gather_rows(widen_bf16(from_device_bf16(o_st)), sel)
    rf, ma = rel_frobenius(got, ref), max_abs(got, ref)
    print("  vs oracle: %d rows (%d in split tiles) rel_F %.3e max %.3e" % (len(sel), n_in, rf, ma),
          flush=True)
    assert rf <= BF16_REL_F and ma <= BF16_MAX_ABS


def test_noalloc_two_calls_second_smaller():
    import joint_attention_amd as ja
    w1 = synth.WORKLOADS["t2i_2048_bf16"]
    n1 = ja.load().joint_attn_fwd_bf16_splitkv_suggest(w1.B, w1.H, w1.N, w1.D)
    assert n1 > 1
    _check(w1, n1, 96)
    # a smaller call after the larger one: fewer split tiles, a ragged last key tile
    w2 = synth.custom("small", B=1, H=3, D=128, stream_lens=(100, 900), outliers=4, seed=5)
    _check(w2, 3, 128)


def test_noalloc_head_size_64_and_no_split():
    # D = 64 (128-row tiles), then a call whose split is 1 (the plain forward, no scratch)
    _check(synth.custom("d64", B=2, H=5, D=64, stream_lens=(64, 700), seed=6), 4, 128)
    _check(synth.custom("nosplit", B=1, H=2, D=128, stream_lens=(32, 500), outliers=4, seed=7),
           1, 64)


def test_noalloc_rejects_partials_beyond_the_scratch():
    # one GPU's share of a 4-way head split of 2048^2 (B = 1, H = 6): 140 split tiles x 7
    # ranges x 256 rows x 129 floats = 129 MB > JA_SCRATCH_BYTES; nothing is launched
    import joint_attention_amd as ja
    import torch
    from joint_attention_amd import _abi
    lib = ja.load()
    q = torch.zeros((1, 6, 16896, 128), dtype=torch.bfloat16, device="cuda")
    vt = torch.zeros((1, 6, 128, 16896), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros((1, 16896, 6, 128), dtype=torch.bfloat16, device="cuda")
    st = lib.joint_attn_fwd_bf16_splitkv_noalloc(q.data_ptr(), q.data_ptr(), vt.data_ptr(), 1, 6,
                                                 16896, 128, 16896, 0.1, 7, o.data_ptr(), None,
                                                 ctypes.c_void_p(0))
    torch.cuda.synchronize()
    assert st == _abi.JA_ESCRATCH
    assert b"scratch" in lib.joint_attn_strerror(st)
    assert torch.count_nonzero(o.view(torch.int16)) == 0
