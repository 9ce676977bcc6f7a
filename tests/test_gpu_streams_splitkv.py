"""GPU: joint_attn_fwd_bf16_streams_splitkv, the split-KV forward over the streams.

Q and K are read in place from the streams; V either in place too (pack_v = 0, transposed
in LDS) or from a V^T copy the call makes in its workspace (pack_v = 1).  Either way the
results must equal, bit for bit, joint_attn_pack x3 + joint_attn_fwd_bf16_splitkv with the
same n_split (the same tiles, key ranges and merge; only where the operands come from
differs), and meet the bf16 bar against the fp64 oracle.  Cases: stream boundaries inside
key tiles, zero-length streams, N below one tile, a grid with whole rounds before the split
round, no split (n_split 1), both head sizes, and the full-size workloads with rows drawn
from the split tiles.
"""
import numpy as np
import pytest

import oracle
from joint_attention_amd import synth

from _common import (BF16_MAX_ABS, BF16_REL_F, device_packed, from_device_bf16, gather_rows,
                     host_streams, max_abs, packed_host, rel_frobenius, to_device, widen_bf16,
                     with_split_tile_rows)

pytestmark = pytest.mark.gpu


def _check(w, n_split, pack_v, sel=None, tag=""):
    import joint_attention_amd as ja
    import torch
    st = host_streams(w)
    scale = 1.0 / np.sqrt(w.D)
    print("streams split-KV %s lens %s D %d split %d pack_v %d" % (tag, w.stream_lens, w.D,
                                                                   n_split, pack_v), flush=True)
    qd = [to_device(x) for x in st.q]
    kd = [to_device(x) for x in st.k]
    vd = [to_device(x) for x in st.v]
    o_s, offs_s, lse_s = ja.joint_attn_fwd_bf16_streams_splitkv(
        qd, kd, vd, scale, n_split=n_split, pack_v=pack_v, return_lse=True)
    q, k, vt, offs_p = device_packed(st)
    o_p, lse_p = ja.joint_attn_fwd_bf16_splitkv(q, k, vt, scale, n_split=n_split,
                                                return_lse=True)
    torch.cuda.synchronize()
    assert offs_s == offs_p == oracle.stream_offsets([x.shape[1] for x in st.q]).tolist()
    assert torch.equal(o_s.view(torch.int16), o_p.view(torch.int16)), "O differs from packed path"
    assert torch.equal(lse_s.view(torch.int32), lse_p.view(torch.int32)), "lse differs"
    qh, kh, vh, _ = packed_host(st)
    if sel is None:
        sel = oracle.all_rows(w.B, w.N, w.H)
    ref, ref_lse = oracle.attention_rows(qh, kh, vh, scale, sel)
    got = gather_rows(widen_bf16(from_device_bf16(o_s)), sel)
    got_lse = lse_s.cpu().numpy()[sel[:, 0], sel[:, 1], sel[:, 2]].astype(np.float64)
    rf, ma = rel_frobenius(got, ref), max_abs(got, ref)
    le = float(np.abs(got_lse - ref_lse).max())
    print("  vs oracle rel_F %.3e max %.3e lse %.2e" % (rf, ma, le), flush=True)
    assert rf <= BF16_REL_F and ma <= BF16_MAX_ABS, (tag, rf, ma)
    assert le <= 1e-2, (tag, le)


@pytest.mark.parametrize("pack_v", [0, 1])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("lens,n_split", [((1,), 3), ((31,), 2), ((100, 29), 3),
                                          ((127, 2, 0, 1), 4), ((0, 45, 0, 300), 5),
                                          ((129, 64, 66), 7), ((17, 300, 0), 1)])
def test_streams_splitkv_small_every_row(lens, n_split, D, pack_v):
    w = synth.custom("sskv", B=2, H=3, D=D, stream_lens=lens,
                     n_reference=max(0, len(lens) - 2), outliers=4 if D == 128 else 0,
                     seed=41 + sum(lens))
    _check(w, n_split, pack_v, tag="small")


@pytest.mark.parametrize("pack_v", [0, 1])
@pytest.mark.parametrize("D,n_split", [(128, 3), (64, 4)])
def test_streams_splitkv_whole_rounds_and_tail(D, n_split, pack_v):
    # more query tiles than one round of workgroups: whole rounds unsplit, the last
    # round's tiles split; a stream boundary (300) inside a key tile
    w = synth.custom("sskvt", B=2, H=65, D=D, stream_lens=(300, 200),
                     outliers=4 if D == 128 else 0, seed=43)
    _check(w, n_split, pack_v, tag="whole rounds + tail")


@pytest.mark.parametrize("pack_v", [0, 1])
@pytest.mark.parametrize("name", ["t2i_2048_bf16", "i2i_1024_r3_bf16"])
def test_streams_splitkv_full_size(name, pack_v):
    import joint_attention_amd as ja
    w = synth.WORKLOADS[name]
    n = ja.load().joint_attn_fwd_bf16_splitkv_suggest(w.B, w.H, w.N, w.D)
    n = n if n > 1 else 5
    sel = synth.row_sample(w, 192, seed=47, n_pairs=min(4, w.B * w.H))
    sel, n_in = with_split_tile_rows(w, sel, "bf16", n_rows=128, seed=47)
    print("%s: %d of %d compared rows in split tiles" % (name, n_in, len(sel)), flush=True)
    assert n_in > 0
    _check(w, n, pack_v, sel=sel, tag=name)
