"""GPU: split-KV bf16 forward (joint_attn_fwd_bf16_splitkv) against the fp64 oracle at the
bf16 bar, for several split counts (1 up to more ranges than key tiles) on ragged shapes,
with whole rounds of unsplit query tiles before a split last round, and at full size with
the suggested split (1024^2 and 2048^2 T2I, one GPU's share of a head split)."""
import numpy as np
import pytest

import oracle
from joint_attention_amd import synth

from _common import (BF16_MAX_ABS, BF16_REL_F, device_packed, from_device_bf16, gather_rows,
                     host_streams, max_abs, packed_host, rel_frobenius, widen_bf16,
                     with_split_tile_rows)

pytestmark = pytest.mark.gpu


def _run(w, n_split, sel=None):
    import joint_attention_amd as ja
    import torch
    st = host_streams(w)
    q, k, vt, offs = device_packed(st)
    scale = 1.0 / np.sqrt(w.D)
    o, lse = ja.joint_attn_fwd_bf16_splitkv(q, k, vt, scale, n_split=n_split, return_lse=True)
    torch.cuda.synchronize()
    qh, kh, vh, _ = packed_host(st)
    if sel is None:
        sel = oracle.all_rows(w.B, w.N, w.H)
    ref, ref_lse = oracle.attention_rows(qh, kh, vh, scale, sel)
    got = gather_rows(widen_bf16(from_device_bf16(o)), sel)
    got_lse = lse.cpu().numpy()[sel[:, 0], sel[:, 1], sel[:, 2]].astype(np.float64)
    return got, ref, got_lse, ref_lse, o


def _assert(tag, got, ref, got_lse, ref_lse):
    rf, ma = rel_frobenius(got, ref), max_abs(got, ref)
    le = float(np.abs(got_lse - ref_lse).max())
    print("%s: rel_F %.3e max %.3e lse %.2e" % (tag, rf, ma, le), flush=True)
    assert rf <= BF16_REL_F and ma <= BF16_MAX_ABS, (tag, rf, ma)
    assert le <= 1e-2, (tag, le)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("lens,n_split", [((32, 256), 2), ((100, 29), 3), ((1,), 4),
                                          ((129, 64, 700), 7), ((63,), 64), ((512, 1000), 1)])
def test_splitkv_every_row(D, lens, n_split):
    w = synth.custom("skv", B=2, H=3, D=D, stream_lens=lens, outliers=4 if D == 128 else 0,
                     seed=13 + sum(lens))
    _assert("split %d %s D=%d" % (n_split, lens, D), *_run(w, n_split)[:4])


@pytest.mark.parametrize("D,n_split", [(128, 3), (64, 4)])
def test_splitkv_whole_rounds_and_tail(D, n_split):
    # more query tiles than one round of workgroups: the whole rounds run unsplit, the
    # last round's tiles split (every row compared)
    w = synth.custom("skvt", B=2, H=65, D=D, stream_lens=(100, 200), outliers=4 if D == 128 else 0,
                     seed=31)
    _assert("whole rounds + tail D=%d split %d" % (D, n_split), *_run(w, n_split)[:4])


@pytest.mark.parametrize("shape", ["t2i_1024", "t2i_2048", "ulysses4_share", "ulysses8_share"])
def test_splitkv_full_size(shape):
    import joint_attention_amd as ja
    base = synth.WORKLOADS["t2i_1024_bf16" if shape == "t2i_1024" else "t2i_2048_bf16"]
    heads = {"t2i_1024": base.H, "t2i_2048": base.H, "ulysses4_share": 6,
             "ulysses8_share": 3}[shape]
    B = base.B if shape in ("t2i_1024", "t2i_2048") else 1
    w = synth.custom(shape, B=B, H=heads, D=base.D, stream_lens=base.stream_lens,
                     outliers=base.outliers)
    # the suggested split, or 5 where the library suggests none (all tiles then split)
    n = ja.load().joint_attn_fwd_bf16_splitkv_suggest(w.B, w.H, w.N, w.D)
    n = n if n > 1 else 5
    # random rows of 4 slices, plus rows of the last round's tiles: the ones cut into key
    # ranges and merged (at 2048^2: slice (1, 22) from row 9216 on and all of (1, 23))
    sel = synth.row_sample(w, 256, seed=23, n_pairs=min(4, w.B * w.H))
    sel, n_in = with_split_tile_rows(w, sel, "bf16", n_rows=160, seed=23)
    print("%s: %d of %d compared rows in split tiles" % (shape, n_in, len(sel)), flush=True)
    assert n_in > 0
    _assert("%s split %d" % (shape, n), *_run(w, n, sel)[:4])


def test_splitkv_deterministic():
    import torch
    w = synth.custom("skvd", B=1, H=2, D=128, stream_lens=(64, 900), outliers=4, seed=2)
    a = _run(w, 5, sel=oracle.all_rows(1, 4, 1))[4].clone()
    b = _run(w, 5, sel=oracle.all_rows(1, 4, 1))[4]
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("B,H,lens,n_split", [(1, 3, (100, 300), 1), (2, 128, (256,), 4)])
def test_splitkv_without_a_tail_is_the_plain_forward(B, H, lens, n_split):
    # n_split = 1, or a grid of whole rounds (2 x 128 heads x one 256-row tile = 256
    # workgroups on 256 CUs): the plain forward runs, bit for bit
    import joint_attention_amd as ja
    import torch
    w = synth.custom("skvp", B=B, H=H, D=128, stream_lens=lens, outliers=4, seed=17)
    q, k, vt, _ = device_packed(host_streams(w))
    a = ja.joint_attn_fwd_bf16(q, k, vt)
    b = ja.joint_attn_fwd_bf16_splitkv(q, k, vt, n_split=n_split)
    torch.cuda.synchronize()
    if torch.cuda.get_device_properties(0).multi_processor_count != 256 and n_split > 1:
        pytest.skip("the whole-rounds case assumes 256 CUs")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
