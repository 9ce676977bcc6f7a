"""GPU: split-KV fp8 forward (joint_attn_fwd_fp8_splitkv), both modes, against the oracle's
fp8 attention at each mode's bar (as for joint_attn_fwd_fp8): ragged shapes whose tiles are
all split, a grid with whole rounds before a split last round, 2048^2 T2I sampled rows with
the suggested split; and equality with the plain forward where no tile is split."""
import numpy as np
import pytest

from joint_attention_amd import synth

from _common import device_packed, host_streams, with_split_tile_rows
from test_gpu_fp8 import _assert_fp8, _fwd_fp8

pytestmark = pytest.mark.gpu

MODES = (0, 1)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("lens,D,n_split", [((100, 29), 128, 2), ((129, 64, 66), 128, 3),
                                            ((63,), 64, 7), ((127, 2, 0, 1), 64, 2),
                                            ((512, 1000), 128, 64)])
def test_fp8_splitkv_every_row(lens, D, n_split, mode):
    w = synth.custom("f8skv", B=2, H=2, D=D, stream_lens=lens, outliers=4 if D == 128 else 0,
                     seed=5 + sum(lens))
    _assert_fp8("fp8 split-KV %s D=%d split %d" % (lens, D, n_split), mode,
                *_fwd_fp8(w, mode, n_split=n_split), outliers=w.outliers > 0)


@pytest.mark.parametrize("mode", MODES)
def test_fp8_splitkv_whole_rounds_and_tail(mode):
    # 2 x 65 heads x 2 tiles = 260 query tiles on 256 CUs: tiles 0..255 unsplit, 256..259
    # (slices (1, 63) and (1, 64)) split; every row of two slices of each kind
    import torch
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the slice choice assumes 256 CUs")
    w = synth.custom("f8skvt", B=2, H=65, D=128, stream_lens=(100, 200), outliers=4, seed=41)
    sel = np.asarray([(b, h, i) for b, h in ((0, 0), (0, 1), (1, 63), (1, 64))
                      for i in range(w.N)], dtype=np.int64)
    _assert_fp8("fp8 whole rounds + tail", mode, *_fwd_fp8(w, mode, sel, n_split=3),
                outliers=True)


@pytest.mark.parametrize("mode", MODES)
def test_fp8_splitkv_t2i_2048_sampled_rows(mode):
    import joint_attention_amd as ja
    w = synth.WORKLOADS["t2i_2048_fp8"]
    n = ja.load().joint_attn_fwd_fp8_splitkv_suggest(w.B, w.H, w.N, w.D, mode)
    assert n > 1, n
    # random rows of 3 slices, plus rows of the last round's tiles (the ones cut into key
    # ranges and merged: slice (1, 22) from row 9216 on and all of (1, 23))
    sel = synth.row_sample(w, 256, seed=14, n_pairs=3)
    sel, n_in = with_split_tile_rows(w, sel, "fp8", n_rows=160, seed=14)
    print("fp8 t2i_2048 mode %d: %d of %d compared rows in split tiles" % (mode, n_in, len(sel)),
          flush=True)
    assert n_in > 0
    _assert_fp8("fp8 split-KV t2i_2048 split %d" % n, mode, *_fwd_fp8(w, mode, sel, n_split=n),
                outliers=True)


@pytest.mark.parametrize("mode", MODES)
def test_fp8_splitkv_t2i_1024_sampled_rows(mode):
    # 1024^2 T2I: 864 query tiles on 256 CUs, the last 96 split (slice (1, 18) from row
    # 3072 on, and (1, 19) .. (1, 23))
    import joint_attention_amd as ja
    base = synth.WORKLOADS["t2i_1024_bf16"]
    w = synth.custom("t2i_1024_fp8", B=base.B, H=base.H, D=base.D, stream_lens=base.stream_lens,
                     outliers=base.outliers)
    n = ja.load().joint_attn_fwd_fp8_splitkv_suggest(w.B, w.H, w.N, w.D, mode)
    n = n if n > 1 else 2
    sel = synth.row_sample(w, 128, seed=15, n_pairs=2)
    sel, n_in = with_split_tile_rows(w, sel, "fp8", n_rows=160, seed=15)
    print("fp8 t2i_1024 mode %d: %d of %d compared rows in split tiles" % (mode, n_in, len(sel)),
          flush=True)
    assert n_in > 0
    _assert_fp8("fp8 split-KV t2i_1024 split %d" % n, mode, *_fwd_fp8(w, mode, sel, n_split=n),
                outliers=True)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("B,H,lens,n_split", [(1, 3, (100, 300), 1), (2, 128, (256,), 4)])
def test_fp8_splitkv_without_a_tail_is_the_plain_forward(B, H, lens, n_split, mode):
    import joint_attention_amd as ja
    import torch
    if torch.cuda.get_device_properties(0).multi_processor_count != 256 and n_split > 1:
        pytest.skip("the whole-rounds case assumes 256 CUs")
    w = synth.custom("f8skvp", B=B, H=H, D=128, stream_lens=lens, outliers=4, seed=19)
    q, k, vt, _ = device_packed(host_streams(w))
    t = ja.joint_attn_quant_fp8(q, k, vt, mode)
    a = ja.joint_attn_fwd_fp8(t)
    b = ja.joint_attn_fwd_fp8_splitkv(t, n_split=n_split)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
