"""GPU: every forward at the longest sequences it is tested for, on sampled rows against
the oracle at each path's own bar.

- sparse (unplanned, and planned bit for bit against it) and token repair: exactly their
  declared maxima, JA_SPARSE_MAX_N and JA_REPAIR_MAX_N (131072 tokens);
- fp8 plain and split: 130771 tokens (a ragged last tile; 511 query tiles, so the split-KV
  call splits the 255 of its last round), plain and split-KV calls;
- dense bf16: 2^20 + 77 tokens, through the plain, split-KV and in-place stream calls.

The dense bf16 length is 16 times the longest workload on the pages (66048 tokens) and an
eighth of the ABI's own bound (one head's V^T at most JA_MAX_HEAD_ELEMS elements, whose
rejection is checked on the CPU).  One (b, h) slice keeps the host-side generation and the
oracle rows small.
"""
import numpy as np
import pytest

import joint_attention_amd as ja
from joint_attention_amd import synth

import test_gpu_fp8
import test_gpu_fp8_repair
import test_gpu_fwd_bf16
import test_gpu_fwd_streams
import test_gpu_sparse
import test_gpu_splitkv
from _common import with_split_tile_rows

pytestmark = pytest.mark.gpu

LONG_BF16 = synth.custom("long_bf16", B=1, H=1, D=128, stream_lens=(512, (1 << 20) + 77 - 512),
                         outliers=4, seed=101)


def _sample(w, n_rows, seed):
    return synth.row_sample(w, n_rows, seed=seed)


def test_bf16_longest_plain():
    w = LONG_BF16
    sel = _sample(w, 48, 5)
    print("bf16 plain N", w.N, flush=True)
    test_gpu_fwd_bf16._assert_parity("bf16 N=%d" % w.N, *test_gpu_fwd_bf16._run(w, sel=sel)[:4])


def test_bf16_longest_splitkv():
    w = LONG_BF16
    n = ja.load().joint_attn_fwd_bf16_splitkv_suggest(w.B, w.H, w.N, w.D)
    n = n if n > 1 else 5
    sel, n_in = with_split_tile_rows(w, _sample(w, 48, 5), "bf16", n_rows=48, seed=5)
    print("bf16 split-KV N %d split %d: %d of %d compared rows in split tiles"
          % (w.N, n, n_in, len(sel)), flush=True)
    test_gpu_splitkv._assert("split-KV N=%d split %d" % (w.N, n),
                             *test_gpu_splitkv._run(w, n, sel)[:4])


def test_bf16_longest_streams():
    # equal to pack + plain forward bit for bit, and the bf16 bar against the oracle
    w = LONG_BF16
    print("bf16 streams N", w.N, flush=True)
    test_gpu_fwd_streams._check(w, sel=_sample(w, 32, 6), tag="longest")


def test_sparse_longest():
    w = synth.custom("long_sparse", B=1, H=2, D=128,
                     stream_lens=(512, ja.JA_SPARSE_MAX_N - 512), outliers=4, seed=102)
    assert w.N == ja.JA_SPARSE_MAX_N
    mask = synth.block_mask(w, "structured", 0.15, band=2, seed=4)
    sel = _sample(w, 96, 7)
    print("sparse N", w.N, flush=True)
    got, ref, got_lse, ref_lse, (q, k, vt, m_dev, o) = test_gpu_sparse._run(w, mask, sel)
    test_gpu_sparse._assert("sparse N=%d" % w.N, got, ref, got_lse, ref_lse)
    # the dispatch plan at the same size: its rule, and the planned forward bit for bit
    import torch
    plan = ja.joint_attn_sparse_plan(m_dev, w.N)
    o2 = ja.joint_attn_fwd_bf16_sparse_planned(q, k, vt, m_dev, plan, 1.0 / np.sqrt(w.D))
    torch.cuda.synchronize()
    assert np.array_equal(plan.cpu().numpy(), test_gpu_sparse._plan_rule(mask))
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("split_kv", [False, True])
@pytest.mark.parametrize("mode", [0, 1])
def test_fp8_longest(mode, split_kv):
    w = synth.custom("long_fp8", B=1, H=1, D=128,
                     stream_lens=(512, ja.JA_REPAIR_MAX_N - 301 - 512), outliers=4, seed=103)
    n = None
    sel = _sample(w, 64, 8)
    if split_kv:
        n = ja.load().joint_attn_fwd_fp8_splitkv_suggest(w.B, w.H, w.N, w.D, mode)
        n = n if n > 1 else 5
        sel, n_in = with_split_tile_rows(w, sel, "fp8", n_rows=48, seed=8)
        print("fp8 N %d: %d of %d compared rows in split tiles" % (w.N, n_in, len(sel)),
              flush=True)
        assert n_in > 0
    print("fp8 N", w.N, "mode", mode, "split", n, flush=True)
    test_gpu_fp8._assert_fp8("fp8 N=%d split %s" % (w.N, n), mode,
                             *test_gpu_fp8._fwd_fp8(w, mode, sel, n_split=n), outliers=True)


@pytest.mark.parametrize("split_kv", [False, True])
@pytest.mark.parametrize("mode", [0, 1])
def test_fp8_beyond_one_scale_table(mode, split_kv):
    # more than 2048 K scale blocks (the fp8 forward's LDS table of block scales is
    # refilled on the way): 2048 * 128 + 12345 keys, ragged last tile
    w = synth.custom("long_fp8_tab", B=1, H=1, D=128, stream_lens=(512, 2048 * 128 + 12345 - 512),
                     outliers=4, seed=105)
    n = None
    sel = _sample(w, 48, 10)
    if split_kv:
        n = ja.load().joint_attn_fwd_fp8_splitkv_suggest(w.B, w.H, w.N, w.D, mode)
        n = n if n > 1 else 5
        sel, n_in = with_split_tile_rows(w, sel, "fp8", n_rows=32, seed=10)
        assert n_in > 0
    print("fp8 N", w.N, "mode", mode, "split", n, flush=True)
    test_gpu_fp8._assert_fp8("fp8 N=%d split %s" % (w.N, n), mode,
                             *test_gpu_fp8._fwd_fp8(w, mode, sel, n_split=n), outliers=True)


def test_repair_longest():
    w = synth.custom("long_rep", B=1, H=1, D=128,
                     stream_lens=(512, ja.JA_REPAIR_MAX_N - 512), outliers=4, seed=104)
    assert w.N == ja.JA_REPAIR_MAX_N
    sel = _sample(w, 64, 9)
    # the sampled rows plus a stride of the repaired rows
    t = test_gpu_fp8_repair._run(w, 0.005, fwd=False)["t"]
    rep = t.q_sel.cpu().numpy()[0, 0]
    extra = [(0, 0, int(i)) for i in rep[::16]]
    sel = np.asarray(sorted(set(map(tuple, sel.tolist())) | set(extra)), dtype=np.int64)
    print("repair N", w.N, "rows", len(sel), flush=True)
    c = test_gpu_fp8_repair._compare(w, 0.005, sel)
    assert c["n"] == 656 and c["rep_row"].sum() >= len(extra)
    test_gpu_fp8_repair._assert_repair("repair N=%d" % w.N, c, outliers=True)
