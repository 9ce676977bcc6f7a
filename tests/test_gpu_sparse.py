"""GPU: block-sparse bf16 attention (joint_attn_fwd_bf16_sparse) against the block-sparse
oracle: random masks of several densities, rows and whole workgroups with no key, the
ragged last block, both head sizes; an all-ones mask equals the dense kernel bit for bit;
structured masks at full size on sampled rows.  Bar: the bf16 one (rel_F <= 5e-3, max |err|
<= 2e-2), empty rows exactly O = 0 and lse = -inf."""
import numpy as np
import pytest

import oracle
from joint_attention_amd import synth

from _common import (BF16_MAX_ABS, BF16_REL_F, device_packed, from_device_bf16, gather_rows,
                     host_streams, max_abs, packed_host, rel_frobenius, widen_bf16)

pytestmark = pytest.mark.gpu


def _run(w, mask, sel=None):
    import joint_attention_amd as ja
    import torch
    st = host_streams(w)
    q, k, vt, offs = device_packed(st)
    m_dev = torch.from_numpy(mask).cuda()
    scale = 1.0 / np.sqrt(w.D)
    o, lse = ja.joint_attn_fwd_bf16_sparse(q, k, vt, m_dev, scale, return_lse=True)
    torch.cuda.synchronize()
    qh, kh, vh, _ = packed_host(st)
    if sel is None:
        sel = oracle.all_rows(w.B, w.N, w.H)
    ref, ref_lse = oracle.sparse_attention_rows(qh, kh, vh, scale, mask, sel)
    got = gather_rows(widen_bf16(from_device_bf16(o)), sel)
    got_lse = lse.cpu().numpy()[sel[:, 0], sel[:, 1], sel[:, 2]].astype(np.float64)
    return got, ref, got_lse, ref_lse, (q, k, vt, m_dev, o)


def _assert(tag, got, ref, got_lse, ref_lse):
    empty = ~np.isfinite(ref_lse)
    assert np.all(got[empty] == 0), (tag, "O of rows without keys")
    assert np.all(got_lse[empty] == -np.inf), (tag, "lse of rows without keys")
    full = ~empty
    if full.any():
        rf, ma = rel_frobenius(got[full], ref[full]), max_abs(got[full], ref[full])
        le = float(np.abs(got_lse[full] - ref_lse[full]).max())
        print("%s: rel_F %.3e max %.3e lse %.2e (%d empty rows)" % (tag, rf, ma, le,
                                                                     int(empty.sum())), flush=True)
        assert rf <= BF16_REL_F and ma <= BF16_MAX_ABS, (tag, rf, ma)
        assert le <= 1e-2, (tag, le)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("lens,density", [((32, 256), 0.5), ((100, 300), 0.3),
                                          ((129, 64, 700), 0.2), ((512, 1000), 0.1),
                                          ((64, 600), 1.0)])
def test_sparse_random_every_row(D, lens, density):
    w = synth.custom("sp", B=2, H=2, D=D, stream_lens=lens, outliers=4 if D == 128 else 0,
                     seed=5 + sum(lens))
    mask = synth.block_mask(w, "random", density, seed=sum(lens))
    _assert("random %s %.1f D=%d" % (lens, density, D), *_run(w, mask)[:4])


def test_sparse_empty_rows_and_workgroups():
    w = synth.custom("spe", B=1, H=3, D=128, stream_lens=(64, 900), outliers=4, seed=3)
    mask = synth.block_mask(w, "random", 0.4, seed=1)
    mask[0, 0, 1, :] = 0            # one query block of head 0 sees nothing
    mask[0, 1, 2:4, :] = 0          # a whole 256-row workgroup of head 1 sees nothing
    mask[0, 2] = 0                  # head 2: no key at all
    _assert("empty rows", *_run(w, mask)[:4])


def test_sparse_all_ones_equals_dense_bitwise():
    import joint_attention_amd as ja
    import torch
    w = synth.custom("spd", B=2, H=2, D=128, stream_lens=(77, 555), outliers=4, seed=9)
    mask = np.ones((w.B, w.H) + oracle.mask_shape(w.N), np.uint8)
    _, _, _, _, (q, k, vt, m_dev, o) = _run(w, mask, sel=oracle.all_rows(1, 4, 1))
    o_d = ja.joint_attn_fwd_bf16(q, k, vt, 1.0 / np.sqrt(w.D))
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_d.view(torch.int16))


@pytest.mark.parametrize("name", ["t2i_1024_bf16", "t2i_2048_bf16"])
def test_sparse_structured_full_size(name):
    w = synth.WORKLOADS[name]
    mask = synth.block_mask(w, "structured", 0.15, band=2, seed=4)
    sel = synth.row_sample(w, 256, seed=17, n_pairs=4)
    _assert("structured " + name, *_run(w, mask, sel)[:4])


# ---- dispatch plan (joint_attn_sparse_plan) and the planned forward

def _plan_rule(mask):
    """The documented order, written out on the host: the B*H*nb workgroups in eight
    contiguous shares (sizes q + 1 for the first total % 8, then q); within a share the
    query blocks whose count of allowed key blocks exceeds twice the share's mean first,
    each group in its given order."""
    nb = mask.shape[-1]
    cnt = (mask.reshape(-1, nb) != 0).sum(-1).astype(np.int64)
    total = cnt.size
    q, r = divmod(total, 8)
    out = []
    for x in range(8):
        c0 = x * (q + 1) if x < r else r * (q + 1) + (x - r) * q
        n = q + (1 if x < r else 0)
        c = cnt[c0:c0 + n]
        idx = np.arange(c0, c0 + n)
        long_ = c * n > 2 * c.sum()
        out += [idx[long_], idx[~long_]]
    return np.concatenate(out).astype(np.int32)


def _plan_masks():
    t2i = synth.WORKLOADS["t2i_2048_bf16"]
    yield "structured 2048", synth.block_mask(t2i, "structured", 0.15, band=2, seed=4)
    yield "structured 1024", synth.block_mask(synth.WORKLOADS["t2i_1024_bf16"], "structured",
                                              0.15, band=2, seed=2)
    small = synth.custom("pl", B=1, H=3, D=128, stream_lens=(100, 600), seed=1)
    yield "random 0.3", synth.block_mask(small, "random", 0.3, seed=3)
    yield "all ones", np.ones((2, 5, 7, 7), np.uint8)
    yield "all zeros", np.zeros((1, 3, 6, 6), np.uint8)
    yield "3 units", synth.block_mask(synth.custom("p3", B=1, H=1, D=64, stream_lens=(40, 300),
                                                   seed=2), "structured", 0.2, seed=5)
    m = np.zeros((1, 2, 9, 9), np.uint8)          # 18 units: long rows in some shares only
    m[0, 0, [0, 4], :] = 1
    m[0, 1, 8, :] = 3                             # any nonzero byte counts
    m[0, 1, :, 2] = 1
    yield "hand", m
    big = np.random.default_rng(7).random((1, 2, 1024, 1024)) < 0.05
    big[:, :, -3:, :] = True                      # long rows at the end of a share
    yield "longest N", big.astype(np.uint8)


@pytest.mark.parametrize("tag,mask", list(_plan_masks()), ids=lambda x: x if isinstance(x, str) else "")
def test_sparse_plan_matches_rule(tag, mask):
    import joint_attention_amd as ja
    import torch
    nb = mask.shape[-1]
    N = nb * 128 - 5 if nb > 1 else 100
    plan = ja.joint_attn_sparse_plan(torch.from_numpy(mask).cuda(), N)
    torch.cuda.synchronize()
    got = plan.cpu().numpy()
    want = _plan_rule(mask)
    assert np.array_equal(np.sort(got), np.arange(mask.shape[0] * mask.shape[1] * nb)), tag
    assert np.array_equal(got, want), (tag, np.flatnonzero(got != want)[:10])


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("lens,kind", [((129, 64, 700), "random"), ((512, 1000), "structured"),
                                       ((32, 256), "random")])
def test_sparse_planned_equals_unplanned_and_oracle(D, lens, kind):
    import joint_attention_amd as ja
    import torch
    w = synth.custom("spp", B=2, H=3, D=D, stream_lens=lens, outliers=4 if D == 128 else 0,
                     seed=11 + sum(lens))
    mask = synth.block_mask(w, kind, 0.25, band=1, seed=sum(lens) + D)
    mask[0, 1, 0, :] = 0                          # a query block with no key
    got, ref, got_lse, ref_lse, (q, k, vt, m_dev, o) = _run(w, mask)
    plan = ja.joint_attn_sparse_plan(m_dev, w.N)
    o2, lse2 = ja.joint_attn_fwd_bf16_sparse_planned(q, k, vt, m_dev, plan, 1.0 / np.sqrt(w.D),
                                                     return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    sel = oracle.all_rows(w.B, w.N, w.H)
    lse2_rows = lse2.cpu().numpy()[sel[:, 0], sel[:, 1], sel[:, 2]].astype(np.float64)
    assert np.array_equal(lse2_rows, got_lse)
    _assert("planned %s %s D=%d" % (lens, kind, D), got, ref, got_lse, ref_lse)


@pytest.mark.parametrize("name", ["t2i_2048_bf16"])
def test_sparse_planned_full_size_bitwise(name):
    # the benchmarked configuration: the planned forward against the unplanned one, all rows
    import joint_attention_amd as ja
    import torch
    w = synth.WORKLOADS[name]
    mask = synth.block_mask(w, "structured", 0.15, band=2, seed=4)
    st = host_streams(w)
    q, k, vt, _ = device_packed(st)
    m_dev = torch.from_numpy(mask).cuda()
    scale = 1.0 / np.sqrt(w.D)
    o1, l1 = ja.joint_attn_fwd_bf16_sparse(q, k, vt, m_dev, scale, return_lse=True)
    plan = ja.joint_attn_sparse_plan(m_dev, w.N)
    o2, l2 = ja.joint_attn_fwd_bf16_sparse_planned(q, k, vt, m_dev, plan, scale, return_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(plan.cpu().numpy(), _plan_rule(mask))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
