"""GPU: token packing through the C ABI is bit-exact against the oracle's packing."""
import numpy as np
import pytest

import oracle
from joint_attention_amd import synth

from _common import from_device_bf16, to_device

pytestmark = pytest.mark.gpu


def _random_streams(B, H, D, lens, seed):
    rng = np.random.default_rng(seed)
    return [rng.integers(0, 65536, size=(B, L, H, D), dtype=np.uint32).astype(np.uint16)
            for L in lens]


def _check(streams_bits, B, H, D):
    import joint_attention_amd as ja
    dev = [to_device(s) for s in streams_bits]
    ref_tok, ref_offs = oracle.pack_tokens(streams_bits)
    N = ref_tok.shape[1]
    got, offs = ja.joint_attn_pack(dev, "bhnd")
    assert offs == ref_offs.tolist()
    assert np.array_equal(from_device_bf16(got), oracle.to_bhnd(ref_tok))
    ld = ja.joint_attn_vt_ld(N)
    got_t, offs_t = ja.joint_attn_pack(dev, "bhdn")
    assert offs_t == ref_offs.tolist()
    assert tuple(got_t.shape) == (B, H, D, ld)
    assert np.array_equal(from_device_bf16(got_t), oracle.to_bhdn(ref_tok, ld))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("lens", [(32, 256), (3, 0, 17, 5), (1,), (0, 7), (129, 64, 1, 66)])
def test_pack_ragged_streams(D, lens):
    print("pack", D, lens, flush=True)
    _check(_random_streams(2, 3, D, lens, seed=sum(lens) + D), 2, 3, D)


def test_pack_wider_pitch_pads_with_zero():
    import torch
    import joint_attention_amd as ja
    print("pack wide pitch", flush=True)
    streams = _random_streams(1, 2, 128, (5, 20), seed=9)
    ref_tok, _ = oracle.pack_tokens(streams)
    ld = 64                                             # N = 25, pitch well past 32
    out = torch.full((1, 2, 128, ld), 7.0, dtype=torch.bfloat16, device="cuda")
    got, _ = ja.joint_attn_pack([to_device(s) for s in streams], "bhdn", ld=ld, out=out)
    assert np.array_equal(from_device_bf16(got), oracle.to_bhdn(ref_tok, ld))


def test_pack_t2i_1024_shape():
    print("pack t2i_1024", flush=True)
    st = synth.make_streams(synth.WORKLOADS["t2i_1024_bf16"])
    for streams in (st.q, st.v):
        _check(streams, 2, 24, 128)
