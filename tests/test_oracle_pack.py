"""Pins for the reference token packing (CPU only)."""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("lens,expected", [
    ([32, 256], [0, 32, 288]),                       # tiny: text + 16x16 image
    ([512, 4096], [0, 512, 4608]),                   # 1024^2 T2I
    ([512, 16384], [0, 512, 16896]),                 # 2048^2 T2I
    ([512, 16384, 16384], [0, 512, 16896, 33280]),   # 2048^2 I2I with one reference
    ([3, 0, 5], [0, 3, 3, 8]),                       # an empty stream repeats its offset
    ([0], [0, 0]),
])
def test_offsets_hand_values(lens, expected):
    assert oracle.stream_offsets(lens).tolist() == expected


def _tagged(s, B, L, H, D):
    """Element value encodes (stream, b, token, h, c) uniquely."""
    b, t, h, c = np.meshgrid(np.arange(B), np.arange(L), np.arange(H), np.arange(D), indexing="ij")
    return (((s * 10 + b) * 1000 + t) * 10 + h) * 1000 + c


def test_pack_places_every_element_by_loop():
    B, H, D = 2, 3, 4
    lens = [5, 0, 7, 2]
    streams = [_tagged(s, B, L, H, D) for s, L in enumerate(lens)]
    packed, offs = oracle.pack_tokens(streams)
    assert packed.shape == (B, sum(lens), H, D)
    for b in range(B):
        for n in range(sum(lens)):
            s = max(i for i in range(len(lens)) if offs[i] <= n and lens[i] > 0 and n < offs[i + 1])
            t = n - offs[s]
            for h in range(H):
                for c in range(D):
                    assert packed[b, n, h, c] == (((s * 10 + b) * 1000 + t) * 10 + h) * 1000 + c


def test_head_major_and_channel_major_views():
    x = _tagged(1, 2, 6, 3, 4)
    bhnd = oracle.to_bhnd(x)
    bhdn = oracle.to_bhdn(x, 8)
    assert bhdn.shape == (2, 3, 4, 8)
    for b in range(2):
        for n in range(6):
            for h in range(3):
                for c in range(4):
                    assert bhnd[b, h, n, c] == x[b, n, h, c]
                    assert bhdn[b, h, c, n] == x[b, n, h, c]
    assert (bhdn[:, :, :, 6:] == 0).all()


def test_rejects_mismatched_streams():
    with pytest.raises(ValueError):
        oracle.pack_tokens([np.zeros((1, 2, 3, 4)), np.zeros((1, 2, 2, 4))])
    with pytest.raises(ValueError):
        oracle.stream_offsets([3, -1])
