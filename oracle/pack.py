"""TEST INFRASTRUCTURE ONLY: reference token packing.

The VisualGen FLUX 3 article (everytik.com translation, section
使用 TensorRT LLM VisualGen 进行 FLUX 3 推理) describes three kinds of token streams --
text, the noisy target image, and optional reference images -- that are processed on
their own and joined only inside joint attention; its offline-inference section
(离线推理) shows that several reference images may be given.  Joining them means
concatenating the streams along the token axis in that order.  Offsets are the
exclusive prefix sums of the stream lengths.
"""
from __future__ import annotations

import numpy as np


def stream_offsets(lens) -> np.ndarray:
    """[0, L0, L0+L1, ...]: where each stream starts in the packed sequence (int64)."""
    lens = np.asarray(lens, dtype=np.int64)
    if lens.ndim != 1 or (lens < 0).any():
        raise ValueError("stream lengths must be a 1-D array of non-negative ints")
    out = np.zeros(len(lens) + 1, dtype=np.int64)
    out[1:] = np.cumsum(lens)
    return out


def pack_tokens(streams) -> tuple[np.ndarray, np.ndarray]:
    """Concatenate per-stream [B, L_s, H, D] arrays along tokens -> ([B, N, H, D], offsets)."""
    streams = list(streams)
    if not streams:
        raise ValueError("need at least one stream")
    B, _, H, D = streams[0].shape
    for s in streams:
        if s.ndim != 4 or s.shape[0] != B or s.shape[2] != H or s.shape[3] != D:
            raise ValueError("every stream must be [B, L_s, H, D] with the same B, H, D")
    packed = np.concatenate(streams, axis=1)
    return packed, stream_offsets([s.shape[1] for s in streams])


def to_bhnd(x_tok: np.ndarray) -> np.ndarray:
    """Token-major [B, N, H, D] -> head-major [B, H, N, D] (a copy)."""
    return np.ascontiguousarray(x_tok.transpose(0, 2, 1, 3))


def to_bhdn(x_tok: np.ndarray, ld: int) -> np.ndarray:
    """Token-major [B, N, H, D] -> channel-major [B, H, D, ld]; columns N..ld-1 are zero."""
    B, N, H, D = x_tok.shape
    if ld < N:
        raise ValueError("ld must be >= N")
    out = np.zeros((B, H, D, ld), dtype=x_tok.dtype)
    out[:, :, :, :N] = x_tok.transpose(0, 2, 3, 1)
    return out
