"""TEST INFRASTRUCTURE ONLY: fp64 joint attention (wraps attention_ref.c).

Definition (unmasked scaled-dot-product softmax attention over the packed text +
target + reference tokens; the VisualGen FLUX 3 article, everytik.com translation,
sections 使用 TensorRT LLM VisualGen 进行 FLUX 3 推理 and 量化注意力与稀疏注意力):

    O[b, i, h, :] = sum_j softmax_j(scale * q_i . k_j) * v_j
    lse[b, h, i]  = ln sum_j exp(scale * q_i . k_j)

All arithmetic is in double precision, two passes per row (max, then weights).
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _native

KIND_F64 = 0
KIND_BF16 = 1


def _as_input(x: np.ndarray) -> tuple[np.ndarray, int]:
    if x.dtype == np.uint16:           # bf16 bit patterns
        return np.ascontiguousarray(x), KIND_BF16
    return np.ascontiguousarray(x, dtype=np.float64), KIND_F64


def attention_rows(q, k, v, softmax_scale: float, sel, threads: int | None = None):
    """Selected query rows of joint attention.

    q: token-major [B, Nq, H, D]; k, v: token-major [B, N, H, D]; all uint16 (bf16
    bits) or all floating point.  sel: int array [n, 3] of (b, h, i), i < Nq.
    Returns (O [n, D] float64, lse [n] float64).
    """
    qa, kind_q = _as_input(q)
    ka, kind_k = _as_input(k)
    va, kind_v = _as_input(v)
    if not (kind_q == kind_k == kind_v):
        raise ValueError("q, k, v must all be bf16 bits or all floating point")
    if ka.shape != va.shape or qa.ndim != 4 or ka.ndim != 4 or \
            qa.shape[0] != ka.shape[0] or qa.shape[2:] != ka.shape[2:]:
        raise ValueError("q must be [B, Nq, H, D] and k, v [B, N, H, D]")
    B, Nq, H, D = qa.shape
    N = ka.shape[1]
    sel = np.ascontiguousarray(np.asarray(sel, dtype=np.int64).reshape(-1, 3))
    n = sel.shape[0]
    out = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    if n == 0:
        return out, lse
    t = threads or _native.default_threads()
    rc = _native.lib().oracle_attention_rows(
        qa.ctypes.data, ka.ctypes.data, va.ctypes.data, kind_q,
        B, Nq, N, H, D, float(softmax_scale), sel.ctypes.data, n,
        out.ctypes.data, lse.ctypes.data, int(t))
    if rc != 0:
        raise RuntimeError("oracle_attention_rows failed with status %d" % rc)
    return out, lse


def all_rows(B: int, N: int, H: int) -> np.ndarray:
    """Every (b, h, i) triple in [B, H, N] order."""
    b, h, i = np.meshgrid(np.arange(B), np.arange(H), np.arange(N), indexing="ij")
    return np.stack([b.ravel(), h.ravel(), i.ravel()], axis=1).astype(np.int64)


def attention(q, k, v, softmax_scale: float, threads: int | None = None):
    """Every row: returns (O [B, N, H, D] float64, lse [B, H, N] float64)."""
    B, N, H, D = q.shape
    o, lse = attention_rows(q, k, v, softmax_scale, all_rows(B, N, H), threads)
    o = o.reshape(B, H, N, D).transpose(0, 2, 1, 3).copy()
    return o, lse.reshape(B, H, N)


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    u = bits.astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)
