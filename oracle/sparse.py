"""TEST INFRASTRUCTURE ONLY: block-sparse joint attention (fp64, numpy).

The VisualGen FLUX 3 article (everytik.com translation, section 量化注意力与稀疏注意力)
offers sparse attention (Sol-Attention) running on a general block-sparse attention
kernel; the rule that chooses the blocks is not given, so here the block mask is an input.
Definition, per (b, h) and query row i:

    allowed(i, j) = mask[b, h, i // BQ, j // BK] != 0
    s_ij = scale * q_i . k_j               for allowed j, and -inf otherwise
    O_i  = sum_j softmax_j(s_ij) v_j,      lse_i = ln sum_{allowed j} exp(s_ij)

A row with no allowed key has O_i = 0 and lse_i = -inf (the empty sum).  All arithmetic is
in double precision: two passes per row, as in the dense oracle.
"""
from __future__ import annotations

import numpy as np

SPARSE_BQ = 128     # query rows per mask block
SPARSE_BK = 128     # keys per mask block


def _widen(x: np.ndarray) -> np.ndarray:
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def mask_shape(N: int, bq: int = SPARSE_BQ, bk: int = SPARSE_BK) -> tuple[int, int]:
    return -(-N // bq), -(-N // bk)


def sparse_attention_rows(q, k, v, softmax_scale: float, mask, sel, bq: int = SPARSE_BQ,
                          bk: int = SPARSE_BK):
    """Selected rows (b, h, i) of block-sparse attention.

    q, k, v: token-major [B, N, H, D], bf16 bits (uint16) or floating point;
    mask: [B, H, ceil(N / bq), ceil(N / bk)], nonzero = the block is attended.
    Returns (O [n, D], lse [n]) in float64.
    """
    B, N, H, D = q.shape
    mask = np.asarray(mask)
    if mask.shape != (B, H) + mask_shape(N, bq, bk):
        raise ValueError("mask must be [B, H, ceil(N/bq), ceil(N/bk)]")
    sel = np.asarray(sel, dtype=np.int64).reshape(-1, 3)
    out = np.zeros((len(sel), D))
    lse = np.full((len(sel),), -np.inf)
    key_block = np.arange(N) // bk
    cache = {}
    for r, (b, h, i) in enumerate(sel):
        if (b, h) not in cache:
            cache = {(b, h): (_widen(k[b, :, h, :]), _widen(v[b, :, h, :]))}
        kd, vd = cache[(b, h)]
        allowed = mask[b, h, i // bq][key_block] != 0
        if not allowed.any():
            continue
        s = (kd[allowed] @ _widen(q[b, i, h, :])) * softmax_scale
        m = s.max()
        w = np.exp(s - m)
        out[r] = (w @ vd[allowed]) / w.sum()
        lse[r] = m + np.log(w.sum())
    return out, lse
