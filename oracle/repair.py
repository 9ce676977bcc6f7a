"""TEST INFRASTRUCTURE ONLY: token repair of fp8 attention (the repair budget of
VC-Attention FP8).

Where it comes from.  The VisualGen FLUX 3 article (everytik.com translation, section
量化注意力与稀疏注意力) recommends VC-Attention FP8 at 2048x2048 with a repair budget
rho = 0.005: that share of the tokens, those with the highest quantisation error, gets a
residual correction.  The article says nothing more.  The plainest reading, taken here:

  * per (b, h), separately for Q and for K, n = ceil(rho * N) tokens are repaired
    (rho in [0, 1]; rho * N is evaluated in binary64, so n is the same on every side);
  * a token's quantisation error is its largest absolute residual over the head's D
    channels, max_c |x_c - decode(code_c) * scale|.  The residual of a bf16 value
    against its e4m3 neighbour times a power-of-two scale is exact in binary32, and so
    is the maximum: every implementation ranks the tokens identically;
  * the n tokens with the largest error are repaired, ties to the lower token index;
  * residual correction: the repaired tokens get their residual x - decode(code) * scale
    back, i.e. they enter Q K^T with their exact bf16 values.  P and V stay as in the
    plain fp8 recipe (fp8.fp8_attention_rows with q_exact / k_exact and q_rep / k_rep).
"""
from __future__ import annotations

import math

import numpy as np

from .fp8 import QK_BLOCK, _widen_f32, e4m3_decode, quantise_qk


def repair_count(N: int, rho: float) -> int:
    """Tokens repaired per (b, h) and operand: ceil(rho * N), rho in [0, 1]."""
    if not (0.0 <= rho <= 1.0):
        raise ValueError("rho must lie in [0, 1]")
    return min(int(N), int(math.ceil(float(rho) * float(N))))


def residual_linf(x_tok: np.ndarray, codes: np.ndarray, scales: np.ndarray,
                  block: int = QK_BLOCK) -> np.ndarray:
    """Per token and head, max over channels of |x - decode(code) * scale| ->
    float64 [B, H, N].  x_tok / codes token-major [B, N, H, D]; scales [B, H, nblk]."""
    B, N, H, D = x_tok.shape
    x = _widen_f32(x_tok).astype(np.float64)
    s_tok = scales[:, :, np.arange(N) // block].astype(np.float64)       # [B, H, N]
    xhat = e4m3_decode(codes) * np.transpose(s_tok, (0, 2, 1))[:, :, :, None]
    return np.transpose(np.abs(x - xhat).max(axis=3), (0, 2, 1))


def select_repair_tokens(err: np.ndarray, n: int) -> np.ndarray:
    """Per (b, h): the n tokens of largest err (ties: lower index), ascending ->
    int32 [B, H, n]."""
    B, H, N = err.shape
    out = np.empty((B, H, n), dtype=np.int32)
    idx = np.arange(N)
    for b in range(B):
        for h in range(H):
            order = np.lexsort((idx, -err[b, h]))[:n]      # by -err, then index
            out[b, h] = np.sort(order)
    return out


def quantise_qk_repair(x_tok: np.ndarray, n: int, block: int = QK_BLOCK):
    """Plain e4m3 quantisation of Q or K plus the repair selection ->
    (codes [B, N, H, D], scales [B, H, nblk], err [B, H, N], sel int32 [B, H, n])."""
    codes, scales = quantise_qk(x_tok, block)
    err = residual_linf(x_tok, codes, scales, block)
    return codes, scales, err, select_repair_tokens(err, n)
