"""TEST INFRASTRUCTURE ONLY: reference fp8 (e4m3) quantisation and fp8 attention.

Where it comes from.  The VisualGen FLUX 3 article (everytik.com translation, section
量化注意力与稀疏注意力) runs attention with fp8 Q/K (qk_dtype) and fp8 V (v_dtype) but
prints no quantisation recipe; the kongchang.com English page ("Accelerated Deployment
of FLUX 3 Klein on NVIDIA Blackwell", section "Reducing Numerical Precision") only says
that narrow formats need block-wise scale factors.  The recipe below is this library's
plainest reading of those two facts:

  * format: OCP FP8 E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa bits,
    subnormal step 2**-9, largest finite 448, no infinities; S.1111.111 is NaN);
  * Q and K: one scale per (b, h, block of 128 consecutive packed tokens);
  * V: one scale per (b, h, channel) over all tokens;
  * every scale is a power of two, as the shared scales of the OCP Microscaling (MX)
    formats are: scale = 2**k with k the smallest integer such that amax <= 448 * 2**k
    (k >= -126; amax == 0 gives scale 1), so x / scale is exact and
    codes = e4m3(x / scale) with e4m3 rounding to nearest even (|x / scale| <= 448);
  * P: the softmax numerators, taken relative to an integer row maximum in base 2
    and multiplied by 2**8, are rounded to e4m3 before the P.V product; the row sum
    uses the unrounded numerators.

A second, corrected mode keeps R = 16 channels of Q and K per (b, h) out of the e4m3
product: the channels with the largest amax(|q_c|) * amax(|k_c|) over all tokens (ties:
lower index).  Their exact bf16 values, divided by the block scale (exact, the scale
being a power of two), enter the same logit accumulation; their e4m3 codes are zero.
This is the residual-correction idea of the article's VC-Attention remark (section
量化注意力与稀疏注意力: the part of the input with the largest quantisation error gets a
correction) applied to whole channels, where activation outliers live.

Scales are dequantisation multipliers: x ~= decode(code) * scale.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
QK_BLOCK = 128          # tokens per Q/K scale block
P_SCALE_LOG2 = 8        # P is stored as e4m3(2**8 * p)
HI_CHANNELS = 16        # channels of Q and K kept out of e4m3 in the corrected mode


# --------------------------------------------------------------------- the format
def e4m3_encode(x) -> np.ndarray:
    """Round to the nearest e4m3 value (ties to even) after clamping to +-448.

    Works on any real array; values are handled in float64, where every step below is
    exact.  NaN maps to 0x7F (with its sign); the sign of zero is kept.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    a = np.minimum(np.abs(x), E4M3_MAX)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, a)
    _, E = np.frexp(a)                      # a = f * 2**E, f in [0.5, 1)
    e = E.astype(np.int64) - 1              # a in [2**e, 2**(e+1))
    normal = a >= 2.0 ** -6
    q = np.where(normal, e - 3, -9)         # spacing of e4m3 values near a
    r = np.rint(a / np.exp2(q.astype(np.float64)))   # ties to even; exact division
    # normal: value = r * 2**(e-3), r in [8, 16] -> code = (e+7)*8 + (r-8);
    #         r == 16 rolls over into the next binade by itself.
    # subnormal: value = r * 2**-9, r in [0, 8] -> code = r (8 is the smallest normal).
    code = np.where(normal, (e + 7) * 8 + (r.astype(np.int64) - 8), r.astype(np.int64))
    code = np.where(nan, 0x7F, code)
    return (code.astype(np.uint8) | sign)


def e4m3_decode(code) -> np.ndarray:
    """e4m3 codes (uint8) -> float64 values (NaN for the two NaN codes)."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(E == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((E - 7).astype(np.float64)))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


# --------------------------------------------------------------------- quantisers
def _widen_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def pow2_scale(amax) -> np.ndarray:
    """Smallest power of two s (>= 2**-126) with amax <= 448 * s; 1 where amax == 0.

    amax = f * 2**E with f in [0.5, 1): 448 * 2**(E-9) = 0.875 * 2**E, so k = E - 9 when
    amax <= 0.875 * 2**E and E - 8 otherwise (all comparisons exact in float64)."""
    a = np.asarray(amax, dtype=np.float64)
    f, E = np.frexp(a)
    k = np.where(f <= 0.875, E - 9, E - 8)
    k = np.maximum(k, -126)
    return np.where(a == 0, 1.0, np.ldexp(1.0, k)).astype(np.float32)


def quantise_qk(x_tok: np.ndarray, block: int = QK_BLOCK):
    """Q or K, token-major [B, N, H, D] bf16 bits -> (codes [B, N, H, D] uint8,
    scales [B, H, ceil(N/block)] float32).  A short last block uses its own rows."""
    B, N, H, D = x_tok.shape
    x = _widen_f32(x_tok)
    nblk = -(-N // block)
    codes = np.empty((B, N, H, D), dtype=np.uint8)
    scales = np.empty((B, H, nblk), dtype=np.float32)
    for blk in range(nblk):
        lo, hi = blk * block, min(N, (blk + 1) * block)
        xb = x[:, lo:hi].astype(np.float64)                # [B, t, H, D]
        scale = pow2_scale(np.abs(xb).max(axis=(1, 3)))    # [B, H]
        scales[:, :, blk] = scale
        codes[:, lo:hi] = e4m3_encode(xb / scale.astype(np.float64)[:, None, :, None])
    return codes, scales


def quantise_v(x_tok: np.ndarray):
    """V, token-major [B, N, H, D] bf16 bits -> (codes [B, N, H, D] uint8,
    scales [B, H, D] float32), one scale per channel over all tokens."""
    x = _widen_f32(x_tok).astype(np.float64)
    scale = pow2_scale(np.abs(x).max(axis=1))               # [B, H, D]
    return e4m3_encode(x / scale.astype(np.float64)[:, None, :, :]), scale


def select_hi_channels(q_tok: np.ndarray, k_tok: np.ndarray, r: int = HI_CHANNELS):
    """Per (b, h): the r channels with the largest amax(|q_c|) * amax(|k_c|) over all
    tokens (ties to the lower index), in ascending channel order -> int32 [B, H, r]."""
    qa = np.abs(_widen_f32(q_tok).astype(np.float64)).max(axis=1)     # [B, H, D]
    ka = np.abs(_widen_f32(k_tok).astype(np.float64)).max(axis=1)
    score = qa * ka                                     # exact: bf16 * bf16
    B, H, D = score.shape
    sel = np.empty((B, H, r), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            order = sorted(range(D), key=lambda c: (-score[b, h, c], c))[:r]
            sel[b, h] = sorted(order)
    return sel


def quantise_qk_split(x_tok: np.ndarray, sel: np.ndarray, block: int = QK_BLOCK):
    """Corrected mode: e4m3 codes as quantise_qk with the selected channels' codes set to
    zero, plus their exact values divided by the block scale -> (codes [B, N, H, D],
    scales [B, H, nblk], hi [B, N, H, r] float64)."""
    codes, scales = quantise_qk(x_tok, block)
    x = _widen_f32(x_tok).astype(np.float64)
    B, N, H, D = x.shape
    r = sel.shape[2]
    blk_of = np.arange(N) // block
    hi = np.empty((B, N, H, r))
    for b in range(B):
        for h in range(H):
            codes[b, :, h, sel[b, h]] = 0
            s_tok = scales[b, h, blk_of].astype(np.float64)
            hi[b, :, h, :] = x[b][:, h, sel[b, h]] / s_tok[:, None]
    return codes, scales, hi


# --------------------------------------------------------------------- fp8 attention
def e4m3_midpoint_distance(x) -> np.ndarray:
    """Distance of each x >= 0 (x <= 448) to the nearest point where e4m3 rounding
    switches between two neighbouring values (the midpoints of the e4m3 grid), and the
    grid step there.  Returns (distance, step), float64."""
    a = np.asarray(x, dtype=np.float64)
    _, E = np.frexp(a)
    e = E.astype(np.int64) - 1
    step = np.where(a >= 2.0 ** -6, np.exp2((e - 3).astype(np.float64)), 2.0 ** -9)
    y = a / step                                  # exact: step is a power of two
    dist = np.abs(y - np.floor(y) - 0.5) * step
    return dist, step


def fp8_attention_rows(q8, k8, v8, q_scale, k_scale, v_scale, softmax_scale: float, sel,
                       block: int = QK_BLOCK, q_hi=None, k_hi=None, rel_window=None,
                       q_exact=None, k_exact=None, q_rep=None, k_rep=None):
    """Attention on the fp8 operands, selected rows (b, h, i).

    For each row, in float64 with exactly dequantised operands:
        t_j  = (q_i . k_j) * softmax_scale / ln 2            (logit in base-2 units)
        M    = ceil(max_j t_j)                               (integer row maximum)
        p_j  = 2 ** (t_j - M)                                (in (0, 1])
        P_j  = decode(e4m3(2**8 * p_j))                      (P rounded to e4m3)
        O[c] = (sum_j P_j * v_j[c]) / (2**8 * sum_j p_j)
        lse  = (M + log2 sum_j p_j) * ln 2
    q8/k8/v8 are token-major [B, N, H, D] codes; q_scale/k_scale [B, H, nblk];
    v_scale [B, H, D].  In the corrected mode q_hi/k_hi [B, N, H, r] hold the kept
    channels divided by their block scale and add (q_hi . k_hi) * qs * ks to the dot
    product.  In the token-repair mode q_rep / k_rep [B, H, n] list, per (b, h), the
    query / key tokens whose exact values (q_exact / k_exact, token-major bf16 bits
    [B, N, H, D]) replace the dequantised ones in the dot product.  Returns
    (O [n, D], lse [n]).

    Rounding P to e4m3 is a decision taken on a floating-point logit: an implementation
    whose logits differ by rounding alone may round 2**8 * p_j the other way where it
    lies within a hair of a midpoint of the e4m3 grid.  With rel_window set, a third
    result [n, D] bounds what that can change: the sum over keys whose 2**8 * p_j lies
    within rel_window * 2**8 * p_j of a midpoint of step_j * |v_j[c]| / (2**8 * sum p).
    """
    B, N, H, D = q8.shape
    sel = np.asarray(sel, dtype=np.int64).reshape(-1, 3)
    out = np.empty((len(sel), D), dtype=np.float64)
    lse = np.empty((len(sel),), dtype=np.float64)
    flip = None if rel_window is None else np.empty((len(sel), D), dtype=np.float64)
    blk_of = np.arange(N) // block
    cache = {}
    for r, (b, h, i) in enumerate(sel):
        key = (int(b), int(h))
        if key not in cache:
            ks_tok = k_scale[b, h, blk_of].astype(np.float64)
            kd = e4m3_decode(k8[b, :, h, :]) * ks_tok[:, None]
            vd = e4m3_decode(v8[b, :, h, :]) * v_scale[b, h][None, :].astype(np.float64)
            kh = None if k_hi is None else k_hi[b, :, h, :] * ks_tok[:, None]
            if k_rep is not None:
                idx = np.asarray(k_rep[b, h], dtype=np.int64)
                kd[idx] = _widen_f32(k_exact[b, idx, h, :]).astype(np.float64)
            qset = set() if q_rep is None else set(int(t) for t in q_rep[b, h])
            cache = {key: (kd, vd, kh, qset)}             # keep one (b, h) at a time
        kd, vd, kh, qset = cache[key]
        qs = float(q_scale[b, h, i // block])
        if int(i) in qset:
            qd = _widen_f32(q_exact[b, i, h, :]).astype(np.float64)
        else:
            qd = e4m3_decode(q8[b, i, h, :]) * qs
        dots = kd @ qd
        if kh is not None:
            dots = dots + kh @ (q_hi[b, i, h, :] * qs)
        t = dots * (softmax_scale / math.log(2.0))
        M = math.ceil(t.max())
        p = np.exp2(t - M)
        x = p * 2.0 ** P_SCALE_LOG2
        P = e4m3_decode(e4m3_encode(x))
        l = p.sum()
        out[r] = (P @ vd) / (2.0 ** P_SCALE_LOG2 * l)
        lse[r] = (M + math.log2(l)) * math.log(2.0)
        if flip is not None:
            dist, step = e4m3_midpoint_distance(x)
            near = dist <= rel_window * x
            flip[r] = (step * near) @ np.abs(vd) / (2.0 ** P_SCALE_LOG2 * l)
    return (out, lse) if flip is None else (out, lse, flip)
