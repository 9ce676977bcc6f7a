"""Seeded synthetic inputs shaped like FLUX 3 Image Klein joint attention.

This module only draws inputs; it holds none of the attention arithmetic, and both the
HIP path's tests/benchmark and the CPU oracle consume exactly what it returns.

Workloads.  The VisualGen FLUX 3 article (everytik.com translation) measures T2I and
I2I generation at 1024x1024 and 2048x2048 with classifier-free guidance (batch 2,
section 使用 TensorRT LLM VisualGen 进行 FLUX 3 推理 / 表 1).  The pages give no head
count, head size, text length or patch size; the shapes below use 24 heads of 128,
512 text tokens and one token per 16x16 pixels (64x64 tokens at 1024^2, 128x128 at
2048^2), plus a two-head, head-size-64 toy case.

Value recipe (stated here because the pages give none):
  * Q and K rows are RMS-normalised standard-normal rows (eps 1e-6) times a per-channel
    gain drawn once from N(1, 0.1) (separately for Q and K, shared by all batches,
    heads and streams) -- the pages say the QKV projection is fused with query/key
    normalisation (section GEMM 内核优化), so Q and K arrive normalised;
  * in the large workloads 4 channels (one seeded draw, the same for Q and K, all
    heads) are multiplied by 8 after the normalisation, as activation outliers;
  * V ~ N(0, 1);
  * reference-image streams draw K and V from a second generator (seed + 1) with half
    the variance (factor sqrt(0.5)); their Q comes from the main generator;
  * draw order: gain_q, gain_k, outlier channels, then per stream Q, K, V;
  * values are drawn in float64 and rounded once to binary32, then to bf16, both with
    round-to-nearest-even.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    D: int
    stream_lens: tuple          # text, target, then reference streams
    n_reference: int = 0        # how many trailing streams are reference images
    outliers: int = 0           # channels scaled x8 in Q and K
    precision: str = "bf16"     # arithmetic of the attention call being measured
    seed: int = 0

    @property
    def N(self) -> int:
        return int(sum(self.stream_lens))

    @property
    def flops(self) -> int:
        """Algorithmic flops of one attention call: 2 GEMMs of 2*B*H*N*N*D each."""
        return 4 * self.B * self.H * self.N * self.N * self.D


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_bf16", B=1, H=2, D=64, stream_lens=(32, 256)),
        Workload("t2i_1024_bf16", B=2, H=24, D=128, stream_lens=(512, 4096), outliers=4),
        Workload("t2i_2048_bf16", B=2, H=24, D=128, stream_lens=(512, 16384), outliers=4),
        Workload("i2i_2048_bf16", B=2, H=24, D=128, stream_lens=(512, 16384, 16384),
                 n_reference=1, outliers=4),
        Workload("t2i_2048_fp8", B=2, H=24, D=128, stream_lens=(512, 16384), outliers=4,
                 precision="fp8"),
        # several reference images: text + target + r references of the target's size
        Workload("i2i_1024_r1_bf16", B=2, H=24, D=128, stream_lens=(512, 4096, 4096),
                 n_reference=1, outliers=4),
        Workload("i2i_1024_r3_bf16", B=2, H=24, D=128,
                 stream_lens=(512, 4096, 4096, 4096, 4096), n_reference=3, outliers=4),
        Workload("i2i_2048_r3_bf16", B=2, H=24, D=128,
                 stream_lens=(512, 16384, 16384, 16384, 16384), n_reference=3, outliers=4),
    ]
}


def custom(name="custom", B=1, H=2, D=128, stream_lens=(32, 256), n_reference=0,
           outliers=0, precision="bf16", seed=0) -> Workload:
    return Workload(name, B, H, D, tuple(stream_lens), n_reference, outliers, precision, seed)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """binary32 -> bf16 bit patterns, round to nearest even (inputs here are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def _to_bf16(x64: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(x64.astype(np.float32))


def _normed(rng, shape, gain, outlier_idx):
    x = rng.standard_normal(shape)
    x /= np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + 1e-6)
    x *= gain
    if len(outlier_idx):
        x[..., outlier_idx] *= 8.0
    return x


@dataclass
class Streams:
    """Per-stream bf16 bit arrays, each [B, L_s, H, D] uint16 (token-major)."""
    workload: Workload
    q: list = field(default_factory=list)
    k: list = field(default_factory=list)
    v: list = field(default_factory=list)
    outlier_channels: np.ndarray = field(default_factory=lambda: np.zeros(0, int))


def make_streams(w: Workload, seed: int | None = None) -> Streams:
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    ref_rng = np.random.default_rng(seed + 1)
    gain_q = rng.normal(1.0, 0.1, size=w.D)
    gain_k = rng.normal(1.0, 0.1, size=w.D)
    outl = rng.choice(w.D, w.outliers, replace=False) if w.outliers else np.zeros(0, int)
    out = Streams(w, outlier_channels=np.sort(outl))
    n_streams = len(w.stream_lens)
    for s, L in enumerate(w.stream_lens):
        shape = (w.B, L, w.H, w.D)
        is_ref = s >= n_streams - w.n_reference
        out.q.append(_to_bf16(_normed(rng, shape, gain_q, outl)))
        src = ref_rng if is_ref else rng
        k = _normed(src, shape, gain_k, outl)
        v = src.standard_normal(shape)
        if is_ref:
            k *= np.sqrt(0.5)
            v *= np.sqrt(0.5)
        out.k.append(_to_bf16(k))
        out.v.append(_to_bf16(v))
        del k, v
    return out


def row_sample(w: Workload, n_rows: int, seed: int = 1234, n_pairs: int | None = None) -> np.ndarray:
    """(b, h, i) triples for sampled parity checks at full size: every row within two
    tokens of each stream boundary and of both ends, plus random rows; restricted to
    n_pairs random (b, h) pairs when given.  Sorted by (b, h, i)."""
    rng = np.random.default_rng(seed)
    all_pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    if n_pairs is not None:
        idx = rng.choice(len(all_pairs), min(n_pairs, len(all_pairs)), replace=False)
        pairs = [all_pairs[i] for i in sorted(idx)]
    else:
        pairs = all_pairs
    offs = np.concatenate([[0], np.cumsum(w.stream_lens)])
    edge = set()
    for o in offs:
        for d in range(-2, 3):
            if 0 <= o + d < w.N:
                edge.add(int(o + d))
    rows = set()
    for i in sorted(edge):
        b, h = pairs[int(rng.integers(len(pairs)))]
        rows.add((b, h, i))
    while len(rows) < n_rows:
        b, h = pairs[int(rng.integers(len(pairs)))]
        rows.add((b, h, int(rng.integers(w.N))))
    return np.asarray(sorted(rows), dtype=np.int64)


def block_mask(w: Workload, kind: str = "structured", density: float = 0.25, band: int = 2,
               seed: int = 0, block: int = 128) -> np.ndarray:
    """Seeded uint8 block mask [B, H, nb, nb] (nb = ceil(N / block)) for block-sparse runs.

    "random": every (query block, key block) on with probability `density`.
    "structured": the text blocks (those holding stream 0's tokens) on in whole rows and
    columns, the key blocks within `band` of each query block's diagonal on, and the other
    image-image blocks on with probability `density`: a stand-in for the per-block selection
    of a sparse-attention method, whose rule is not given.
    """
    rng = np.random.default_rng(seed)
    nb = -(-w.N // block)
    m = (rng.random((w.B, w.H, nb, nb)) < density).astype(np.uint8)
    if kind == "structured":
        n_text = -(-w.stream_lens[0] // block) if w.stream_lens[0] > 0 else 0
        m[:, :, :n_text, :] = 1
        m[:, :, :, :n_text] = 1
        qb, kb = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
        m[:, :, np.abs(qb - kb) <= band] = 1
    elif kind != "random":
        raise ValueError("kind must be 'random' or 'structured'")
    return m
