"""TEST INFRASTRUCTURE ONLY -- the CPU oracle for joint multi-stream attention.

Plain, slow, obviously correct reference implementations, written from the VisualGen
FLUX 3 article (everytik.com translation) and the mathematics of softmax attention:

  pack       -- token concatenation of text / target / reference streams + offsets
  attention  -- fp64 two-pass softmax attention (C, OpenMP over rows)
  fp8        -- OCP e4m3 codec, the block/channel quantiser, fp8 attention
  sparse     -- block-sparse attention with an input block mask
  repair     -- token repair of fp8 attention (repair budget, error measure, selection)

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this
package.  The product path (joint_attention_amd) never imports it, and this package
never imports the product path; the two share no code.
"""
from .pack import stream_offsets, pack_tokens, to_bhnd, to_bhdn
from .attention import attention, attention_rows, all_rows, widen_bf16
from .fp8 import (E4M3_MAX, QK_BLOCK, P_SCALE_LOG2, HI_CHANNELS, e4m3_encode, e4m3_decode,
                  pow2_scale, quantise_qk, quantise_v, select_hi_channels, quantise_qk_split,
                  fp8_attention_rows, e4m3_midpoint_distance)
from .sparse import SPARSE_BQ, SPARSE_BK, mask_shape, sparse_attention_rows
from .repair import repair_count, residual_linf, select_repair_tokens, quantise_qk_repair
from ._native import build, default_threads

__all__ = [
    "stream_offsets", "pack_tokens", "to_bhnd", "to_bhdn",
    "attention", "attention_rows", "all_rows", "widen_bf16",
    "E4M3_MAX", "QK_BLOCK", "P_SCALE_LOG2", "HI_CHANNELS", "e4m3_encode", "e4m3_decode",
    "pow2_scale", "quantise_qk", "quantise_v", "select_hi_channels", "quantise_qk_split",
    "fp8_attention_rows", "e4m3_midpoint_distance",
    "SPARSE_BQ", "SPARSE_BK", "mask_shape", "sparse_attention_rows", "build", "default_threads",
    "repair_count", "residual_linf", "select_repair_tokens", "quantise_qk_repair",
]
