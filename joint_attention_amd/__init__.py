"""joint_attention_amd -- joint multi-stream attention on AMD MI355X (gfx950).

The compute path is libjoint_attn.so (hand-written HIP kernels behind a C ABI, see
include/joint_attn.h); this package is its thin Python binding plus the seeded
synthetic-input generator used by the tests and the benchmark.
"""
from ._abi import (JointAttnError, Fp8Tensors, load, joint_attn_vt_ld, joint_attn_pack,
                   joint_attn_fwd_bf16, joint_attn_fwd_bf16_sparse, joint_attn_fwd_bf16_splitkv,
                   joint_attn_sparse_plan, joint_attn_fwd_bf16_sparse_planned,
                   joint_attn_fwd_bf16_streams, joint_attn_fwd_bf16_splitkv_noalloc,
                   joint_attn_fwd_bf16_streams_splitkv,
                   joint_attn_quant_fp8,
                   joint_attn_quant_fp8_streams, joint_attn_fwd_fp8, joint_attn_fwd_fp8_splitkv,
                   joint_attn_repair_count,
                   joint_attn_quant_fp8_repair, joint_attn_fwd_fp8_repair, EXPORTS, LIB_PATH,
                   JA_QK_BLOCK, JA_HI_CHANNELS, JA_FP8_PLAIN, JA_FP8_SPLIT, JA_FP8_REPAIR,
                   JA_SPARSE_BLOCK, JA_SPARSE_MAX_N, JA_SPARSE_PLAN_MAX, JA_REPAIR_MAX_N)

__all__ = ["JointAttnError", "Fp8Tensors", "load", "joint_attn_vt_ld", "joint_attn_pack",
           "joint_attn_fwd_bf16", "joint_attn_fwd_bf16_sparse", "joint_attn_fwd_bf16_splitkv",
           "joint_attn_sparse_plan", "joint_attn_fwd_bf16_sparse_planned",
           "joint_attn_fwd_bf16_streams", "joint_attn_fwd_bf16_splitkv_noalloc",
           "joint_attn_fwd_bf16_streams_splitkv",
           "joint_attn_quant_fp8",
           "joint_attn_quant_fp8_streams", "joint_attn_fwd_fp8", "joint_attn_fwd_fp8_splitkv",
           "joint_attn_repair_count",
           "joint_attn_quant_fp8_repair", "joint_attn_fwd_fp8_repair", "JA_FP8_REPAIR",
           "JA_REPAIR_MAX_N",
           "EXPORTS", "LIB_PATH", "JA_QK_BLOCK", "JA_HI_CHANNELS", "JA_FP8_PLAIN",
           "JA_FP8_SPLIT", "JA_SPARSE_BLOCK", "JA_SPARSE_MAX_N", "JA_SPARSE_PLAN_MAX"]
