// Host-side launchers of the gfx950 kernels (internal to libjoint_attn; arguments are
// validated by the C entry points before any of these is called).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "joint_attn.h"

namespace ja {

// Per-stream source tensors of one joint sequence (Q, K and V, each bf16 [B][L_s][H][D])
// with the packed offsets: stream s holds packed tokens off[s] .. off[s+1]-1.  Passed to
// kernels by value.
struct StreamTable {
    const void* q[JA_MAX_STREAMS];
    const void* k[JA_MAX_STREAMS];
    const void* v[JA_MAX_STREAMS];
    int64_t off[JA_MAX_STREAMS + 1];
    int n;
};

hipError_t launch_pack(int n_streams, const void* const* src, const int64_t* offsets, int B,
                       int H, int D, int layout, int64_t ld, void* dst, hipStream_t stream);

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* vt, int B, int H, int N,
                           int D, int64_t ldv, float softmax_scale, void* o, float* lse,
                           hipStream_t stream);

// plan: the dispatch order of joint_attn_sparse_plan, or nullptr for the given order
hipError_t launch_fwd_bf16_sparse(const void* q, const void* k, const void* vt,
                                  const uint8_t* mask, int B, int H, int N, int D, int64_t ldv,
                                  float softmax_scale, void* o, float* lse, hipStream_t stream,
                                  const int32_t* plan = nullptr);
// units = B * H * nb query blocks of an nb x nb mask per (b, h)
hipError_t launch_sparse_plan(const uint8_t* mask, int units, int nb, int32_t* plan,
                              hipStream_t stream);

// split-KV planning: workgroups that run at once on the current device, and query rows
// per workgroup of the bf16 forward for head size D.  The launch takes the slot count the
// caller sized the workspace with, so that both use one answer of the device query.
int splitkv_slots(int D);
int splitkv_rows_per_tile(int D);
hipError_t launch_fwd_bf16_splitkv(const void* q, const void* k, const void* vt, int B, int H,
                                   int N, int D, int64_t ldv, float softmax_scale, int n_split,
                                   int slots, float* o_part, float* lse_part, void* o,
                                   float* lse, hipStream_t stream);

// the same with the partial results in the library's static per-device scratch array
// (parts = split tiles x key ranges, within JA_SCRATCH_BYTES; 0 runs the plain forward)
hipError_t launch_fwd_bf16_splitkv_noalloc(const void* q, const void* k, const void* vt, int B,
                                           int H, int N, int D, int64_t ldv, float softmax_scale,
                                           int n_split, int slots, int64_t parts, void* o,
                                           float* lse, hipStream_t stream);

hipError_t launch_fwd_bf16_streams(const StreamTable& st, int B, int H, int N, int D,
                                   float softmax_scale, void* o, float* lse,
                                   hipStream_t stream);

// split-KV over the streams: with vt == nullptr Q, K and V are all read in place (V
// transposed in LDS); otherwise Q and K are read in place and V^T from the packed copy
// vt (BHDN, pitch ldv).  o_part / lse_part as for launch_fwd_bf16_splitkv.
hipError_t launch_fwd_bf16_streams_splitkv(const StreamTable& st, const void* vt, int64_t ldv,
                                           int B, int H, int N, int D, float softmax_scale,
                                           int n_split, int slots, float* o_part,
                                           float* lse_part, void* o, float* lse,
                                           hipStream_t stream);

hipError_t launch_quant_fp8(const void* q, const void* k, const void* vt, int B, int H, int N,
                            int D, int64_t ldv, int mode, void* q8, void* k8, void* v8t,
                            float* q_scale, float* k_scale, float* v_scale, void* q_hi,
                            void* k_hi, int32_t* hi_idx, float* ch_amax, hipStream_t stream);

hipError_t launch_quant_fp8_streams(const StreamTable& st, int B, int H, int N, int D,
                                    int64_t ldv, int mode, void* q8, void* k8, void* v8t,
                                    float* q_scale, float* k_scale, float* v_scale, void* q_hi,
                                    void* k_hi, int32_t* hi_idx, float* ch_amax,
                                    hipStream_t stream);

hipError_t launch_quant_fp8_repair(const void* q, const void* k, const void* vt, int B, int H,
                                   int N, int D, int64_t ldv, int n_repair, void* q8, void* k8,
                                   void* v8t, float* q_scale, float* k_scale, float* v_scale,
                                   float* q_err, float* k_err, int32_t* q_sel, int32_t* k_sel,
                                   void* v8t_sel, hipStream_t stream);
hipError_t launch_fwd_fp8_repair(const void* q8, const void* k8, const void* v8t,
                                 const float* q_scale, const float* k_scale, const float* v_scale,
                                 const void* q, const void* k, const int32_t* q_sel,
                                 const int32_t* k_sel, const void* v8t_sel, int n_repair, int B,
                                 int H, int N, int D, int64_t ldv, float softmax_scale, void* o,
                                 float* lse, hipStream_t stream);
// fp8 split-KV planning and launch (as for the bf16 forward; 64-key tiles)
int fp8_splitkv_slots(int D, int mode);
int fp8_splitkv_rows_per_tile(int D);
hipError_t launch_fwd_fp8_splitkv(const void* q8, const void* k8, const void* v8t,
                                  const float* q_scale, const float* k_scale,
                                  const float* v_scale, int B, int H, int N, int D, int64_t ldv,
                                  float softmax_scale, int mode, const void* q_hi,
                                  const void* k_hi, int n_split, int slots, float* o_part,
                                  float* lse_part, void* o, float* lse, hipStream_t stream);
hipError_t launch_fwd_fp8(const void* q8, const void* k8, const void* v8t, const float* q_scale,
                          const float* k_scale, const float* v_scale, int B, int H, int N, int D,
                          int64_t ldv, float softmax_scale, int mode, const void* q_hi,
                          const void* k_hi, void* o, float* lse, hipStream_t stream);

}  // namespace ja
