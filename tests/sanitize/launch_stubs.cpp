// Host-only stand-ins for the kernel launchers of libjoint_attn, for building the C-ABI
// layer (joint_attn.cpp) under AddressSanitizer / UndefinedBehaviorSanitizer on a machine
// without a GPU.  Each stub reads every host-side array it is handed (so that an argument
// count the ABI layer got wrong shows up as an out-of-bounds read), checks the invariants
// the real launchers rely on, and returns hipSuccess without touching device memory.
// A broken invariant returns hipErrorInvalidValue, which the ABI reports as JA_EHIP.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ja_launch.h"

namespace ja {
namespace {

volatile int64_t g_sink = 0;

hipError_t shape_ok(int B, int H, int N, int D) {
    return (B > 0 && H > 0 && N > 0 && (D == 64 || D == 128)) ? hipSuccess
                                                              : hipErrorInvalidValue;
}

hipError_t table_ok(const StreamTable& st, int N) {
    if (st.n < 1 || st.n > JA_MAX_STREAMS || st.off[0] != 0 || st.off[st.n] != N)
        return hipErrorInvalidValue;
    for (int s = 0; s < st.n; ++s) {
        if (st.off[s + 1] < st.off[s]) return hipErrorInvalidValue;
        if (st.off[s + 1] > st.off[s] && (!st.q[s] || !st.k[s] || !st.v[s]))
            return hipErrorInvalidValue;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_pack(int n_streams, const void* const* src, const int64_t* offsets, int B,
                       int H, int D, int layout, int64_t ld, void* dst, hipStream_t) {
    int64_t acc = 0;
    for (int s = 0; s < n_streams; ++s) acc += reinterpret_cast<uintptr_t>(src[s]) & 1;
    for (int s = 0; s <= n_streams; ++s) acc += offsets[s];
    g_sink = acc;
    if (offsets[0] != 0 || !dst || B <= 0 || H <= 0 || (D != 64 && D != 128)) return hipErrorInvalidValue;
    if (layout == JA_LAYOUT_BHDN && (ld < offsets[n_streams] || ld % 16 != 0))
        return hipErrorInvalidValue;
    return hipSuccess;
}

hipError_t launch_fwd_bf16(const void*, const void*, const void*, int B, int H, int N, int D,
                           int64_t ldv, float, void*, float*, hipStream_t) {
    return ldv >= N ? shape_ok(B, H, N, D) : hipErrorInvalidValue;
}

hipError_t launch_fwd_bf16_sparse(const void*, const void*, const void*, const uint8_t* mask,
                                  int B, int H, int N, int D, int64_t ldv, float, void*, float*,
                                  hipStream_t, const int32_t* plan) {
    if (!mask || N > JA_SPARSE_MAX_N || ldv < N) return hipErrorInvalidValue;
    if (plan && (int64_t)B * H * ((N + JA_SPARSE_BLOCK - 1) / JA_SPARSE_BLOCK) > JA_SPARSE_PLAN_MAX)
        return hipErrorInvalidValue;
    return shape_ok(B, H, N, D);
}

hipError_t launch_sparse_plan(const uint8_t* mask, int units, int nb, int32_t* plan, hipStream_t) {
    if (!mask || !plan || units <= 0 || units > JA_SPARSE_PLAN_MAX || nb <= 0 ||
        nb > JA_SPARSE_MAX_N / JA_SPARSE_BLOCK || units % nb != 0)
        return hipErrorInvalidValue;
    return hipSuccess;
}

// what the library reports without a GPU: 256 compute units, one workgroup each
int splitkv_slots(int) { return 256; }
int splitkv_rows_per_tile(int D) { return D == 64 ? 128 : 256; }

hipError_t launch_fwd_bf16_splitkv(const void*, const void*, const void*, int B, int H, int N,
                                   int D, int64_t ldv, float, int n_split, int slots,
                                   float* o_part, float* lse_part, void*, float*, hipStream_t) {
    if (n_split < 1 || slots != splitkv_slots(D) || !o_part || !lse_part || ldv < N)
        return hipErrorInvalidValue;
    return shape_ok(B, H, N, D);
}

hipError_t launch_fwd_bf16_splitkv_noalloc(const void*, const void*, const void*, int B, int H,
                                           int N, int D, int64_t ldv, float, int n_split,
                                           int slots, int64_t parts, void*, float*, hipStream_t) {
    const int64_t bytes = parts * splitkv_rows_per_tile(D) * (D + 1) * (int64_t)sizeof(float);
    if (n_split < 1 || slots != splitkv_slots(D) || parts < 0 || bytes > JA_SCRATCH_BYTES ||
        ldv < N)
        return hipErrorInvalidValue;
    return shape_ok(B, H, N, D);
}

hipError_t launch_fwd_bf16_streams(const StreamTable& st, int B, int H, int N, int D, float,
                                   void* o, float*, hipStream_t) {
    if (!o) return hipErrorInvalidValue;
    const hipError_t e = table_ok(st, N);
    return e != hipSuccess ? e : shape_ok(B, H, N, D);
}

hipError_t launch_fwd_bf16_streams_splitkv(const StreamTable& st, const void* vt, int64_t ldv,
                                           int B, int H, int N, int D, float, int n_split,
                                           int slots, float* o_part, float* lse_part, void* o,
                                           float*, hipStream_t) {
    if (!o || n_split < 1 || slots != splitkv_slots(D) || !o_part || !lse_part ||
        (vt && ldv < N))
        return hipErrorInvalidValue;
    const hipError_t e = table_ok(st, N);
    return e != hipSuccess ? e : shape_ok(B, H, N, D);
}

hipError_t launch_quant_fp8(const void*, const void*, const void*, int B, int H, int N, int D,
                            int64_t ldv, int mode, void*, void*, void*, float*, float*, float*,
                            void* q_hi, void* k_hi, int32_t* hi_idx, float* ch_amax,
                            hipStream_t) {
    if (ldv < N || (mode == JA_FP8_SPLIT && (!q_hi || !k_hi || !hi_idx || !ch_amax)))
        return hipErrorInvalidValue;
    return shape_ok(B, H, N, D);
}

hipError_t launch_quant_fp8_streams(const StreamTable& st, int B, int H, int N, int D,
                                    int64_t ldv, int mode, void*, void*, void*, float*, float*,
                                    float*, void* q_hi, void* k_hi, int32_t* hi_idx,
                                    float* ch_amax, hipStream_t) {
    if (ldv < N || (mode == JA_FP8_SPLIT && (!q_hi || !k_hi || !hi_idx || !ch_amax)))
        return hipErrorInvalidValue;
    const hipError_t e = table_ok(st, N);
    return e != hipSuccess ? e : shape_ok(B, H, N, D);
}

hipError_t launch_quant_fp8_repair(const void*, const void*, const void*, int B, int H, int N,
                                   int D, int64_t ldv, int n_repair, void*, void*, void*, float*,
                                   float*, float*, float* q_err, float* k_err, int32_t* q_sel,
                                   int32_t* k_sel, void* v8t_sel, hipStream_t) {
    if (ldv < N || n_repair < 0 || n_repair > N || !q_err || !k_err ||
        (n_repair > 0 && (!q_sel || !k_sel || !v8t_sel)))
        return hipErrorInvalidValue;
    return shape_ok(B, H, N, D);
}

hipError_t launch_fwd_fp8_repair(const void*, const void*, const void*, const float*,
                                 const float*, const float*, const void* q, const void* k,
                                 const int32_t* q_sel, const int32_t* k_sel, const void* v8t_sel,
                                 int n_repair, int B, int H, int N, int D, int64_t ldv, float,
                                 void*, float* lse, hipStream_t) {
    if (!q || !k || !lse || ldv < N || N > JA_REPAIR_MAX_N ||
        (n_repair > 0 && (!q_sel || !k_sel || !v8t_sel)))
        return hipErrorInvalidValue;
    return shape_ok(B, H, N, D);
}

int fp8_splitkv_slots(int, int) { return 256; }
int fp8_splitkv_rows_per_tile(int D) { return D == 64 ? 128 : 256; }

hipError_t launch_fwd_fp8_splitkv(const void*, const void*, const void*, const float*,
                                  const float*, const float*, int B, int H, int N, int D,
                                  int64_t ldv, float, int mode, const void* q_hi,
                                  const void* k_hi, int n_split, int slots, float* o_part,
                                  float* lse_part, void*, float*, hipStream_t) {
    if (n_split < 1 || slots != fp8_splitkv_slots(D, mode) || !o_part || !lse_part || ldv < N ||
        (mode == JA_FP8_SPLIT && (!q_hi || !k_hi)))
        return hipErrorInvalidValue;
    return shape_ok(B, H, N, D);
}

hipError_t launch_fwd_fp8(const void*, const void*, const void*, const float*, const float*,
                          const float*, int B, int H, int N, int D, int64_t ldv, float, int mode,
                          const void* q_hi, const void* k_hi, void*, float*, hipStream_t) {
    if (ldv < N || (mode == JA_FP8_SPLIT && (!q_hi || !k_hi))) return hipErrorInvalidValue;
    return shape_ok(B, H, N, D);
}

}  // namespace ja
