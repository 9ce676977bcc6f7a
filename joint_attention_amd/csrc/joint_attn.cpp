// C-ABI entry points of libjoint_attn: argument validation, then kernel launches.
// Declarations and the contract of every call are in include/joint_attn.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>

#include "joint_attn.h"
#include "ja_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxInt = 2147483647;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool head_size_ok(int D) { return D == 64 || D == 128; }

int hip_status(hipError_t e) {
    if (e == hipSuccess) return JA_OK;
    g_last_hip_error = static_cast<int>(e);
    return JA_EHIP;
}

// Test hook for the launch-failure path: with JOINT_ATTN_SIMULATE_HIP_ERROR set to a
// positive hipError_t code, every call that passes validation reports that code as a
// launch failure (JA_EHIP) without enqueuing anything.
hipError_t simulated_hip_error() {
    const char* s = std::getenv("JOINT_ATTN_SIMULATE_HIP_ERROR");
    if (s == nullptr || *s == '\0') return hipSuccess;
    const long v = std::strtol(s, nullptr, 10);
    return v > 0 && v < 100000 ? static_cast<hipError_t>(v) : hipSuccess;
}

#define JA_LAUNCH(expr)                                        \
    do {                                                        \
        const hipError_t sim_ = simulated_hip_error();          \
        return hip_status(sim_ != hipSuccess ? sim_ : (expr));  \
    } while (0)

// Shared checks of the attention-shaped calls: sizes, pitch, and that every launch
// dimension and 32-bit in-kernel index stays in range.
int check_shape(int B, int H, int64_t N, int D, int64_t ldv) {
    if (B <= 0 || H <= 0 || N < 0 || D <= 0) return JA_EINVAL;
    if (!head_size_ok(D)) return JA_EUNSUPPORTED;
    if (N > kMaxInt / 2 || ldv < N || ldv % 16 != 0) return JA_EINVAL;
    if ((int64_t)D * ldv > JA_MAX_HEAD_ELEMS) return JA_EINVAL;   // 32-bit V^T offsets
    if ((int64_t)B * H > 65535) return JA_EINVAL;
    const int64_t qtiles = (N + 63) / 64;             // finest query tiling any kernel uses
    if (qtiles * B * H > kMaxInt) return JA_EINVAL;
    if ((int64_t)B * H * D * ldv > ((int64_t)1 << 46)) return JA_EINVAL;   // element counts
    return JA_OK;
}

// The stream table of the *_streams calls: lengths, non-NULL and 16-byte aligned
// pointers for every non-empty stream, offsets.
int stream_table(int n_streams, const void* const* q, const void* const* k,
                 const void* const* v, const int64_t* lens, ja::StreamTable& st) {
    if (n_streams <= 0 || !q || !k || !v || !lens) return JA_EINVAL;
    if (n_streams > JA_MAX_STREAMS) return JA_EUNSUPPORTED;
    st.n = n_streams;
    st.off[0] = 0;
    for (int s = 0; s < n_streams; ++s) {
        if (lens[s] < 0 || lens[s] > kMaxInt) return JA_EINVAL;
        if (lens[s] > 0) {
            if (!q[s] || !k[s] || !v[s]) return JA_EINVAL;
            if (!aligned16(q[s]) || !aligned16(k[s]) || !aligned16(v[s])) return JA_EUNSUPPORTED;
            st.q[s] = q[s];
            st.k[s] = k[s];
            st.v[s] = v[s];
        }
        st.off[s + 1] = st.off[s] + lens[s];
    }
    return JA_OK;
}

// Output checks of the fp8 quantiser (shared by the packed and the streams call).
int check_quant_outputs(int mode, const void* q8, const void* k8, const void* v8t,
                        const float* q_scale, const float* k_scale, const float* v_scale,
                        const void* q_hi, const void* k_hi, const int32_t* hi_idx,
                        const float* ch_amax) {
    if (!q8 || !k8 || !v8t || !q_scale || !k_scale || !v_scale) return JA_EINVAL;
    if (mode == JA_FP8_SPLIT && (!q_hi || !k_hi || !hi_idx || !ch_amax)) return JA_EINVAL;
    if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8t)) return JA_EUNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(q_scale) | reinterpret_cast<uintptr_t>(k_scale) |
         reinterpret_cast<uintptr_t>(v_scale)) & 3u)
        return JA_EUNSUPPORTED;
    if (mode == JA_FP8_SPLIT &&
        ((reinterpret_cast<uintptr_t>(q_hi) | reinterpret_cast<uintptr_t>(k_hi)) & 15u ||
         (reinterpret_cast<uintptr_t>(hi_idx) | reinterpret_cast<uintptr_t>(ch_amax)) & 3u))
        return JA_EUNSUPPORTED;
    return JA_OK;
}

}  // namespace

extern "C" {

const char* joint_attn_strerror(int status) {
    switch (status) {
        case JA_OK: return "ok";
        case JA_EINVAL: return "invalid argument";
        case JA_EUNSUPPORTED: return "unsupported argument (head size, alignment, stream count or mode)";
        case JA_EHIP: return "HIP runtime error";
        case JA_ESCRATCH:
            return "partial results larger than the static scratch buffer (JA_SCRATCH_BYTES); "
                   "use joint_attn_fwd_bf16_splitkv with a workspace, or a smaller n_split";
        default: return "unknown status";
    }
}

int joint_attn_last_hip_error(void) { return g_last_hip_error; }

int64_t joint_attn_vt_ld(int64_t N) { return N <= 0 ? 0 : (N + 15) / 16 * 16; }

int joint_attn_pack(int n_streams, const void* const* src, const int64_t* lens, int B, int H,
                    int D, int layout, int64_t ld, void* dst, int64_t* offsets, void* stream) {
    if (n_streams <= 0 || !src || !lens || !offsets) return JA_EINVAL;
    if (n_streams > JA_MAX_STREAMS) return JA_EUNSUPPORTED;
    if (B <= 0 || H <= 0 || D <= 0) return JA_EINVAL;
    if (!head_size_ok(D)) return JA_EUNSUPPORTED;
    if (layout != JA_LAYOUT_BHND && layout != JA_LAYOUT_BHDN) return JA_EINVAL;
    int64_t off[JA_MAX_STREAMS + 1];
    off[0] = 0;
    for (int s = 0; s < n_streams; ++s) {
        if (lens[s] < 0 || lens[s] > kMaxInt) return JA_EINVAL;
        if (lens[s] > 0 && !src[s]) return JA_EINVAL;
        if (lens[s] > 0 && !aligned16(src[s])) return JA_EUNSUPPORTED;
        off[s + 1] = off[s] + lens[s];
    }
    const int64_t N = off[n_streams];
    if (N > kMaxInt / 2 || (int64_t)B * N > kMaxInt || (int64_t)B * H > 65535) return JA_EINVAL;
    if (layout == JA_LAYOUT_BHDN && (ld < N || ld % 16 != 0)) return JA_EINVAL;
    const int64_t cols = layout == JA_LAYOUT_BHDN ? ld : N;
    if (cols > 0 && !dst) return JA_EINVAL;
    if (cols > 0 && !aligned16(dst)) return JA_EUNSUPPORTED;
    for (int s = 0; s <= n_streams; ++s) offsets[s] = off[s];
    if (cols == 0) return JA_OK;
    JA_LAUNCH(ja::launch_pack(n_streams, src, off, B, H, D, layout, ld, dst,
                              static_cast<hipStream_t>(stream)));
}

int joint_attn_fwd_bf16(const void* q, const void* k, const void* vt, int B, int H, int64_t N,
                        int D, int64_t ldv, float softmax_scale, void* o, float* lse,
                        void* stream) {
    const int st = check_shape(B, H, N, D, ldv);
    if (st != JA_OK) return st;
    if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return JA_EINVAL;
    if (N == 0) return JA_OK;
    if (!q || !k || !vt || !o) return JA_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned16(o)) return JA_EUNSUPPORTED;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return JA_EUNSUPPORTED;
    JA_LAUNCH(ja::launch_fwd_bf16(q, k, vt, B, H, (int)N, D, ldv, softmax_scale, o, lse,
                                  static_cast<hipStream_t>(stream)));
}

int joint_attn_fwd_bf16_sparse(const void* q, const void* k, const void* vt, int B, int H,
                               int64_t N, int D, int64_t ldv, const uint8_t* block_mask,
                               float softmax_scale, void* o, float* lse, void* stream) {
    const int st = check_shape(B, H, N, D, ldv);
    if (st != JA_OK) return st;
    if (N > JA_SPARSE_MAX_N) return JA_EUNSUPPORTED;
    if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return JA_EINVAL;
    if (N == 0) return JA_OK;
    if (!q || !k || !vt || !o || !block_mask) return JA_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned16(o)) return JA_EUNSUPPORTED;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return JA_EUNSUPPORTED;
    JA_LAUNCH(ja::launch_fwd_bf16_sparse(q, k, vt, block_mask, B, H, (int)N, D, ldv,
                                         softmax_scale, o, lse,
                                         static_cast<hipStream_t>(stream)));
}

int64_t joint_attn_sparse_plan_bytes(int B, int H, int64_t N) {
    if (B <= 0 || H <= 0 || N < 0 || N > JA_SPARSE_MAX_N) return -1;
    const int64_t units = (int64_t)B * H * ((N + JA_SPARSE_BLOCK - 1) / JA_SPARSE_BLOCK);
    if (units > JA_SPARSE_PLAN_MAX) return -1;
    return units * (int64_t)sizeof(int32_t);
}

int joint_attn_sparse_plan(const uint8_t* block_mask, int B, int H, int64_t N, int32_t* plan,
                           int64_t plan_bytes, void* stream) {
    if (B <= 0 || H <= 0 || N < 0) return JA_EINVAL;
    if (N > JA_SPARSE_MAX_N) return JA_EUNSUPPORTED;
    const int64_t nb = (N + JA_SPARSE_BLOCK - 1) / JA_SPARSE_BLOCK;
    const int64_t units = (int64_t)B * H * nb;
    if (units > JA_SPARSE_PLAN_MAX) return JA_EUNSUPPORTED;
    if (N == 0) return JA_OK;
    if (!block_mask || !plan) return JA_EINVAL;
    if (plan_bytes < units * (int64_t)sizeof(int32_t)) return JA_EINVAL;
    if (reinterpret_cast<uintptr_t>(plan) & 3u) return JA_EUNSUPPORTED;
    JA_LAUNCH(ja::launch_sparse_plan(block_mask, (int)units, (int)nb, plan,
                                     static_cast<hipStream_t>(stream)));
}

int joint_attn_fwd_bf16_sparse_planned(const void* q, const void* k, const void* vt, int B,
                                       int H, int64_t N, int D, int64_t ldv,
                                       const uint8_t* block_mask, const int32_t* plan,
                                       float softmax_scale, void* o, float* lse, void* stream) {
    const int st = check_shape(B, H, N, D, ldv);
    if (st != JA_OK) return st;
    if (N > JA_SPARSE_MAX_N) return JA_EUNSUPPORTED;
    if ((int64_t)B * H * ((N + JA_SPARSE_BLOCK - 1) / JA_SPARSE_BLOCK) > JA_SPARSE_PLAN_MAX)
        return JA_EUNSUPPORTED;
    if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return JA_EINVAL;
    if (N == 0) return JA_OK;
    if (!q || !k || !vt || !o || !block_mask || !plan) return JA_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned16(o)) return JA_EUNSUPPORTED;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return JA_EUNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(plan) & 3u) return JA_EUNSUPPORTED;
    JA_LAUNCH(ja::launch_fwd_bf16_sparse(q, k, vt, block_mask, B, H, (int)N, D, ldv,
                                         softmax_scale, o, lse,
                                         static_cast<hipStream_t>(stream), plan));
}

int64_t joint_attn_fwd_bf16_splitkv_workspace(int B, int H, int64_t N, int D, int n_split) {
    if (B <= 0 || H <= 0 || N < 0 || D <= 0 || n_split <= 0 || !head_size_ok(D)) return -1;
    // only the query tiles of the last, partial round are split: fewer than the slots
    // (workgroups running at once on the current device) and than all tiles
    const int64_t br = ja::splitkv_rows_per_tile(D);
    const int64_t units = (N + br - 1) / br * B * H;
    const int64_t split_tiles = std::min<int64_t>(units, ja::splitkv_slots(D));
    return (int64_t)n_split * split_tiles * br * (D + 1) * (int64_t)sizeof(float);
}

int joint_attn_fwd_bf16_splitkv_suggest(int B, int H, int64_t N, int D) {
    if (B <= 0 || H <= 0 || N <= 0 || !head_size_ok(D)) return 1;
    const int64_t br = ja::splitkv_rows_per_tile(D);
    const int64_t units = (N + br - 1) / br * B * H;
    const int64_t slots = ja::splitkv_slots(D);
    const int64_t tail = units % slots;                 // query tiles of the last round
    if (tail == 0) return 1;
    const int64_t tiles = (N + 31) / 32;
    // In units of one round of full-length workgroups: the tail unsplit costs 1; split s
    // ways it takes ceil(tail * s / slots) rounds of 1/s length, plus about 6 key tiles of
    // fixed cost per workgroup (prologue, epilogue), plus reading its fp32 partials back
    // in the merge (at ~4 TB/s, against a round of ~1 PFLOP/s work; their writes overlap
    // the forward).  A split
    // is suggested only where it should save over a twentieth of a round (measured on 9
    // shapes from 1024^2 T2I to 2048^2 I2I and head-split shares of 2048^2: at this
    // threshold the pick is the fastest split measured or within 0.7 % of it; at a tenth, a
    // grid of one partial round, 198 tiles, kept the plain forward, 17 % slower than 5 ranges).
    const double round_s = (double)slots * br * tiles * 32.0 * 4.0 * D / 1.0e15;
    double best = 0.95;
    int best_s = 1;
    for (int s = 2; s <= 16 && s <= tiles; ++s) {
        const double rounds = (double)((tail * s + slots - 1) / slots);
        const double merge = (double)tail * s * br * (D + 1) * 4.0 / 4.0e12 / round_s;
        const double cost = rounds * (1.0 / s + 6.0 / (double)tiles) + merge;
        if (cost < best - 1e-9) {
            best = cost;
            best_s = s;
        }
    }
    return best_s;
}

int joint_attn_fwd_bf16_splitkv(const void* q, const void* k, const void* vt, int B, int H,
                                int64_t N, int D, int64_t ldv, float softmax_scale, int n_split,
                                void* workspace, int64_t workspace_bytes, void* o, float* lse,
                                void* stream) {
    const int st = check_shape(B, H, N, D, ldv);
    if (st != JA_OK) return st;
    if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return JA_EINVAL;
    if (n_split <= 0 || n_split > 64) return JA_EINVAL;
    if (N == 0) return JA_OK;
    if (!q || !k || !vt || !o || !workspace) return JA_EINVAL;
    // one device query sizes the workspace check, the partial layout and the launch
    const int slots = ja::splitkv_slots(D);
    const int64_t br = ja::splitkv_rows_per_tile(D);
    const int64_t split_tiles = std::min<int64_t>((N + br - 1) / br * B * H, slots);
    if (workspace_bytes < (int64_t)n_split * split_tiles * br * (D + 1) * (int64_t)sizeof(float))
        return JA_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned16(o) ||
        !aligned16(workspace))
        return JA_EUNSUPPORTED;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return JA_EUNSUPPORTED;
    float* o_part = static_cast<float*>(workspace);
    float* lse_part = o_part + (int64_t)n_split * split_tiles * br * D;
    JA_LAUNCH(ja::launch_fwd_bf16_splitkv(q, k, vt, B, H, (int)N, D, ldv, softmax_scale,
                                          n_split, slots, o_part, lse_part, o, lse,
                                          static_cast<hipStream_t>(stream)));
}

int joint_attn_fwd_bf16_splitkv_noalloc(const void* q, const void* k, const void* vt, int B,
                                        int H, int64_t N, int D, int64_t ldv,
                                        float softmax_scale, int n_split, void* o, float* lse,
                                        void* stream) {
    const int st = check_shape(B, H, N, D, ldv);
    if (st != JA_OK) return st;
    if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return JA_EINVAL;
    if (n_split <= 0 || n_split > 64) return JA_EINVAL;
    if (N == 0) return JA_OK;
    if (!q || !k || !vt || !o) return JA_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned16(o))
        return JA_EUNSUPPORTED;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return JA_EUNSUPPORTED;
    // the split tiles are those of the last, partial round (as in the workspace variant);
    // each of their key ranges needs rows * (D + 1) floats of scratch
    const int slots = ja::splitkv_slots(D);
    const int64_t br = ja::splitkv_rows_per_tile(D);
    const int64_t ranges = std::min<int64_t>(n_split, (N + 31) / 32);
    const int64_t tail = (N + br - 1) / br * B * H % slots;
    const int64_t parts = (ranges <= 1 || tail == 0) ? 0 : tail * ranges;
    if (parts * br * (D + 1) * (int64_t)sizeof(float) > JA_SCRATCH_BYTES) return JA_ESCRATCH;
    JA_LAUNCH(ja::launch_fwd_bf16_splitkv_noalloc(q, k, vt, B, H, (int)N, D, ldv, softmax_scale,
                                                  n_split, slots, parts, o, lse,
                                                  static_cast<hipStream_t>(stream)));
}

int joint_attn_fwd_bf16_streams(int n_streams, const void* const* q, const void* const* k,
                                const void* const* v, const int64_t* lens, int B, int H, int D,
                                float softmax_scale, void* o, float* lse, int64_t* offsets,
                                void* stream) {
    ja::StreamTable st{};
    const int tst = stream_table(n_streams, q, k, v, lens, st);
    if (tst != JA_OK) return tst;
    const int64_t N = st.off[n_streams];
    const int sh = check_shape(B, H, N, D, joint_attn_vt_ld(N));
    if (sh != JA_OK) return sh;
    if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return JA_EINVAL;
    if (offsets)
        for (int s = 0; s <= n_streams; ++s) offsets[s] = st.off[s];
    if (N == 0) return JA_OK;
    if (!o) return JA_EINVAL;
    if (!aligned16(o)) return JA_EUNSUPPORTED;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return JA_EUNSUPPORTED;
    JA_LAUNCH(ja::launch_fwd_bf16_streams(st, B, H, (int)N, D, softmax_scale, o, lse,
                                          static_cast<hipStream_t>(stream)));
}

namespace {
// bytes of the packed V^T copy at the head of the streams split-KV workspace (256-aligned)
int64_t streams_vt_bytes(int B, int H, int64_t N, int D) {
    return ((int64_t)B * H * D * joint_attn_vt_ld(N) * 2 + 255) / 256 * 256;
}
}  // namespace

int64_t joint_attn_fwd_bf16_streams_splitkv_workspace(int B, int H, int64_t N, int D,
                                                      int n_split, int pack_v) {
    if (pack_v != 0 && pack_v != 1) return -1;
    const int64_t part = joint_attn_fwd_bf16_splitkv_workspace(B, H, N, D, n_split);
    if (part < 0) return -1;
    return part + (pack_v ? streams_vt_bytes(B, H, N, D) : 0);
}

int joint_attn_fwd_bf16_streams_splitkv(int n_streams, const void* const* q,
                                        const void* const* k, const void* const* v,
                                        const int64_t* lens, int B, int H, int D,
                                        float softmax_scale, int n_split, int pack_v,
                                        void* workspace, int64_t workspace_bytes, void* o,
                                        float* lse, int64_t* offsets, void* stream) {
    ja::StreamTable st{};
    const int tst = stream_table(n_streams, q, k, v, lens, st);
    if (tst != JA_OK) return tst;
    const int64_t N = st.off[n_streams];
    const int64_t ldv = joint_attn_vt_ld(N);
    const int sh = check_shape(B, H, N, D, ldv);
    if (sh != JA_OK) return sh;
    if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return JA_EINVAL;
    if (n_split <= 0 || n_split > 64 || (pack_v != 0 && pack_v != 1)) return JA_EINVAL;
    if (offsets)
        for (int s = 0; s <= n_streams; ++s) offsets[s] = st.off[s];
    if (N == 0) return JA_OK;
    if (!o || !workspace) return JA_EINVAL;
    // one device query sizes the workspace check, the partial layout and the launch
    const int slots = ja::splitkv_slots(D);
    const int64_t br = ja::splitkv_rows_per_tile(D);
    const int64_t split_tiles = std::min<int64_t>((N + br - 1) / br * B * H, slots);
    const int64_t vt_bytes = pack_v ? streams_vt_bytes(B, H, N, D) : 0;
    const int64_t part_floats = (int64_t)n_split * split_tiles * br * (D + 1);
    if (workspace_bytes < vt_bytes + part_floats * (int64_t)sizeof(float)) return JA_EINVAL;
    if (!aligned16(o) || !aligned16(workspace)) return JA_EUNSUPPORTED;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return JA_EUNSUPPORTED;
    char* ws = static_cast<char*>(workspace);
    void* vt = pack_v ? ws : nullptr;
    float* o_part = reinterpret_cast<float*>(ws + vt_bytes);
    float* lse_part = o_part + (int64_t)n_split * split_tiles * br * D;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    const hipError_t sim = simulated_hip_error();       // (test hook: nothing is launched)
    if (sim != hipSuccess) return hip_status(sim);
    if (pack_v) {
        const hipError_t e = ja::launch_pack(n_streams, v, st.off, B, H, D, JA_LAYOUT_BHDN, ldv,
                                             vt, hs);
        if (e != hipSuccess) return hip_status(e);
    }
    return hip_status(ja::launch_fwd_bf16_streams_splitkv(st, vt, ldv, B, H, (int)N, D,
                                                          softmax_scale, n_split, slots, o_part,
                                                          lse_part, o, lse, hs));
}

int joint_attn_quant_fp8(const void* q, const void* k, const void* vt, int B, int H, int64_t N,
                         int D, int64_t ldv, int mode, void* q8, void* k8, void* v8t,
                         float* q_scale, float* k_scale, float* v_scale, void* q_hi, void* k_hi,
                         int32_t* hi_idx, float* ch_amax, void* stream) {
    const int st = check_shape(B, H, N, D, ldv);
    if (st != JA_OK) return st;
    if (mode != JA_FP8_PLAIN && mode != JA_FP8_SPLIT) return JA_EUNSUPPORTED;
    if (N == 0) return JA_OK;
    if (!q || !k || !vt) return JA_EINVAL;
    const int ost = check_quant_outputs(mode, q8, k8, v8t, q_scale, k_scale, v_scale, q_hi, k_hi,
                                        hi_idx, ch_amax);
    if (ost != JA_OK) return ost;
    if (!aligned16(q) || !aligned16(k) || !aligned16(vt)) return JA_EUNSUPPORTED;
    JA_LAUNCH(ja::launch_quant_fp8(q, k, vt, B, H, (int)N, D, ldv, mode, q8, k8, v8t,
                                   q_scale, k_scale, v_scale, q_hi, k_hi, hi_idx,
                                   ch_amax, static_cast<hipStream_t>(stream)));
}

int joint_attn_quant_fp8_streams(int n_streams, const void* const* q, const void* const* k,
                                 const void* const* v, const int64_t* lens, int B, int H, int D,
                                 int64_t ldv, int mode, void* q8, void* k8, void* v8t,
                                 float* q_scale, float* k_scale, float* v_scale, void* q_hi,
                                 void* k_hi, int32_t* hi_idx, float* ch_amax, int64_t* offsets,
                                 void* stream) {
    ja::StreamTable st{};
    const int tst = stream_table(n_streams, q, k, v, lens, st);
    if (tst != JA_OK) return tst;
    const int64_t N = st.off[n_streams];
    const int sh = check_shape(B, H, N, D, ldv);
    if (sh != JA_OK) return sh;
    if (mode != JA_FP8_PLAIN && mode != JA_FP8_SPLIT) return JA_EUNSUPPORTED;
    if (offsets)
        for (int s = 0; s <= n_streams; ++s) offsets[s] = st.off[s];
    if (N == 0) return JA_OK;
    const int ost = check_quant_outputs(mode, q8, k8, v8t, q_scale, k_scale, v_scale, q_hi, k_hi,
                                        hi_idx, ch_amax);
    if (ost != JA_OK) return ost;
    JA_LAUNCH(ja::launch_quant_fp8_streams(st, B, H, (int)N, D, ldv, mode, q8, k8, v8t,
                                           q_scale, k_scale, v_scale, q_hi, k_hi, hi_idx,
                                           ch_amax, static_cast<hipStream_t>(stream)));
}

int joint_attn_fwd_fp8(const void* q8, const void* k8, const void* v8t, const float* q_scale,
                       const float* k_scale, const float* v_scale, int B, int H, int64_t N, int D,
                       int64_t ldv, float softmax_scale, int mode, const void* q_hi,
                       const void* k_hi, void* o, float* lse, void* stream) {
    const int st = check_shape(B, H, N, D, ldv);
    if (st != JA_OK) return st;
    if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return JA_EINVAL;
    if (mode != JA_FP8_PLAIN && mode != JA_FP8_SPLIT) return JA_EUNSUPPORTED;
    if (N == 0) return JA_OK;
    if (!q8 || !k8 || !v8t || !q_scale || !k_scale || !v_scale || !o) return JA_EINVAL;
    if (mode == JA_FP8_SPLIT && (!q_hi || !k_hi)) return JA_EINVAL;
    if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8t) || !aligned16(o))
        return JA_EUNSUPPORTED;
    if (mode == JA_FP8_SPLIT && (!aligned16(q_hi) || !aligned16(k_hi))) return JA_EUNSUPPORTED;
    if (((reinterpret_cast<uintptr_t>(q_scale) | reinterpret_cast<uintptr_t>(k_scale) |
          reinterpret_cast<uintptr_t>(v_scale)) & 3u) ||
        (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
        return JA_EUNSUPPORTED;
    JA_LAUNCH(ja::launch_fwd_fp8(q8, k8, v8t, q_scale, k_scale, v_scale, B, H, (int)N, D,
                                 ldv, softmax_scale, mode, q_hi, k_hi, o, lse,
                                 static_cast<hipStream_t>(stream)));
}

int64_t joint_attn_fwd_fp8_splitkv_workspace(int B, int H, int64_t N, int D, int n_split) {
    if (B <= 0 || H <= 0 || N < 0 || n_split <= 0 || !head_size_ok(D)) return -1;
    // only the query tiles of the last, partial round are split: fewer than the slots of
    // either mode's kernel on the current device, and than all tiles
    const int64_t br = ja::fp8_splitkv_rows_per_tile(D);
    const int64_t units = (N + br - 1) / br * B * H;
    const int64_t slots = std::max(ja::fp8_splitkv_slots(D, JA_FP8_PLAIN),
                                   ja::fp8_splitkv_slots(D, JA_FP8_SPLIT));
    return (int64_t)n_split * std::min(units, slots) * br * (D + 1) * (int64_t)sizeof(float);
}

int joint_attn_fwd_fp8_splitkv_suggest(int B, int H, int64_t N, int D, int mode) {
    if (B <= 0 || H <= 0 || N <= 0 || !head_size_ok(D) ||
        (mode != JA_FP8_PLAIN && mode != JA_FP8_SPLIT))
        return 1;
    const int64_t br = ja::fp8_splitkv_rows_per_tile(D);
    const int64_t units = (N + br - 1) / br * B * H;
    const int64_t slots = ja::fp8_splitkv_slots(D, mode);
    const int64_t tail = units % slots;
    if (tail == 0) return 1;
    const int64_t tiles = (N + 63) / 64;
    // the bf16 model (one round of full-length workgroups = 1; about 6 key tiles of fixed
    // cost per workgroup; the merge reading the partials at ~4 TB/s) with 64-key tiles
    // and ~1.7 PFLOP/s rounds
    const double round_s = (double)slots * br * tiles * 64.0 * 4.0 * D / 1.7e15;
    double best = 0.9;
    int best_s = 1;
    for (int s = 2; s <= 16 && s <= tiles; ++s) {
        const double rounds = (double)((tail * s + slots - 1) / slots);
        const double merge = (double)tail * s * br * (D + 1) * 4.0 / 4.0e12 / round_s;
        const double cost = rounds * (1.0 / s + 6.0 / (double)tiles) + merge;
        if (cost < best - 1e-9) {
            best = cost;
            best_s = s;
        }
    }
    return best_s;
}

int joint_attn_fwd_fp8_splitkv(const void* q8, const void* k8, const void* v8t,
                               const float* q_scale, const float* k_scale, const float* v_scale,
                               int B, int H, int64_t N, int D, int64_t ldv, float softmax_scale,
                               int mode, const void* q_hi, const void* k_hi, int n_split,
                               void* workspace, int64_t workspace_bytes, void* o, float* lse,
                               void* stream) {
    const int st = check_shape(B, H, N, D, ldv);
    if (st != JA_OK) return st;
    if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return JA_EINVAL;
    if (mode != JA_FP8_PLAIN && mode != JA_FP8_SPLIT) return JA_EUNSUPPORTED;
    if (n_split <= 0 || n_split > 64) return JA_EINVAL;
    if (N == 0) return JA_OK;
    if (!q8 || !k8 || !v8t || !q_scale || !k_scale || !v_scale || !o || !workspace)
        return JA_EINVAL;
    if (mode == JA_FP8_SPLIT && (!q_hi || !k_hi)) return JA_EINVAL;
    // one device query per mode: the launch's slots never exceed the ones the partial
    // layout and the workspace check are sized with (their maximum over both modes)
    const int slots = ja::fp8_splitkv_slots(D, mode);
    const int64_t br = ja::fp8_splitkv_rows_per_tile(D);
    const int64_t slots_ws = std::max<int64_t>(
        slots, ja::fp8_splitkv_slots(D, mode == JA_FP8_PLAIN ? JA_FP8_SPLIT : JA_FP8_PLAIN));
    const int64_t split_tiles = std::min<int64_t>((N + br - 1) / br * B * H, slots_ws);
    if (workspace_bytes < (int64_t)n_split * split_tiles * br * (D + 1) * (int64_t)sizeof(float))
        return JA_EINVAL;
    if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8t) || !aligned16(o) ||
        !aligned16(workspace))
        return JA_EUNSUPPORTED;
    if (mode == JA_FP8_SPLIT && (!aligned16(q_hi) || !aligned16(k_hi))) return JA_EUNSUPPORTED;
    if (((reinterpret_cast<uintptr_t>(q_scale) | reinterpret_cast<uintptr_t>(k_scale) |
          reinterpret_cast<uintptr_t>(v_scale)) & 3u) ||
        (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
        return JA_EUNSUPPORTED;
    float* o_part = static_cast<float*>(workspace);
    float* lse_part = o_part + (int64_t)n_split * split_tiles * br * D;
    JA_LAUNCH(ja::launch_fwd_fp8_splitkv(q8, k8, v8t, q_scale, k_scale, v_scale, B, H,
                                         (int)N, D, ldv, softmax_scale, mode, q_hi, k_hi,
                                         n_split, slots, o_part, lse_part, o, lse,
                                         static_cast<hipStream_t>(stream)));
}

int64_t joint_attn_repair_count(int64_t N, double rho) {
    if (N < 0 || !(rho >= 0.0 && rho <= 1.0)) return -1;
    const double x = std::ceil(rho * (double)N);
    return x > (double)N ? N : (int64_t)x;
}

static bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int joint_attn_quant_fp8_repair(const void* q, const void* k, const void* vt, int B, int H,
                                int64_t N, int D, int64_t ldv, int64_t n_repair, void* q8,
                                void* k8, void* v8t, float* q_scale, float* k_scale,
                                float* v_scale, float* q_err, float* k_err, int32_t* q_sel,
                                int32_t* k_sel, void* v8t_sel, void* stream) {
    const int st = check_shape(B, H, N, D, ldv);
    if (st != JA_OK) return st;
    if (n_repair < 0 || n_repair > N) return JA_EINVAL;
    if (N == 0) return JA_OK;
    if (!q || !k || !vt) return JA_EINVAL;
    const int ost = check_quant_outputs(JA_FP8_PLAIN, q8, k8, v8t, q_scale, k_scale, v_scale,
                                        nullptr, nullptr, nullptr, nullptr);
    if (ost != JA_OK) return ost;
    if (!q_err || !k_err || (n_repair > 0 && (!q_sel || !k_sel || !v8t_sel))) return JA_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(vt)) return JA_EUNSUPPORTED;
    if (!aligned4(q_err) || !aligned4(k_err) || (n_repair > 0 && (!aligned4(q_sel) ||
                                                                   !aligned4(k_sel))))
        return JA_EUNSUPPORTED;
    JA_LAUNCH(ja::launch_quant_fp8_repair(q, k, vt, B, H, (int)N, D, ldv, (int)n_repair,
                                          q8, k8, v8t, q_scale, k_scale, v_scale, q_err,
                                          k_err, q_sel, k_sel, v8t_sel,
                                          static_cast<hipStream_t>(stream)));
}

int joint_attn_fwd_fp8_repair(const void* q8, const void* k8, const void* v8t,
                              const float* q_scale, const float* k_scale, const float* v_scale,
                              const void* q, const void* k, const int32_t* q_sel,
                              const int32_t* k_sel, const void* v8t_sel, int64_t n_repair, int B,
                              int H, int64_t N, int D, int64_t ldv, float softmax_scale, void* o,
                              float* lse, void* stream) {
    const int st = check_shape(B, H, N, D, ldv);
    if (st != JA_OK) return st;
    if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return JA_EINVAL;
    if (n_repair < 0 || n_repair > N) return JA_EINVAL;
    if (N == 0) return JA_OK;
    if (N > JA_REPAIR_MAX_N) return JA_EUNSUPPORTED;
    if (!q8 || !k8 || !v8t || !q_scale || !k_scale || !v_scale || !o || !q || !k || !lse)
        return JA_EINVAL;
    if (n_repair > 0 && (!q_sel || !k_sel || !v8t_sel)) return JA_EINVAL;
    if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8t) || !aligned16(o) || !aligned16(q) ||
        !aligned16(k))
        return JA_EUNSUPPORTED;
    if (!aligned4(q_scale) || !aligned4(k_scale) || !aligned4(v_scale) ||
        !aligned4(lse) || (n_repair > 0 && (!aligned4(q_sel) || !aligned4(k_sel) ||
                                            !aligned16(v8t_sel))))
        return JA_EUNSUPPORTED;
    JA_LAUNCH(ja::launch_fwd_fp8_repair(q8, k8, v8t, q_scale, k_scale, v_scale, q, k,
                                        q_sel, k_sel, v8t_sel, (int)n_repair, B, H, (int)N, D,
                                        ldv, softmax_scale, o, lse,
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"
