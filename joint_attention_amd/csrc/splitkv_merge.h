// split-KV merge, shared by the bf16 and fp8 forwards (included inside their anonymous
// namespaces).  The forwards' PARTIAL variants run the query tiles n_full .. of the
// last, partial round of workgroups as n_split key ranges each, and write per range the
// normalised fp32 output and natural-log lse of its keys: OP [part][BR][D], LP [part][BR],
// part = (tile - n_full) * n_split + range.
#pragma once

#include "ja_device.h"

namespace ja {
namespace {

// split-KV merge -- grid ((n_units - n_full) * BR / RPB), 256 threads: RPB rows x (D / 4)
// channel quads of one split query tile.  O = sum_s w_s O_s / sum_s w_s,
// w_s = exp(lse_s - max lse), lse = max + ln sum_s w_s (the log-sum-exp rule for attention
// over a union of key sets).
template <int D, int BR>
__global__ __launch_bounds__(256) void splitkv_merge_kernel(const float* __restrict__ OP,
                                                           const float* __restrict__ LP,
                                                           int n_split, int n_full, int n_qtiles,
                                                           int H, int N, __bf16* __restrict__ O,
                                                           float* __restrict__ LSE) {
    constexpr int TPR = D / 4;                    // threads per row
    constexpr int RPB = 256 / TPR;                // rows per block
    constexpr int BPU = BR / RPB;                 // blocks per query tile
    const int ut = blockIdx.x / BPU;              // split tile index, 0 ..
    const int unit = n_full + ut;
    const int bh = unit / n_qtiles, qt = unit - bh * n_qtiles, b = bh / H, h = bh - b * H;
    const int r = (blockIdx.x - ut * BPU) * RPB + threadIdx.x / TPR, c = (threadIdx.x % TPR) * 4;
    const int row = qt * BR + r;
    if (row >= N) return;
    const int64_t base = (int64_t)ut * n_split * BR + r;   // part (ut, 0), row r
    float mx = -INFINITY;
    for (int s = 0; s < n_split; ++s) mx = fmaxf(mx, LP[base + (int64_t)s * BR]);
    float den = 0.f;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < n_split; ++s) {
        const int64_t pr = base + (int64_t)s * BR;
        const float wgt = expf(LP[pr] - mx);
        const floatx4 o = *reinterpret_cast<const floatx4*>(OP + pr * D + c);
        den += wgt;
        acc += o * wgt;
    }
    const float inv = 1.f / den;
    *reinterpret_cast<bf16x4*>(O + (((int64_t)b * N + row) * H + h) * D + c) =
        __builtin_convertvector(acc * inv, bf16x4);
    if (LSE != nullptr && c == 0) LSE[(int64_t)bh * N + row] = mx + logf(den);
}

}  // namespace
}  // namespace ja
