// Token packing: concatenate text / target / reference streams along tokens.
//
// The streams are kept apart in the FLUX 3 Image Klein transformer and only meet in joint
// attention (VisualGen FLUX 3 article, everytik.com translation, section
// 使用 TensorRT LLM VisualGen 进行 FLUX 3 推理).  Both kernels are plain copies bound by HBM
// bandwidth: 16-byte loads and stores, each 256-byte (b, n, h) row moved by 16 lanes.
#include "ja_device.h"
#include "ja_launch.h"

namespace ja {

struct PackStreams {
    const uint16_t* src[JA_MAX_STREAMS];
    int64_t off[JA_MAX_STREAMS + 1];
    int n;
};

// Stream holding packed token n: the last stream whose start is <= n (zero-length
// streams share their start with the next stream and are skipped this way).
__device__ inline int stream_of(const PackStreams& s, int64_t n) {
    int r = 0;
    for (int i = 1; i < s.n; ++i)
        if (n >= s.off[i]) r = i;
    return r;
}

// BHND: one workgroup per packed token (b, n); copies its H*D elements to H rows.
template <int D>
__global__ __launch_bounds__(128) void pack_bhnd_kernel(PackStreams s, int H, int64_t N,
                                                        uint16_t* __restrict__ dst) {
    constexpr int CPR = D / 8;                       // 16-byte chunks per (token, head)
    const int64_t row = blockIdx.x;
    const int64_t b = row / N, n = row - b * N;
    const int st = stream_of(s, n);
    const int64_t L = s.off[st + 1] - s.off[st], t = n - s.off[st];
    const uint4* src = reinterpret_cast<const uint4*>(s.src[st] + (b * L + t) * H * D);
    for (int c = threadIdx.x; c < H * CPR; c += blockDim.x) {
        const int h = c / CPR, ch = c % CPR;
        const uint4 v = src[c];
        *reinterpret_cast<uint4*>(dst + ((b * H + h) * N + n) * D + ch * 8) = v;
    }
}

// BHDN: one workgroup per (64-token tile, h, b); transposes through LDS so that both
// the token-major reads and the channel-major writes are 16-byte vectors.  Columns
// N..ld-1 are written as zero.
template <int D>
__global__ __launch_bounds__(256) void pack_bhdn_kernel(PackStreams s, int H, int64_t N,
                                                        int64_t ld, uint16_t* __restrict__ dst) {
    constexpr int T = 64;
    constexpr int CPR = D / 8;
    constexpr int PITCH = D + 2;                     // odd word pitch: column reads hit distinct banks
    __shared__ uint16_t tile[T * PITCH];
    const int64_t n0 = (int64_t)blockIdx.x * T;
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;

    for (int c = threadIdx.x; c < T * CPR; c += blockDim.x) {
        const int r = c / CPR, ch = c % CPR;
        const int64_t n = n0 + r;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (n < N) {
            const int st = stream_of(s, n);
            const int64_t L = s.off[st + 1] - s.off[st], t = n - s.off[st];
            v = *reinterpret_cast<const uint4*>(s.src[st] + ((b * L + t) * H + h) * D + ch * 8);
        }
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            tile[r * PITCH + ch * 8 + 2 * e] = (uint16_t)(w[e] & 0xFFFF);
            tile[r * PITCH + ch * 8 + 2 * e + 1] = (uint16_t)(w[e] >> 16);
        }
    }
    __syncthreads();

    for (int c = threadIdx.x; c < D * (T / 8); c += blockDim.x) {
        const int ch = c / (T / 8), tg = c % (T / 8);
        const int64_t n = n0 + tg * 8;
        if (n >= ld) continue;                       // ld % 16 == 0, so n + 8 <= ld here
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = (uint32_t)tile[(tg * 8 + 2 * e) * PITCH + ch] |
                   ((uint32_t)tile[(tg * 8 + 2 * e + 1) * PITCH + ch] << 16);
        *reinterpret_cast<uint4*>(dst + ((b * H + h) * D + ch) * ld + n) =
            make_uint4(w[0], w[1], w[2], w[3]);
    }
}

template <int D>
static hipError_t launch_pack_d(const PackStreams& s, int B, int H, int64_t N, int layout,
                                int64_t ld, void* dst, hipStream_t stream) {
    if (layout == JA_LAYOUT_BHND) {
        hipLaunchKernelGGL(pack_bhnd_kernel<D>, dim3((unsigned)(B * N)), dim3(128), 0, stream,
                           s, H, N, static_cast<uint16_t*>(dst));
    } else {
        const unsigned tiles = (unsigned)((ld + 63) / 64);
        hipLaunchKernelGGL(pack_bhdn_kernel<D>, dim3(tiles, H, B), dim3(256), 0, stream,
                           s, H, N, ld, static_cast<uint16_t*>(dst));
    }
    return hipGetLastError();
}

hipError_t launch_pack(int n_streams, const void* const* src, const int64_t* offsets, int B,
                       int H, int D, int layout, int64_t ld, void* dst, hipStream_t stream) {
    PackStreams s{};
    s.n = n_streams;
    for (int i = 0; i < n_streams; ++i) s.src[i] = static_cast<const uint16_t*>(src[i]);
    for (int i = 0; i <= n_streams; ++i) s.off[i] = offsets[i];
    const int64_t N = offsets[n_streams];
    return D == 64 ? launch_pack_d<64>(s, B, H, N, layout, ld, dst, stream)
                   : launch_pack_d<128>(s, B, H, N, layout, ld, dst, stream);
}

}  // namespace ja
