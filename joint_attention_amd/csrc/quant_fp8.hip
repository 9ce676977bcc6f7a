// fp8 (OCP E4M3) quantisation of packed Q, K and V with dequantisation scales.
//
// The VisualGen FLUX 3 article (everytik.com translation, section 量化注意力与稀疏注意力)
// runs attention with fp8 Q/K and V; the block-wise scale factors follow the
// kongchang.com English page (section "Reducing Numerical Precision").  Granularity:
// Q and K one scale per (b, h, 128 packed tokens), V one scale per (b, h, channel).
//
// Both kernels are bound by HBM bandwidth.  One workgroup owns one scale segment, which
// is contiguous in memory in the layouts used here (a 128-token block of a BHND tensor
// is 128 * D consecutive elements; a V channel is one BHDN row): pass 1 takes the
// absolute maximum, pass 2 re-reads the segment (now in L2) and writes the codes.
//
// Codes are bit-exact: scale = amax / 448 and inv = 448 / amax are correctly rounded
// binary32 quotients, y = x * inv is one binary32 product, and y is clamped to +-448 and
// rounded to e4m3 (nearest, ties to even) by the integer encoder below, written from
// the OCP E4M3 definition.
#include "ja_device.h"
#include "ja_launch.h"

namespace ja {
namespace {

constexpr int NT = 256;

// binary32 (finite) -> e4m3 code, round to nearest even, saturating at +-448.
__device__ inline uint32_t e4m3_from_f32(float y) {
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fminf(fabsf(y), 448.0f);
    uint32_t code;
    if (a >= 0.015625f) {                              // normal range, >= 2^-6
        const uint32_t u = __float_as_uint(a);
        // keep 3 of the 23 mantissa bits, ties to even; a carry bumps the exponent
        const uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;
        code = r - ((127u - 7u) << 3);                 // rebias the exponent 127 -> 7
    } else {                                           // subnormal: multiples of 2^-9
        code = (uint32_t)rintf(a * 512.0f);            // exact product, ties to even
    }
    return code | sign;
}

__device__ inline void bf16x2_to_f32(uint32_t w, float& lo, float& hi) {
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xFFFF0000u);
}

__device__ inline float block_max(float v, float* red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) r = fmaxf(r, red[i]);
    return r;
}

__device__ inline void scale_pair(float amax, float& scale, float& inv) {
    if (amax == 0.f) {
        scale = 1.f;
        inv = 1.f;
    } else {
        scale = __fdiv_rn(amax, 448.0f);
        inv = __fdiv_rn(448.0f, amax);
    }
}

// 8 bf16 (one uint4) -> 8 e4m3 codes (one uint2)
__device__ inline uint2 quant8(uint4 v, float inv) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[2] = {0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float lo, hi;
        bf16x2_to_f32(w[e], lo, hi);
        const uint32_t c = e4m3_from_f32(lo * inv) | (e4m3_from_f32(hi * inv) << 8);
        out[e / 2] |= c << (16 * (e % 2));
    }
    return make_uint2(out[0], out[1]);
}

__device__ inline float amax8(uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float lo, hi;
        bf16x2_to_f32(w[e], lo, hi);
        m = fmaxf(m, fmaxf(fabsf(lo), fabsf(hi)));
    }
    return m;
}

// grid: (n_blocks, B*H, 2) -- z selects Q (0) or K (1)
__global__ __launch_bounds__(NT) void quant_qk_kernel(const uint16_t* __restrict__ q,
                                                     const uint16_t* __restrict__ k, int N, int D,
                                                     uint8_t* __restrict__ q8,
                                                     uint8_t* __restrict__ k8,
                                                     float* __restrict__ qs,
                                                     float* __restrict__ ks, int nblk) {
    __shared__ float red[NT / 64];
    const uint16_t* x = blockIdx.z ? k : q;
    uint8_t* y = blockIdx.z ? k8 : q8;
    float* sc = blockIdx.z ? ks : qs;
    const int blk = blockIdx.x, bh = blockIdx.y;
    const int t0 = blk * JA_QK_BLOCK;
    const int rows = min(JA_QK_BLOCK, N - t0);
    const int64_t base = ((int64_t)bh * N + t0) * D;
    const int nch = rows * D / 8;                       // 16-byte input chunks in the segment
    const uint4* src = reinterpret_cast<const uint4*>(x + base);

    float m = 0.f;
    for (int c = threadIdx.x; c < nch; c += NT) m = fmaxf(m, amax8(src[c]));
    const float amax = block_max(m, red);
    float scale, inv;
    scale_pair(amax, scale, inv);
    if (threadIdx.x == 0) sc[(int64_t)bh * nblk + blk] = scale;

    uint2* dst = reinterpret_cast<uint2*>(y + base);
    for (int c = threadIdx.x; c < nch; c += NT) dst[c] = quant8(src[c], inv);
}

// grid: (D, B*H) -- one V^T row (b, h, channel) per workgroup
__global__ __launch_bounds__(NT) void quant_v_kernel(const uint16_t* __restrict__ vt, int N,
                                                    int D, int64_t ldv,
                                                    uint8_t* __restrict__ v8t,
                                                    float* __restrict__ vs) {
    __shared__ float red[NT / 64];
    const int c = blockIdx.x, bh = blockIdx.y;
    const int64_t base = ((int64_t)bh * D + c) * ldv;
    const uint4* src = reinterpret_cast<const uint4*>(vt + base);
    const int nfull = N / 8;                           // chunks entirely inside [0, N)
    const int rem = N - nfull * 8;
    const int nch = (int)(ldv / 8);                    // chunks in the padded row

    float m = 0.f;
    for (int i = threadIdx.x; i < nfull; i += NT) m = fmaxf(m, amax8(src[i]));
    if (rem && threadIdx.x == 0) {
        const uint4 v = src[nfull];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        for (int e = 0; e < rem; ++e) {
            const uint32_t bits = (e & 1) ? (w[e / 2] >> 16) : (w[e / 2] & 0xFFFFu);
            m = fmaxf(m, fabsf(__uint_as_float(bits << 16)));
        }
    }
    const float amax = block_max(m, red);
    float scale, inv;
    scale_pair(amax, scale, inv);
    if (threadIdx.x == 0) vs[(int64_t)bh * D + c] = scale;

    uint2* dst = reinterpret_cast<uint2*>(v8t + base);
    for (int i = threadIdx.x; i < nch; i += NT) {
        if (i < nfull) {
            dst[i] = quant8(src[i], inv);
        } else if (i == nfull && rem) {
            uint4 v = src[i];
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
            for (int e = 0; e < 4; ++e) {             // zero the elements at or past N
                if (2 * e >= rem) w[e] = 0;
                else if (2 * e + 1 >= rem) w[e] &= 0xFFFFu;
            }
            uint2 cde = quant8(make_uint4(w[0], w[1], w[2], w[3]), inv);
            // a zero input encodes as code 0 (positive zero), as padding must be
            dst[i] = cde;
        } else {
            dst[i] = make_uint2(0, 0);
        }
    }
}

}  // namespace

hipError_t launch_quant_fp8(const void* q, const void* k, const void* vt, int B, int H, int N,
                            int D, int64_t ldv, void* q8, void* k8, void* v8t, float* q_scale,
                            float* k_scale, float* v_scale, hipStream_t stream) {
    const int nblk = (N + JA_QK_BLOCK - 1) / JA_QK_BLOCK;
    hipLaunchKernelGGL(quant_qk_kernel, dim3(nblk, B * H, 2), dim3(NT), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), N, D,
                       static_cast<uint8_t*>(q8), static_cast<uint8_t*>(k8), q_scale, k_scale,
                       nblk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(quant_v_kernel, dim3(D, B * H), dim3(NT), 0, stream,
                       static_cast<const uint16_t*>(vt), N, D, ldv, static_cast<uint8_t*>(v8t),
                       v_scale);
    return hipGetLastError();
}

}  // namespace ja
