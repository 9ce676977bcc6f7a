// Joint attention forward on fp8 (OCP E4M3) operands (gfx950).
//
// The fp8 attention variant of the VisualGen FLUX 3 article (everytik.com translation,
// section 量化注意力与稀疏注意力: fp8 Q/K and fp8 V), on the codes and scales that
// quant_fp8 produces.  Same work split and operand mapping as the bf16 kernel (S^T =
// K Q^T with one query per lane, O^T = V^T P^T with P^T taken from the score
// registers), on v_mfma_f32_32x32x64_f8f6f4 (both operands e4m3).
//
// Scales.  A workgroup's 128 query rows are exactly one Q scale block and a 64-key
// tile lies inside one K scale block, so scale * qs * ks * log2(e) is one factor per
// tile, applied in the same FMA that subtracts the running maximum.  The running
// maximum is kept as an integer (base 2), so every rescale of the accumulators is an
// exact power of two and P's e4m3 rounding does not depend on the order keys arrive
// in.  P is stored as e4m3(2^8 * p); the 2^8 is folded into the exponent and the row
// sum is taken over the same 2^8-scaled fp32 values, so it cancels in O = acc / l.
// The per-channel V scale is applied in the epilogue.
//
// Split mode (HI): the 16 kept channels of Q and K (bf16, already divided by their
// power-of-two block scales) add one v_mfma_f32_32x32x16_bf16 per 32x32 score block
// into the same accumulator, so t = (q8.k8 + q_hi.k_hi) * qs * ks * scale * log2 e.
#include "ja_device.h"
#include "ja_launch.h"

namespace ja {
namespace {

constexpr int BR = 128;          // query rows per workgroup (= one Q scale block)
constexpr int BC = 64;           // keys per tile (half a K scale block)
constexpr int NTHREADS = 256;
static_assert(BR == JA_QK_BLOCK && JA_QK_BLOCK % BC == 0, "scale blocks must align with tiles");

__device__ inline int swap_bits23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

template <int D, bool HI>
__global__ __launch_bounds__(NTHREADS, 2) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8, const uint8_t* __restrict__ V8T,
    const float* __restrict__ QS, const float* __restrict__ KS, const float* __restrict__ VS,
    const __bf16* __restrict__ QH, const __bf16* __restrict__ KH,
    int H, int N, int64_t ldv, float c2, __bf16* __restrict__ O, float* __restrict__ LSE,
    int n_qtiles, int total) {
    constexpr int KROWB = D;                 // bytes per K row
    constexpr int DC = D / 16;               // 16-byte chunks per K row
    constexpr int NQC = D / 64;              // k-steps of the QK product (64 channels each)
    constexpr int NOB = D / 32;              // 32-channel output blocks
    constexpr int KCH = BC * DC / NTHREADS;  // K staging chunks per thread
    constexpr int VCH = D * (BC / 16) / NTHREADS;
    static_assert(KCH >= 1 && VCH >= 1, "tile too small for the workgroup");
    __shared__ __attribute__((aligned(16))) uint8_t sk[BC * KROWB];
    __shared__ __attribute__((aligned(16))) uint8_t sv[D * BC];
    constexpr int HC = JA_HI_CHANNELS;           // kept channels (bf16), 2 x 16 bytes per key
    __shared__ __attribute__((aligned(16))) __bf16 skh[HI ? BC * HC : 8];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r32 = lane & 31, hh = lane >> 5;
    const int wg = xcd_remap(blockIdx.x, total);
    const int bh = wg / n_qtiles, qt = wg - bh * n_qtiles;
    const int b = bh / H, h = bh - b * H;
    const int nblk = (N + JA_QK_BLOCK - 1) / JA_QK_BLOCK;
    const uint8_t* Qbh = Q8 + (int64_t)bh * N * D;
    const uint8_t* Kbh = K8 + (int64_t)bh * N * D;
    const uint8_t* Vbh = V8T + (int64_t)bh * D * ldv;
    const float qscale_c2 = QS[(int64_t)bh * nblk + qt] * c2;

    const int q_row = qt * BR + w * 32 + r32;
    const int q_ld = min(q_row, N - 1);
    const __bf16* KHbh = HI ? KH + (int64_t)bh * N * HC : nullptr;
    bf16x8 qhf = {};
    if (HI) qhf = *reinterpret_cast<const bf16x8*>(QH + ((int64_t)bh * N + q_ld) * HC + 8 * hh);
    intx8 qf[NQC];
#pragma unroll
    for (int c = 0; c < NQC; ++c) {
        const uint4* p = reinterpret_cast<const uint4*>(Qbh + (int64_t)q_ld * D + 64 * c + 32 * hh);
        const uint4 x0 = p[0], x1 = p[1];
        qf[c] = intx8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                      (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    }

    floatx16 oacc[NOB];
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
        for (int a = 0; a < 16; ++a) oacc[ob][a] = 0.f;
    float m = -INFINITY, l = 0.f;

    const int nkt = (N + BC - 1) / BC;
    uint4 kreg[KCH], vreg[VCH], khreg = make_uint4(0, 0, 0, 0);

    auto load_tile = [&](int kt) {
        const int k0 = kt * BC;
        const bool full = k0 + BC <= N;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int idx = tid + i * NTHREADS, row = idx / DC, ch = idx % DC;
            const int key = k0 + row;
            kreg[i] = make_uint4(0, 0, 0, 0);
            if (full || key < N)
                kreg[i] = *reinterpret_cast<const uint4*>(Kbh + (int64_t)key * D + ch * 16);
        }
        if (HI && tid < BC * 2) {               // 2 chunks of 8 kept channels per key
            const int key = k0 + tid / 2;
            khreg = make_uint4(0, 0, 0, 0);
            if (full || key < N)
                khreg = *reinterpret_cast<const uint4*>(KHbh + (int64_t)key * HC + (tid % 2) * 8);
        }
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int idx = tid + i * NTHREADS, row = idx / (BC / 16), ch = idx % (BC / 16);
            const int key = k0 + ch * 16;
            vreg[i] = make_uint4(0, 0, 0, 0);
            if (full || key < N) {
                // key < N, key % 16 == 0 and ldv % 16 == 0 keep the 16 bytes in the row
                uint4 v = *reinterpret_cast<const uint4*>(Vbh + (int64_t)row * ldv + key);
                if (!full) {
                    uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        if (key + e >= N) wv[e / 4] &= ~(0xFFu << (8 * (e % 4)));
                    v = make_uint4(wv[0], wv[1], wv[2], wv[3]);
                }
                vreg[i] = v;
            }
        }
    };
    auto store_tile = [&]() {
        if (HI && tid < BC * 2) {
            const int row = tid / 2, half = (tid % 2) ^ ((row >> 3) & 1);
            *reinterpret_cast<uint4*>(&skh[row * HC + half * 8]) = khreg;
        }
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int idx = tid + i * NTHREADS, row = idx / DC, ch = idx % DC;
            *reinterpret_cast<uint4*>(&sk[row * KROWB + ((ch ^ (row % DC)) * 16)]) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            // 16 keys (16j .. 16j+15) of channel `row`, stored as two 8-byte units so that
            // lane half hh later finds its keys {16j + 8hh + e} as 8-byte unit 2j + hh
            const int idx = tid + i * NTHREADS, row = idx / (BC / 16), j = idx % (BC / 16);
            const uint4 v = vreg[i];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int unit = (2 * j + half) ^ (row % 8);
                *reinterpret_cast<uint2*>(&sv[row * BC + unit * 8]) =
                    half ? make_uint2(v.z, v.w) : make_uint2(v.x, v.y);
            }
        }
    };

    load_tile(0);
    for (int kt = 0; kt < nkt; ++kt) {
        store_tile();
        __syncthreads();
        if (kt + 1 < nkt) load_tile(kt + 1);

        floatx16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int a = 0; a < 16; ++a) s[kb][a] = 0.f;
            const int krow = kb * 32 + swap_bits23(r32);
#pragma unroll
            for (int c = 0; c < NQC; ++c) {
                const int u0 = 4 * c + 2 * hh;       // two 16-byte chunks: channels 64c+32hh..+31
                const uint4 x0 = *reinterpret_cast<const uint4*>(
                    &sk[krow * KROWB + ((u0 ^ (krow % DC)) * 16)]);
                const uint4 x1 = *reinterpret_cast<const uint4*>(
                    &sk[krow * KROWB + (((u0 + 1) ^ (krow % DC)) * 16)]);
                const intx8 av = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                                  (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
                s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    av, qf[c], s[kb], 0, 0, 0, 0, 0, 0);
            }
            if (HI) {
                const int half = hh ^ ((krow >> 3) & 1);
                const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&skh[krow * HC + half * 8]);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, qhf, s[kb], 0, 0, 0);
            }
        }

        const int k0 = kt * BC;
        if (k0 + BC > N) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int a = 0; a < 16; ++a) {
                    const int key = k0 + kb * 32 + 16 * (a / 8) + 8 * hh + (a % 8);
                    if (key >= N) s[kb][a] = -INFINITY;
                }
        }

        // base-2 logits t = s * f; integer running maximum
        const float f = qscale_c2 * KS[(int64_t)bh * nblk + (k0 / JA_QK_BLOCK)];
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int a = 0; a < 16; ++a) mx = fmaxf(mx, s[kb][a]);
        mx = wave_halves_max(mx);
        const float m_new = fmaxf(m, ceilf(mx * f));
        const float alpha = (m == -INFINITY) ? 0.f : ldexpf(1.f, (int)(m - m_new));
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
            for (int a = 0; a < 16; ++a) oacc[ob][a] *= alpha;

        // P^T as e4m3 of 2^8 * 2^(t - m), 32 bytes per lane: slot kb*16 + a
        const float bias = 8.f - m;
        intx8 pb;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                float p[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    p[e] = fast_exp2(fmaf(s[kb][4 * d + e], f, bias));
                    l += p[e];
                }
                int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
                word = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], word, true);
                pb[4 * kb + d] = word;
            }

        // O^T += V^T P^T; A-operand slot s of half hh holds key kb*32 + 16u + 8hh + e
        // for s = 16kb + 8u + e, i.e. the 8-byte units 2(2kb + u) + hh of the V^T row
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob) {
            const int vrow = ob * 32 + r32;
            intx8 av;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int unit = (2 * j + hh) ^ (vrow % 8);
                const uint2 x = *reinterpret_cast<const uint2*>(&sv[vrow * BC + unit * 8]);
                av[2 * j] = (int)x.x;
                av[2 * j + 1] = (int)x.y;
            }
            oacc[ob] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                av, pb, oacc[ob], 0, 0, 0, 0, 0, 0);
        }
        __syncthreads();
    }

    const float l_tot = wave_halves_sum(l);
    const float inv = 1.f / l_tot;
    if (q_row < N) {
        __bf16* orow = O + (((int64_t)b * N + q_row) * H + h) * D;
        const float* vs = VS + (int64_t)bh * D;
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c0 = ob * 32 + j * 8 + hh * 4;
                // v_scale is only 4-byte aligned by contract: four scalar loads
                floatx4 v = {oacc[ob][4 * j] * inv * vs[c0], oacc[ob][4 * j + 1] * inv * vs[c0 + 1],
                             oacc[ob][4 * j + 2] * inv * vs[c0 + 2],
                             oacc[ob][4 * j + 3] * inv * vs[c0 + 3]};
                *reinterpret_cast<bf16x4*>(orow + c0) = __builtin_convertvector(v, bf16x4);
            }
        if (LSE != nullptr && hh == 0)
            LSE[(int64_t)bh * N + q_row] = (m - 8.f + log2f(l_tot)) * kLn2;
    }
}

template <int D, bool HI>
hipError_t launch_d(const void* q8, const void* k8, const void* v8t, const float* qs,
                    const float* ks, const float* vs, const void* qh, const void* kh, int B,
                    int H, int N, int64_t ldv, float softmax_scale, void* o, float* lse,
                    hipStream_t stream) {
    const int n_qtiles = (N + BR - 1) / BR;
    const int total = n_qtiles * B * H;
    hipLaunchKernelGGL((fwd_fp8_kernel<D, HI>), dim3(total), dim3(NTHREADS), 0, stream,
                       static_cast<const uint8_t*>(q8), static_cast<const uint8_t*>(k8),
                       static_cast<const uint8_t*>(v8t), qs, ks, vs,
                       static_cast<const __bf16*>(qh), static_cast<const __bf16*>(kh), H, N, ldv,
                       softmax_scale * kLog2e, static_cast<__bf16*>(o), lse, n_qtiles, total);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const void* q8, const void* k8, const void* v8t, const float* q_scale,
                          const float* k_scale, const float* v_scale, int B, int H, int N, int D,
                          int64_t ldv, float softmax_scale, int mode, const void* q_hi,
                          const void* k_hi, void* o, float* lse, hipStream_t stream) {
    if (mode == JA_FP8_SPLIT)
        return D == 64 ? launch_d<64, true>(q8, k8, v8t, q_scale, k_scale, v_scale, q_hi, k_hi, B,
                                            H, N, ldv, softmax_scale, o, lse, stream)
                       : launch_d<128, true>(q8, k8, v8t, q_scale, k_scale, v_scale, q_hi, k_hi,
                                             B, H, N, ldv, softmax_scale, o, lse, stream);
    return D == 64 ? launch_d<64, false>(q8, k8, v8t, q_scale, k_scale, v_scale, nullptr, nullptr,
                                         B, H, N, ldv, softmax_scale, o, lse, stream)
                   : launch_d<128, false>(q8, k8, v8t, q_scale, k_scale, v_scale, nullptr, nullptr,
                                          B, H, N, ldv, softmax_scale, o, lse, stream);
}

}  // namespace ja
